"""GPU parity of p3d_projection_stats over a seeded sweep of shapes, against
the CPU oracle.

Each case draws (from one fixed seed) the dtype, one map or two (equal
channel counts, so the cosine is taken, or unequal), channel counts that
leave a ragged share for the 16 lanes of a token's row, map sizes, cell
centres or grid nodes, batch and resolution, and a token count from 1 to
about 40000 (ragged quads of 4, ragged 64-token projection groups, and more
than one group per wave). Bar as in the fixed diagnostics tests: counts
exact, sums within one bf16 rounding (2^-8) / 1e-5 of sum |S|, the cosine
count exact and its mean within 1e-3 / 1e-6.
"""
import os
import sys

import numpy as np
import pytest

import oracle
import p3d_synth as synth
import pixel_aligned_image_amd as p3d
from parity_util import run_stats

pytestmark = pytest.mark.gpu


def say(*a):
    print("[random stats]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def orc():
    o = oracle.get()
    o.set_threads(min(16, os.cpu_count() or 1))
    return o


def _draw(i):
    rng = np.random.default_rng(5100 + i)
    bf16 = i % 4 != 3
    step = 8 if bf16 else 4
    n = [1, 3, 4, 5, 63, 65, 129][i] if i < 7 else int(rng.integers(6, 40000))
    kind = ("one", "cosine", "unequal")[i % 3]
    c0 = step * int(rng.integers(1, 41))
    if kind == "one":
        chans = [c0]
    elif kind == "cosine":
        chans = [c0, c0]
    else:
        chans = [c0, c0 + step * int(rng.integers(1, 9))]
    maps = [(int(rng.integers(2, 64)), int(rng.integers(2, 64)), c) for c in chans]
    B = int(rng.integers(1, 4))
    R = int(max(4, np.ceil((n / B) ** (1 / 3))) + rng.integers(0, 24))
    return dict(i=i, bf16=bf16, n=n, maps=maps, B=B, R=R, kind=kind,
                points="grid_nodes" if rng.random() < 0.3 else "cell_centres",
                spill=int(rng.integers(0, 3)))


CASES = [_draw(i) for i in range(24)]


@pytest.mark.parametrize("case", CASES, ids=["%d_%s_n%d" % (c["i"], c["kind"], c["n"])
                                              for c in CASES])
def test_stats_random_shape(orc, case):
    say(case)
    rng = np.random.default_rng(6100 + case["i"])
    B, n = case["B"], case["n"]
    coords = synth.random_coords(case["R"], B, n, seed=n + 31 * case["i"], spill=case["spill"])
    maps = [rng.standard_normal((B, h, w, c)).astype(np.float32) + 0.2 * k
            for k, (h, w, c) in enumerate(case["maps"])]
    if case["bf16"]:
        maps = [synth.bf16_bits(m) for m in maps]
    got, want = run_stats(p3d, orc, coords, n, case["R"], [35.0 + 6 * b for b in range(B)],
                          [None] * B, maps, case["bf16"], case["points"], case["maps"][0][1])
    say("  coverage %d/%d cos_count %d" % (got["inside"], got["tokens"], got["cos_count"]))
