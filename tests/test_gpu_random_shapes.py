"""GPU parity of p3d_proj_cond over a seeded sweep of shapes, against the CPU
oracle: the combinations the fixed cases do not enumerate.

Each case draws (from one fixed seed) the dtype, one map or two, channel
counts (ragged K tails; map 0 a multiple of 64 when there are two), map
sizes, feature width D (not a multiple of 512, up to three 512-wide tiles),
bias or none, cell centres or grid nodes, and a token count picked so that
the launch runs as 32-token parts only, as whole tiles only, or as whole
tiles plus parts; a further set draws 65 to 128 tiles past a full round, so
that the leftover tiles run as 64-token parts. A bf16 launch of fewer whole
tiles than compute units that fits one round of 96-token tiles runs as
those ("round96"). Each case is named by the regime its tile count takes on
256 compute units. Null rows range from none
to several 128-row blocks per tile. Bar as in the other fused tests: masks bit-exact, null rows equal to
the bias bit for bit, token rows within 2e-2 (bf16) / 1e-5 (fp32), and
every checked row written (the output starts as NaN).
"""
import os
import sys

import numpy as np
import pytest

import oracle
import p3d_synth as synth
import pixel_aligned_image_amd as p3d
from parity_util import run_fused

pytestmark = pytest.mark.gpu

CUS = 256          # the tile-count regimes below assume the MI355X's compute units


def say(*a):
    print("[random shapes]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def orc():
    o = oracle.get()
    o.set_threads(min(16, os.cpu_count() or 1))
    return o


def _draw(i):
    rng = np.random.default_rng(9000 + i)
    bf16 = i % 5 != 4
    two = bf16 and rng.random() < 0.4
    D = int(rng.integers(1, 138)) * 8                       # 8 .. 1096
    n_tiles = -(-D // 512)
    regime = ("parts", "whole", "mixed")[i % 3]
    if regime == "parts":
        T = int(rng.integers(1, 65 // n_tiles + 1)) * n_tiles if n_tiles <= 64 else n_tiles
        T = max(n_tiles, min(T, 64 - 64 % n_tiles))
    elif regime == "whole":
        T = int(rng.integers(66 // n_tiles + 1, 200 // n_tiles + 1)) * n_tiles
    else:
        D, n_tiles = int(rng.integers(1, 64)) * 8, 1            # keep the oracle quick
        T = CUS + int(rng.integers(1, 65))
    m_tiles = T // n_tiles
    n = (m_tiles - 1) * 128 + int(rng.integers(1, 129))
    if two:
        maps = [(int(rng.integers(2, 33)), int(rng.integers(2, 33)), 64 * int(rng.integers(1, 3))),
                (int(rng.integers(2, 49)), int(rng.integers(2, 49)), 8 * int(rng.integers(1, 17)))]
    else:
        c = 8 * int(rng.integers(1, 33)) if bf16 else 4 * int(rng.integers(1, 65))
        maps = [(int(rng.integers(2, 65)), int(rng.integers(2, 65)), c)]
    null_choice = rng.integers(0, 4)
    n_null = [0, int(rng.integers(1, 300)), n, int(2.5 * n) + 3][null_choice]
    B = int(rng.integers(1, 4))
    R = int(max(8, np.ceil((n / B) ** (1 / 3))) + rng.integers(0, 16))
    return dict(i=i, bf16=bf16, maps=maps, D=D, n=n, B=B, R=R, n_null=n_null,
                bias=bool(rng.random() < 0.6), regime=regime, T=T,
                points="grid_nodes" if rng.random() < 0.3 else "cell_centres")


def _draw_half(i):
    """Whole tiles plus 65 to 128 leftover tiles, or 65 to 128 tiles alone."""
    c = _draw(i)
    rng = np.random.default_rng(9500 + i)
    D = int(rng.integers(1, 64)) * 8
    T = (CUS if i % 2 else 0) + int(rng.integers(65, 129))
    n = (T - 1) * 128 + int(rng.integers(1, 129))
    c.update(i=i, D=D, T=T, n=n, n_null=[0, int(rng.integers(1, 300)), n][i % 3],
             R=int(max(8, np.ceil((n / c["B"]) ** (1 / 3))) + rng.integers(0, 16)))
    return c


def _regime(c):
    """How a launch of T tiles (of 128 tokens) runs on CUS compute units, by
    the library's tiling rule (p3d_proj_cond_plan; the fp32 path has no
    parts or 96-token tiles, so its cases are named by the same counts)."""
    plan = p3d.p3d_proj_cond_plan(c["n"], c["D"], CUS)
    if plan["tile_rows"] != 128:
        return "round96" if c["bf16"] else "whole"
    tail = {32: "quarters", 64: "halves"}.get(plan["part_rows"], "")
    return "+".join(x for x in (["whole"] if plan["whole_tiles"] else []) + ([tail] if tail else []))


CASES = ([_draw(i) for i in range(40)] + [_draw_half(i) for i in range(40, 52)] +
         [_draw(i) for i in range(1000, 1040)])


@pytest.mark.parametrize("case", CASES, ids=["%d_%s_T%d" % (c["i"], _regime(c), c["T"])
                                              for c in CASES])
def test_proj_cond_random_shape(orc, case):
    say(case)
    rng = np.random.default_rng(7000 + case["i"])
    B, n, R = case["B"], case["n"], case["R"]
    coords = synth.random_coords(R, B, n, seed=n + case["i"])
    maps = [rng.standard_normal((B, h, w, c)).astype(np.float32) for h, w, c in case["maps"]]
    K = sum(c for _, _, c in case["maps"])
    Wf = (rng.standard_normal((case["D"], K)) * 0.05).astype(np.float32)
    bf = (rng.standard_normal(case["D"]) * 0.05).astype(np.float32) if case["bias"] else None
    if case["bf16"]:
        maps = [synth.bf16_bits(m) for m in maps]
        Wf = synth.bf16_bits(Wf)
        bf = synth.bf16_bits(bf) if bf is not None else None
    nn = case["n_null"]
    if n * case["D"] <= 4_000_000:
        rows = np.arange(n + nn)
    else:
        # tile edges, the last 64 tiles' tokens (the parts of a mixed launch)
        # and a sample of the rest; null rows: the first and last blocks and
        # a sample
        edge = np.concatenate([np.arange(0, n, 128), np.arange(127, n, 128),
                               np.arange(0, n, 96), np.arange(95, n, 96),
                               np.arange(max(0, n - 64 * 128), n)])
        pick = rng.choice(n, size=min(n, 3000), replace=False)
        nulls = np.concatenate([np.arange(n, min(n + 256, n + nn)),
                                np.arange(max(n, n + nn - 256), n + nn),
                                n + rng.choice(nn, size=min(nn, 512), replace=False)]) \
            if nn else np.zeros(0, np.int64)
        rows = np.unique(np.concatenate([edge, pick, nulls]).astype(np.int64))
    fovs = [30.0 + 7.0 * b for b in range(B)]
    st = run_fused(p3d, orc, coords, n, R, fovs, [None] * B, maps, Wf, bf, nn, case["bf16"],
                   rows, case["points"], case["maps"][0][1])
    if st is not None:
        say("  rows %d  max|diff|/max|Y| %.3e corr %.8f" % (len(rows), st[0], st[1]))
