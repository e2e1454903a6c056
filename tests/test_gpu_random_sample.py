"""GPU parity of p3d_bilinear_sample over a seeded sweep of shapes, against
the CPU oracle.

Each case draws (from one fixed seed) the dtype mode (f32 -> f32,
bf16 -> f32, bf16 -> bf16), the batch, map sizes from 1 x 1 up to a few
hundred pixels a side, a channel count that leaves a ragged share of the
last 1 KB channel slice, and a point count from 1 to about 60000 (ragged
16-point tiles). The points mix uniform draws over and past the image,
exact pixel centres and edges, and non-finite values; with more than one
batch item the indices include out-of-range ones. Bar as in the fixed
sampling tests: every value within 1e-5 of sum_k w_k |F_k|, plus one bf16
rounding for bf16 output.
"""
import os
import sys

import numpy as np
import pytest

import oracle
import p3d_synth as synth
import pixel_aligned_image_amd as p3d
from parity_util import run_sample

pytestmark = pytest.mark.gpu


def say(*a):
    print("[random sample]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def orc():
    o = oracle.get()
    o.set_threads(min(16, os.cpu_count() or 1))
    return o


def _draw(i):
    rng = np.random.default_rng(8100 + i)
    mode = ("f32>f32", "bf16>f32", "bf16>bf16")[i % 3]
    step = 4 if mode == "f32>f32" else 8
    C = step * int(rng.integers(1, 2049 // step + 1)) if i % 4 else step * int(rng.integers(1, 9))
    B = int(rng.integers(1, 4))
    H = [1, 2, 3][i] if i < 3 else int(rng.integers(1, 320))
    W = [1, 3, 2][i] if i < 3 else int(rng.integers(1, 320))
    n = [1, 15, 17, 16][i - 3] if 3 <= i < 7 else int(rng.integers(2, 60000))
    n = max(1, min(n, 16_000_000 // C))                     # keep the oracle quick
    while B * H * W * C > 50_000_000:                         # and the host maps small
        H, W = max(1, H // 2), max(1, W // 2)
    return dict(i=i, mode=mode, B=B, H=H, W=W, C=C, n=n)


CASES = [_draw(i) for i in range(24)]


@pytest.mark.parametrize("case", CASES, ids=["%d_%s_%dx%dx%dx%d_n%d" % (
    c["i"], c["mode"].replace(">", "to"), c["B"], c["H"], c["W"], c["C"], c["n"]) for c in CASES])
def test_bilinear_sample_random_shape(orc, case):
    say(case)
    rng = np.random.default_rng(9100 + case["i"])
    B, H, W, C, n = case["B"], case["H"], case["W"], case["C"], case["n"]
    bf16_in = case["mode"].startswith("bf16")
    featf = rng.standard_normal((B, H, W, C)).astype(np.float32)
    feat = synth.bf16_bits(featf) if bf16_in else featf
    pts = rng.uniform(-1.2, 1.2, size=(n, 2))
    # a share of exact pixel centres (x = (2j + 1) / W - 1) and edges (+-1)
    k = n // 4
    if k:
        pts[:k, 0] = (2 * rng.integers(0, W, size=k) + 1) / W - 1
        pts[:k, 1] = (2 * rng.integers(0, H, size=k) + 1) / H - 1
        pts[k:k + k // 4, :] = rng.choice([-1.0, 1.0], size=(k // 4, 2))
    special = np.array([np.nan, np.inf, -np.inf, 5.0, -5.0])
    m = min(n, 5)
    pts[n - m:, 0] = special[:m]
    grid = pts.astype(np.float32)
    bidx = rng.integers(-1, B + 1, size=n).astype(np.int32) if B > 1 else None
    st = run_sample(p3d, orc, feat, grid, bidx, bf16_in, case["mode"].endswith("bf16"))
    say("  max err %.3e corr %.8f" % st)
