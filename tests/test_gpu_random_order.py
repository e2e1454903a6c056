"""The image-space token order over a seeded sweep of 60 inputs.

Each case draws (from one fixed seed) the grid resolution, the batch, the
token count (1 to about 60000, so the 1024-token bin workgroups end ragged),
how far the coords spill past the grid, the point mode, and a key map from
1 x 1 to 1024 x 1024 (block sizes from 4 texels up to coarser blocks when
the bins would pass 16384). For every case:
- the order is a permutation of [0, n) whose block keys, computed from the
  oracle's projection, never decrease along it;
- the standalone gather at the tokens' projected points, given the order,
  writes the bytes of the unordered call;
- on every third case, the fused bf16 call through the order writes the
  bytes of the unordered call (rows, null rows, mask).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import p3d_synth as synth
import pixel_aligned_image_amd as p3d
from parity_util import product_cameras, to_dev
from test_gpu_order import _check_order, _order

pytestmark = pytest.mark.gpu


def say(*a):
    print("[random order]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def _draw(i):
    rng = np.random.default_rng(9100 + i)
    R = int(rng.choice([2, 5, 16, 33, 64, 128, 257, 1024]))
    B = int(rng.integers(1, 5)) if i % 5 else int(rng.integers(1, 40))
    n = int(rng.integers(1, 60000)) if i % 3 else int(rng.choice([1, 1023, 1024, 1025, 4097]))
    kH = int(rng.choice([1, 3, 17, 64, 100, 256, 512, 1024]))
    kW = int(rng.choice([1, 5, 16, 64, 129, 256, 512, 1024]))
    spill = int(rng.integers(0, 4))
    pts = "grid_nodes" if (i % 4 == 1 and R >= 2) else "cell_centres"
    return dict(i=i, R=R, B=B, n=n, kH=kH, kW=kW, spill=spill, pts=pts)


CASES = [_draw(i) for i in range(60)]


@pytest.mark.parametrize("case", CASES, ids=["%d_R%d_b%d_n%d_%dx%d_%s" % (
    c["i"], c["R"], c["B"], c["n"], c["kH"], c["kW"], c["pts"][:4]) for c in CASES])
def test_token_order_random(orc, case):
    say(case)
    i, R, B, n, kH, kW = case["i"], case["R"], case["B"], case["n"], case["kH"], case["kW"]
    coords = synth.random_coords(R, B, n, seed=9200 + i, spill=case["spill"])
    fovs = [25.0 + 4 * b for b in range(B)]
    cams = product_cameras(p3d, fovs, [None] * B, kW)
    cd = to_dev(coords)
    order = _order(cd, n, R, cams, B, kH, kW, case["pts"])
    torch.cuda.synchronize()
    _check_order(orc, coords, n, R, fovs, kW, kH, kW, case["pts"], order)
    # the standalone gather through the order: same bytes
    rng = np.random.default_rng(9300 + i)
    C = 8 * int(rng.integers(1, 33))
    while B * kH * kW * C > (1 << 26) and C > 8:             # keep the host map small
        C //= 2
    C = max(8, C - C % 8)
    if B * kH * kW * C > (1 << 26):
        pytest.skip("map too large for a host draw")
    feat = to_dev(synth.bf16_bits(rng.standard_normal((B, kH, kW, C)).astype(np.float32)), True)
    grid = torch.empty((n, 2), device="cuda")
    p3d.p3d_project_points(cd, n, R, cams, kH, kW, grid=grid, points=case["pts"])
    bidx = to_dev(coords[:, 0].copy())
    ref = torch.full((n, C), float("nan"), dtype=torch.bfloat16, device="cuda")
    got = torch.full_like(ref, float("nan"))
    p3d.p3d_bilinear_sample(feat, grid, ref, batch_index=bidx)
    p3d.p3d_bilinear_sample(feat, grid, got, batch_index=bidx, order=order)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    if i % 3 == 0:
        D = 8 * int(rng.integers(1, 80))
        weight = to_dev(synth.bf16_bits((rng.standard_normal((D, C)) * 0.05).astype(np.float32)),
                        True)
        nn = int(rng.integers(0, 2 * n + 1))
        outs, masks = [], []
        for o in (None, order):
            y = torch.full((n + nn, D), float("nan"), dtype=torch.bfloat16, device="cuda")
            m = torch.full((n,), 7, dtype=torch.uint8, device="cuda")
            p3d.p3d_proj_cond(cd, n, R, cams, feat, weight, y, n_null=nn, mask=m,
                              points=case["pts"], order=o)
            outs.append(y)
            masks.append(m)
        torch.cuda.synchronize()
        assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
        assert torch.equal(masks[0], masks[1])
