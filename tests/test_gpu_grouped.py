"""GPU parity of "gather once, apply every block's proj_linear": the
gathered samples (p3d_proj_sample) and the per-block linears over them
(p3d_proj_linear_grouped, with and without the residual add), through the C
ABI, against the CPU oracle.

Bar: samples within the sampling tolerance (fp32: 1e-5 of sum_k w_k |F_k|;
bf16: that plus one bf16 ulp, since both sides round); masks bit-exact; one-map bf16 samples
bit-identical to p3d_bilinear_sample at the same projected points (the same
arithmetic); per-block outputs within the bf16 proj_linear tolerance (2e-2
of |Y| + rms(row) per element, 2e-2 of max |Y| overall), residual included.
Besides the fixed cases, a seeded sweep draws token counts, ragged K and D,
the number of blocks, the residual add and the bias, and checks every row.
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import p3d_synth as synth
import pixel_aligned_image_amd as p3d
from parity_util import (bf16_to_f64, check_bf16_linear, oracle_cameras, product_cameras,
                         to_dev, to_host)

pytestmark = pytest.mark.gpu


def say(*a):
    print("[grouped]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def orc():
    o = oracle.get()
    o.set_threads(min(16, os.cpu_count() or 1))
    return o


def _gather(o, coords, n, R, fovs, maps_np, bf16, points, image_size, rows):
    cp = product_cameras(p3d, fovs, [None] * len(fovs), image_size)
    fo, do = oracle_cameras(o, fovs, [None] * len(fovs), image_size)
    K = sum(m.shape[3] for m in maps_np)
    dt = torch.bfloat16 if bf16 else torch.float32
    S = torch.full((n, K), float("nan"), dtype=dt, device="cuda")
    mask = torch.full((n,), 7, dtype=torch.uint8, device="cuda")
    feats = [to_dev(m, bf16) for m in maps_np]
    p3d.p3d_proj_sample(to_dev(coords), n, R, cp, feats if len(feats) > 1 else feats[0], S,
                        mask=mask, points=points)
    torch.cuda.synchronize()
    Sref, mref = o.proj_sample_rows(coords, n, R, fo, do, list(maps_np), rows, points=points)
    absm = [np.abs(bf16_to_f64(m)).astype(np.float32) if bf16 else np.abs(m) for m in maps_np]
    mag, _ = o.proj_sample_rows(coords, n, R, fo, do, absm, rows, points=points)
    got = to_host(S[torch.from_numpy(rows).cuda()])
    g = bf16_to_f64(got) if bf16 else got.astype(np.float64)
    # bf16: both sides are rounded (GPU: binary32 blend, oracle: binary64), so
    # near a rounding boundary they may sit one bf16 ulp (2^-7 relative) apart
    bound = 1e-5 * mag + (2.0 ** -7 * np.abs(Sref) if bf16 else 0.0) + 1e-30
    assert np.all(np.abs(g - Sref) <= bound), (np.abs(g - Sref) / bound).max()
    assert np.array_equal(to_host(mask)[rows], mref)
    return S, cp, feats, Sref


GATHER = [
    dict(name="bf16_one_map", bf16=True, R=32, B=2, n=1000, maps=[(24, 24, 136)], pts="cell_centres"),
    dict(name="f32_one_map_nodes", bf16=False, R=17, B=1, n=300, maps=[(13, 11, 36)],
         pts="grid_nodes"),
    dict(name="bf16_two_maps", bf16=True, R=40, B=2, n=777, maps=[(8, 8, 72), (40, 32, 64)],
         pts="cell_centres"),
    dict(name="f32_two_maps_nodes", bf16=False, R=20, B=3, n=260, maps=[(9, 9, 12), (30, 27, 20)],
         pts="grid_nodes"),
]


@pytest.mark.parametrize("case", GATHER, ids=[c["name"] for c in GATHER])
def test_proj_sample(orc, case):
    say(case)
    rng = np.random.default_rng(len(case["name"]) * 3)
    B, n = case["B"], case["n"]
    coords = synth.random_coords(case["R"], B, n, seed=n, spill=2)
    maps = [rng.standard_normal((B, h, w, c)).astype(np.float32) for h, w, c in case["maps"]]
    if case["bf16"]:
        maps = [synth.bf16_bits(m) for m in maps]
    _gather(orc, coords, n, case["R"], [40.0 + 3 * b for b in range(B)], maps, case["bf16"],
            case["pts"], case["maps"][0][1], np.arange(n))


def test_proj_sample_matches_bilinear_sample(orc):
    """One bf16 map: the gathered samples are bit-identical to
    p3d_bilinear_sample at the GPU's projected points."""
    rng = np.random.default_rng(5)
    R, B, n = 64, 2, 3000
    coords = synth.random_coords(R, B, n, seed=9, spill=3)
    m = synth.bf16_bits(rng.standard_normal((B, 32, 48, 256)).astype(np.float32))
    cp = product_cameras(p3d, [35.0, 45.0], [None, None], 48)
    feat = to_dev(m, True)
    S = torch.empty((n, 256), dtype=torch.bfloat16, device="cuda")
    p3d.p3d_proj_sample(to_dev(coords), n, R, cp, feat, S)
    grid = torch.empty((n, 2), device="cuda")
    p3d.p3d_project_points(to_dev(coords), n, R, cp, 32, 48, grid=grid)
    S2 = torch.empty_like(S)
    p3d.p3d_bilinear_sample(feat, grid, S2, batch_index=to_dev(coords[:, 0].copy()))
    torch.cuda.synchronize()
    assert torch.equal(S.view(torch.int16), S2.view(torch.int16))


def _grouped(o, S_np, n, K, D, G, accumulate, with_bias, rows, seed):
    rng = np.random.default_rng(seed)
    Ws = [synth.bf16_bits((rng.standard_normal((D, K)) * 0.05).astype(np.float32))
          for _ in range(G)]
    bs = [synth.bf16_bits((rng.standard_normal(D) * 0.05).astype(np.float32))
          if with_bias and g % 2 == 0 else None for g in range(G)]
    R0 = [synth.bf16_bits(rng.standard_normal((n, D)).astype(np.float32)) for _ in range(G)]
    S = to_dev(S_np, True)
    outs = [to_dev(r, True) if accumulate else torch.full((n, D), float("nan"),
                                                          dtype=torch.bfloat16, device="cuda")
            for r in R0]
    p3d.p3d_proj_linear_grouped(S, [to_dev(w, True) for w in Ws], outs,
                                biases=[None if b is None else to_dev(b, True) for b in bs]
                                if with_bias else None, accumulate=accumulate)
    torch.cuda.synchronize()
    Srows = bf16_to_f64(S_np[rows])
    res = [bf16_to_f64(r[rows]) for r in R0] if accumulate else None
    Y = o.linear_grouped(Srows, Ws, bs if with_bias else None, res)
    stats = []
    for g in range(G):
        got = to_host(outs[g][torch.from_numpy(rows).cuda()])
        stats.append(check_bf16_linear(got, Y[g]))
    return stats


CASES = [
    dict(name="ragged_tails", n=300, K=200, D=264, G=3, acc=False, bias=True),
    dict(name="residual_add", n=513, K=128, D=520, G=2, acc=True, bias=True),
    dict(name="one_block_no_bias", n=129, K=8, D=8, G=1, acc=False, bias=False),
    dict(name="many_blocks", n=260, K=64, D=64, G=64, acc=True, bias=True),
]


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_grouped_small(orc, case):
    say(case)
    rng = np.random.default_rng(len(case["name"]))
    n, K = case["n"], case["K"]
    S_np = synth.bf16_bits(rng.standard_normal((n, K)).astype(np.float32))
    _grouped(orc, S_np, n, K, case["D"], case["G"], case["acc"], case["bias"], np.arange(n),
             len(case["name"]) + 1)


def _draw_grouped(i):
    rng = np.random.default_rng(4300 + i)
    n = [1, 127, 128, 129][i] if i < 4 else int(rng.integers(2, 20000))
    K = 8 * int(rng.integers(1, 66))                          # 8 .. 520
    D = 8 * int(rng.integers(1, 138))                         # 8 .. 1096
    G = int(rng.integers(1, 9))
    while n * K * D * G > 2.5e9:                              # keep the oracle quick
        n //= 2
    return dict(i=i, n=max(n, 1), K=K, D=D, G=G, acc=bool(rng.random() < 0.5),
                bias=bool(rng.random() < 0.5))


SWEEP = [_draw_grouped(i) for i in range(20)]


@pytest.mark.parametrize("case", SWEEP, ids=["%d_n%d_K%d_D%d_G%d" % (c["i"], c["n"], c["K"], c["D"],
                                                                   c["G"]) for c in SWEEP])
def test_grouped_random_shape(orc, case):
    """A seeded sweep of shapes: ragged K and D, 1 to 8 blocks, with and
    without the residual add and the bias, every row."""
    say(case)
    rng = np.random.default_rng(4400 + case["i"])
    n, K = case["n"], case["K"]
    S_np = synth.bf16_bits(rng.standard_normal((n, K)).astype(np.float32))
    _grouped(orc, S_np, n, K, case["D"], case["G"], case["acc"], case["bias"], np.arange(n),
             4500 + case["i"])


def test_gather_once_then_blocks_full_size(orc):
    """The texture-stage workload: two maps gathered once into S [100k, 2048],
    then four blocks' 2048 -> 1536 linears with residual add, on sampled rows;
    block 0 without residual equals the fused path."""
    w = synth.workload("shell1024_cfg_twomap_bf16_c1024x2_d1536")
    coords = synth.coords(w)
    n = w.n_tokens
    maps = synth.feature_maps(w)
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([rng.choice(n, 256, replace=False), [0, 127, 128, n - 1]]))
    S, cp, feats, Sref = _gather(orc, coords, n, w.resolution, synth.fovs(w), maps, True,
                                 w.points, w.width, rows)
    K = S.shape[1]
    Wn = [synth.bf16_bits((rng.standard_normal((w.out_dim, K)) * 0.02).astype(np.float32))
          for _ in range(4)]
    Ws = [to_dev(x, True) for x in Wn]
    outs = [torch.zeros((n, w.out_dim), dtype=torch.bfloat16, device="cuda") for _ in range(4)]
    p3d.p3d_proj_linear_grouped(S, Ws, outs, accumulate=True)
    y = torch.empty((n, w.out_dim), dtype=torch.bfloat16, device="cuda")
    p3d.p3d_proj_cond(to_dev(coords), n, w.resolution, cp, feats, Ws[0], y)
    torch.cuda.synchronize()
    Y = orc.linear_grouped(Sref, Wn)          # the oracle's own samples and the drawn weights
    for g in range(4):
        st = check_bf16_linear(to_host(outs[g][torch.from_numpy(rows).cuda()]), Y[g])
        say("  block %d max|diff|/max|Y| %.3e corr %.8f" % (g, st[0], st[1]))
    a, b = outs[0].float(), y.float()
    rel = ((a - b).abs().max() / b.abs().max()).item()
    say("  grouped block 0 vs fused path: max|diff|/max|Y| %.3e" % rel)
    assert rel <= 2e-2
