"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Bar: pixel indices, fractions, normalised coordinates, depths and masks are
bit-exact (both sides take those binary32 decisions with the same operations
in the same order); fp32 samples within 1e-5 of the interpolated magnitude
sum_k w_k |F_k|; bf16 samples within half a bf16 ulp plus that; fp32
proj_linear within 1e-5 of sum_c |W||S| + |b|; bf16 proj_linear within 2e-2
of |Y| + rms(row) per element and 2e-2 of max |Y| overall; null rows
bit-exact. Small cases cover several tiles, ragged tails in tokens, channels
and outputs, odd map sizes, points outside the image and behind the camera.
The five workloads run at full size, compared on seeded samples of rows.
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import p3d_synth as synth
import pixel_aligned_image_amd as p3d
from parity_util import (Inputs, bf16_to_f64, check_bf16_linear, check_fp32_linear,
                         oracle_cameras, product_cameras, run_sample, tile_edge_rows, to_dev,
                         to_host)

pytestmark = pytest.mark.gpu


def say(*a):
    print("[parity]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def orc():
    o = oracle.get()
    o.set_threads(min(16, os.cpu_count() or 1))
    return o


@pytest.fixture(scope="module", params=range(len(synth.WORKLOADS)),
                ids=[w.name for w in synth.WORKLOADS])
def wl(request):
    w = synth.WORKLOADS[request.param]
    say("generating inputs", w.name)
    return Inputs(w)


def cams_both(o, fovs, dists, size):
    cp = product_cameras(p3d, fovs, dists, size)
    fo, do = oracle_cameras(o, fovs, dists, size)
    return cp, fo, do


# ------------------------------------------------------------------ cameras
def test_cameras_bit_identical(orc):
    fovs = [40.0, 25.0, 49.13, 30.0, 50.0, 1.0, 179.0] + list(
        np.random.default_rng(3).uniform(5, 170, 40))
    for a in fovs:
        for d in (None, 2.0, 1.6, 0.3):
            cp = product_cameras(p3d, [a], [d], 512)[0]
            fo, do = oracle_cameras(orc, [a], [d], 512)
            assert np.float32(cp[0]).tobytes() == fo[0].tobytes(), (a, d)
            assert np.float32(cp[1]).tobytes() == do[0].tobytes(), (a, d)
    for e in (0, 64, 128):
        assert p3d.p3d_distance_from_fov(49.13, 512, e) == orc.distance_from_fov(49.13, 512, e)


# ------------------------------------------------------------- projection
def _project_both(o, coords, n, R, fovs, dists, H, W, size=512):
    cp, fo, do = cams_both(o, fovs, dists, size)
    ref = o.project(coords, n, R, fo, do, H, W)
    out = dict(grid=torch.empty((n, 2), device="cuda"),
               pixel=torch.empty((n, 2), dtype=torch.int32, device="cuda"),
               frac=torch.empty((n, 2), device="cuda"),
               depth=torch.empty((n,), device="cuda"),
               mask=torch.empty((n,), dtype=torch.uint8, device="cuda"))
    p3d.p3d_project_points(to_dev(coords), n, R, cp, H, W, **out)
    torch.cuda.synchronize()
    return ref, {k: to_host(v) for k, v in out.items()}


def _assert_bitwise(ref, got, what):
    for k in ref:
        a, b = np.ascontiguousarray(ref[k]), np.ascontiguousarray(got[k])
        if not np.array_equal(a.view(np.uint8), b.view(np.uint8)):
            idx = np.nonzero((a != b).reshape(len(a), -1).any(axis=1))[0]
            raise AssertionError("%s: %s differs at %d tokens, first %s: oracle %s gpu %s" % (
                what, k, len(idx), idx[:5], a[idx[:3]], b[idx[:3]]))


def test_project_points_workloads(orc, wl):
    w = wl.w
    say("project", w.name, "n =", wl.n)
    ref, got = _project_both(orc, wl.coords, wl.n, w.resolution, wl.fovs, wl.dists,
                             w.height, w.width)
    _assert_bitwise(ref, got, w.name)
    say("  coverage (mask mean) %.4f" % got["mask"].mean())


@pytest.mark.parametrize("case", [
    dict(R=1, B=1, H=1, W=1, dense=True, fovs=[40.0], dists=[2.0]),
    dict(R=2, B=2, H=2, W=3, dense=True, fovs=[40.0, 60.0], dists=[2.0, 1.1]),
    dict(R=3, B=1, H=3, W=2, dense=True, fovs=[90.0], dists=[0.3]),      # behind camera
    dict(R=5, B=3, H=8, W=8, dense=True, fovs=[20.0, 40.0, 80.0], dists=[None, 1.5, None]),
    dict(R=16, B=3, H=7, W=9, dense=False, n=1000, spill=6, fovs=[35.0, 45.0, 55.0],
         dists=[None, None, 0.9]),
    dict(R=1024, B=2, H=512, W=512, dense=False, n=777, spill=0, fovs=[40.0, 30.0],
         dists=[None, None]),
    # distance 0.25 with R = 2: the far layer of cell centres sits at z =
    # 0.25, depth exactly 0, so gx, gy are +-inf (or NaN on the axis) and
    # the index clamp picks the edge texel (texel 0 for NaN); mask 0
    dict(R=2, B=1, H=4, W=5, dense=True, fovs=[40.0], dists=[0.25]),
    dict(R=4, B=2, H=6, W=6, dense=True, fovs=[60.0, 30.0], dists=[0.125, 0.375]),
], ids=["R1", "R2_b2", "behind_camera", "R5_b3", "spill_outside_cube", "R1024",
        "depth_zero_R2", "depth_zero_R4_b2"])
def test_project_points_edges(orc, case):
    say("project edge", case)
    R, B = case["R"], case["B"]
    if case["dense"]:
        coords, n = None, B * R ** 3
    else:
        n = case["n"]
        coords = synth.random_coords(R, B, n, seed=R + n, spill=case["spill"])
        coords[::97, 0] = B + 3       # batch column out of range -> mask 0
        coords[5::101, 0] = -1
    ref, got = _project_both(orc, coords, n, R, case["fovs"], case["dists"], case["H"],
                             case["W"])
    _assert_bitwise(ref, got, str(case))


def test_project_points_optional_outputs_and_empty(orc):
    w = synth.workload(2)
    coords = synth.coords(w)
    n = len(coords)
    cp, fo, do = cams_both(orc, synth.fovs(w), [None, None], 128)
    mask = torch.full((n,), 7, dtype=torch.uint8, device="cuda")
    p3d.p3d_project_points(to_dev(coords), n, w.resolution, cp, 128, 128, mask=mask)
    ref = orc.project(coords, n, w.resolution, fo, do, 128, 128)
    assert np.array_equal(to_host(mask), ref["mask"])
    sentinel = torch.full((4,), 9, dtype=torch.uint8, device="cuda")
    p3d.p3d_project_points(to_dev(coords[:0]), 0, w.resolution, cp, 128, 128)
    torch.cuda.synchronize()
    assert to_host(sentinel).tolist() == [9, 9, 9, 9]


# --------------------------------------------------------------- sampling
def _sample_check(o, feat_np, grid_np, bidx_np, bf16_in, out_bf16):
    return run_sample(p3d, o, feat_np, grid_np, bidx_np, bf16_in, out_bf16)


@pytest.mark.parametrize("shape", [(1, 1, 1, 8), (2, 2, 3, 16), (1, 3, 2, 8), (2, 8, 8, 64),
                                   (1, 5, 7, 24), (3, 16, 9, 2048)])
@pytest.mark.parametrize("mode", ["f32>f32", "bf16>f32", "bf16>bf16"])
def test_bilinear_sample_edges(orc, shape, mode):
    say("sample edge", shape, mode)
    bf16_in = mode.startswith("bf16")
    out_bf16 = mode.endswith("bf16")
    B, H, W, C = shape
    if (not bf16_in) and C % 4:
        pytest.skip("f32 maps need C % 4 == 0")
    rng = np.random.default_rng(sum(shape))
    featf = rng.standard_normal(shape).astype(np.float32)
    feat = synth.bf16_bits(featf) if bf16_in else featf
    pts = [rng.uniform(-1.5, 1.5, size=(300, 2))]
    special = np.array([-1.0, 1.0, -1.05, 1.05, 3.0, -5.0, 0.0, np.nan, np.inf, -np.inf,
                        -1.0 + 1.0 / max(W, 1), 1.0 - 1.0 / max(W, 1)])
    sx, sy = np.meshgrid(special, special)
    pts.append(np.stack([sx.ravel(), sy.ravel()], 1))
    grid = np.concatenate(pts).astype(np.float32)
    bidx = rng.integers(-1, B + 1, size=len(grid)).astype(np.int32) if B > 1 else None
    _sample_check(orc, feat, grid, bidx, bf16_in, out_bf16)


def test_bilinear_sample_workloads(orc, wl):
    """The workload's own map sampled at the GPU's projected points, against the
    oracle sampling the same map at its own (bit-identical) points; a seeded
    sample of points for the large workloads."""
    w = wl.w
    n = wl.n
    cp, fo, do = cams_both(orc, wl.fovs, wl.dists, w.width)
    grid = torch.empty((n, 2), device="cuda")
    p3d.p3d_project_points(to_dev(wl.coords), n, w.resolution, cp, w.height, w.width, grid=grid)
    ref_p = orc.project(wl.coords, n, w.resolution, fo, do, w.height, w.width)
    bidx_np = wl.coords[:, 0].copy() if wl.coords is not None else np.zeros(n, np.int32)
    feat = to_dev(wl.feat, bf16=wl.bf16)
    out = torch.empty((n, w.channels), dtype=torch.bfloat16 if wl.bf16 else torch.float32,
                      device="cuda")
    say("sample", w.name, "n =", n)
    p3d.p3d_bilinear_sample(feat, grid, out, batch_index=to_dev(bidx_np))
    torch.cuda.synchronize()
    assert np.array_equal(to_host(grid), ref_p["grid"])
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, size=min(n, 1500),
                                                             replace=False)]))
    got = to_host(out[torch.from_numpy(rows).cuda()])
    ref = orc.sample(wl.feat, ref_p["grid"][rows], bidx_np[rows])
    absf = np.abs(bf16_to_f64(wl.feat) if wl.bf16 else wl.feat)
    mag = orc.sample(absf.astype(np.float32), ref_p["grid"][rows], bidx_np[rows])
    g = bf16_to_f64(got) if wl.bf16 else got.astype(np.float64)
    bound = 1e-5 * mag + (2.0 ** -8 * np.abs(ref) if wl.bf16 else 0.0) + 1e-30
    err = np.abs(g - ref)
    assert np.all(err <= bound), "%d off, worst %.3e" % ((err > bound).sum(), (err / bound).max())


# ---------------------------------------------------------- fused path
def _run_proj_cond(o, coords, n, R, fovs, dists, feat_np, W_np, b_np, n_null, bf16, rows,
                   image_size, stream=None, keep=False, workspace=None):
    B, H, Wd, C = feat_np.shape
    D = W_np.shape[0]
    cp, fo, do = cams_both(o, fovs, dists, image_size)
    dt = torch.bfloat16 if bf16 else torch.float32
    out = torch.full((n + n_null, D), float("nan"), dtype=dt, device="cuda")
    mask = torch.full((n,), 7, dtype=torch.uint8, device="cuda")
    ws = None if workspace is None else p3d.proj_cond_workspace(n, B, feat_np)
    p3d.p3d_proj_cond(to_dev(coords), n, R, cp, to_dev(feat_np, bf16), to_dev(W_np, bf16),
                      out, bias=to_dev(b_np, bf16), n_null=n_null, mask=mask, stream=stream,
                      workspace=ws)
    torch.cuda.synchronize()
    Yref, mref = o.proj_cond_rows(coords, n, R, fo, do, feat_np, W_np, b_np, n_null, rows)
    got = to_host(out[torch.from_numpy(rows).cuda()])
    gmask = to_host(mask)
    tok = rows[rows < n]
    assert np.array_equal(gmask[tok], mref[rows < n]), "mask differs"
    # null rows: exactly the bias (or +0)
    null = rows >= n
    if null.any():
        want = (b_np if b_np is not None else np.zeros(D, W_np.dtype))
        assert np.array_equal(got[null], np.broadcast_to(want, (null.sum(), D))), "null rows"
    if bf16:
        stats = check_bf16_linear(got[~null], Yref[~null]) if (~null).any() else (0, 1)
    else:
        # |W| |S| + |b| magnitudes from the oracle on |map|, |W|
        S = o.proj_cond_rows(coords, n, R, fo, do, np.abs(feat_np), np.abs(W_np),
                             None if b_np is None else np.abs(b_np), n_null, rows[~null])[0]
        check_fp32_linear(got[~null], Yref[~null], S)
        stats = (np.abs(got[~null] - Yref[~null]).max() if (~null).any() else 0, 1)
    if keep:
        return gmask, stats, out
    return gmask, stats


SMALL = [
    dict(name="bf16_ragged_bias_null", bf16=True, R=32, B=2, n=300, H=24, W=24, C=136, D=264,
         bias=True, n_null=70),
    dict(name="f32_ragged", bf16=False, R=32, B=1, n=200, H=17, W=13, C=36, D=132, bias=False,
         n_null=0),
    dict(name="f32_dense_b2", bf16=False, R=5, B=2, n=None, H=8, W=8, C=64, D=64, bias=True,
         n_null=3),
    dict(name="bf16_one_token", bf16=True, R=8, B=1, n=1, H=2, W=2, C=8, D=8, bias=True,
         n_null=1),
    dict(name="bf16_tiles_2x3", bf16=True, R=64, B=3, n=129 * 2, H=64, W=48, C=192, D=520,
         bias=False, n_null=0),
    dict(name="f32_wide", bf16=False, R=40, B=2, n=390, H=33, W=31, C=260, D=300, bias=True,
         n_null=17),
    dict(name="bf16_outside_frame", bf16=True, R=16, B=1, n=400, H=16, W=16, C=64, D=256,
         bias=True, n_null=0, fov=70.0, dist=0.8, spill=4),
    # depth exactly 0 (distance 0.25, R = 2): infinite normalised coordinates
    # reach the sampler from coords; the clamp picks the edge texel
    dict(name="bf16_depth_zero", bf16=True, R=2, B=1, n=None, H=4, W=4, C=64, D=64, bias=True,
         n_null=2, dist=0.25),
    dict(name="f32_depth_zero", bf16=False, R=2, B=1, n=None, H=5, W=3, C=16, D=24, bias=False,
         n_null=0, dist=0.25),
    # null rows far beyond the token rows, ragged, 25 vectors per row
    dict(name="bf16_null_heavy", bf16=True, R=16, B=1, n=130, H=8, W=8, C=64, D=200,
         bias=True, n_null=700),
    # 300 tiles of 128 tokens: on 256 compute units the first 256 run whole
    # and the 44 past the last full round as 32-token parts, one launch; the
    # null blocks reach the split tiles too (block q goes with token tile q)
    dict(name="bf16_whole_and_split_tiles", bf16=True, R=64, B=1, n=299 * 128 + 77, H=48,
         W=40, C=136, D=264, bias=True, n_null=299 * 128 + 77),
    # 357 tiles: 256 run whole and the 101 past the last full round (too
    # many for 32-token parts) as 64-token parts, null blocks included
    dict(name="bf16_whole_and_half_tiles", bf16=True, R=64, B=1, n=356 * 128 + 45, H=48,
         W=40, C=136, D=264, bias=True, n_null=200 * 128 + 3),
    # 230 whole tiles: one round, too many to split and too many for one
    # round of 96-token tiles; each writes two or three null blocks inside a
    # three-chunk K loop
    dict(name="bf16_whole_tiles_null_blocks", bf16=True, R=48, B=2, n=230 * 128 - 5, H=32,
         W=36, C=136, D=264, bias=True, n_null=80000),
    # 140 tiles of 128 tokens (too many to split) run as one round of 187
    # 96-token tiles, each writing two or three 96-row null blocks
    dict(name="bf16_round_tiles_null_blocks", bf16=True, R=48, B=2, n=140 * 128 - 5, H=32,
         W=36, C=136, D=264, bias=True, n_null=50000),
    # exactly 256 96-token tiles (192 of 128), and one token more: 257 would
    # not fit one round, so that launch runs 193 whole tiles
    dict(name="bf16_round_tiles_every_cu", bf16=True, R=48, B=1, n=256 * 96, H=32, W=36,
         C=72, D=264, bias=True, n_null=300),
    dict(name="bf16_round_tiles_one_past", bf16=True, R=48, B=1, n=256 * 96 + 1, H=32, W=36,
         C=72, D=264, bias=True, n_null=300),
    # two N tiles, the second ragged (features 512 .. 999): 158 tiles of 128
    # tokens run as 210 of 96; 72 channels (one whole chunk and one vector)
    dict(name="bf16_round_tiles_two_n", bf16=True, R=40, B=2, n=10000, H=24, W=20, C=72,
         D=1000, bias=False, n_null=96 * 3 + 1),
    # 70 tiles as 140 64-token parts, each writing its half of two or three
    # null blocks
    dict(name="bf16_half_parts_null_blocks", bf16=True, R=48, B=2, n=70 * 128 - 5, H=32,
         W=36, C=136, D=264, bias=True, n_null=25000),
]


@pytest.mark.parametrize("case", SMALL, ids=[c["name"] for c in SMALL])
def test_proj_cond_small(orc, case):
    say("proj_cond small", case)
    rng = np.random.default_rng(len(case["name"]))
    R, B = case["R"], case["B"]
    if case["n"] is None:
        coords, n = None, B * R ** 3
    else:
        n = case["n"]
        coords = synth.random_coords(R, B, n, seed=n + R, spill=case.get("spill", 0))
    featf = rng.standard_normal((B, case["H"], case["W"], case["C"])).astype(np.float32)
    Wf = (rng.standard_normal((case["D"], case["C"])) * 0.05).astype(np.float32)
    bf = (rng.standard_normal(case["D"]) * 0.05).astype(np.float32) if case["bias"] else None
    if case["bf16"]:
        featf, Wf = synth.bf16_bits(featf), synth.bf16_bits(Wf)
        bf = synth.bf16_bits(bf) if bf is not None else None
    fovs = [case.get("fov", 40.0 + 5 * b) for b in range(B)]
    dists = [case.get("dist", None) for _ in range(B)]
    rows = np.arange(n + case["n_null"])
    _run_proj_cond(orc, coords, n, R, fovs, dists, featf, Wf, bf, case["n_null"],
                   case["bf16"], rows, case["W"])
    # the same case with the tokens in image-space order: every row and mask
    # byte against the oracle again
    _run_proj_cond(orc, coords, n, R, fovs, dists, featf, Wf, bf, case["n_null"],
                   case["bf16"], rows, case["W"], workspace=True)


def test_proj_cond_workloads(orc, wl):
    """Full size, in the launch configuration the bench times. Every row up to
    16384 tokens; above: 16384 seeded token rows, the first and last row of
    every whole tile and tail part, the first and last row of every 128-row null block
    plus 64 seeded null rows against the oracle; the mask of every token
    against the oracle's projection; and no output element left unwritten
    (the output starts as NaN)."""
    w = wl.w
    n, nn = wl.n, wl.n_null
    rng = np.random.default_rng(9)
    if n <= 16384:
        rows = np.arange(n + nn)
    else:
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        pick = rng.choice(n, size=16384, replace=False)
        edge = tile_edge_rows(n, w.out_dim, cus)
        nulls = []
        if nn:
            nb = np.arange(0, nn, 128)
            nulls = np.concatenate([n + nb, n + np.minimum(nb + 127, nn - 1),
                                    rng.integers(n, n + nn, 64)])
        rows = np.unique(np.concatenate([pick, edge, nulls]).astype(np.int64))
        say("proj_cond", w.name, "rows checked: %d (16384 seeded, %d tile/part edges, %d null)"
            % (len(rows), len(edge), len(nulls)))
    say("proj_cond", w.name, "n =", n, "n_null =", nn, "rows checked =", len(rows))
    gmask, stats, out = _run_proj_cond(orc, wl.coords, n, w.resolution, wl.fovs, wl.dists,
                                       wl.feat, wl.weight, wl.bias, nn, wl.bf16, rows, w.width,
                                       keep=True)
    assert not torch.isnan(out.float()).any().item(), "an output element was not written"
    fo, do = oracle_cameras(orc, wl.fovs, wl.dists, w.width)
    ref = orc.project(wl.coords, n, w.resolution, fo, do, w.height, w.width)
    ref_mask = ref["mask"] if isinstance(ref, dict) else ref[-1]
    assert np.array_equal(gmask, ref_mask), "fused mask differs from the oracle on %d of %d" % (
        int((gmask != ref_mask).sum()), n)
    say("  mask: all %d tokens equal; max|diff| stat %.3e corr %.8f coverage %.4f"
        % (n, stats[0], stats[1], gmask.mean()))


def test_proj_cond_ws_workloads_bitwise(orc, wl):
    """p3d_proj_cond_ws (tokens in image-space order) writes the same bytes
    as p3d_proj_cond on every row and mask byte of the full-size workload;
    with the row checks above that carries the oracle comparison over."""
    w = wl.w
    n, nn = wl.n, wl.n_null
    cp = product_cameras(p3d, wl.fovs, wl.dists, w.width)
    dt = torch.bfloat16 if wl.bf16 else torch.float32
    args = (to_dev(wl.coords), n, w.resolution, cp, to_dev(wl.feat, wl.bf16),
            to_dev(wl.weight, wl.bf16))
    bias = to_dev(wl.bias, wl.bf16)
    outs, masks = [], []
    for ws in (None, p3d.proj_cond_workspace(n, w.batch, args[4])):
        out = torch.full((n + nn, w.out_dim), float("nan"), dtype=dt, device="cuda")
        mask = torch.full((n,), 7, dtype=torch.uint8, device="cuda")
        p3d.p3d_proj_cond(*args, out, bias=bias, n_null=nn, mask=mask, workspace=ws)
        outs.append(out)
        masks.append(mask)
    torch.cuda.synchronize()
    bits = torch.int16 if wl.bf16 else torch.int32
    assert torch.equal(outs[0].view(bits), outs[1].view(bits)), "ordered rows differ"
    assert torch.equal(masks[0], masks[1]), "ordered mask differs"
    say("proj_cond_ws", w.name, "all %d rows and %d mask bytes bit-identical" % (n + nn, n))


def test_proj_cond_side_stream_matches_default(orc):
    w = synth.workload(2)
    inp = Inputs(w)
    rows = np.arange(0, inp.n, 37)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        m1, _ = _run_proj_cond(orc, inp.coords, inp.n, w.resolution, inp.fovs, inp.dists,
                               inp.feat, inp.weight, inp.bias, 5, True, rows, w.width, stream=s)
    m0, _ = _run_proj_cond(orc, inp.coords, inp.n, w.resolution, inp.fovs, inp.dists, inp.feat,
                           inp.weight, inp.bias, 5, True, rows, w.width)
    assert np.array_equal(m0, m1)


def test_proj_cond_null_only_and_empty(orc):
    D = 64
    bias = synth.bf16_bits(np.linspace(-1, 1, D).astype(np.float32))
    W_np = synth.bf16_bits(np.ones((D, 16), np.float32))
    feat = synth.bf16_bits(np.ones((1, 4, 4, 16), np.float32))
    out = torch.full((10, D), 3.0, dtype=torch.bfloat16, device="cuda")
    cams = product_cameras(p3d, [40.0], [None], 4)
    # nothing at all: no launch, out untouched
    p3d.p3d_proj_cond(None, 0, 8, cams, to_dev(feat, True), to_dev(W_np, True), out[:0],
                      bias=to_dev(bias, True), n_null=0)
    torch.cuda.synchronize()
    assert np.all(bf16_to_f64(to_host(out)) == 3.0)
    # n = 0 tokens, 10 null rows: the bias broadcast, no map or weight read
    p3d.p3d_proj_cond(None, 0, 8, cams, to_dev(feat, True), to_dev(W_np, True), out,
                      bias=to_dev(bias, True), n_null=10)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(out), np.broadcast_to(bias, (10, D)))
    # no bias: +0.0 rows
    p3d.p3d_proj_cond(None, 0, 8, cams, to_dev(feat, True), to_dev(W_np, True), out,
                      bias=None, n_null=10)
    torch.cuda.synchronize()
    assert np.all(to_host(out) == 0)


def test_proj_cond_channel_mismatch_names_both_shapes():
    feat = torch.zeros((1, 4, 4, 16), dtype=torch.bfloat16, device="cuda")
    weight = torch.zeros((32, 24), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((8, 32), dtype=torch.bfloat16, device="cuda")
    coords = torch.zeros((8, 4), dtype=torch.int32, device="cuda")
    with pytest.raises(p3d.P3DError) as e:
        p3d.p3d_proj_cond(coords, 8, 8, [(2.0, 2.0)], feat, weight, out)
    assert e.value.status == p3d.P3D_ERR_SHAPE
    assert "[32, 24]" in e.value.message and "[1, 4, 4, 16]" in e.value.message


def test_proj_cond_ws_errors():
    """A short or misaligned workspace is refused before anything runs, with
    both sizes in the message; an F32 call ignores the workspace."""
    feat = torch.zeros((1, 8, 8, 16), dtype=torch.bfloat16, device="cuda")
    weight = torch.zeros((32, 16), dtype=torch.bfloat16, device="cuda")
    out = torch.full((40, 32), 5.0, dtype=torch.bfloat16, device="cuda")
    coords = torch.zeros((40, 4), dtype=torch.int32, device="cuda")
    need = p3d.p3d_proj_cond_workspace_size(40, 1, feat)
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(p3d.P3DError) as e:
        p3d.p3d_proj_cond(coords, 40, 8, [(2.0, 2.0)], feat, weight, out, workspace=small)
    assert e.value.status == p3d.P3D_ERR_INVALID_ARG
    assert str(need) in e.value.message and str(need - 256) in e.value.message
    torch.cuda.synchronize()
    assert np.all(bf16_to_f64(to_host(out)) == 5.0)
    big = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(p3d.P3DError) as e:
        p3d.p3d_proj_cond(coords, 40, 8, [(2.0, 2.0)], feat, weight, out, workspace=big[1:])
    assert e.value.status == p3d.P3D_ERR_UNSUPPORTED and "256-byte" in e.value.message
