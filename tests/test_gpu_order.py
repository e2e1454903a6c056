"""GPU tests of the image-space token order (p3d_token_order) and of the
calls that take it (p3d_proj_sample_ordered, p3d_projection_stats_ordered).

The order among tokens of one texel block is unspecified, so the order is
checked for what is unique about it: it is a permutation of [0, n), and the
key of the token at each sorted position -- batch item, then the Morton
index of the block holding its top-left corner texel on the key map,
computed here from the oracle's projection -- never decreases. Results of
the ordered calls must not depend on which valid order they get: the ordered
samples and mask are bit-identical to the unordered call's, for the token
order and for a random permutation; the ordered diagnostics meet the oracle
bar of the unordered ones (counts exact, sums within the sampling bound).
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import p3d_synth as synth
import pixel_aligned_image_amd as p3d
from parity_util import oracle_cameras, product_cameras, run_stats, to_dev, to_host

pytestmark = pytest.mark.gpu


def say(*a):
    print("[order]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def orc():
    o = oracle.get()
    o.set_threads(min(16, os.cpu_count() or 1))
    return o


def _blocks(batch, kH, kW):
    """Block side (log2 texels) and blocks per item of the documented rule:
    4-texel blocks, coarser until batch * P^2 <= 16384, P the blocks per
    axis rounded up to a power of two."""
    side = max(kH, kW)
    shift = 2
    while True:
        P = 1
        while P * (1 << shift) < side:
            P *= 2
        if batch * P * P <= 16384:
            return shift, P * P
        shift += 1


def _morton(x, y):
    key = np.zeros_like(x, dtype=np.int64)
    for bit in range(16):
        key |= ((x >> bit) & 1) << (2 * bit)
        key |= ((y >> bit) & 1) << (2 * bit + 1)
    return key


def _order(coords_d, n, R, cams, batch, kH, kW, points="cell_centres"):
    order = torch.full((max(n, 1),), -1, dtype=torch.int32, device="cuda")[:n]
    p3d.p3d_token_order(coords_d, n, R, cams, kH, kW, order, points=points)
    return order


def _check_order(o, coords, n, R, fovs, image_size, kH, kW, points, order):
    got = to_host(order).astype(np.int64)
    assert got.shape == (n,)
    assert np.array_equal(np.sort(got), np.arange(n)), "not a permutation"
    fo, do = oracle_cameras(o, fovs, [None] * len(fovs), image_size)
    pr = o.project(coords, n, R, fo, do, kH, kW, points=points)
    batch = len(fovs)
    b = np.clip(coords[:, 0].astype(np.int64), 0, batch - 1)
    shift, per_item = _blocks(batch, kH, kW)
    key = b * per_item + _morton(pr["pixel"][:, 0].astype(np.int64) >> shift,
                                 pr["pixel"][:, 1].astype(np.int64) >> shift)
    ks = key[got]
    assert np.all(np.diff(ks) >= 0), "keys decrease at %d places" % int((np.diff(ks) < 0).sum())
    return key


ORDER_CASES = [
    dict(name="one_token", R=8, B=1, n=1, key=(16, 16), spill=0, pts="cell_centres"),
    dict(name="ragged_1025", R=24, B=2, n=1025, key=(17, 13), spill=3, pts="cell_centres"),
    dict(name="nodes_3000", R=33, B=1, n=3000, key=(64, 64), spill=0, pts="grid_nodes"),
    dict(name="coarse_blocks_b20", R=64, B=20, n=40000, key=(512, 512), spill=2,
         pts="cell_centres"),
    dict(name="wide_key_one_block_row", R=40, B=3, n=5000, key=(1, 700), spill=1,
         pts="cell_centres"),
]


@pytest.mark.parametrize("case", ORDER_CASES, ids=[c["name"] for c in ORDER_CASES])
def test_token_order_small(orc, case):
    say(case)
    B, n, R = case["B"], case["n"], case["R"]
    coords = synth.random_coords(R, B, n, seed=n + 17, spill=case["spill"])
    fovs = [30.0 + 5 * b for b in range(B)]
    kH, kW = case["key"]
    cams = product_cameras(p3d, fovs, [None] * B, kW)
    order = _order(to_dev(coords), n, R, cams, B, kH, kW, case["pts"])
    torch.cuda.synchronize()
    _check_order(orc, coords, n, R, fovs, kW, kH, kW, case["pts"], order)


def test_token_order_empty():
    cams = product_cameras(p3d, [40.0], [None], 16)
    order = torch.empty((0,), dtype=torch.int32, device="cuda")
    p3d.p3d_token_order(torch.empty((0, 4), dtype=torch.int32, device="cuda"), 0, 8, cams, 16,
                        16, order)
    torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["shell1024_cfg_bf16_c2048_d1536",
                                  "shell1024_cfg_twomap_bf16_c1024x2_d1536",
                                  "shell64x2_bf16_c2048_d1536"])
def test_token_order_workloads(orc, name):
    w = synth.workload(name)
    coords = synth.coords(w)
    n = w.n_tokens
    fovs = synth.fovs(w)
    cams = product_cameras(p3d, fovs, [None] * w.batch, w.width)
    # the key map is the one with the most texels
    kH, kW = max([(w.height, w.width)] + ([w.map1[:2]] if w.map1 else []),
                 key=lambda hw: hw[0] * hw[1])
    order = _order(to_dev(coords), n, w.resolution, cams, w.batch, kH, kW, w.points)
    torch.cuda.synchronize()
    key = _check_order(orc, coords, n, w.resolution, fovs, w.width, kH, kW, w.points, order)
    say(name, "tokens", n, "distinct blocks", np.unique(key).size)


def _sample_pair(coords, n, R, cams, feats, order, points):
    K = sum(f.shape[3] for f in feats)
    S0 = torch.full((n, K), float("nan"), dtype=feats[0].dtype, device="cuda")
    S1 = torch.full((n, K), float("nan"), dtype=feats[0].dtype, device="cuda")
    m0 = torch.full((n,), 7, dtype=torch.uint8, device="cuda")
    m1 = torch.full((n,), 7, dtype=torch.uint8, device="cuda")
    cd = to_dev(coords)
    p3d.p3d_proj_sample(cd, n, R, cams, feats, S0, mask=m0, points=points)
    p3d.p3d_proj_sample(cd, n, R, cams, feats, S1, mask=m1, points=points, order=order)
    torch.cuda.synchronize()
    iv = torch.int16 if S0.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(S0.view(iv), S1.view(iv))
    assert torch.equal(m0, m1)


SAMPLE_CASES = [
    dict(name="bf16_two_maps", bf16=True, R=40, B=2, n=2777, maps=[(8, 8, 72), (40, 32, 64)],
         pts="cell_centres"),
    dict(name="f32_one_map_nodes", bf16=False, R=17, B=1, n=1300, maps=[(13, 11, 36)],
         pts="grid_nodes"),
    dict(name="bf16_one_map_ragged", bf16=True, R=64, B=3, n=4099, maps=[(32, 48, 256)],
         pts="cell_centres"),
]


@pytest.mark.parametrize("case", SAMPLE_CASES, ids=[c["name"] for c in SAMPLE_CASES])
def test_ordered_sample_bitwise(case):
    """Token order and a random permutation both reproduce the unordered
    samples and mask bit for bit."""
    say(case)
    rng = np.random.default_rng(len(case["name"]))
    B, n, R = case["B"], case["n"], case["R"]
    coords = synth.random_coords(R, B, n, seed=n, spill=2)
    maps = [rng.standard_normal((B, h, w, c)).astype(np.float32) for h, w, c in case["maps"]]
    if case["bf16"]:
        maps = [synth.bf16_bits(m) for m in maps]
    feats = [to_dev(m, case["bf16"]) for m in maps]
    fovs = [40.0 + 3 * b for b in range(B)]
    cams = product_cameras(p3d, fovs, [None] * B, case["maps"][0][1])
    kH = max(m[0] for m in case["maps"])
    kW = max(m[1] for m in case["maps"])
    order = _order(to_dev(coords), n, R, cams, B, kH, kW, case["pts"])
    _sample_pair(coords, n, R, cams, feats, order, case["pts"])
    perm = torch.from_numpy(rng.permutation(n).astype(np.int32)).cuda()
    _sample_pair(coords, n, R, cams, feats, perm, case["pts"])


def test_ordered_sample_twomap_workload():
    w = synth.workload("shell1024_cfg_twomap_bf16_c1024x2_d1536")
    coords = synth.coords(w)
    n = w.n_tokens
    feats = [to_dev(m, True) for m in synth.feature_maps(w)]
    cams = product_cameras(p3d, synth.fovs(w), [None] * w.batch, w.width)
    kH = max(f.shape[1] for f in feats)
    kW = max(f.shape[2] for f in feats)
    order = _order(to_dev(coords), n, w.resolution, cams, w.batch, kH, kW, w.points)
    say("two-map workload", n, "tokens, key", kH, kW)
    _sample_pair(coords, n, w.resolution, cams, feats, order, w.points)


STATS_CASES = [
    dict(name="f32_one_map", bf16=False, R=24, B=2, n=1000, maps=[(17, 13, 36)], spill=3,
         pts="cell_centres"),
    dict(name="bf16_two_maps_cosine", bf16=True, R=40, B=2, n=2049,
         maps=[(16, 16, 128), (64, 48, 128)], spill=2, pts="cell_centres"),
    dict(name="bf16_two_maps_nodes", bf16=True, R=16, B=1, n=130, maps=[(8, 8, 64), (20, 20, 72)],
         spill=0, pts="grid_nodes"),
]


@pytest.mark.parametrize("case", STATS_CASES, ids=[c["name"] for c in STATS_CASES])
def test_ordered_stats_small(orc, case):
    say(case)
    rng = np.random.default_rng(len(case["name"]) * 13)
    B, n, R = case["B"], case["n"], case["R"]
    coords = synth.random_coords(R, B, n, seed=n, spill=case["spill"])
    maps = [rng.standard_normal((B, h, w, c)).astype(np.float32) + 0.1 * i
            for i, (h, w, c) in enumerate(case["maps"])]
    if case["bf16"]:
        maps = [synth.bf16_bits(m) for m in maps]
    fovs = [40.0 + 7 * b for b in range(B)]
    image = case["maps"][0][1]
    cams = product_cameras(p3d, fovs, [None] * B, image)
    kH = max(m[0] for m in case["maps"])
    kW = max(m[1] for m in case["maps"])
    order = _order(to_dev(coords), n, R, cams, B, kH, kW, case["pts"])
    run_stats(p3d, orc, coords, n, R, fovs, [None] * B, maps, case["bf16"], case["pts"], image,
              order=order)


def test_ordered_stats_twomap_workload(orc):
    w = synth.workload("shell1024_cfg_twomap_bf16_c1024x2_d1536")
    coords = synth.coords(w)
    maps = synth.feature_maps(w)
    n = w.n_tokens
    cams = product_cameras(p3d, synth.fovs(w), [None] * w.batch, w.width)
    kH = max(m.shape[1] for m in maps)
    kW = max(m.shape[2] for m in maps)
    order = _order(to_dev(coords), n, w.resolution, cams, w.batch, kH, kW, w.points)
    got, _ = run_stats(p3d, orc, coords, n, w.resolution, synth.fovs(w), [None] * w.batch, maps,
                       True, w.points, w.width, order=order)
    say("two-map workload ordered", p3d.p3d_stats_figures(got, [m.shape[3] for m in maps]))


def _fused_pair(coords, n, R, cams, feats, weight, bias, n_null, order, points):
    D = weight.shape[0]
    outs, masks = [], []
    for o in (None, order):
        y = torch.full((n + n_null, D), float("nan"), dtype=weight.dtype, device="cuda")
        m = torch.full((n,), 7, dtype=torch.uint8, device="cuda")
        p3d.p3d_proj_cond(to_dev(coords), n, R, cams, feats, weight, y, bias=bias, n_null=n_null,
                          mask=m, points=points, order=o)
        outs.append(y)
        masks.append(m)
    torch.cuda.synchronize()
    iv = torch.int16 if weight.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(outs[0].view(iv), outs[1].view(iv))
    assert torch.equal(masks[0], masks[1])


FUSED_CASES = [
    dict(name="bf16_one_map_ragged", bf16=True, R=48, B=2, n=3001, maps=[(24, 24, 256)], D=520,
         nn=130, pts="cell_centres", bias=True),
    dict(name="bf16_two_maps_nodes", bf16=True, R=40, B=1, n=1500, maps=[(8, 8, 64), (40, 32, 128)],
         D=256, nn=0, pts="grid_nodes", bias=False),
    dict(name="f32_ignores_order", bf16=False, R=20, B=1, n=700, maps=[(16, 16, 64)], D=96, nn=5,
         pts="cell_centres", bias=True),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=[c["name"] for c in FUSED_CASES])
def test_proj_cond_ordered_bitwise(case):
    """p3d_proj_cond_ordered with the token order and with a random
    permutation writes the same bytes as p3d_proj_cond_ex."""
    say(case)
    rng = np.random.default_rng(len(case["name"]) + 5)
    B, n, R = case["B"], case["n"], case["R"]
    coords = synth.random_coords(R, B, n, seed=n + 3, spill=2)
    maps = [rng.standard_normal((B, h, w, c)).astype(np.float32) for h, w, c in case["maps"]]
    K = sum(c for _, _, c in case["maps"])
    W = (rng.standard_normal((case["D"], K)) * 0.05).astype(np.float32)
    b = (rng.standard_normal(case["D"]) * 0.05).astype(np.float32) if case["bias"] else None
    bf = case["bf16"]
    if bf:
        maps = [synth.bf16_bits(m) for m in maps]
        W = synth.bf16_bits(W)
        b = synth.bf16_bits(b) if b is not None else None
    feats = [to_dev(m, bf) for m in maps]
    fovs = [40.0 + 3 * i for i in range(B)]
    cams = product_cameras(p3d, fovs, [None] * B, case["maps"][0][1])
    kH = max(m[0] for m in case["maps"])
    kW = max(m[1] for m in case["maps"])
    order = _order(to_dev(coords), n, R, cams, B, kH, kW, case["pts"])
    for o in (order, torch.from_numpy(rng.permutation(n).astype(np.int32)).cuda()):
        _fused_pair(coords, n, R, cams, feats, to_dev(W, bf), to_dev(b, bf), case["nn"], o,
                    case["pts"])


def test_proj_cond_ordered_workload():
    w = synth.workload("shell1024_cfg_bf16_c2048_d1536")
    coords = synth.coords(w)
    n = w.n_tokens
    feat = to_dev(synth.feature_map(w), True)
    weight = to_dev(synth.weight(w), True)
    cams = product_cameras(p3d, synth.fovs(w), [None] * w.batch, w.width)
    order = _order(to_dev(coords), n, w.resolution, cams, w.batch, w.height, w.width, w.points)
    say(w.name, n, "tokens +", w.n_null, "null rows")
    _fused_pair(coords, n, w.resolution, cams, feat, weight, None, w.n_null, order, w.points)


GATHER_CASES = [
    dict(name="bf16_to_bf16", R=48, B=2, n=3001, H=24, W=40, C=256, out="bf16"),
    dict(name="bf16_to_f32_one_item", R=33, B=1, n=1025, H=17, W=13, C=72, out="f32"),
    dict(name="f32_to_f32", R=20, B=3, n=700, H=9, W=30, C=36, out="f32"),
]


@pytest.mark.parametrize("case", GATHER_CASES, ids=[c["name"] for c in GATHER_CASES])
def test_ordered_bilinear_sample_bitwise(case):
    """p3d_bilinear_sample_ordered at the tokens' projected points, with the
    token order and with a random permutation, writes the bytes of
    p3d_bilinear_sample."""
    say(case)
    rng = np.random.default_rng(len(case["name"]) + 11)
    B, n, R, H, W, C = case["B"], case["n"], case["R"], case["H"], case["W"], case["C"]
    coords = synth.random_coords(R, B, n, seed=n + 1, spill=2)
    featf = rng.standard_normal((B, H, W, C)).astype(np.float32)
    bf_in = case["name"].startswith("bf16")
    feat = to_dev(synth.bf16_bits(featf), True) if bf_in else to_dev(featf)
    odt = torch.bfloat16 if case["out"] == "bf16" else torch.float32
    cams = product_cameras(p3d, [40.0 + 3 * b for b in range(B)], [None] * B, W)
    cd = to_dev(coords)
    grid = torch.empty((n, 2), device="cuda")
    p3d.p3d_project_points(cd, n, R, cams, H, W, grid=grid)
    bidx = to_dev(coords[:, 0].copy())
    order = _order(cd, n, R, cams, B, H, W)
    ref = torch.full((n, C), float("nan"), dtype=odt, device="cuda")
    p3d.p3d_bilinear_sample(feat, grid, ref, batch_index=bidx)
    iv = torch.int16 if odt == torch.bfloat16 else torch.int32
    for o in (order, torch.from_numpy(rng.permutation(n).astype(np.int32)).cuda()):
        got = torch.full_like(ref, float("nan"))
        p3d.p3d_bilinear_sample(feat, grid, got, batch_index=bidx, order=o)
        torch.cuda.synchronize()
        assert torch.equal(got.view(iv), ref.view(iv))


def test_ordered_bilinear_sample_workload():
    w = synth.workload("shell1024_cfg_bf16_c2048_d1536")
    coords = synth.coords(w)
    n = w.n_tokens
    feat = to_dev(synth.feature_map(w), True)
    cams = product_cameras(p3d, synth.fovs(w), [None] * w.batch, w.width)
    cd = to_dev(coords)
    grid = torch.empty((n, 2), device="cuda")
    p3d.p3d_project_points(cd, n, w.resolution, cams, w.height, w.width, grid=grid)
    bidx = to_dev(coords[:, 0].copy())
    order = _order(cd, n, w.resolution, cams, w.batch, w.height, w.width)
    ref = torch.empty((n, w.channels), dtype=torch.bfloat16, device="cuda")
    got = torch.full_like(ref, float("nan"))
    p3d.p3d_bilinear_sample(feat, grid, ref, batch_index=bidx)
    p3d.p3d_bilinear_sample(feat, grid, got, batch_index=bidx, order=order)
    torch.cuda.synchronize()
    say(w.name, "ordered gather of", n, "points")
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


def test_proj_cond_ordered_twomap_workload():
    """The texture stage's two maps at full size: the fused call through the
    token order (key map: the 512 x 512 one) writes the bytes of the
    unordered call, null rows and mask included."""
    w = synth.workload("shell1024_cfg_twomap_bf16_c1024x2_d1536")
    coords = synth.coords(w)
    n = w.n_tokens
    feats = [to_dev(m, True) for m in synth.feature_maps(w)]
    weight = to_dev(synth.weight(w), True)
    cams = product_cameras(p3d, synth.fovs(w), [None] * w.batch, w.width)
    kH = max(f.shape[1] for f in feats)
    kW = max(f.shape[2] for f in feats)
    order = _order(to_dev(coords), n, w.resolution, cams, w.batch, kH, kW, w.points)
    say(w.name, n, "tokens +", w.n_null, "null rows, two maps")
    _fused_pair(coords, n, w.resolution, cams, feats, weight, None, w.n_null, order, w.points)
