"""GPU parity of the adjacent parts: grid-node points, cascade
requantization and the two-map (concatenated) gather, through the C ABI,
against the CPU oracle on the same seeded inputs.

Bar: requantized coords bit-exact (integer work); projections (grid, pixel,
frac, depth, mask) bit-exact; proj_linear within the tolerances of the main
parity tests (fp32: 1e-5 of sum |W||S| + |b|; bf16: 2e-2 of |Y| + rms(row),
2e-2 of max |Y| overall); null rows bit-exact.
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import p3d_synth as synth
import pixel_aligned_image_amd as p3d
from parity_util import (check_bf16_linear, check_fp32_linear, oracle_cameras, run_fused,
                         product_cameras, to_dev, to_host)

pytestmark = pytest.mark.gpu


def say(*a):
    print("[nodes/maps]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def orc():
    o = oracle.get()
    o.set_threads(min(16, os.cpu_count() or 1))
    return o


# ------------------------------------------------------------ requantization
@pytest.mark.parametrize("src_res,grid", [(512, 64), (512, 63), (512, 65), (1024, 64),
                                          (64, 64), (7, 3), (3, 4), (1, 2), (100, 1)])
@pytest.mark.parametrize("mode", ["round_nodes", "floor_cells"])
def test_requantize_every_coordinate(orc, src_res, grid, mode):
    if mode == "round_nodes" and grid < 2:
        pytest.skip("nearest-node rounding needs grid >= 2")
    say("requantize", src_res, grid, mode)
    c = np.arange(-3, src_res + 3, dtype=np.int32)          # includes out-of-range
    toks = np.stack([np.arange(len(c), dtype=np.int32) % 5, c, c[::-1], (c * 7) % (src_res + 6) - 3],
                    1).astype(np.int32)
    src = to_dev(toks)
    dst = torch.full_like(src, -99)
    p3d.p3d_requantize_coords(src, src_res, grid, dst, mode=mode)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(dst), orc.requantize(toks, src_res, grid, mode))


def test_requantize_in_place_and_workload(orc):
    w = synth.workload("cascade512_grid64_nodes_bf16_c2048_d1536")
    coords = synth.coords(w)
    say("requantize workload", w.name, len(coords))
    t = to_dev(coords)
    p3d.p3d_requantize_coords(t, w.coords_resolution, w.resolution, t, mode="round_nodes")
    torch.cuda.synchronize()
    want = orc.requantize(coords, w.coords_resolution, w.resolution, "round_nodes")
    assert np.array_equal(to_host(t), want)
    floor = orc.requantize(coords, w.coords_resolution, w.resolution, "floor_cells")
    moved = np.any(want[:, 1:] != floor[:, 1:], axis=1).mean()
    say("  tokens that flooring would misregister: %.4f" % moved)


# ------------------------------------------------------------ grid nodes
def _project_both(o, coords, n, R, fovs, dists, H, W, points):
    cp = product_cameras(p3d, fovs, dists, W)
    fo, do = oracle_cameras(o, fovs, dists, W)
    ref = o.project(coords, n, R, fo, do, H, W, points=points)
    out = dict(grid=torch.empty((n, 2), device="cuda"),
               pixel=torch.empty((n, 2), dtype=torch.int32, device="cuda"),
               frac=torch.empty((n, 2), device="cuda"),
               depth=torch.empty((n,), device="cuda"),
               mask=torch.empty((n,), dtype=torch.uint8, device="cuda"))
    p3d.p3d_project_points(to_dev(coords), n, R, cp, H, W, points=points, **out)
    torch.cuda.synchronize()
    got = {k: to_host(v) for k, v in out.items()}
    for k in ref:
        assert np.array_equal(np.ascontiguousarray(ref[k]).view(np.uint8),
                              np.ascontiguousarray(got[k]).view(np.uint8)), k
    return got


@pytest.mark.parametrize("R,B,H,W,dense", [(2, 1, 4, 4, True), (5, 2, 9, 7, True),
                                           (17, 1, 32, 32, True), (64, 2, 128, 128, False),
                                           (1025, 1, 512, 512, False)])
def test_project_grid_nodes(orc, R, B, H, W, dense):
    say("grid nodes", R, B, H, W, dense)
    if dense:
        coords, n = None, B * R ** 3
    else:
        n = 5000
        coords = synth.random_coords(R, B, n, seed=R)
    _project_both(orc, coords, n, R, [40.0, 33.0][:B], [None, 1.9][:B], H, W, "grid_nodes")


def test_cascade_requantize_then_project(orc):
    """res-512 coords -> 64 nodes (nearest node) -> node projection, every
    step on the GPU, against the oracle doing the same steps."""
    w = synth.workload("cascade512_grid64_nodes_bf16_c2048_d1536")
    coords = synth.coords(w)
    n = len(coords)
    t = to_dev(coords)
    q = torch.empty_like(t)
    p3d.p3d_requantize_coords(t, w.coords_resolution, w.resolution, q)
    torch.cuda.synchronize()
    qc = orc.requantize(coords, w.coords_resolution, w.resolution, "round_nodes")
    assert np.array_equal(to_host(q), qc)
    got = _project_both(orc, qc, n, w.resolution, synth.fovs(w), [None], w.height, w.width,
                        "grid_nodes")
    say("  cascade coverage %.4f" % got["mask"].mean())


# ------------------------------------------------ fused: nodes and two maps
def _run(o, coords, n, R, fovs, dists, maps_np, W_np, b_np, n_null, bf16, rows, points,
         image_size):
    return run_fused(p3d, o, coords, n, R, fovs, dists, maps_np, W_np, b_np, n_null, bf16,
                     rows, points, image_size)


CASES = [
    dict(name="bf16_nodes_one_map", bf16=True, R=33, B=2, n=300, maps=[(24, 24, 136)], D=264,
         bias=True, n_null=20, points="grid_nodes"),
    dict(name="f32_nodes_one_map", bf16=False, R=17, B=1, n=260, maps=[(13, 17, 36)], D=132,
         bias=False, n_null=0, points="grid_nodes"),
    dict(name="bf16_two_maps", bf16=True, R=32, B=2, n=300, maps=[(8, 8, 64), (40, 24, 72)],
         D=264, bias=True, n_null=33, points="cell_centres"),
    dict(name="bf16_two_maps_one_chunk", bf16=True, R=16, B=1, n=200,
         maps=[(5, 7, 64), (16, 16, 8)], D=520, bias=False, n_null=0, points="cell_centres"),
    dict(name="bf16_two_maps_nodes", bf16=True, R=40, B=3, n=390,
         maps=[(16, 16, 128), (64, 48, 192)], D=136, bias=True, n_null=5, points="grid_nodes"),
    dict(name="f32_two_maps", bf16=False, R=24, B=2, n=270, maps=[(6, 6, 64), (31, 29, 36)],
         D=100, bias=True, n_null=7, points="cell_centres"),
    # 230 whole tiles on 256 compute units; map 0 is one K chunk, so the
    # switch to map 1 comes right after the consumers' chunk 0
    dict(name="bf16_two_maps_whole_tiles", bf16=True, R=48, B=2, n=230 * 128 - 3,
         maps=[(16, 16, 64), (40, 24, 72)], D=136, bias=True, n_null=200,
         points="cell_centres"),
    # 140 tiles of 128 tokens, run as 187 of 96 tokens, the same switch
    dict(name="bf16_two_maps_round_tiles", bf16=True, R=48, B=2, n=140 * 128 - 3,
         maps=[(16, 16, 64), (40, 24, 72)], D=136, bias=True, n_null=200,
         points="cell_centres"),
    # 70 tiles, run as 140 64-token parts, the same switch
    dict(name="bf16_two_maps_half_parts", bf16=True, R=48, B=2, n=70 * 128 - 3,
         maps=[(16, 16, 64), (40, 24, 72)], D=136, bias=True, n_null=200,
         points="cell_centres"),
]


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_proj_cond_nodes_and_maps(orc, case):
    say("proj_cond", case)
    rng = np.random.default_rng(len(case["name"]) * 7)
    R, B, n = case["R"], case["B"], case["n"]
    coords = synth.random_coords(R, B, n, seed=n + R)
    maps = [rng.standard_normal((B, h, w, c)).astype(np.float32) for h, w, c in case["maps"]]
    K = sum(c for _, _, c in case["maps"])
    Wf = (rng.standard_normal((case["D"], K)) * 0.05).astype(np.float32)
    bf = (rng.standard_normal(case["D"]) * 0.05).astype(np.float32) if case["bias"] else None
    if case["bf16"]:
        maps = [synth.bf16_bits(m) for m in maps]
        Wf = synth.bf16_bits(Wf)
        bf = synth.bf16_bits(bf) if bf is not None else None
    rows = np.arange(n + case["n_null"])
    _run(orc, coords, n, R, [40.0 + 4 * b for b in range(B)], [None] * B, maps, Wf, bf,
         case["n_null"], case["bf16"], rows, case["points"], case["maps"][0][1])


@pytest.mark.parametrize("name", [w.name for w in synth.EXTRA_WORKLOADS])
def test_proj_cond_extra_workloads(orc, name):
    """The cascade and two-map workloads at full size, in the launch
    configuration the benchmark times, on sampled rows."""
    w = synth.workload(name)
    coords = synth.coords(w)
    n = w.n_tokens
    if w.coords_resolution:
        coords = orc.requantize(coords, w.coords_resolution, w.resolution, "round_nodes")
    maps = synth.feature_maps(w)
    Wt, b = synth.weight(w), synth.bias(w)
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([rng.choice(n, 384, replace=False), [0, 127, 128, n - 1],
                                     [n, n + w.n_null - 1] if w.n_null else []]).astype(np.int64))
    say(name, "rows checked", len(rows))
    st = _run(orc, coords, n, w.resolution, synth.fovs(w), [None] * w.batch, maps, Wt, b,
              w.n_null, w.dtype == "bf16", rows, w.points, w.width)
    say("  max|diff|/max|Y| %.3e corr %.8f" % st)


@pytest.mark.parametrize("n", [1500, 9000, 20000, 28000],
                         ids=["quarter_parts", "half_parts", "round_tiles", "whole_tiles"])
@pytest.mark.parametrize("two_maps", [False, True], ids=["one_map", "two_maps"])
def test_proj_cond_map_of_4gib(orc, two_maps, n):
    """A bf16 map of exactly 4 GiB (1 x 1024 x 1024 x 2048): its corner
    offsets no longer fit 32 bits, so the fused kernel takes its 64-bit
    gather addressing (launches whose maps are all smaller take the 32-bit
    one). Alone, or as map 1 behind a small seeded 32 x 32 x 64 map 0; 12
    tiles of 128 tokens (run as 32-token parts), 71 (as 64-token parts), 157
    (as one round of 209 96-token tiles on 256 compute units) or 219 (run
    whole). The large map is zero except around the pixels the tokens
    project to (chosen by the oracle's projection), which hold seeded
    values; every row is checked."""
    B, H, W, C, D, R, n_null = 1, 1024, 1024, 2048, 264, 256, 7
    coords = synth.random_coords(R, B, n, seed=4242)
    fovs = [40.0]
    fo, do = oracle_cameras(orc, fovs, [None], W)
    pix = orc.project(coords, n, R, fo, do, H, W)["pixel"]
    say("4 GiB map: %d tokens, two maps %s" % (n, two_maps))
    feat = np.zeros((B, H, W, C), np.uint16)
    rng = np.random.default_rng(4243)
    ys = np.clip(pix[:, 1:2] + np.arange(-1, 3), 0, H - 1)
    xs = np.clip(pix[:, 0:1] + np.arange(-1, 3), 0, W - 1)
    rows = np.unique((ys[:, :, None] * W + xs[:, None, :]).reshape(-1))
    flat = feat.reshape(-1, C)
    flat[rows] = synth.bf16_bits(rng.standard_normal((len(rows), C)).astype(np.float32))
    maps = [feat]
    if two_maps:
        maps = [synth.bf16_bits(rng.standard_normal((B, 32, 32, 64)).astype(np.float32)), feat]
    K = sum(m.shape[3] for m in maps)
    Wt = synth.bf16_bits((rng.standard_normal((D, K)) * 0.05).astype(np.float32))
    b = synth.bf16_bits((rng.standard_normal(D) * 0.05).astype(np.float32))
    st = _run(orc, coords, n, R, fovs, [None], maps, Wt, b, n_null, True,
              np.arange(n + n_null), "cell_centres", W)
    say("  max|diff|/max|Y| %.3e corr %.8f" % st)
