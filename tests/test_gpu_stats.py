"""GPU parity of the projection diagnostics (p3d_projection_stats) against
the CPU oracle: token and in-frame counts exact; per-map sums and sums of
squares within 1e-5 of sum |S| for binary32 maps and within one bf16
rounding (2^-8 of sum |S|) for bf16 maps, where a sample's rounding may fall
on the other side of a tie between the kernel's binary32 blend and the
oracle's binary64 one; the cosine count exact, its mean within 1e-6 (fp32)
or 1e-3 (bf16); the printed figures (p3d_stats_figures on the GPU's sums)
against the oracle's derivation (orc_stats_figures on its sums) within the
bounds those sums imply."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import p3d_synth as synth
import pixel_aligned_image_amd as p3d
from parity_util import run_stats

pytestmark = pytest.mark.gpu


def say(*a):
    print("[stats]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def orc():
    o = oracle.get()
    o.set_threads(min(16, os.cpu_count() or 1))
    return o


def _check(o, coords, n, R, fovs, dists, maps_np, bf16, points, image_size):
    return run_stats(p3d, o, coords, n, R, fovs, dists, maps_np, bf16, points, image_size)


CASES = [
    dict(name="f32_one_map", bf16=False, R=24, B=2, n=1000, maps=[(17, 13, 36)], spill=3,
         points="cell_centres"),
    dict(name="bf16_one_map_nodes", bf16=True, R=33, B=1, n=777, maps=[(32, 32, 136)], spill=0,
         points="grid_nodes"),
    dict(name="bf16_two_maps_cosine", bf16=True, R=40, B=2, n=2049,
         maps=[(16, 16, 128), (64, 48, 128)], spill=2, points="cell_centres"),
    dict(name="f32_two_maps_cosine", bf16=False, R=20, B=3, n=300,
         maps=[(9, 9, 64), (30, 27, 64)], spill=0, points="cell_centres"),
    dict(name="bf16_two_maps_unequal", bf16=True, R=16, B=1, n=130,
         maps=[(8, 8, 64), (20, 20, 72)], spill=0, points="grid_nodes"),
    dict(name="bf16_wide_rows", bf16=True, R=64, B=1, n=70, maps=[(8, 8, 1032), (16, 16, 1032)],
         spill=0, points="cell_centres"),
]


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_stats_small(orc, case):
    say(case)
    rng = np.random.default_rng(len(case["name"]) * 13)
    B, n = case["B"], case["n"]
    coords = synth.random_coords(case["R"], B, n, seed=n, spill=case["spill"])
    maps = [rng.standard_normal((B, h, w, c)).astype(np.float32) + 0.1 * i
            for i, (h, w, c) in enumerate(case["maps"])]
    if case["bf16"]:
        maps = [synth.bf16_bits(m) for m in maps]
    _check(orc, coords, n, case["R"], [40.0 + 7 * b for b in range(B)], [None] * B, maps,
           case["bf16"], case["points"], case["maps"][0][1])


def test_stats_empty_zeroes(orc):
    stats = torch.full((8,), 5.0, dtype=torch.float64, device="cuda")
    feat = torch.zeros((1, 4, 4, 8), dtype=torch.bfloat16, device="cuda")
    p3d.p3d_projection_stats(torch.zeros((0, 4), dtype=torch.int32, device="cuda"), 0, 8,
                             [(2.0, 2.0)], feat, stats)
    torch.cuda.synchronize()
    assert np.all(stats.cpu().numpy() == 0.0)


@pytest.mark.parametrize("name", ["shell1024_cfg_twomap_bf16_c1024x2_d1536",
                                  "shell64x2_bf16_c2048_d1536"])
def test_stats_workloads(orc, name):
    w = synth.workload(name)
    coords = synth.coords(w)
    maps = synth.feature_maps(w)
    say(name, "tokens", w.n_tokens)
    got, want = _check(orc, coords, w.n_tokens, w.resolution, synth.fovs(w), [None] * w.batch,
                       maps, w.dtype == "bf16", w.points, w.width)
    say("  ", p3d.p3d_stats_figures(got, [m.shape[3] for m in maps]))
