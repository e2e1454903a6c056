"""HIP graph capture. The library's device calls only enqueue kernels (no
allocation, memset, copy or synchronisation inside a call), so a caller can
capture them in a graph and replay it. Each graph is replayed several times,
with eager work and synchronisations between the replays, and every replay
is checked bit for bit against the same calls run eagerly:
- the sorted fused call of one step (p3d_proj_cond_ws: four sort kernels,
  then the fused kernel and its null rows);
- a stage's per-step linears over samples gathered once (p3d_proj_sample,
  then p3d_proj_linear_grouped with the residual add, so every replay adds
  once more and is compared with the same number of eager adds).
"""
import sys

import numpy as np
import pytest
import torch

import p3d_synth as synth
import pixel_aligned_image_amd as p3d
from parity_util import product_cameras, to_dev

pytestmark = pytest.mark.gpu


def say(*a):
    print("[graph]", *a, flush=True)
    sys.stdout.flush()


def _bf16(rng, shape, scale=1.0):
    return to_dev(synth.bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32)), True)


def test_graph_of_the_sorted_fused_call():
    rng = np.random.default_rng(31)
    R, B, n, C, D, nn = 96, 2, 20000, 256, 776, 4000
    say("sorted fused call: n %d, C %d, D %d, null rows %d" % (n, C, D, nn))
    coords = to_dev(synth.random_coords(R, B, n, seed=32))
    feat = _bf16(rng, (B, 64, 64, C))
    W = _bf16(rng, (D, C), 0.05)
    bias = _bf16(rng, (D,), 0.05)
    cams = product_cameras(p3d, [38.0, 44.0], [None, None], 64)
    ws = p3d.proj_cond_workspace(n, B, feat)
    mask = torch.empty((n,), dtype=torch.uint8, device="cuda")
    ref = torch.empty((n + nn, D), dtype=torch.bfloat16, device="cuda")
    p3d.p3d_proj_cond(coords, n, R, cams, feat, W, ref, bias=bias, n_null=nn, mask=mask,
                      workspace=ws)
    torch.cuda.synchronize()
    ref_mask = mask.clone()
    out = torch.empty_like(ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                       # warm-up off the capture
        p3d.p3d_proj_cond(coords, n, R, cams, feat, W, out, bias=bias, n_null=nn, mask=mask,
                          workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        p3d.p3d_proj_cond(coords, n, R, cams, feat, W, out, bias=bias, n_null=nn, mask=mask,
                          workspace=ws)
    for r in range(4):
        out.fill_(float("nan"))
        mask.fill_(7)
        ws.fill_(0xA5)                                  # the sort must not rely on old contents
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), "replay %d" % r
        assert torch.equal(mask, ref_mask), "replay %d mask" % r
    say("  4 replays equal the eager call")


def test_graph_of_the_per_step_linears():
    rng = np.random.default_rng(33)
    R, B, n, D, G = 64, 1, 12000, 520, 3
    maps = [_bf16(rng, (B, 16, 16, 128)), _bf16(rng, (B, 48, 48, 64))]
    K = 192
    say("gather once + %d per-block linears: n %d, K %d, D %d" % (G, n, K, D))
    coords = to_dev(synth.random_coords(R, B, n, seed=34))
    cams = product_cameras(p3d, [40.0], [None], 48)
    S = torch.empty((n, K), dtype=torch.bfloat16, device="cuda")
    p3d.p3d_proj_sample(coords, n, R, cams, maps, S)
    Ws = [_bf16(rng, (D, K), 0.05) for _ in range(G)]
    bs = [_bf16(rng, (D,), 0.05) for _ in range(G)]
    Y0 = [_bf16(rng, (n, D)) for _ in range(G)]
    torch.cuda.synchronize()
    # eager: the residual add applied 1, 2, 3 and 4 times
    eager, Ye = [], [y.clone() for y in Y0]
    for r in range(4):
        p3d.p3d_proj_linear_grouped(S, Ws, Ye, biases=bs, accumulate=True)
        torch.cuda.synchronize()
        eager.append([y.clone() for y in Ye])
    Yg = [y.clone() for y in Y0]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                       # warm-up off the capture
        scratch = [y.clone() for y in Y0]
        p3d.p3d_proj_linear_grouped(S, Ws, scratch, biases=bs, accumulate=True)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        p3d.p3d_proj_linear_grouped(S, Ws, Yg, biases=bs, accumulate=True)
    torch.cuda.synchronize()
    for r in range(4):
        g.replay()
        torch.cuda.synchronize()
        _ = torch.zeros(1024, device="cuda").sum().item()   # eager work between replays
        for gi in range(G):
            assert torch.equal(Yg[gi].view(torch.int16), eager[r][gi].view(torch.int16)), \
                "replay %d block %d" % (r, gi)
    say("  4 replays equal 1..4 eager residual adds")
