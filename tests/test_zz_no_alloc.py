"""p3d_proj_cond_noalloc (the allocation-free entry point, scratch in a static
device array of the library) against p3d_proj_cond_ws (caller workspace),
called through the C ABI: two calls in a row, the second with fewer tokens,
so the second runs on scratch the first one left behind. Both must write the
same bytes in every output row and mask byte; the noalloc call also stays
within the fused path's bar against the oracle on sampled rows. Too many
tokens is refused before anything runs."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import p3d_synth as synth
import pixel_aligned_image_amd as p3d
from parity_util import (check_bf16_linear, oracle_cameras, product_cameras, to_dev, to_host)

pytestmark = pytest.mark.gpu


def say(*a):
    print("[noalloc]", *a, flush=True)


def _case(n_per_item, B, R, H, W, C, D, n_null, seed):
    rng = np.random.default_rng(seed)
    coords = synth.shell_coords(R, B, n_per_item, seed=seed)
    feat = synth.bf16_bits(rng.standard_normal((B, H, W, C)).astype(np.float32))
    weight = synth.bf16_bits((rng.standard_normal((D, C)) * 0.03).astype(np.float32))
    bias = synth.bf16_bits((rng.standard_normal(D) * 0.03).astype(np.float32))
    fovs = [40.0 + 3 * b for b in range(B)]
    return coords, feat, weight, bias, fovs, n_null


def test_noalloc_matches_workspace_path_twice():
    o = oracle.get()
    o.set_threads(min(16, os.cpu_count() or 1))
    # the second call is the smaller one: it reuses the scratch of the first
    for k, (npi, B, R, H, W, C, D, nn, seed) in enumerate([
            (12000, 2, 128, 96, 80, 520, 776, 3000, 11),
            (1500, 1, 64, 40, 48, 136, 264, 77, 12)]):
        coords, feat, weight, bias, fovs, n_null = _case(npi, B, R, H, W, C, D, nn, seed)
        n = coords.shape[0]
        say("call %d: n = %d, null rows %d, map %s, D %d" % (k + 1, n, n_null, feat.shape, D))
        cams = product_cameras(p3d, fovs, [None] * B, W)
        args = (to_dev(coords), n, R, cams, to_dev(feat, True), to_dev(weight, True))
        outs, masks = [], []
        for mode in ("workspace", "noalloc"):
            out = torch.full((n + n_null, D), float("nan"), dtype=torch.bfloat16, device="cuda")
            mask = torch.full((n,), 7, dtype=torch.uint8, device="cuda")
            kw = dict(bias=to_dev(bias, True), n_null=n_null, mask=mask)
            if mode == "workspace":
                kw["workspace"] = p3d.proj_cond_workspace(n, B, args[4])
            else:
                kw["noalloc"] = True
            p3d.p3d_proj_cond(*args, out, **kw)
            outs.append(out)
            masks.append(mask)
        torch.cuda.synchronize()
        assert not torch.isnan(outs[1].float()).any().item(), "unwritten output"
        assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)), "rows differ"
        assert torch.equal(masks[0], masks[1]), "masks differ"
        # the fused path's bar against the oracle on seeded rows
        rows = np.unique(np.concatenate([np.random.default_rng(seed).choice(n, 600, replace=False),
                                         [0, n - 1, n, n + n_null - 1]]))
        fo, do = oracle_cameras(o, fovs, [None] * B, W)
        Yref, mref = o.proj_cond_rows(coords, n, R, fo, do, feat, weight, bias, n_null, rows)
        got = to_host(outs[1][torch.from_numpy(rows).cuda()])
        tok = rows < n
        assert np.array_equal(to_host(masks[1])[rows[tok]], mref[tok])
        assert np.array_equal(got[~tok], np.broadcast_to(bias, ((~tok).sum(), D)))
        check_bf16_linear(got[tok], Yref[tok])
        say("  call %d: every row and mask byte equals the workspace path; %d rows checked "
            "against the oracle" % (k + 1, len(rows)))


def test_noalloc_refuses_too_many_tokens():
    feat = torch.zeros((1, 8, 8, 16), dtype=torch.bfloat16, device="cuda")
    weight = torch.zeros((32, 16), dtype=torch.bfloat16, device="cuda")
    n = p3d.P3D_NOALLOC_MAX_TOKENS + 1
    out = torch.zeros((1, 32), dtype=torch.bfloat16, device="cuda")
    # the size check runs before any pointer is touched: tiny buffers suffice
    cams = p3d.make_cameras([(2.0, 2.0)])
    maps = (p3d.p3d_map * 1)()
    maps[0].feat, maps[0].height, maps[0].width, maps[0].channels = feat.data_ptr(), 8, 8, 16
    coords = torch.zeros((1, 4), dtype=torch.int32, device="cuda")
    st = p3d.lib.p3d_proj_cond_noalloc(coords.data_ptr(), n, 8, 0, cams, 1, p3d.P3D_BF16, maps,
                                       1, weight.data_ptr(), 32, 16, None, 0, out.data_ptr(),
                                       None, None)
    assert st == p3d.P3D_ERR_UNSUPPORTED
    msg = p3d.p3d_last_error()
    assert "P3D_NOALLOC_MAX_TOKENS" in msg and str(n) in msg
