"""Shared helpers of the GPU parity tests: seeded inputs from p3d_synth, the
two independent camera constructions, host<->device transfers and the
tolerance checks. Each side computes from the same drawn inputs; nothing the
GPU produces is ever fed to the oracle."""
import numpy as np
import torch

import p3d_synth as synth


def to_dev(a, bf16=False):
    """numpy -> cuda tensor; uint16 arrays holding bf16 bits -> bfloat16."""
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    if bf16:
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.cuda()


def to_host(t):
    """cuda tensor -> numpy (bfloat16 -> uint16 bits)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32).astype(np.float64)


def distances_spec(w):
    return [w.distance] * w.batch


def product_cameras(p3d, fovs, dists, image_size):
    cams = []
    for a, d in zip(fovs, dists):
        if d is None:
            d = p3d.p3d_distance_from_fov(a, image_size, 0)
        cams.append(p3d.p3d_make_camera(a, d))
    return cams


def oracle_cameras(o, fovs, dists, image_size):
    fs, ds = [], []
    for a, d in zip(fovs, dists):
        if d is None:
            d = o.distance_from_fov(a, image_size, 0)
        f, dd = o.camera(a, d)
        fs.append(f)
        ds.append(dd)
    return np.array(fs, np.float32), np.array(ds, np.float32)


class Inputs:
    """Seeded inputs of one workload (numpy, host)."""

    def __init__(self, w):
        self.w = w
        self.coords = synth.coords(w)
        self.n = w.n_tokens
        self.n_null = w.n_null
        self.feat = synth.feature_map(w)
        self.weight = synth.weight(w)
        self.bias = synth.bias(w)
        self.fovs = synth.fovs(w)
        self.dists = distances_spec(w)
        self.bf16 = w.dtype == "bf16"


def check_fp32_linear(Y_gpu, Y_orc, absmag, tol=1e-5):
    """|Y_gpu - Y| <= tol * (sum_c |W||S| + |b|) per element."""
    err = np.abs(Y_gpu.astype(np.float64) - Y_orc)
    bad = err > tol * absmag + 1e-30
    assert not bad.any(), "fp32 proj_linear: %d elements off, worst %.3e (bound %.3e)" % (
        bad.sum(), (err / (absmag + 1e-30)).max(), tol)


def check_bf16_linear(Y_gpu_bits, Y_orc, tol=2e-2):
    """bf16 proj_linear output: per element |Y_gpu - Y| <= tol (|Y| + rms of
    its row), and max |diff| / max |Y| <= tol over the whole output."""
    Yg = bf16_to_f64(Y_gpu_bits)
    err = np.abs(Yg - Y_orc)
    rms = np.sqrt(np.mean(Y_orc ** 2, axis=1, keepdims=True))
    bad = err > tol * (np.abs(Y_orc) + rms)
    assert not bad.any(), "bf16 proj_linear: %d elements off, worst rel %.3e" % (
        bad.sum(), (err / (np.abs(Y_orc) + rms + 1e-30)).max())
    scale = np.abs(Y_orc).max()
    assert err.max() <= tol * scale, "bf16 proj_linear: max|diff| %.3e vs max|Y| %.3e" % (
        err.max(), scale)
    return err.max() / max(scale, 1e-30), np.corrcoef(Yg.ravel(), Y_orc.ravel())[0, 1]


def run_fused(p3d, o, coords, n, R, fovs, dists, maps_np, W_np, b_np, n_null, bf16, rows,
              points, image_size):
    """One p3d_proj_cond call (one map, or a list of two) on the GPU against the
    oracle's rows `rows`: every checked row must have been written (out starts
    as NaN), masks bit-exact, null rows equal to the bias bit for bit, token
    rows within the bf16 / fp32 tolerances. Returns the bf16 statistics."""
    D = W_np.shape[0]
    cp = product_cameras(p3d, fovs, dists, image_size)
    fo, do = oracle_cameras(o, fovs, dists, image_size)
    dt = torch.bfloat16 if bf16 else torch.float32
    out = torch.full((n + n_null, D), float("nan"), dtype=dt, device="cuda")
    mask = torch.full((n,), 7, dtype=torch.uint8, device="cuda")
    feats = [to_dev(m, bf16) for m in maps_np]
    p3d.p3d_proj_cond(to_dev(coords), n, R, cp, feats if len(feats) > 1 else feats[0],
                      to_dev(W_np, bf16), out, bias=to_dev(b_np, bf16), n_null=n_null,
                      mask=mask, points=points)
    torch.cuda.synchronize()
    Yref, mref = o.proj_cond_rows(coords, n, R, fo, do, list(maps_np), W_np, b_np, n_null, rows,
                                  points=points)
    got = to_host(out[torch.from_numpy(rows).cuda()])
    tok = rows < n
    assert np.array_equal(to_host(mask)[rows[tok]], mref[tok]), "mask differs"
    null = ~tok
    if null.any():
        want = b_np if b_np is not None else np.zeros(D, W_np.dtype)
        assert np.array_equal(got[null], np.broadcast_to(want, (null.sum(), D))), "null rows"
    if not tok.any():
        return None
    if bf16:
        return check_bf16_linear(got[tok], Yref[tok])
    absmaps = [np.abs(m) for m in maps_np]
    S = o.proj_cond_rows(coords, n, R, fo, do, absmaps, np.abs(W_np),
                         None if b_np is None else np.abs(b_np), n_null, rows[tok],
                         points=points)[0]
    check_fp32_linear(got[tok], Yref[tok], S)
    return None


def run_stats(p3d, o, coords, n, R, fovs, dists, maps_np, bf16, points, image_size,
              order=None):
    """p3d_projection_stats (p3d_projection_stats_ordered with a device
    order) on the GPU against the oracle: counts exact, sums within 1e-5
    (fp32) or one bf16 rounding (2^-8) of sum |S|, the cosine count exact and
    its mean within 1e-6 / 1e-3. Returns (got, want)."""
    cp = product_cameras(p3d, fovs, dists, image_size)
    fo, do = oracle_cameras(o, fovs, dists, image_size)
    stats = torch.full((8,), float("nan"), dtype=torch.float64, device="cuda")
    feats = [to_dev(m, bf16) for m in maps_np]
    p3d.p3d_projection_stats(to_dev(coords), n, R, cp, feats, stats, points=points, order=order)
    torch.cuda.synchronize()
    got = dict(zip(p3d.STAT_FIELDS, stats.cpu().numpy().tolist()))
    want = o.projection_stats(coords, n, R, fo, do, list(maps_np), points=points)
    assert got["tokens"] == want["tokens"] == n
    assert got["inside"] == want["inside"]
    tol = 2.0 ** -8 if bf16 else 1e-5
    for h in range(len(maps_np)):
        c = maps_np[h].shape[3]
        mag = np.sqrt(n * c * want["sum_sq%d" % h])        # >= sum |S|
        assert abs(got["sum%d" % h] - want["sum%d" % h]) <= tol * mag + 1e-300, h
        assert abs(got["sum_sq%d" % h] - want["sum_sq%d" % h]) <= 2 * tol * want["sum_sq%d" % h] \
            + 1e-300, h
    assert got["cos_count"] == want["cos_count"]
    if want["cos_count"]:
        dc = abs(got["cos_sum"] - want["cos_sum"]) / want["cos_count"]
        assert dc <= (1e-3 if bf16 else 1e-6), dc
    else:
        assert got["cos_sum"] == 0.0
    # the printed figures: the library's p3d_stats_figures on the GPU's sums
    # against the oracle's own derivation on its sums. With the sums' bounds
    # above: |d mean| <= tol rms, |d std^2| <= 4 tol E[x^2], so
    # |d std| <= 2 tol E[x^2] / std.
    ch = [m.shape[3] for m in maps_np]
    gf = p3d.p3d_stats_figures(stats, ch)
    wf = o.stats_figures(want, ch)
    assert gf["coverage"] == wf["coverage"]
    for h in range(2):
        if h >= len(ch):
            assert gf["mean%d" % h] is None and gf["std%d" % h] is None
            continue
        e2 = want["sum_sq%d" % h] / (n * ch[h])
        assert abs(gf["mean%d" % h] - wf["mean%d" % h]) <= tol * np.sqrt(e2) + 1e-300, h
        assert abs(gf["std%d" % h] - wf["std%d" % h]) <= \
            2 * tol * e2 / max(wf["std%d" % h], 1e-300) + 1e-300, h
    if want["cos_count"]:
        assert abs(gf["cosine"] - wf["cosine"]) <= (1e-3 if bf16 else 1e-6)
    else:
        assert gf["cosine"] is None and wf["cosine"] is None
    return got, want


def run_sample(p3d, o, feat_np, grid_np, bidx_np, bf16_in, out_bf16):
    """p3d_bilinear_sample of feat_np at grid_np (batch indices bidx_np or
    None) against the oracle: every value within 1e-5 of sum_k w_k |F_k|,
    plus one bf16 rounding (2^-8 |ref|) for bf16 output. Returns the largest
    error and the correlation."""
    n = len(grid_np)
    feat = to_dev(feat_np, bf16=bf16_in)
    grid = to_dev(grid_np.astype(np.float32))
    bidx = to_dev(bidx_np) if bidx_np is not None else None
    C = feat_np.shape[-1]
    out = torch.empty((n, C), dtype=torch.bfloat16 if out_bf16 else torch.float32,
                      device="cuda")
    p3d.p3d_bilinear_sample(feat, grid, out, batch_index=bidx)
    torch.cuda.synchronize()
    got = to_host(out)
    ref = o.sample(feat_np, grid_np, bidx_np)
    absf = np.abs(bf16_to_f64(feat_np) if bf16_in else feat_np.astype(np.float64))
    mag = o.sample(absf.astype(np.float32), grid_np, bidx_np)      # sum_k w_k |F_k|
    g = bf16_to_f64(got) if out_bf16 else got.astype(np.float64)
    err = np.abs(g - ref)
    bound = 1e-5 * mag + (2.0 ** -8 * np.abs(ref) if out_bf16 else 0.0) + 1e-30
    assert np.all(err <= bound), "sample: %d off, worst %.3e" % ((err > bound).sum(),
                                                                (err / bound).max())
    return np.max(err), np.corrcoef(g.ravel(), ref.ravel())[0, 1] if g.size > 1 else 1.0


def tile_edge_rows(n, D, cus):
    """First and last token row of every whole tile and of every tail part of
    the fused bf16 launch of n tokens and D features on `cus` compute units,
    as the library's tiling rule (p3d_proj_cond_plan) cuts it."""
    import pixel_aligned_image_amd as p3d
    plan = p3d.p3d_proj_cond_plan(n, D, cus)
    bm, nt = plan["tile_rows"], plan["feature_tiles"]
    first_split = plan["whole_tiles"] // nt          # token tiles before the split ones
    rows = []
    for mt in range(plan["token_tiles"]):
        step = plan["part_rows"] if plan["parts"] and mt >= first_split else bm
        for lo in range(mt * bm, min((mt + 1) * bm, n), step):
            rows += [lo, min(lo + step, n) - 1]
    return np.unique(np.array(rows, np.int64))
