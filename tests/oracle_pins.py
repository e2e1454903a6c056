"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Every pin is a function ``pin_<name>(o)`` taking an ``oracle.Oracle`` and
raising AssertionError when the oracle disagrees with:
  * values the pages print (the camera-distance worked example),
  * closed forms that follow from the pages' statements (corner registration
    at the closed-form distance, the half-texel mapping, border clamping of
    the source index, on-axis points at the image centre, the -Z view),
  * brute force (bilinear weights as tent functions summed over every pixel),
  * library routines the special cases reduce to (torch grid_sample on CPU,
    numpy float64 matmul, torch's bfloat16 rounding).
The same functions run against deliberately broken oracle builds (see
test_oracle_mutants.py) to show that each plausible mistake fails one of them.

Sources, by page title and section:
  pixal3d_mrp_mlx, history of tests/, commit landing the pixel-aligned head
    (grid_sample mapping, border clamp of the source index, -Z camera);
  trellis.cpp PR #38 "Initial support for Pixal3D": commit adding pixal3d.cpp
    (closed-form camera solve), commit exposing extend_pixel (worked example),
    commit adding projection diagnostics (cube corners legitimately leave the
    frame), commit introducing FlowCond (null proj zeroed), commit on the
    cascade requantization (endpoint-inclusive projection grid, nearest-node
    rounding; a quarter of the coordinates per axis and 58 % of tokens move
    under flooring at grid 64, in stripes of period 8), commit adding the NAF
    upsampler (two maps concatenated into 2048 proj channels).
"""
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rel(a, b, scale):
    return np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)) / scale)


# ----------------------------------------------------------------- camera ---
def pin_camera_distance_worked_example(o):
    """The printed distances at 49.13 deg / 512 px / e = 0, 64, 128."""
    rows = [l.split() for l in open(os.path.join(GOLDEN, "camera_distance.txt"))
            if l.strip() and not l.startswith("#")]
    assert len(rows) == 3
    for fov, size, ext, printed in rows:
        d = o.distance_from_fov(float(fov), int(size), int(ext))
        assert abs(d - float(printed)) <= 5e-4 + 1e-12, (fov, size, ext, d, printed)
        assert "%.3f" % d == printed, (d, printed)


def pin_corner_registration(o):
    """At the closed-form distance the cube's z = 0 corners land on the frame
    border (|g| -> 1), which holds only for focal = 1/tan(fov/2) with the
    full-angle FOV, depth = d - z and unit-cube extent +-1/2. Cell centres
    approach the corner as 1/2 - 1/(2R); the exact g is 1 - 1/R."""
    R = 1001
    mid = (R - 1) // 2
    cells = np.array([[0, R - 1, R - 1, mid], [0, 0, 0, mid],
                      [0, R - 1, 0, mid], [0, 0, R - 1, mid]], np.int32)
    for fov in (30.0, 40.0, 49.13, 60.0):
        f, d = o.camera(fov, o.distance_from_fov(fov, 512, 0))
        p = o.project(cells, 4, R, [f], [d], 64, 64)
        want = 1.0 - 1.0 / R
        sx = np.array([1, -1, 1, -1])
        sy = np.array([-1, 1, 1, -1])
        assert _rel(p["grid"][:, 0], sx * want, 1.0) < 2e-6, (fov, p["grid"])
        assert _rel(p["grid"][:, 1], sy * want, 1.0) < 2e-6, (fov, p["grid"])
        assert p["mask"].tolist() == [1, 1, 1, 1]


def pin_near_far_corners(o):
    """Camera at +d looking down -Z: the near face (z = +1/2) is magnified past
    the border and the far face (z = -1/2) shrinks inside it, so near corners
    fall outside the frame (as the pages say they legitimately do) and far
    corners inside. Exact closed form in binary64 for the cell centres."""
    R = 64
    h = 0.5 - 0.5 / R
    for fov in (30.0, 40.0, 50.0):
        f, d = o.camera(fov, o.distance_from_fov(fov, 512, 0))
        cells = np.array([[0, R - 1, R - 1, R - 1], [0, 0, 0, R - 1],
                          [0, R - 1, R - 1, 0], [0, 0, 0, 0]], np.int32)
        p = o.project(cells, 4, R, [f], [d], 128, 128)
        near = float(f) * h / (float(d) - h)
        far = float(f) * h / (float(d) + h)
        assert near > 1.0 > far
        want_x = np.array([near, -near, far, -far])
        want_y = -want_x
        assert _rel(p["grid"][:, 0], want_x, 1.0) < 2e-6, (fov, p["grid"], want_x)
        assert _rel(p["grid"][:, 1], want_y, 1.0) < 2e-6
        assert _rel(p["depth"], [d - h, d - h, d + h, d + h], 1.0) < 1e-6
        assert p["mask"].tolist() == [0, 0, 1, 1]


def pin_on_axis_centre(o):
    """Points on the optical axis (x = y = 0, odd R) land exactly on the image
    centre: g = (0, 0), source index (W-1)/2, i.e. for even W the corners
    W/2-1 and W/2 with fraction 1/2; for odd W the centre texel, fraction 0."""
    R = 5
    c = (R - 1) // 2
    cells = np.array([[0, c, c, z] for z in range(R)], np.int32)
    for H, W in ((1, 1), (2, 2), (3, 3), (8, 8), (3, 8), (8, 3)):
        p = o.project(cells, R, R, [2.0], [1.7], H, W)
        assert np.all(p["grid"] == 0.0), p["grid"]
        for axis, size in ((0, W), (1, H)):
            want_i0 = (size - 1) // 2
            want_t = 0.5 if size % 2 == 0 else 0.0
            assert np.all(p["pixel"][:, axis] == want_i0), (H, W, p["pixel"])
            assert np.all(p["frac"][:, axis] == want_t), (H, W, p["frac"])
        assert np.all(p["mask"] == 1)


def pin_view_handedness(o):
    """Looking down -Z from +Z: world +x appears on the right half of the
    image (a camera looking down +Z would mirror it), world +y on the top
    rows; mirrored cells give mirrored normalised coordinates."""
    R = 16
    rng = np.random.default_rng(7)
    cells = np.concatenate([np.zeros((200, 1), np.int32),
                            rng.integers(0, R, size=(200, 3)).astype(np.int32)], axis=1)
    mirror = cells.copy()
    mirror[:, 1] = R - 1 - cells[:, 1]
    f, d = o.camera(40.0, 2.0)
    p = o.project(cells, 200, R, [f], [d], 32, 32)
    q = o.project(mirror, 200, R, [f], [d], 32, 32)
    x = (cells[:, 1] + 0.5) / R - 0.5
    y = (cells[:, 2] + 0.5) / R - 0.5
    assert np.all(np.sign(p["grid"][:, 0]) == np.sign(x))
    assert np.all(np.sign(p["grid"][:, 1]) == -np.sign(y))
    ix = p["pixel"][:, 0] + p["frac"][:, 0]
    iy = p["pixel"][:, 1] + p["frac"][:, 1]
    assert np.all((ix > 15.5) == (x > 0)) and np.all((iy < 15.5) == (y > 0))
    assert _rel(p["grid"][:, 0], -q["grid"][:, 0], 1.0) < 1e-6
    assert _rel(p["grid"][:, 1], q["grid"][:, 1], 1.0) == 0.0


def pin_mask_bounds(o):
    """Mask = depth > 0 and both normalised coordinates within [-1, 1]
    (inclusive). With focal 2, distance 3/4 and R = 2, the cell (1, 1, 1) sits
    at (1/4, 1/4, 1/4): depth 1/2 and g = (1, -1) exactly."""
    p = o.project(np.array([[0, 1, 1, 1], [0, 0, 0, 1]], np.int32), 2, 2,
                  [2.0], [0.75], 4, 4)
    assert p["grid"].tolist() == [[1.0, -1.0], [-1.0, 1.0]]
    assert p["mask"].tolist() == [1, 1]
    # distance 0.3: the near half of the cube is behind the camera.
    R = 8
    cells = np.array([[0, 3, 4, z] for z in range(R)], np.int32)
    p = o.project(cells, R, R, [1.0], [0.3], 16, 16)
    pz = (np.arange(R) + 0.5) / R - 0.5
    assert np.all((p["depth"] > 0) == (0.3 - pz > 0))
    assert np.all(p["mask"][0.3 - pz <= 0] == 0)
    assert np.any(p["mask"][0.3 - pz > 0] == 1)


def pin_dense_order_and_batch(o):
    """Dense enumeration n = ((b R + x) R + y) R + z equals explicit coords
    in that order; each batch item uses its own camera; a batch column
    outside [0, batch) is masked out."""
    R, B = 4, 2
    n = B * R ** 3
    t = np.arange(n)
    coords = np.stack([t // R ** 3, (t // R ** 2) % R, (t // R) % R, t % R], 1).astype(np.int32)
    fo, di = [1.5, 2.5], [1.2, 2.0]
    a = o.project(None, n, R, fo, di, 8, 8)
    b = o.project(coords, n, R, fo, di, 8, 8)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    solo = o.project(coords[R ** 3:] * np.array([0, 1, 1, 1], np.int32), R ** 3, R,
                     [fo[1]], [di[1]], 8, 8)
    assert np.array_equal(solo["grid"], a["grid"][R ** 3:])
    bad = coords[:3].copy()
    bad[:, 0] = [-1, 2, 7]
    p = o.project(bad, 3, R, fo, di, 8, 8)
    assert p["mask"].tolist() == [0, 0, 0]


# ----------------------------------------------------------- index mapping ---
def pin_half_texel(o):
    """align_corners=False: g = -1 + (2k+1)/W is the centre of texel k, so the
    source index is exactly k (fraction 0) and the sample is F[k]."""
    for W in (1, 2, 4, 8, 512):
        for k in range(W):
            g = np.float32(-1.0 + (2 * k + 1) / W)
            i0, i1, t = o.source_index(g, W)
            assert (i0, i1, t) == (k, min(k + 1, W - 1), 0.0), (W, k, i0, i1, t)
    for W in (3, 5, 7, 13):
        feat = np.arange(W, dtype=np.float32).reshape(1, 1, W, 1)
        g = np.array([[-1.0 + (2 * k + 1) / W, 0.0] for k in range(W)], np.float32)
        s = o.sample(feat, g)[:, 0]
        assert _rel(s, np.arange(W), 1.0) < 1e-5, (W, s)


def pin_not_align_corners(o):
    """On the map F[x] = x, g = -0.875 (W = 8) samples 0.0 and g = 0.5 samples
    5.5; align_corners=True would give 0.4375 and 5.25."""
    feat = np.arange(8, dtype=np.float32).reshape(1, 1, 8, 1)
    s = o.sample(feat, np.array([[-0.875, 0.0], [0.5, 0.0]], np.float32))[:, 0]
    assert s.tolist() == [0.0, 5.5], s


def pin_border_clamp_index(o):
    """padding_mode='border' clamps the SOURCE INDEX before the corners are
    taken: any g at or beyond the border gives the edge texel with fraction 0
    (clamping the corners afterwards would give fraction 1/2 at g = +-1 and
    other weights further out); NaN clamps to texel 0."""
    for W in (1, 2, 3, 8, 64):
        for g in (1.0, 1.05, 3.0, 5.0, 1e30, math.inf):
            assert o.source_index(g, W) == (W - 1, W - 1, 0.0), (W, g, o.source_index(g, W))
        for g in (-1.0, -1.05, -3.0, -5.0, -1e30, -math.inf, math.nan):
            assert o.source_index(g, W) == (0, min(1, W - 1), 0.0), (W, g)
    # inside the outer half texel: clamped to the edge texel, weight 0 on the
    # (clamped) neighbour
    assert o.source_index(np.float32(-1.0 + 0.5 / 8), 8) == (0, 1, 0.0)
    i0, i1, t = o.source_index(np.float32(1.0 - 0.5 / 8), 8)
    assert (i0, i1, t) == (7, 7, 0.0)


# ---------------------------------------------------------------- sampling ---
def _grid(rng, n, lo=-1.3, hi=1.3):
    return rng.uniform(lo, hi, size=(n, 2)).astype(np.float32)


def _ix(g, size):
    ix = ((g.astype(np.float64) + 1.0) * size - 1.0) / 2.0
    return np.clip(ix, 0.0, size - 1.0)


def pin_constant_map(o):
    rng = np.random.default_rng(11)
    for dt in (np.float32, np.uint16):
        for (B, H, W, C) in ((1, 5, 7, 3), (2, 8, 8, 4)):
            k = np.float32(rng.uniform(-4, 4))
            if dt == np.uint16:
                feat = np.full((B, H, W, C), o.f32_to_bf16(np.array([k]))[0], np.uint16)
                k = o.bf16_to_f32(feat.ravel()[:1])[0]
            else:
                feat = np.full((B, H, W, C), k, np.float32)
            g = _grid(rng, 300)
            bi = rng.integers(0, B, size=300).astype(np.int32)
            s = o.sample(feat, g, bi)
            assert _rel(s, k, abs(float(k))) < 4 * 2.0 ** -24, (dt, k)


def pin_linear_ramp_map(o):
    """F = a_c x + b_c (resp. y): bilinear interpolation reproduces the ramp at
    the clamped source index exactly (up to binary32 weights)."""
    rng = np.random.default_rng(12)
    for (H, W) in ((1, 1), (2, 3), (7, 5), (16, 16)):
        C = 3
        a = rng.uniform(-2, 2, C)
        b = rng.uniform(-2, 2, C)
        xs = np.arange(W, dtype=np.float64)
        ys = np.arange(H, dtype=np.float64)
        fx = (a[None, None, :] * xs[None, :, None] + b).astype(np.float32)
        fx = np.broadcast_to(fx, (H, W, C))[None].copy()
        fy = (a[None, None, :] * ys[:, None, None] + b).astype(np.float32)
        fy = np.broadcast_to(fy, (H, W, C))[None].copy()
        g = _grid(rng, 400, -1.5, 1.5)
        sx = o.sample(fx, g)
        sy = o.sample(fy, g)
        wx = a[None, :] * _ix(g[:, 0], W)[:, None] + b[None, :]
        wy = a[None, :] * _ix(g[:, 1], H)[:, None] + b[None, :]
        scale = np.abs(a).max() * max(H, W) + np.abs(b).max()
        assert _rel(sx, wx, scale) < 1e-6, (H, W)
        assert _rel(sy, wy, scale) < 1e-6, (H, W)


def _tent(u):
    return np.maximum(0.0, 1.0 - np.abs(u))


def pin_brute_force_tent(o):
    """Bilinear sampling = sum over EVERY texel of tent(ix - j) tent(iy - i)
    F[i, j], with (ix, iy) the border-clamped source index."""
    rng = np.random.default_rng(13)
    for (B, H, W, C) in ((1, 2, 2, 2), (2, 3, 5, 3), (1, 8, 8, 4), (2, 1, 6, 2)):
        feat = rng.standard_normal((B, H, W, C)).astype(np.float32)
        g = _grid(rng, 200, -1.6, 1.6)
        bi = rng.integers(0, B, size=200).astype(np.int32)
        s = o.sample(feat, g, bi)
        ix = _ix(g[:, 0], W)
        iy = _ix(g[:, 1], H)
        wx = _tent(ix[:, None] - np.arange(W)[None, :])      # [n, W]
        wy = _tent(iy[:, None] - np.arange(H)[None, :])      # [n, H]
        want = np.einsum("nh,nw,nhwc->nc", wy, wx, feat[bi].astype(np.float64))
        # the oracle's source index is binary32 (an ulp of W-1 moves a weight
        # by ~W 2^-24), the tent sums use the binary64 index
        assert _rel(s, want, np.abs(feat).max()) < 1e-5, (B, H, W, C)


def pin_torch_grid_sample(o):
    """torch.nn.functional.grid_sample(bilinear, align_corners=False,
    padding_mode='border') on CPU, the routine the pages diffed against."""
    import torch
    rng = np.random.default_rng(14)
    for (B, H, W, C, n) in ((1, 8, 8, 4, 300), (2, 13, 9, 3, 300), (1, 1, 7, 2, 50),
                            (2, 32, 32, 16, 500)):
        feat = rng.standard_normal((B, H, W, C)).astype(np.float32)
        g = _grid(rng, n, -1.4, 1.4)
        bi = rng.integers(0, B, size=n).astype(np.int32)
        s = o.sample(feat, g, bi)
        inp = torch.from_numpy(feat).permute(0, 3, 1, 2).contiguous()
        want = np.empty((n, C))
        for b in range(B):
            sel = np.nonzero(bi == b)[0]
            gr = torch.from_numpy(g[sel]).reshape(1, 1, -1, 2)
            r = torch.nn.functional.grid_sample(inp[b:b + 1], gr, mode="bilinear",
                                                padding_mode="border", align_corners=False)
            want[sel] = r[0, :, 0, :].T.double().numpy()
        scale = np.abs(feat).max()
        assert _rel(s, want, scale) < 1e-6, (B, H, W, C)


# ------------------------------------------------------------------ linear ---
def pin_numpy_matmul(o):
    rng = np.random.default_rng(15)
    for (n, C, D, bf16, with_bias) in ((7, 16, 32, False, True), (33, 64, 48, True, True),
                                       (5, 8, 16, True, False), (1, 4, 4, False, False)):
        S = rng.standard_normal((n, C))
        Wf = (rng.standard_normal((D, C)) * 0.02).astype(np.float32)
        bf = (rng.standard_normal(D) * 0.02).astype(np.float32)
        if bf16:
            Wq, bq = o.f32_to_bf16(Wf), o.f32_to_bf16(bf)
            Wd, bd = o.bf16_to_f32(Wq).astype(np.float64), o.bf16_to_f32(bq).astype(np.float64)
        else:
            Wq, bq, Wd, bd = Wf, bf, Wf.astype(np.float64), bf.astype(np.float64)
        Y = o.linear(S, Wq, bq if with_bias else None)
        want = S @ Wd.T + (bd if with_bias else 0.0)
        scale = np.abs(S) @ np.abs(Wd).T + (np.abs(bd) if with_bias else 0.0)
        assert np.max(np.abs(Y - want) / scale) < 1e-12


# -------------------------------------------------------------------- bf16 ---
def pin_bf16_rounding(o):
    """binary32 -> bf16 against torch's round-to-nearest-even conversion, on
    ties, subnormals, overflow to infinity, infinities and NaN; binary64 ->
    bf16 against the nearest-even bf16 found by brute force."""
    import torch
    edge = np.array([0.0, -0.0, 1.0, -1.0, 1.00390625, 1.01171875, 1.0 + 2 ** -8,
                     1.0 + 3 * 2 ** -8, 3.3895314e38, 3.3961776e38, 3.4e38, 1e-40, -1e-40,
                     1.18e-38, 2 ** -133, np.inf, -np.inf], np.float32)
    rng = np.random.default_rng(16)
    x = np.concatenate([edge, (rng.standard_normal(4000) * 10.0 ** rng.integers(-30, 30, 4000)
                               ).astype(np.float32)])
    got = o.f32_to_bf16(x)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
    nan = o.f32_to_bf16(np.array([np.nan], np.float32))[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x007F) != 0
    # binary64: candidates are the bf16 values bracketing x
    xd = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-20, 20, 3000),
                         1.0 + np.array([2 ** -8, 3 * 2 ** -8, 2 ** -8 + 2 ** -40,
                                         2 ** -8 - 2 ** -40, 2 ** -9 * 3])])
    got = o.f64_to_bf16(xd)
    for v, gbits in zip(xd, got):
        t = np.float32(v)
        base = int(np.array([t], np.float32).view(np.uint32)[0] >> 16)
        cands = [(base + k) & 0xFFFF for k in (-1, 0, 1, 2)]
        vals = [float(o.bf16_to_f32(np.array([c], np.uint16))[0]) for c in cands]
        errs = [abs(val - v) for val in vals]
        best = min(errs)
        ties = [c for c, e in zip(cands, errs) if e == best]
        pick = ties[0] if len(ties) == 1 else [c for c in ties if c % 2 == 0][0]
        assert gbits == pick, (v, gbits, pick)


# -------------------------------------------------------------- whole path ---
def pin_whole_path_composition(o):
    """Whole path on a tiny dense 2^3 grid and a few sparse cells equals the
    library composition: the oracle's projection, torch grid_sample (the
    pages' reference routine) on CPU, bf16 rounding by torch, numpy matmul;
    null rows equal the bias exactly."""
    import torch
    rng = np.random.default_rng(17)
    for dt in ("f32", "bf16"):
        R, B, H, W, C, D = 2, 1, 6, 6, 16, 32
        n = B * R ** 3
        featf = rng.standard_normal((B, H, W, C)).astype(np.float32)
        Wf = (rng.standard_normal((D, C)) * 0.1).astype(np.float32)
        bf = (rng.standard_normal(D) * 0.1).astype(np.float32)
        if dt == "bf16":
            feat, Wq, bq = o.f32_to_bf16(featf), o.f32_to_bf16(Wf), o.f32_to_bf16(bf)
            featv = o.bf16_to_f32(feat)
            Wd, bd = o.bf16_to_f32(Wq).astype(np.float64), o.bf16_to_f32(bq).astype(np.float64)
        else:
            feat, Wq, bq, featv = featf, Wf, bf, featf
            Wd, bd = Wf.astype(np.float64), bf.astype(np.float64)
        f, d = o.camera(40.0, 1.4)
        n_null = 3
        Y, mask = o.proj_cond_rows(None, n, R, [f], [d], feat, Wq, bq, n_null,
                                   np.arange(n + n_null))
        p = o.project(None, n, R, [f], [d], H, W)
        inp = torch.from_numpy(featv).permute(0, 3, 1, 2).contiguous()
        gr = torch.from_numpy(p["grid"]).reshape(1, 1, n, 2)
        S = torch.nn.functional.grid_sample(inp, gr, mode="bilinear", padding_mode="border",
                                            align_corners=False)[0, :, 0, :].T
        if dt == "bf16":
            S = S.to(torch.bfloat16)
        S = S.double().numpy()
        want = S @ Wd.T + bd
        tol = 1e-5 if dt == "f32" else 2e-2
        scale = np.abs(S) @ np.abs(Wd).T + np.abs(bd)
        assert np.max(np.abs(Y[:n] - want) / scale) < tol, dt
        assert np.array_equal(mask[:n], p["mask"])
        assert np.array_equal(Y[n:], np.broadcast_to(bd, (n_null, D)))
        assert np.all(mask[n:] == 0)
        Y0, _ = o.proj_cond_rows(None, n, R, [f], [d], feat, Wq, None, n_null, [n, n + 2])
        assert np.all(Y0 == 0.0)


# ---------------------------------------------------- grid nodes, cascade ---
def pin_requant_pages_fractions(o):
    """Res-512 coordinates requantized to a grid of 64: flooring u*64 and
    rounding u*63 disagree on exactly a quarter of the coordinates of each
    axis, always by one full cell, in stripes of period 8 (res-512 units);
    over the cube that is 1 - (3/4)^3 = 57.8 % of tokens off on at least one
    axis (the pages' 58 %)."""
    c = np.arange(512, dtype=np.int32)
    toks = np.stack([np.zeros_like(c), c, c, c], 1)
    r = o.requantize(toks, 512, 64, "round_nodes")[:, 1]
    f = o.requantize(toks, 512, 64, "floor_cells")[:, 1]
    d = r != f
    assert d.sum() == 128, d.sum()
    assert set(np.abs(r - f).tolist()) == {0, 1}
    # stripes of period 8: within each aligned block of 8 coordinates (one
    # grid-64 cell) the disagreements form one contiguous run, whose width
    # shrinks from 4 at the faces to 0 at the centre (mirror symmetric)
    for blk in d.reshape(-1, 8):
        idx = np.nonzero(blk)[0]
        assert idx.size == 0 or idx[-1] - idx[0] + 1 == idx.size, blk
    assert np.array_equal(d, d[::-1])
    assert d[:8].sum() == 4 and d[252:260].sum() == 0
    assert r.min() == 0 and r.max() == 63 and f.min() == 0 and f.max() == 63
    assert np.all(np.diff(r) >= 0) and np.all(np.diff(f) >= 0)
    # every token of the 512^3 cube: the per-axis disagreement is independent
    keep = 1.0 - d.mean()
    assert abs((1.0 - keep ** 3) - 0.578125) < 1e-12
    rng = np.random.default_rng(67)
    t = np.concatenate([np.zeros((200000, 1), np.int32),
                        rng.integers(0, 512, (200000, 3)).astype(np.int32)], 1)
    moved = np.any(o.requantize(t, 512, 64, "round_nodes")[:, 1:] !=
                   o.requantize(t, 512, 64, "floor_cells")[:, 1:], axis=1).mean()
    assert abs(moved - 0.578125) < 0.005, moved


def pin_requant_identity(o):
    """A grid requantized to its own size is unchanged in both modes."""
    for R in (1, 2, 3, 7, 64, 100, 512):
        c = np.arange(R, dtype=np.int32)
        toks = np.stack([np.full_like(c, 3), c, c[::-1], c], 1)
        for mode in ("round_nodes", "floor_cells"):
            if R == 1 and mode == "round_nodes":
                continue
            assert np.array_equal(o.requantize(toks, R, R, mode), toks), (R, mode)


def pin_requant_brute_force(o):
    """Against exact rationals: round half to even of (c+1/2)(G-1)/R and
    floor of (c+1/2)G/R, for every coordinate of small grids."""
    from fractions import Fraction
    for R in range(1, 41):
        c = np.arange(R, dtype=np.int32)
        toks = np.stack([np.zeros_like(c), c, c, c], 1)
        for G in range(2, 41):
            r = o.requantize(toks, R, G, "round_nodes")[:, 1]
            f = o.requantize(toks, R, G, "floor_cells")[:, 1]
            for ci in range(R):
                u = Fraction(2 * ci + 1, 2 * R)
                assert r[ci] == round(u * (G - 1)), (R, G, ci)
                assert f[ci] == math.floor(u * G), (R, G, ci)


def pin_grid_node_endpoints(o):
    """Node i of linspace(-1, 1, R) at half scale: the end nodes sit exactly on
    the cube faces (+-1/2), the middle node of an odd grid on the axis, so
    on-axis nodes land on the image centre exactly."""
    for R in (2, 3, 5, 64, 65, 1025):
        cells = np.array([[0, 0, R - 1, 0], [0, R - 1, 0, R - 1]], np.int32)
        f, d = 2.0, 3.0
        p = o.project(cells, 2, R, [f], [d], 8, 8, points="grid_nodes")
        # z = -1/2 and +1/2 exactly: depth = d -+ 1/2
        assert p["depth"].tolist() == [np.float32(d + 0.5), np.float32(d - 0.5)]
        want = np.float32(f) * np.float32(0.5) / np.array([d + 0.5, d - 0.5], np.float32)
        assert p["grid"][0, 0] == -want[0] and p["grid"][1, 0] == want[1]
        if R % 2:
            m = (R - 1) // 2
            q = o.project(np.array([[0, m, m, 0]], np.int32), 1, R, [f], [d], 8, 8,
                          points="grid_nodes")
            assert np.all(q["grid"] == 0.0) and q["pixel"].tolist() == [[3, 3]]


def pin_grid_node_registration(o):
    """The camera solve registers the grid so that its z = 0 corner nodes
    land on the frame border: |g| = 1 up to binary32 rounding of focal and
    distance (cell centres only approach it, as 1 - 1/R)."""
    R = 65
    m = (R - 1) // 2
    cells = np.array([[0, R - 1, R - 1, m], [0, 0, 0, m], [0, R - 1, 0, m]], np.int32)
    for fov in (30.0, 40.0, 49.13):
        f, d = o.camera(fov, o.distance_from_fov(fov, 512, 0))
        p = o.project(cells, 3, R, [f], [d], 64, 64, points="grid_nodes")
        assert np.max(np.abs(np.abs(p["grid"]) - 1.0)) < 4e-7, (fov, p["grid"])


# ---------------------------------------------------------------- two maps ---
def _affine_map(B, H, W, a, b, g):
    """map[y][x][c] = a_c * xn + b_c * yn + g_c at pixel centres in normalised
    coordinates (xn = (2x+1)/W - 1), binary32."""
    xn = ((2 * np.arange(W) + 1) / W - 1).astype(np.float64)
    yn = ((2 * np.arange(H) + 1) / H - 1).astype(np.float64)
    m = a[None, None, :] * xn[None, :, None] + b[None, None, :] * yn[:, None, None] + g
    return np.ascontiguousarray(np.broadcast_to(m, (B, H, W, len(a))).astype(np.float32))


def pin_two_map_affine_maps(o):
    """Bilinear interpolation reproduces an affine function of the normalised
    coordinates on any grid, so two affine maps of different sizes sampled at
    one point give each its own a*g + b*gy + c, concatenated map 0 first;
    with an identity proj_linear that is the output."""
    rng = np.random.default_rng(23)
    C0, C1 = 8, 12
    a0, b0, g0 = rng.standard_normal((3, C0))
    a1, b1, g1 = rng.standard_normal((3, C1))
    m0 = _affine_map(1, 16, 24, a0, b0, g0)
    m1 = _affine_map(1, 40, 32, a1, b1, g1)
    Wt = np.eye(C0 + C1, dtype=np.float32)
    R = 16
    coords = np.array([[0, x, y, z] for x, y, z in rng.integers(3, R - 3, (40, 3))], np.int32)
    f, d = o.camera(30.0, 2.5)
    for points in ("cell_centres", "grid_nodes"):
        Y, _ = o.proj_cond_rows(coords, len(coords), R, [f], [d], [m0, m1], Wt, None, 0,
                                np.arange(len(coords)), points=points)
        p = o.project(coords, len(coords), R, [f], [d], 16, 16, points=points)
        gx = p["grid"][:, :1].astype(np.float64)
        gy = p["grid"][:, 1:].astype(np.float64)
        assert np.all(np.abs(p["grid"]) < 0.9)       # away from every border clamp
        want = np.concatenate([a0 * gx + b0 * gy + g0, a1 * gx + b1 * gy + g1], 1)
        assert _rel(Y, want, np.abs(want).max()) < 2e-6, points


def pin_two_map_linearity(o):
    """proj_linear over the concatenated sample splits over the halves:
    Y([m0, m1]; [W0 | W1], b) = Y(m0; W0, b) + Y(m1; W1, no bias)."""
    rng = np.random.default_rng(29)
    m0 = rng.standard_normal((2, 9, 7, 8)).astype(np.float32)
    m1 = rng.standard_normal((2, 5, 11, 16)).astype(np.float32)
    W0 = rng.standard_normal((20, 8)).astype(np.float32)
    W1 = rng.standard_normal((20, 16)).astype(np.float32)
    bias = rng.standard_normal(20).astype(np.float32)
    coords = np.concatenate([rng.integers(0, 2, (50, 1)), rng.integers(0, 12, (50, 3))],
                            1).astype(np.int32)
    fo, do = o.cameras([35.0, 45.0], [None, 1.8])
    rows = np.arange(50)
    Y, mask = o.proj_cond_rows(coords, 50, 12, fo, do, [m0, m1], np.concatenate([W0, W1], 1),
                               bias, 0, rows)
    Ya, ma = o.proj_cond_rows(coords, 50, 12, fo, do, m0, W0, bias, 0, rows)
    Yb, mb = o.proj_cond_rows(coords, 50, 12, fo, do, m1, W1, None, 0, rows)
    assert np.array_equal(mask, ma) and np.array_equal(mask, mb)
    assert _rel(Y, Ya + Yb, np.abs(Y).max()) < 1e-12


# ------------------------------------------------------------ diagnostics ---
def _torch_samples(o, feats, coords, n, R, focal, dist, points, bf16):
    """Per map, torch grid_sample (bilinear, border, align_corners=False) of
    the map at the oracle's projected points; bf16 maps give bf16-rounded
    samples, as fed to proj_linear."""
    import torch
    p = o.project(coords, n, R, focal, dist, 4, 4, points=points)
    bidx = coords[:, 0] if coords is not None else np.zeros(n, np.int64)
    out = []
    for f in feats:
        v = o.bf16_to_f32(f) if bf16 else f
        inp = torch.from_numpy(np.ascontiguousarray(v)).permute(0, 3, 1, 2).contiguous()
        S = np.empty((n, f.shape[3]), np.float64)
        for b in range(f.shape[0]):
            sel = np.nonzero(bidx == b)[0]
            if sel.size == 0:
                continue
            gr = torch.from_numpy(p["grid"][sel]).reshape(1, 1, -1, 2)
            r = torch.nn.functional.grid_sample(inp[b:b + 1], gr, mode="bilinear",
                                                padding_mode="border",
                                                align_corners=False)[0, :, 0, :].T
            if bf16:
                r = r.to(torch.bfloat16)
            S[sel] = r.double().numpy()
        out.append(S)
    return out, p["mask"]


def pin_stats_torch_numpy(o):
    """Coverage, per-half sums and the mean cosine against torch grid_sample
    samples reduced with numpy, for two maps of different sizes, fp32 and
    bf16, with tokens outside the frame and behind the camera."""
    rng = np.random.default_rng(31)
    R, n = 12, 300
    coords = np.concatenate([rng.integers(0, 2, (n, 1)), rng.integers(-4, R + 4, (n, 3))],
                            1).astype(np.int32)
    fo, do = o.cameras([45.0, 60.0], [1.2, 0.55])
    for bf16 in (False, True):
        m0 = rng.standard_normal((2, 7, 9, 16)).astype(np.float32)
        m1 = rng.standard_normal((2, 20, 13, 16)).astype(np.float32) + 0.3
        feats = [o.f32_to_bf16(m0), o.f32_to_bf16(m1)] if bf16 else [m0, m1]
        for points in ("cell_centres", "grid_nodes"):
            st = o.projection_stats(coords, n, R, fo, do, feats, points=points)
            (S0, S1), mask = _torch_samples(o, feats, coords, n, R, fo, do, points, bf16)
            assert st["tokens"] == n and st["inside"] == mask.sum()
            assert 0 < mask.sum() < n
            for h, S in enumerate((S0, S1)):
                assert abs(st["sum%d" % h] - S.sum()) <= 1e-5 * np.abs(S).sum()
                assert abs(st["sum_sq%d" % h] - (S * S).sum()) <= 1e-5 * (S * S).sum()
            n0, n1 = np.linalg.norm(S0, axis=1), np.linalg.norm(S1, axis=1)
            ok = (n0 > 0) & (n1 > 0)
            cos = (S0 * S1).sum(1)[ok] / (n0[ok] * n1[ok])
            assert st["cos_count"] == ok.sum()
            assert abs(st["cos_sum"] - cos.sum()) <= 1e-5 * n, (st["cos_sum"], cos.sum())


def pin_stats_figures_numpy(o):
    """The printed figures from the raw sums (orc_stats_figures) against
    numpy's own statistics of torch grid_sample samples: coverage =
    mask.mean(), mean and population std (np.std, two-pass) of each map's
    samples, mean cosine over the tokens where both samples are non-zero.
    Maps with an offset (mean 0.3 or 2.5 against std 1) make a dropped
    mean^2 term, a sample (N - 1) std or a wrong count show; a constant map
    must give std exactly 0 (the radicand may round below 0)."""
    rng = np.random.default_rng(41)
    R, n = 12, 300
    coords = np.concatenate([rng.integers(0, 2, (n, 1)), rng.integers(-4, R + 4, (n, 3))],
                            1).astype(np.int32)
    fo, do = o.cameras([45.0, 60.0], [1.2, 0.55])
    for bf16 in (False, True):
        m0 = (rng.standard_normal((2, 7, 9, 16)) + 0.3).astype(np.float32)
        m1 = (rng.standard_normal((2, 20, 13, 16)) * 0.5 + 2.5).astype(np.float32)
        feats = [o.f32_to_bf16(m0), o.f32_to_bf16(m1)] if bf16 else [m0, m1]
        st = o.projection_stats(coords, n, R, fo, do, feats)
        fig = o.stats_figures(st, [16, 16])
        (S0, S1), mask = _torch_samples(o, feats, coords, n, R, fo, do, "cell_centres", bf16)
        assert abs(fig["coverage"] - mask.mean()) < 1e-15
        for h, S in enumerate((S0, S1)):
            assert abs(fig["mean%d" % h] - S.mean()) <= 1e-6 * np.abs(S).mean(), (h, fig)
            assert abs(fig["std%d" % h] - S.std()) <= 1e-5 * S.std(), (h, fig, S.std())
        n0, n1 = np.linalg.norm(S0, axis=1), np.linalg.norm(S1, axis=1)
        ok = (n0 > 0) & (n1 > 0)
        cos = (S0 * S1).sum(1)[ok] / (n0[ok] * n1[ok])
        assert abs(fig["cosine"] - cos.mean()) <= 1e-6, (fig["cosine"], cos.mean())
        # one map: no second half, no cosine
        fig1 = o.stats_figures(o.projection_stats(coords, n, R, fo, do, feats[:1]), [16])
        assert fig1["mean1"] is None and fig1["std1"] is None and fig1["cosine"] is None
        assert abs(fig1["std0"] - fig["std0"]) <= 1e-12 * fig["std0"]
    c = np.full((1, 5, 6, 8), 0.1, np.float32)
    f, d = o.camera(40.0, 1.5)
    fig = o.stats_figures(o.projection_stats(coords[:40] * 0, 40, R, [f], [d], [c]), [8])
    assert fig["std0"] == 0.0 and abs(fig["mean0"] - 0.1) < 1e-7
    assert o.stats_figures([0.0] * 8, [8])["coverage"] is None


def pin_stats_scaled_copies(o):
    """A map and a scaled copy of it on the same grid: the cosine is exactly
    +1 (or -1 for a negative scale) at every token, mean and std scale with
    it; constant maps give their constants as means, std 0, and the sign of
    their product as cosine."""
    rng = np.random.default_rng(37)
    m0 = rng.standard_normal((1, 11, 8, 24)).astype(np.float32)
    coords = np.concatenate([np.zeros((80, 1)), rng.integers(0, 10, (80, 3))], 1).astype(np.int32)
    f, d = o.camera(40.0, 1.5)
    for a in (3.0, -0.5):
        st = o.projection_stats(coords, 80, 10, [f], [d], [m0, (a * m0).astype(np.float32)])
        assert st["cos_count"] == 80
        assert abs(st["cos_sum"] - 80 * np.sign(a)) < 1e-9
        mag = abs(a) * math.sqrt(80 * 24 * st["sum_sq0"])    # >= sum |a S0|
        assert abs(st["sum1"] - a * st["sum0"]) <= 1e-6 * mag
        assert abs(st["sum_sq1"] - a * a * st["sum_sq0"]) <= 1e-6 * st["sum_sq1"]
    c0 = np.full((1, 3, 5, 8), 0.25, np.float32)
    c1 = np.full((1, 6, 4, 8), -2.0, np.float32)
    st = o.projection_stats(coords, 80, 10, [f], [d], [c0, c1])
    # binary32 bilinear weights sum to 1 within a few ulp
    assert abs(st["sum0"] - 0.25 * 80 * 8) < 1e-6 * 0.25 * 80 * 8
    assert abs(st["sum1"] + 2.0 * 80 * 8) < 1e-6 * 2.0 * 80 * 8
    assert abs(st["sum_sq0"] - 0.0625 * 80 * 8) < 1e-6 * 0.0625 * 80 * 8
    assert abs(st["sum_sq1"] - 4.0 * 80 * 8) < 1e-6 * 4.0 * 80 * 8
    assert st["cos_count"] == 80 and abs(st["cos_sum"] + 80) < 1e-12


def pin_stats_coverage_corners(o):
    """At the closed-form distance the two near cube corners leave the frame
    and the two far ones stay inside (coverage is a ratio, not a pass/fail);
    a token behind the camera counts as outside."""
    R = 64
    f, d = o.camera(40.0, o.distance_from_fov(40.0, 512, 0))
    cells = np.array([[0, R - 1, R - 1, R - 1], [0, 0, 0, R - 1],
                      [0, R - 1, R - 1, 0], [0, 0, 0, 0]], np.int32)
    m = np.ones((1, 4, 4, 8), np.float32)
    st = o.projection_stats(cells, 4, R, [f], [d], m)
    assert st["tokens"] == 4 and st["inside"] == 2
    f2, d2 = o.camera(40.0, 0.3)          # z = +0.49 cells sit behind this camera
    st = o.projection_stats(np.array([[0, 32, 32, R - 1], [0, 32, 32, 0]], np.int32), 2, R,
                            [f2], [d2], m)
    assert st["inside"] == 1


def pin_stats_zero_map(o):
    """A half that samples to zero has no direction: no cosine is counted."""
    coords = np.array([[0, 1, 2, 3], [0, 3, 3, 3]], np.int32)
    f, d = o.camera(40.0, 2.0)
    z = np.zeros((1, 4, 4, 8), np.float32)
    st = o.projection_stats(coords, 2, 5, [f], [d], [z, z + 1])
    assert st["cos_count"] == 0 and st["cos_sum"] == 0 and st["sum0"] == 0
    assert abs(st["sum1"] - 16) < 1e-6


# ------------------------------------------------- gather once, per-block ---
def pin_proj_sample_torch(o):
    """The gathered samples S (one or two maps, bf16-rounded for bf16 maps)
    equal torch grid_sample of each map at the projected points, map 0's
    channels first."""
    rng = np.random.default_rng(41)
    R, n = 10, 120
    coords = np.concatenate([rng.integers(0, 2, (n, 1)), rng.integers(-2, R + 2, (n, 3))],
                            1).astype(np.int32)
    fo, do = o.cameras([38.0, 52.0], [None, 1.3])
    m0 = rng.standard_normal((2, 6, 11, 8)).astype(np.float32)
    m1 = rng.standard_normal((2, 17, 9, 24)).astype(np.float32)
    for bf16 in (False, True):
        feats = [o.f32_to_bf16(m0), o.f32_to_bf16(m1)] if bf16 else [m0, m1]
        for points in ("cell_centres", "grid_nodes"):
            S, mask = o.proj_sample_rows(coords, n, R, fo, do, feats, np.arange(n),
                                         points=points)
            (T0, T1), tm = _torch_samples(o, feats, coords, n, R, fo, do, points, bf16)
            T = np.concatenate([T0, T1], 1)
            # scale: the interpolated magnitude sum_k w_k |F_k| (torch, on |map|)
            (A0, A1), _ = _torch_samples(o, [np.abs(m0), np.abs(m1)], coords, n, R, fo, do,
                                         points, False)
            mag = np.concatenate([A0, A1], 1)
            assert np.array_equal(mask, tm)
            # fp32: the sampling tolerance (torch forms the source index in
            # another operation order); bf16: one rounding of the sample
            tol = 2.0 ** -8 if bf16 else 1e-5
            assert np.all(np.abs(S - T) <= tol * (mag + np.abs(T)) + 1e-30), (bf16, points)


def pin_linear_grouped_numpy(o):
    """Per block g: numpy float64 S @ W_g^T + b_g (+ the block's residual)."""
    rng = np.random.default_rng(43)
    S = rng.standard_normal((33, 24))
    for bf16 in (False, True):
        ws = [rng.standard_normal((16, 24)).astype(np.float32) for _ in range(3)]
        bs = [rng.standard_normal(16).astype(np.float32), None, rng.standard_normal(16).astype(
            np.float32)]
        if bf16:
            ws = [o.f32_to_bf16(w) for w in ws]
            bs = [None if b is None else o.f32_to_bf16(b) for b in bs]
        wv = [(o.bf16_to_f32(w) if bf16 else w).astype(np.float64) for w in ws]
        bv = [None if b is None else (o.bf16_to_f32(b) if bf16 else b).astype(np.float64)
              for b in bs]
        res = [rng.standard_normal((33, 16)), None, rng.standard_normal((33, 16))]
        Y = o.linear_grouped(S, ws, bs, res)
        for g in range(3):
            want = S @ wv[g].T + (0 if bv[g] is None else bv[g]) + (0 if res[g] is None
                                                                  else res[g])
            assert np.max(np.abs(Y[g] - want)) <= 1e-12 * np.abs(want).max(), (bf16, g)
        Y2 = o.linear_grouped(S, ws)
        for g in range(3):
            assert np.max(np.abs(Y2[g] - S @ wv[g].T)) <= 1e-12 * np.abs(Y2[g]).max()


def pin_grouped_block_is_the_path(o):
    """Gather once, then block g's linear without residual equals the whole
    path run with that block's weight and bias."""
    rng = np.random.default_rng(47)
    feat = o.f32_to_bf16(rng.standard_normal((1, 12, 12, 16)).astype(np.float32))
    coords = np.concatenate([np.zeros((40, 1)), rng.integers(0, 8, (40, 3))], 1).astype(np.int32)
    f, d = o.camera(40.0, 1.8)
    ws = [o.f32_to_bf16(rng.standard_normal((8, 16)).astype(np.float32)) for _ in range(2)]
    bs = [o.f32_to_bf16(rng.standard_normal(8).astype(np.float32)) for _ in range(2)]
    S, _ = o.proj_sample_rows(coords, 40, 8, [f], [d], feat, np.arange(40))
    Y = o.linear_grouped(S, ws, bs)
    for g in range(2):
        want, _ = o.proj_cond_rows(coords, 40, 8, [f], [d], feat, ws[g], bs[g], 0, np.arange(40))
        assert np.max(np.abs(Y[g] - want)) <= 1e-12 * np.abs(want).max()


ALL_PINS = {name[len("pin_"):]: fn for name, fn in sorted(globals().items())
            if name.startswith("pin_") and callable(fn)}
