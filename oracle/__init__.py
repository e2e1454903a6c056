"""CPU oracle for pixel-aligned projection conditioning -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product library never does; the two
share no code. Every function below is a numpy marshalling layer over the plain
C loops in ``p3d_oracle.c``, which cite the passages they follow.

Arrays are numpy: maps are channels-last ``[B, H, W, C]`` float32, or uint16
holding bf16 bit patterns; coords ``[N, 4]`` int32 (b, x, y, z).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# P3D_ORACLE_LIB names another build of the same source (the sanitizer
# runs load an AddressSanitizer/UBSan build through it)
LIB_PATH = os.environ.get("P3D_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


def _ptr(a, typ):
    return None if a is None else a.ctypes.data_as(typ)


def _vptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _declare(lib):
    lib.orc_version.restype = ctypes.c_int
    lib.orc_set_threads.restype = ctypes.c_int
    lib.orc_set_threads.argtypes = [ctypes.c_int]
    lib.orc_bf16_to_f32.restype = ctypes.c_float
    lib.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.orc_f32_to_bf16.restype = ctypes.c_uint16
    lib.orc_f32_to_bf16.argtypes = [ctypes.c_float]
    lib.orc_f64_to_bf16.restype = ctypes.c_uint16
    lib.orc_f64_to_bf16.argtypes = [ctypes.c_double]
    lib.orc_quantize_bf16.restype = None
    lib.orc_quantize_bf16.argtypes = [_f64p, _i64, _u16p]
    lib.orc_distance_from_fov.restype = ctypes.c_double
    lib.orc_distance_from_fov.argtypes = [ctypes.c_double, _i32, _i32]
    lib.orc_camera.restype = None
    lib.orc_camera.argtypes = [ctypes.c_double, ctypes.c_double, _f32p, _f32p]
    lib.orc_source_index.restype = None
    lib.orc_source_index.argtypes = [ctypes.c_float, _i32, _i32p, _i32p, _f32p]
    lib.orc_project.restype = None
    lib.orc_project.argtypes = [_i32p, _i64, _i32, _f32p, _f32p, _i32, _i32, _i32,
                                _f32p, _i32p, _f32p, _f32p, _u8p]
    lib.orc_project_ex.restype = None
    lib.orc_project_ex.argtypes = [_i32p, _i64, _i32, _i32, _f32p, _f32p, _i32, _i32, _i32,
                                   _f32p, _i32p, _f32p, _f32p, _u8p]
    lib.orc_requantize.restype = None
    lib.orc_requantize.argtypes = [_i32p, _i64, _i32, _i32, _i32, _i32p]
    lib.orc_sample.restype = None
    lib.orc_sample.argtypes = [_vp, _i32, _i32, _i32, _i32, _i32, _f32p, _i32p, _i64, _f64p]
    lib.orc_linear.restype = None
    lib.orc_linear.argtypes = [_f64p, _i64, _i32, _vp, _vp, _i32, _i32, _f64p]
    lib.orc_proj_cond_rows.restype = None
    lib.orc_proj_cond_rows.argtypes = [_i32p, _i64, _i32, _f32p, _f32p, _vp, _i32, _i32,
                                       _i32, _i32, _i32, _vp, _vp, _i32, _i64,
                                       _i64p, _i64, _f64p, _u8p, _f64p]
    lib.orc_proj_cond_rows_ex.restype = None
    lib.orc_proj_cond_rows_ex.argtypes = [_i32p, _i64, _i32, _i32, _f32p, _f32p, _i32, _i32,
                                          ctypes.POINTER(_vp), _i32p, _i32p, _i32p, _i32,
                                          _vp, _vp, _i32, _i64, _i64p, _i64, _f64p, _u8p,
                                          _f64p]
    lib.orc_projection_stats.restype = None
    lib.orc_projection_stats.argtypes = [_i32p, _i64, _i32, _i32, _f32p, _f32p, _i32, _i32,
                                         ctypes.POINTER(_vp), _i32p, _i32p, _i32p, _i32,
                                         _f64p, _f64p]
    lib.orc_stats_figures.restype = None
    lib.orc_stats_figures.argtypes = [_f64p, _i32p, _i32, _f64p]
    lib.orc_proj_sample_rows.restype = None
    lib.orc_proj_sample_rows.argtypes = [_i32p, _i64, _i32, _i32, _f32p, _f32p, _i32, _i32,
                                         ctypes.POINTER(_vp), _i32p, _i32p, _i32p, _i32,
                                         _i64p, _i64, _f64p, _u8p]
    lib.orc_linear_grouped.restype = None
    lib.orc_linear_grouped.argtypes = [_f64p, _i64, _i32, _i32, ctypes.POINTER(_vp),
                                       ctypes.POINTER(_vp), _i32, _i32,
                                       ctypes.POINTER(_vp), _f64p]
    return lib


STAT_FIELDS = ("tokens", "inside", "sum0", "sum1", "sum_sq0", "sum_sq1", "cos_sum",
               "cos_count")


POINTS = {"cell_centres": 0, "grid_nodes": 1}
REQUANT = {"round_nodes": 0, "floor_cells": 1}


class Oracle:
    """numpy front end of one build of the oracle library."""

    def __init__(self, path=LIB_PATH):
        if not os.path.exists(path):
            from . import build as _build
            _build.build(out=path)
        self.path = path
        self.lib = _declare(ctypes.CDLL(path))

    def set_threads(self, n):
        """Threads for the row-parallel loops; returns the count in effect."""
        return self.lib.orc_set_threads(int(n))

    # -------------------------------------------------------------- bf16 ---
    @staticmethod
    def bf16_to_f32(bits):
        bits = np.ascontiguousarray(bits, dtype=np.uint16)
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)

    def f32_to_bf16(self, x):
        x = np.asarray(x, dtype=np.float32)
        return np.array([self.lib.orc_f32_to_bf16(ctypes.c_float(v)) for v in x.ravel()],
                        dtype=np.uint16).reshape(x.shape)

    def f64_to_bf16(self, x):
        x = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty(x.shape, dtype=np.uint16)
        self.lib.orc_quantize_bf16(_ptr(x, _f64p), x.size, _ptr(out, _u16p))
        return out

    # ------------------------------------------------------------ camera ---
    def distance_from_fov(self, fov_deg, image_size, extend_px=0):
        return self.lib.orc_distance_from_fov(float(fov_deg), int(image_size), int(extend_px))

    def camera(self, fov_deg, distance):
        """(focal, distance) as binary32, focal = 1/tan(fov/2)."""
        f = ctypes.c_float()
        d = ctypes.c_float()
        self.lib.orc_camera(float(fov_deg), float(distance), ctypes.byref(f), ctypes.byref(d))
        return np.float32(f.value), np.float32(d.value)

    def cameras(self, fovs_deg, distances):
        """Arrays (focal[B], distance[B]) float32 for per-item FOVs/distances;
        a distance of None takes the closed form for that FOV."""
        fs, ds = [], []
        for a, d in zip(fovs_deg, distances):
            if d is None:
                d = self.distance_from_fov(a, 512, 0)
            f, dd = self.camera(a, d)
            fs.append(f)
            ds.append(dd)
        return np.array(fs, dtype=np.float32), np.array(ds, dtype=np.float32)

    # -------------------------------------------------------- projection ---
    def source_index(self, g, size):
        """(i0, i1, t) of the border-clamped align_corners=False mapping."""
        i0 = ctypes.c_int32()
        i1 = ctypes.c_int32()
        t = ctypes.c_float()
        self.lib.orc_source_index(ctypes.c_float(g), int(size), ctypes.byref(i0),
                                  ctypes.byref(i1), ctypes.byref(t))
        return i0.value, i1.value, np.float32(t.value)

    def project(self, coords, n, resolution, focal, dist, height, width,
                points="cell_centres"):
        """dict grid[n,2] f32, pixel[n,2] i32, frac[n,2] f32, depth[n] f32,
        mask[n] u8. coords None = dense grid (n = B*R^3). points:
        "cell_centres" or "grid_nodes"."""
        focal = np.ascontiguousarray(focal, dtype=np.float32).reshape(-1)
        dist = np.ascontiguousarray(dist, dtype=np.float32).reshape(-1)
        assert focal.shape == dist.shape
        if coords is not None:
            coords = np.ascontiguousarray(coords, dtype=np.int32)
            assert coords.shape == (n, 4)
        out = dict(grid=np.empty((n, 2), np.float32), pixel=np.empty((n, 2), np.int32),
                   frac=np.empty((n, 2), np.float32), depth=np.empty(n, np.float32),
                   mask=np.empty(n, np.uint8))
        self.lib.orc_project_ex(_ptr(coords, _i32p), n, resolution, POINTS[points],
                                _ptr(focal, _f32p), _ptr(dist, _f32p), len(focal), height,
                                width, _ptr(out["grid"], _f32p), _ptr(out["pixel"], _i32p),
                                _ptr(out["frac"], _f32p), _ptr(out["depth"], _f32p),
                                _ptr(out["mask"], _u8p))
        return out

    def requantize(self, coords, src_res, grid, mode="round_nodes"):
        """(b, x, y, z) on a src_res grid -> (b, X, Y, Z) on `grid`:
        "round_nodes" = round(u (grid-1)), "floor_cells" = floor(u grid),
        u = (c + 1/2)/src_res; exact."""
        coords = np.ascontiguousarray(coords, dtype=np.int32).reshape(-1, 4)
        out = np.empty_like(coords)
        self.lib.orc_requantize(_ptr(coords, _i32p), len(coords), int(src_res), int(grid),
                                REQUANT[mode], _ptr(out, _i32p))
        return out

    # ---------------------------------------------------------- sampling ---
    def sample(self, feat, grid, batch_index=None):
        """grid_sample(bilinear, align_corners=False, border) of a channels-last
        map at normalised points; float64 [n, C]."""
        feat = np.ascontiguousarray(feat)
        is_bf16 = feat.dtype == np.uint16
        assert is_bf16 or feat.dtype == np.float32
        B, H, W, C = feat.shape
        grid = np.ascontiguousarray(grid, dtype=np.float32).reshape(-1, 2)
        n = grid.shape[0]
        if batch_index is not None:
            batch_index = np.ascontiguousarray(batch_index, dtype=np.int32)
            assert batch_index.shape == (n,)
        out = np.empty((n, C), np.float64)
        self.lib.orc_sample(_vptr(feat), int(is_bf16), B, H, W, C, _ptr(grid, _f32p),
                            _ptr(batch_index, _i32p), n, _ptr(out, _f64p))
        return out

    # ------------------------------------------------------------ linear ---
    def linear(self, S, weight, bias=None):
        """Y = S @ W^T + b in float64; weight [D, C] float32 or bf16 bits."""
        S = np.ascontiguousarray(S, dtype=np.float64)
        weight = np.ascontiguousarray(weight)
        is_bf16 = weight.dtype == np.uint16
        D, C = weight.shape
        assert S.shape[1] == C
        if bias is not None:
            bias = np.ascontiguousarray(bias)
            assert bias.dtype == weight.dtype and bias.shape == (D,)
        Y = np.empty((S.shape[0], D), np.float64)
        self.lib.orc_linear(_ptr(S, _f64p), S.shape[0], C, _vptr(weight), _vptr(bias),
                            int(is_bf16), D, _ptr(Y, _f64p))
        return Y

    # -------------------------------------------------------- whole path ---
    def projection_stats(self, coords, n, resolution, focal, dist, feat,
                         points="cell_centres"):
        """Raw diagnostic sums over tokens [0, n) (dict of STAT_FIELDS);
        feat is one map or a list of two."""
        feats = [np.ascontiguousarray(f) for f in (feat if isinstance(feat, (list, tuple))
                                                    else [feat])]
        is_bf16 = feats[0].dtype == np.uint16
        B = feats[0].shape[0]
        Hs = np.array([f.shape[1] for f in feats], np.int32)
        Ws = np.array([f.shape[2] for f in feats], np.int32)
        Cs = np.array([f.shape[3] for f in feats], np.int32)
        if coords is not None:
            coords = np.ascontiguousarray(coords, dtype=np.int32)
            assert coords.shape == (n, 4)
        focal = np.ascontiguousarray(focal, dtype=np.float32).reshape(-1)
        dist = np.ascontiguousarray(dist, dtype=np.float32).reshape(-1)
        out = np.zeros(8, np.float64)
        S = np.empty(int(Cs.sum()), np.float64)
        fp = (_vp * len(feats))(*[f.ctypes.data for f in feats])
        self.lib.orc_projection_stats(_ptr(coords, _i32p), n, resolution, POINTS[points],
                                      _ptr(focal, _f32p), _ptr(dist, _f32p), B, len(feats), fp,
                                      _ptr(Hs, _i32p), _ptr(Ws, _i32p), _ptr(Cs, _i32p),
                                      int(is_bf16), _ptr(out, _f64p), _ptr(S, _f64p))
        return dict(zip(STAT_FIELDS, out.tolist()))

    def stats_figures(self, raw, channels):
        """Coverage, per-map mean and population std, mean cosine from the
        raw sums (a dict of STAT_FIELDS, or 8 numbers in that order): a dict
        with None for a figure whose denominator is empty."""
        r = np.array([raw[k] for k in STAT_FIELDS] if isinstance(raw, dict) else raw,
                     np.float64)
        ch = np.array(list(channels) + [0] * (2 - len(channels)), np.int32)
        out = np.empty(6, np.float64)
        self.lib.orc_stats_figures(_ptr(r, _f64p), _ptr(ch, _i32p), len(channels),
                                   _ptr(out, _f64p))
        names = ("coverage", "mean0", "std0", "mean1", "std1", "cosine")
        return {k: (None if np.isnan(v) else float(v)) for k, v in zip(names, out)}

    def proj_sample_rows(self, coords, n, resolution, focal, dist, feat, rows,
                         points="cell_centres"):
        """The samples S of tokens `rows` as the whole path forms them before
        proj_linear: float64 [len(rows), sum C] (bf16-rounded values for bf16
        maps) and the mask. feat: one map or a list of two."""
        feats = [np.ascontiguousarray(f) for f in (feat if isinstance(feat, (list, tuple))
                                                    else [feat])]
        is_bf16 = feats[0].dtype == np.uint16
        B = feats[0].shape[0]
        Hs = np.array([f.shape[1] for f in feats], np.int32)
        Ws = np.array([f.shape[2] for f in feats], np.int32)
        Cs = np.array([f.shape[3] for f in feats], np.int32)
        if coords is not None:
            coords = np.ascontiguousarray(coords, dtype=np.int32)
            assert coords.shape == (n, 4)
        focal = np.ascontiguousarray(focal, dtype=np.float32).reshape(-1)
        dist = np.ascontiguousarray(dist, dtype=np.float32).reshape(-1)
        rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1)
        assert rows.size == 0 or (rows.min() >= 0 and rows.max() < n)
        S = np.empty((rows.size, int(Cs.sum())), np.float64)
        mask = np.empty(rows.size, np.uint8)
        fp = (_vp * len(feats))(*[f.ctypes.data for f in feats])
        self.lib.orc_proj_sample_rows(_ptr(coords, _i32p), n, resolution, POINTS[points],
                                      _ptr(focal, _f32p), _ptr(dist, _f32p), B, len(feats), fp,
                                      _ptr(Hs, _i32p), _ptr(Ws, _i32p), _ptr(Cs, _i32p),
                                      int(is_bf16), _ptr(rows, _i64p), rows.size,
                                      _ptr(S, _f64p), _ptr(mask, _u8p))
        return S, mask

    def linear_grouped(self, S, weights, biases=None, residuals=None):
        """Per block g: Y_g = S @ W_g^T + b_g (+ residual_g), float64
        [G, rows, D]. weights: list of [D, K] (f32 or bf16 bits); biases:
        list (entries may be None) or None; residuals: list of float64
        [rows, D] (entries may be None) or None."""
        S = np.ascontiguousarray(S, dtype=np.float64)
        ws = [np.ascontiguousarray(w) for w in weights]
        G = len(ws)
        D, K = ws[0].shape
        assert S.shape[1] == K and all(w.shape == (D, K) and w.dtype == ws[0].dtype for w in ws)
        is_bf16 = ws[0].dtype == np.uint16
        bs = None
        if biases is not None:
            bs = [None if b is None else np.ascontiguousarray(b) for b in biases]
            assert all(b is None or (b.shape == (D,) and b.dtype == ws[0].dtype) for b in bs)
        rs = None
        if residuals is not None:
            rs = [None if r is None else np.ascontiguousarray(r, dtype=np.float64)
                  for r in residuals]
            assert all(r is None or r.shape == (S.shape[0], D) for r in rs)
        Y = np.empty((G, S.shape[0], D), np.float64)
        wp = (_vp * G)(*[w.ctypes.data for w in ws])
        bp = None if bs is None else (_vp * G)(*[None if b is None else b.ctypes.data for b in bs])
        rp = None if rs is None else (_vp * G)(*[None if r is None else r.ctypes.data for r in rs])
        self.lib.orc_linear_grouped(_ptr(S, _f64p), S.shape[0], K, G, wp, bp, int(is_bf16), D,
                                    rp, _ptr(Y, _f64p))
        return Y

    def proj_cond_rows(self, coords, n, resolution, focal, dist, feat, weight, bias,
                       n_null, rows, points="cell_centres"):
        """Rows `rows` (indices into [0, n + n_null)) of the whole path:
        float64 [len(rows), D] before rounding to the output type, and mask.
        feat is one map or a list of maps (same batch, own H, W, C) whose
        samples are concatenated; weight is [D, sum of C]."""
        feats = [np.ascontiguousarray(f) for f in (feat if isinstance(feat, (list, tuple))
                                                    else [feat])]
        weight = np.ascontiguousarray(weight)
        is_bf16 = feats[0].dtype == np.uint16
        assert all(f.dtype == feats[0].dtype for f in feats) and weight.dtype == feats[0].dtype
        B = feats[0].shape[0]
        assert all(f.shape[0] == B for f in feats)
        Hs = np.array([f.shape[1] for f in feats], np.int32)
        Ws = np.array([f.shape[2] for f in feats], np.int32)
        Cs = np.array([f.shape[3] for f in feats], np.int32)
        C = int(Cs.sum())
        D = weight.shape[0]
        assert weight.shape == (D, C)
        if bias is not None:
            bias = np.ascontiguousarray(bias)
            assert bias.dtype == feats[0].dtype and bias.shape == (D,)
        if coords is not None:
            coords = np.ascontiguousarray(coords, dtype=np.int32)
            assert coords.shape == (n, 4)
        focal = np.ascontiguousarray(focal, dtype=np.float32).reshape(-1)
        dist = np.ascontiguousarray(dist, dtype=np.float32).reshape(-1)
        assert len(focal) == B and len(dist) == B
        rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1)
        assert rows.size == 0 or (rows.min() >= 0 and rows.max() < n + n_null)
        Y = np.empty((rows.size, D), np.float64)
        mask = np.empty(rows.size, np.uint8)
        S = np.empty((rows.size, C), np.float64)
        fp = (_vp * len(feats))(*[f.ctypes.data for f in feats])
        self.lib.orc_proj_cond_rows_ex(_ptr(coords, _i32p), n, resolution, POINTS[points],
                                       _ptr(focal, _f32p), _ptr(dist, _f32p), B, len(feats),
                                       fp, _ptr(Hs, _i32p), _ptr(Ws, _i32p), _ptr(Cs, _i32p),
                                       int(is_bf16), _vptr(weight), _vptr(bias), D, n_null,
                                       _ptr(rows, _i64p), rows.size, _ptr(Y, _f64p),
                                       _ptr(mask, _u8p), _ptr(S, _f64p))
        return Y, mask


_default = None


def get():
    """The oracle built from this directory's source (built on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
