"""pixel_aligned_image_amd -- Python binding of libp3d (MI355X / gfx950).

Thin ctypes marshalling over the C ABI in ``include/p3d.h``: every function
here has the name of its C entry point, checks that the torch tensors it is
given are on the GPU, contiguous and of the declared dtype, and passes their
device pointers plus torch's current HIP stream. All computation happens in
the HIP kernels of libp3d; there is no fallback. If ``libp3d.so`` is missing
the import fails loudly (build it with ``__graft_entry__.build()`` or
``python pixel_aligned_image_amd/build.py``).

torch is imported before libp3d is loaded so that the library binds to the
same HIP runtime as torch (both carry the soname libamdhip64.so.7).
"""
import ctypes
import os

import torch

__all__ = ["P3DError", "P3D_F32", "P3D_BF16", "P3D_MAX_BATCH", "lib", "p3d_version",
           "p3d_status_string", "p3d_last_error", "p3d_distance_from_fov", "p3d_make_camera",
           "p3d_project_points", "p3d_bilinear_sample", "p3d_proj_cond",
           "p3d_requantize_coords", "p3d_projection_stats", "p3d_stats_figures",
           "p3d_proj_sample", "p3d_proj_linear_grouped", "P3D_MAX_GROUPS",
           "p3d_proj_cond_workspace_size", "proj_cond_workspace", "P3D_NOALLOC_MAX_TOKENS",
           "p3d_token_order", "p3d_token_order_workspace_size", "p3d_stream_copy",
           "p3d_proj_cond_plan", "make_cameras", "POINTS", "REQUANT", "LIB_PATH"]

# P3D_LIB names another build of the same sources (the sanitizer run of the
# host validation layer loads a host-AddressSanitizer build through it)
LIB_PATH = os.environ.get("P3D_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                      "libp3d.so")

P3D_OK, P3D_ERR_INVALID_ARG, P3D_ERR_SHAPE, P3D_ERR_DTYPE, P3D_ERR_UNSUPPORTED, P3D_ERR_HIP = range(6)
P3D_F32, P3D_BF16 = 0, 1
P3D_MAX_BATCH = 256
P3D_MAX_GROUPS = 64
P3D_NOALLOC_MAX_TOKENS = 1048576
POINTS = {"cell_centres": 0, "grid_nodes": 1}          # p3d_points
REQUANT = {"round_nodes": 0, "floor_cells": 1}          # p3d_requant


class p3d_camera(ctypes.Structure):
    _fields_ = [("focal", ctypes.c_float), ("distance", ctypes.c_float)]


class p3d_map(ctypes.Structure):
    _fields_ = [("feat", ctypes.c_void_p), ("height", ctypes.c_int32),
                ("width", ctypes.c_int32), ("channels", ctypes.c_int32)]


class P3DError(RuntimeError):
    """A libp3d call returned a status other than P3D_OK."""

    def __init__(self, status, message):
        super().__init__("%s: %s" % (_status_name(status), message))
        self.status = status
        self.message = message


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libp3d.so is not built at %s; run __graft_entry__.build() "
                          "(or python pixel_aligned_image_amd/build.py)" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    cam_p = ctypes.POINTER(p3d_camera)
    L.p3d_version.restype = ctypes.c_char_p
    L.p3d_version.argtypes = []
    L.p3d_status_string.restype = ctypes.c_char_p
    L.p3d_status_string.argtypes = [ctypes.c_int]
    L.p3d_last_error.restype = ctypes.c_char_p
    L.p3d_last_error.argtypes = []
    L.p3d_distance_from_fov.restype = ctypes.c_double
    L.p3d_distance_from_fov.argtypes = [ctypes.c_double, i32, i32]
    L.p3d_make_camera.restype = ctypes.c_int
    L.p3d_make_camera.argtypes = [ctypes.c_double, ctypes.c_double, cam_p]
    L.p3d_project_points.restype = ctypes.c_int
    L.p3d_project_points.argtypes = [vp, i64, i32, cam_p, i32, i32, i32, vp, vp, vp, vp, vp, vp]
    L.p3d_bilinear_sample.restype = ctypes.c_int
    L.p3d_bilinear_sample.argtypes = [vp, ctypes.c_int, i32, i32, i32, i32, vp, vp, i64, vp,
                                      ctypes.c_int, vp]
    L.p3d_bilinear_sample_ordered.restype = ctypes.c_int
    L.p3d_bilinear_sample_ordered.argtypes = [vp, ctypes.c_int, i32, i32, i32, i32, vp, vp, i64,
                                              vp, vp, ctypes.c_int, vp]
    L.p3d_proj_cond.restype = ctypes.c_int
    L.p3d_proj_cond.argtypes = [vp, i64, i32, cam_p, i32, vp, ctypes.c_int, i32, i32, i32,
                                vp, i32, i32, vp, i64, vp, vp, vp]
    L.p3d_project_points_ex.restype = ctypes.c_int
    L.p3d_project_points_ex.argtypes = [vp, i64, i32, ctypes.c_int, cam_p, i32, i32, i32, vp,
                                        vp, vp, vp, vp, vp]
    L.p3d_requantize_coords.restype = ctypes.c_int
    L.p3d_requantize_coords.argtypes = [vp, i64, i32, i32, ctypes.c_int, vp, vp]
    L.p3d_projection_stats.restype = ctypes.c_int
    L.p3d_projection_stats.argtypes = [vp, i64, i32, ctypes.c_int, cam_p, i32, ctypes.c_int,
                                       ctypes.POINTER(p3d_map), i32, vp, vp]
    L.p3d_proj_sample.restype = ctypes.c_int
    L.p3d_proj_sample.argtypes = [vp, i64, i32, ctypes.c_int, cam_p, i32, ctypes.c_int,
                                  ctypes.POINTER(p3d_map), i32, vp, vp, vp]
    L.p3d_proj_linear_grouped.restype = ctypes.c_int
    L.p3d_proj_linear_grouped.argtypes = [vp, i64, i32, ctypes.c_int, i32,
                                          ctypes.POINTER(vp), ctypes.POINTER(vp), i32,
                                          ctypes.POINTER(vp), i32, vp]
    L.p3d_proj_cond_ex.restype = ctypes.c_int
    L.p3d_proj_cond_ex.argtypes = [vp, i64, i32, ctypes.c_int, cam_p, i32, ctypes.c_int,
                                   ctypes.POINTER(p3d_map), i32, vp, i32, i32, vp, i64, vp, vp,
                                   vp]
    L.p3d_proj_cond_workspace_size.restype = ctypes.c_size_t
    L.p3d_proj_cond_workspace_size.argtypes = [i64, i32, ctypes.POINTER(p3d_map), i32]
    L.p3d_proj_cond_ws.restype = ctypes.c_int
    L.p3d_proj_cond_ws.argtypes = [vp, i64, i32, ctypes.c_int, cam_p, i32, ctypes.c_int,
                                   ctypes.POINTER(p3d_map), i32, vp, i32, i32, vp, i64, vp, vp,
                                   vp, ctypes.c_size_t, vp]
    L.p3d_proj_cond_ordered.restype = ctypes.c_int
    L.p3d_proj_cond_ordered.argtypes = [vp, i64, i32, ctypes.c_int, cam_p, i32, ctypes.c_int,
                                        ctypes.POINTER(p3d_map), i32, vp, i32, i32, vp, i64, vp,
                                        vp, vp, vp]
    L.p3d_stream_copy.restype = ctypes.c_int
    L.p3d_stream_copy.argtypes = [vp, vp, i64, vp]
    L.p3d_token_order_workspace_size.restype = ctypes.c_size_t
    L.p3d_token_order_workspace_size.argtypes = [i64, i32, i32, i32]
    L.p3d_token_order.restype = ctypes.c_int
    L.p3d_token_order.argtypes = [vp, i64, i32, ctypes.c_int, cam_p, i32, i32, i32, vp, vp,
                                  ctypes.c_size_t, vp]
    L.p3d_projection_stats_ordered.restype = ctypes.c_int
    L.p3d_projection_stats_ordered.argtypes = [vp, i64, i32, ctypes.c_int, cam_p, i32,
                                               ctypes.c_int, ctypes.POINTER(p3d_map), i32, vp,
                                               vp, vp]
    L.p3d_proj_sample_ordered.restype = ctypes.c_int
    L.p3d_proj_sample_ordered.argtypes = [vp, i64, i32, ctypes.c_int, cam_p, i32, ctypes.c_int,
                                          ctypes.POINTER(p3d_map), i32, vp, vp, vp, vp]
    L.p3d_stats_figures.restype = ctypes.c_int
    L.p3d_stats_figures.argtypes = [vp, vp, i32, vp]
    L.p3d_proj_cond_plan.restype = ctypes.c_int
    L.p3d_proj_cond_plan.argtypes = [i64, i32, i32, vp]
    L.p3d_proj_cond_noalloc.restype = ctypes.c_int
    L.p3d_proj_cond_noalloc.argtypes = [vp, i64, i32, ctypes.c_int, cam_p, i32, ctypes.c_int,
                                        ctypes.POINTER(p3d_map), i32, vp, i32, i32, vp, i64, vp,
                                        vp, vp]
    return L


lib = _load()


def _status_name(s):
    return lib.p3d_status_string(int(s)).decode()


def _check(status):
    if status != P3D_OK:
        raise P3DError(status, lib.p3d_last_error().decode())


def p3d_version():
    return lib.p3d_version().decode()


def p3d_status_string(status):
    return _status_name(status)


def p3d_last_error():
    return lib.p3d_last_error().decode()


def p3d_distance_from_fov(fov_deg, image_size, extend_px=0):
    d = lib.p3d_distance_from_fov(float(fov_deg), int(image_size), int(extend_px))
    if d != d:
        raise P3DError(P3D_ERR_INVALID_ARG, lib.p3d_last_error().decode())
    return d


def p3d_make_camera(fov_deg, distance):
    """(focal, distance) of the camera, as binary32 Python floats."""
    c = p3d_camera()
    _check(lib.p3d_make_camera(float(fov_deg), float(distance), ctypes.byref(c)))
    return c.focal, c.distance


def make_cameras(cams):
    """ctypes array of p3d_camera from a sequence of (focal, distance)."""
    arr = (p3d_camera * len(cams))()
    for i, (f, d) in enumerate(cams):
        arr[i].focal = f
        arr[i].distance = d
    return arr


# ----------------------------------------------------------------- helpers ---
_DT = {torch.float32: P3D_F32, torch.bfloat16: P3D_BF16}


def _dev(t, name, dtype=None, shape=None):
    """Device pointer of an optional tensor after checking it."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on the GPU, got %s" % (name, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    return t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _cams(cams):
    if isinstance(cams, ctypes.Array):
        return cams, len(cams)
    arr = make_cameras(list(cams))
    return arr, len(arr)


# -------------------------------------------------------------- entry points ---
def p3d_project_points(coords, n, resolution, cams, height, width, grid=None, pixel=None,
                       frac=None, depth=None, mask=None, stream=None, points="cell_centres"):
    """Enqueue p3d_project_points (points="cell_centres") or
    p3d_project_points_ex. coords: int32 [n, 4] device tensor or None (dense
    grid); cams: sequence of (focal, distance) per batch item; outputs are
    preallocated device tensors or None; points: "cell_centres" or
    "grid_nodes"."""
    camarr, batch = _cams(cams)
    n = int(n)
    args = (_dev(grid, "grid", torch.float32, (n, 2)), _dev(pixel, "pixel", torch.int32, (n, 2)),
            _dev(frac, "frac", torch.float32, (n, 2)), _dev(depth, "depth", torch.float32, (n,)),
            _dev(mask, "mask", torch.uint8, (n,)), _stream(stream))
    c = _dev(coords, "coords", torch.int32, (n, 4))
    if points == "cell_centres":
        _check(lib.p3d_project_points(c, n, int(resolution), camarr, batch, int(height),
                                      int(width), *args))
    else:
        _check(lib.p3d_project_points_ex(c, n, int(resolution), POINTS[points], camarr, batch,
                                         int(height), int(width), *args))


def p3d_requantize_coords(src, src_resolution, grid, dst, mode="round_nodes", stream=None):
    """Enqueue p3d_requantize_coords: int32 [n, 4] (b, x, y, z) on a
    src_resolution grid -> dst int32 [n, 4] on `grid`; mode "round_nodes"
    (round(u (grid-1))) or "floor_cells" (floor(u grid))."""
    n = int(src.shape[0])
    _check(lib.p3d_requantize_coords(_dev(src, "src", torch.int32, (n, 4)), n,
                                     int(src_resolution), int(grid), REQUANT[mode],
                                     _dev(dst, "dst", torch.int32, (n, 4)), _stream(stream)))


def p3d_bilinear_sample(feat, grid, out, batch_index=None, stream=None, order=None):
    """Enqueue p3d_bilinear_sample (p3d_bilinear_sample_ordered with an
    order, int32 [n] device tensor). feat: [B, H, W, C] float32/bfloat16;
    grid: float32 [n, 2]; out: [n, C] float32 (any map) or bfloat16 (bf16
    map); batch_index: int32 [n] or None."""
    if feat.dim() != 4:
        raise ValueError("feat must be [B, H, W, C], got %s" % (tuple(feat.shape),))
    B, H, W, C = feat.shape
    n = grid.shape[0]
    fdt = _DT.get(feat.dtype)
    odt = _DT.get(out.dtype)
    if fdt is None or odt is None:
        raise TypeError("feat/out must be float32 or bfloat16")
    _check(lib.p3d_bilinear_sample_ordered(
        _dev(feat, "feat"), fdt, B, H, W, C, _dev(grid, "grid", torch.float32, (n, 2)),
        _dev(batch_index, "batch_index", torch.int32, (n,)), n,
        _dev(order, "order", torch.int32, (n,)), _dev(out, "out", None, (n, C)), odt,
        _stream(stream)))


def _map_array(feats):
    maps = (p3d_map * len(feats))()
    for i, f in enumerate(feats):
        maps[i].feat = _dev(f, "feat[%d]" % i) if isinstance(f, torch.Tensor) else None
        maps[i].height, maps[i].width, maps[i].channels = f.shape[1], f.shape[2], f.shape[3]
    return maps


def p3d_proj_cond_workspace_size(n, batch, feat):
    """Bytes of device workspace p3d_proj_cond_ws needs; feat: one map or a
    list of two (tensors, or anything with a 4-entry .shape)."""
    feats = list(feat) if isinstance(feat, (list, tuple)) else [feat]
    maps = (p3d_map * len(feats))()
    for i, f in enumerate(feats):
        maps[i].height, maps[i].width, maps[i].channels = f.shape[1], f.shape[2], f.shape[3]
    size = lib.p3d_proj_cond_workspace_size(int(n), int(batch), maps, len(feats))
    if size == 0:
        raise P3DError(P3D_ERR_INVALID_ARG, lib.p3d_last_error().decode())
    return int(size)


def proj_cond_workspace(n, batch, feat, device="cuda"):
    """A fresh uint8 device tensor large enough for p3d_proj_cond_ws."""
    return torch.empty(p3d_proj_cond_workspace_size(n, batch, feat), dtype=torch.uint8,
                       device=device)


def p3d_proj_cond(coords, n, resolution, cams, feat, weight, out, bias=None, n_null=0,
                  mask=None, stream=None, points="cell_centres", workspace=None, noalloc=False,
                  order=None):
    """Enqueue p3d_proj_cond (one map, cell centres), p3d_proj_cond_ex, or
    p3d_proj_cond_ws when `workspace` (a uint8 device tensor, e.g. from
    proj_cond_workspace) is given, or p3d_proj_cond_noalloc when noalloc is
    true (the library's own scratch), or p3d_proj_cond_ordered when `order`
    (int32 [n] device tensor from p3d_token_order) is given. feat: [B, H, W, C], or a list of two such
    maps (own H, W, C; samples concatenated, map 0 first); weight: [D, C_w]
    (torch Linear layout; C_w is checked against the summed C by the
    library); bias: [D] or None; out: [n + n_null, D]; all of one dtype
    (float32 or bfloat16); mask: uint8 [n] or None; points: "cell_centres" or
    "grid_nodes"."""
    camarr, batch = _cams(cams)
    feats = list(feat) if isinstance(feat, (list, tuple)) else [feat]
    for f in feats:
        if f.dim() != 4:
            raise ValueError("feat must be [B, H, W, C], got %s" % (tuple(f.shape),))
        if f.shape[0] != batch:
            raise ValueError("feat has %d batch items but %d cameras were given"
                             % (f.shape[0], batch))
        if f.dtype != feats[0].dtype:
            raise TypeError("all maps must have one dtype")
    if weight.dim() != 2:
        raise ValueError("weight must be [out_dim, in_dim], got %s" % (tuple(weight.shape),))
    D, Cw = weight.shape
    dt = _DT.get(feats[0].dtype)
    if dt is None:
        raise TypeError("feat must be float32 or bfloat16, got %s" % feats[0].dtype)
    n, n_null = int(n), int(n_null)
    dtype = feats[0].dtype
    common = (_dev(weight, "weight", dtype), D, Cw, _dev(bias, "bias", dtype, (D,)), n_null,
              _dev(out, "out", dtype, (n + n_null, D)), _dev(mask, "mask", torch.uint8, (n,)),
              _stream(stream))
    c = _dev(coords, "coords", torch.int32, (n, 4))
    if order is not None:
        _check(lib.p3d_proj_cond_ordered(c, n, int(resolution), POINTS[points], camarr, batch, dt,
                                         _map_array(feats), len(feats), *common[:-1],
                                         _dev(order, "order", torch.int32, (n,)), common[-1]))
        return
    if noalloc:
        _check(lib.p3d_proj_cond_noalloc(c, n, int(resolution), POINTS[points], camarr, batch, dt,
                                         _map_array(feats), len(feats), *common))
        return
    if workspace is not None:
        ws = _dev(workspace, "workspace", torch.uint8)
        _check(lib.p3d_proj_cond_ws(c, n, int(resolution), POINTS[points], camarr, batch, dt,
                                    _map_array(feats), len(feats), *common[:-1], ws,
                                    workspace.numel(), common[-1]))
        return
    if len(feats) == 1 and points == "cell_centres":
        B, H, W, C = feats[0].shape
        _check(lib.p3d_proj_cond(c, n, int(resolution), camarr, batch, _dev(feats[0], "feat"), dt,
                                 H, W, C, *common))
        return
    maps = (p3d_map * len(feats))()
    for i, f in enumerate(feats):
        maps[i].feat = _dev(f, "feat[%d]" % i)
        maps[i].height, maps[i].width, maps[i].channels = f.shape[1], f.shape[2], f.shape[3]
    _check(lib.p3d_proj_cond_ex(c, n, int(resolution), POINTS[points], camarr, batch, dt, maps,
                                len(feats), *common))


STAT_FIELDS = ("tokens", "inside", "sum0", "sum1", "sum_sq0", "sum_sq1", "cos_sum",
               "cos_count")        # the eight doubles of p3d_proj_stats, in order


def p3d_projection_stats(coords, n, resolution, cams, feat, stats, points="cell_centres",
                         stream=None, order=None):
    """Enqueue p3d_projection_stats (p3d_projection_stats_ordered with an
    order from p3d_token_order). feat: one [B, H, W, C] map or a list of
    two; stats: float64 device tensor of 8 elements (p3d_proj_stats, in
    STAT_FIELDS order), overwritten."""
    camarr, batch = _cams(cams)
    feats = list(feat) if isinstance(feat, (list, tuple)) else [feat]
    dt = _DT.get(feats[0].dtype)
    if dt is None or any(f.dtype != feats[0].dtype for f in feats):
        raise TypeError("maps must all be float32 or all bfloat16")
    maps = (p3d_map * len(feats))()
    for i, f in enumerate(feats):
        if f.dim() != 4 or f.shape[0] != batch:
            raise ValueError("map %d must be [%d, H, W, C], got %s" % (i, batch, tuple(f.shape)))
        maps[i].feat = _dev(f, "feat[%d]" % i)
        maps[i].height, maps[i].width, maps[i].channels = f.shape[1], f.shape[2], f.shape[3]
    n = int(n)
    _check(lib.p3d_projection_stats_ordered(_dev(coords, "coords", torch.int32, (n, 4)), n,
                                            int(resolution), POINTS[points], camarr, batch, dt,
                                            maps, len(feats),
                                            _dev(order, "order", torch.int32, (n,)),
                                            _dev(stats, "stats", torch.float64, (8,)),
                                            _stream(stream)))


class p3d_proj_stats(ctypes.Structure):
    _fields_ = [(k, ctypes.c_double) for k in ("tokens", "inside", "sum0", "sum1", "sum_sq0",
                                               "sum_sq1", "cos_sum", "cos_count")]


class p3d_stats_fig(ctypes.Structure):
    _fields_ = [("coverage", ctypes.c_double), ("mean", ctypes.c_double * 2),
                ("std", ctypes.c_double * 2), ("cosine", ctypes.c_double)]


def p3d_stats_figures(raw, channels):
    """Coverage, per-map mean and std, mean cosine (p3d_stats_figures) from
    the sums of p3d_projection_stats: raw is the stats tensor (8 float64,
    any device) or a dict of STAT_FIELDS. Returns a dict; a figure whose
    denominator is empty is None."""
    if isinstance(raw, torch.Tensor):
        vals = raw.detach().double().cpu().tolist()
    else:
        vals = [float(raw[k]) for k in STAT_FIELDS]
    st = p3d_proj_stats(*vals)
    ch = (ctypes.c_int32 * len(channels))(*[int(c) for c in channels])
    fig = p3d_stats_fig()
    _check(lib.p3d_stats_figures(ctypes.byref(st), ch, len(channels), ctypes.byref(fig)))
    out = {"coverage": fig.coverage, "mean0": fig.mean[0], "std0": fig.std[0],
           "mean1": fig.mean[1], "std1": fig.std[1], "cosine": fig.cosine}
    return {k: (None if v != v else v) for k, v in out.items()}


class p3d_tile_plan(ctypes.Structure):
    _fields_ = [("tile_rows", ctypes.c_int32), ("token_tiles", ctypes.c_int32),
                ("feature_tiles", ctypes.c_int32), ("whole_tiles", ctypes.c_int32),
                ("part_rows", ctypes.c_int32), ("parts", ctypes.c_int32)]


def p3d_proj_cond_plan(n, out_dim, compute_units):
    """How a bf16 fused call of n tokens and out_dim features is cut into
    tiles on compute_units CUs (p3d_proj_cond_plan; host-only). Returns a
    dict of the p3d_tile_plan fields."""
    plan = p3d_tile_plan()
    _check(lib.p3d_proj_cond_plan(int(n), int(out_dim), int(compute_units), ctypes.byref(plan)))
    return {k: getattr(plan, k) for k, _ in p3d_tile_plan._fields_}


def _maps(feat, batch):
    feats = list(feat) if isinstance(feat, (list, tuple)) else [feat]
    dt = _DT.get(feats[0].dtype)
    if dt is None or any(f.dtype != feats[0].dtype for f in feats):
        raise TypeError("maps must all be float32 or all bfloat16")
    maps = (p3d_map * len(feats))()
    for i, f in enumerate(feats):
        if f.dim() != 4 or f.shape[0] != batch:
            raise ValueError("map %d must be [%d, H, W, C], got %s" % (i, batch, tuple(f.shape)))
        maps[i].feat = _dev(f, "feat[%d]" % i)
        maps[i].height, maps[i].width, maps[i].channels = f.shape[1], f.shape[2], f.shape[3]
    return feats, maps, dt


def p3d_proj_sample(coords, n, resolution, cams, feat, S, mask=None, points="cell_centres",
                    stream=None, order=None):
    """Enqueue p3d_proj_sample (p3d_proj_sample_ordered with an order from
    p3d_token_order): S [n, sum C] (dtype of the maps) receives the samples
    the fused path would feed to proj_linear; feat is one map or a list of
    two."""
    camarr, batch = _cams(cams)
    feats, maps, dt = _maps(feat, batch)
    n = int(n)
    K = sum(f.shape[3] for f in feats)
    _check(lib.p3d_proj_sample_ordered(_dev(coords, "coords", torch.int32, (n, 4)), n,
                                       int(resolution), POINTS[points], camarr, batch, dt, maps,
                                       len(feats), _dev(order, "order", torch.int32, (n,)),
                                       _dev(S, "S", feats[0].dtype, (n, K)),
                                       _dev(mask, "mask", torch.uint8, (n,)), _stream(stream)))


def p3d_stream_copy(src, dst, stream=None):
    """Enqueue p3d_stream_copy: dst[:] = src[:] (contiguous device tensors of
    equal byte size, a multiple of 16); a measurement helper, not a step of
    the method."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must have the same size in bytes")
    _check(lib.p3d_stream_copy(_dev(src, "src"), _dev(dst, "dst"), nbytes, _stream(stream)))


def p3d_token_order_workspace_size(n, batch, key_height, key_width):
    """Bytes of device workspace p3d_token_order needs."""
    size = lib.p3d_token_order_workspace_size(int(n), int(batch), int(key_height),
                                              int(key_width))
    if size == 0:
        raise P3DError(P3D_ERR_INVALID_ARG, lib.p3d_last_error().decode())
    return int(size)


def p3d_token_order(coords, n, resolution, cams, key_height, key_width, order, workspace=None,
                    points="cell_centres", stream=None):
    """Enqueue p3d_token_order: order (int32 [n] device tensor) receives an
    image-space permutation of the tokens for a key_height x key_width map
    (the largest the tokens sample). workspace: uint8 device tensor, or None
    for a fresh one (allocated by torch here, not by the library)."""
    camarr, batch = _cams(cams)
    n = int(n)
    if workspace is None:
        workspace = torch.empty(p3d_token_order_workspace_size(n, batch, key_height, key_width),
                                dtype=torch.uint8, device="cuda")
    _check(lib.p3d_token_order(_dev(coords, "coords", torch.int32, (n, 4)), n, int(resolution),
                               POINTS[points], camarr, batch, int(key_height), int(key_width),
                               _dev(order, "order", torch.int32, (n,)),
                               _dev(workspace, "workspace", torch.uint8), workspace.numel(),
                               _stream(stream)))


def p3d_proj_linear_grouped(S, weights, outs, biases=None, accumulate=False, stream=None):
    """Enqueue p3d_proj_linear_grouped: for every block g, outs[g] = W_g S +
    b_g (accumulate: outs[g] += ...). S: bf16 [n, K]; weights: list of bf16
    [D, K]; biases: list (entries may be None) or None; outs: list of bf16
    [n, D]."""
    n, K = S.shape
    G = len(weights)
    D = weights[0].shape[0]
    if len(outs) != G or (biases is not None and len(biases) != G):
        raise ValueError("weights, biases and outs need one entry per block")
    wp = (ctypes.c_void_p * G)(*[_dev(w, "weights[%d]" % g, torch.bfloat16, (D, K))
                                 for g, w in enumerate(weights)])
    op = (ctypes.c_void_p * G)(*[_dev(o, "outs[%d]" % g, torch.bfloat16, (n, D))
                                 for g, o in enumerate(outs)])
    bp = None
    if biases is not None:
        bp = (ctypes.c_void_p * G)(*[_dev(b, "biases[%d]" % g, torch.bfloat16, (D,))
                                     for g, b in enumerate(biases)])
    _check(lib.p3d_proj_linear_grouped(_dev(S, "S", torch.bfloat16, (n, K)), n, K, P3D_BF16, G,
                                       wp, bp, D, op, int(bool(accumulate)), _stream(stream)))
