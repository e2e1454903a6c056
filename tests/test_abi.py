"""The C-ABI library loads and exports every entry point include/p3d.h
declares; host-only helpers and argument validation behave as documented.
CPU only: no call here reaches a kernel launch (each one fails validation
first, or enqueues nothing), and the module skips itself on a machine with a
GPU, where the parity tests cover the same calls for real."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "p3d.h")


def _gpu_present():
    import torch
    return torch.cuda.device_count() > 0


pytestmark = pytest.mark.skipif(_gpu_present(), reason="host-only checks (with a GPU the parity tests run instead)")


@pytest.fixture(scope="module")
def p3d():
    import pixel_aligned_image_amd
    return pixel_aligned_image_amd


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(p3d_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol(p3d):
    names = declared_functions()
    assert len(names) == 26, names
    lib = ctypes.CDLL(p3d.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name


def test_version_and_status_strings(p3d):
    assert "gfx950" in p3d.p3d_version()
    for s, name in enumerate(["P3D_OK", "P3D_ERR_INVALID_ARG", "P3D_ERR_SHAPE", "P3D_ERR_DTYPE",
                              "P3D_ERR_UNSUPPORTED", "P3D_ERR_HIP"]):
        assert p3d.p3d_status_string(s) == name


def test_distance_worked_example(p3d):
    for e, printed in ((0, "1.094"), (64, "0.875"), (128, "0.729")):
        assert "%.3f" % p3d.p3d_distance_from_fov(49.13, 512, e) == printed


def test_camera_matches_oracle_bits(p3d):
    import numpy as np
    import oracle
    o = oracle.get()
    for fov in np.linspace(1.0, 179.0, 357):
        for d in (0.3, 1.0, 1.6, 2.0):
            f1, d1 = p3d.p3d_make_camera(fov, d)
            f2, d2 = o.camera(fov, d)
            assert np.float32(f1) == f2 and np.float32(d1) == d2
        assert p3d.p3d_distance_from_fov(fov, 512, 0) == o.distance_from_fov(fov, 512, 0)


@pytest.mark.parametrize("fov,size,ext", [(0.0, 512, 0), (180.0, 512, 0), (-5.0, 512, 0),
                                          (float("nan"), 512, 0), (40.0, 0, 0), (40.0, 512, -256)])
def test_distance_rejects(p3d, fov, size, ext):
    with pytest.raises(p3d.P3DError) as e:
        p3d.p3d_distance_from_fov(fov, size, ext)
    assert e.value.status == p3d.P3D_ERR_INVALID_ARG


def test_make_camera_rejects(p3d):
    for fov, d in ((0.0, 1.0), (40.0, 0.0), (40.0, float("inf")), (40.0, -1.0)):
        with pytest.raises(p3d.P3DError):
            p3d.p3d_make_camera(fov, d)


# ---------------------------------------------------- validation (raw C ABI)
NULL = None
FAKE = 0x100000  # never dereferenced: every call below fails validation first


def _cams(p3d, vals):
    return p3d.make_cameras(vals)


def _pc(p3d, **kw):
    a = dict(coords=FAKE, n=16, R=8, cams=_cams(p3d, [(2.0, 2.0)]), batch=1, feat=FAKE,
             dtype=p3d.P3D_BF16, H=4, W=4, C=64, weight=FAKE, D=64, Cw=64, bias=NULL,
             n_null=0, out=FAKE, mask=NULL, stream=NULL)
    a.update(kw)
    st = p3d.lib.p3d_proj_cond(a["coords"], a["n"], a["R"], a["cams"], a["batch"], a["feat"],
                               a["dtype"], a["H"], a["W"], a["C"], a["weight"], a["D"], a["Cw"],
                               a["bias"], a["n_null"], a["out"], a["mask"], a["stream"])
    return st, p3d.p3d_last_error()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(n=-1), 1, "n must be >= 0"),
    (dict(R=0), 1, "resolution"),
    (dict(batch=0), 1, "batch"),
    (dict(batch=300), 1, "batch"),
    (dict(H=0), 1, "height/width"),
    (dict(coords=NULL, n=100), 2, "batch*R^3"),
    (dict(coords=FAKE + 4), 4, "16-byte aligned"),
    (dict(dtype=7), 3, "dtype"),
    (dict(Cw=48), 2, "[64, 48]"),
    (dict(C=60, Cw=60), 4, "multiple of 8"),
    (dict(D=60), 4, "out_dim must be a multiple of 8"),
    (dict(dtype=0, C=62, Cw=62), 4, "multiple of 4"),
    (dict(n_null=-3), 1, "n_null"),
    (dict(out=FAKE + 8), 4, "16-byte aligned"),
    (dict(H=65536, W=65536), 4, "2^31"),
    (dict(n=(1 << 30) + 1), 4, "n must be <="),
    (dict(D=(1 << 20) + 8), 4, "out_dim must be <="),
    # 2^23 token tiles x 2048 feature tiles: past the int32 tile counts
    (dict(n=1 << 30, D=1 << 20), 4, "tiles"),
    (dict(dtype=0, C=64, n=1 << 30, D=1 << 18), 4, "tiles"),
], ids=lambda v: str(v)[:40])
def test_proj_cond_validation(p3d, kw, status, needle):
    st, msg = _pc(p3d, **kw)
    assert st == status, (st, msg)
    assert needle in msg, msg


def test_proj_cond_camera_validation(p3d):
    for cam in ((0.0, 2.0), (2.0, 0.0), (float("nan"), 2.0), (2.0, float("inf"))):
        st, msg = _pc(p3d, cams=_cams(p3d, [cam]))
        assert st == p3d.P3D_ERR_INVALID_ARG and "cams[0]" in msg
    st, msg = _pc(p3d, cams=_cams(p3d, [(2.0, 2.0), (2.0, -1.0)]), batch=2)
    assert st == p3d.P3D_ERR_INVALID_ARG and "cams[1].distance" in msg


def test_zero_work_is_ok_without_touching_memory(p3d):
    st, msg = _pc(p3d, n=0, n_null=0, coords=NULL)
    assert st == 0, msg
    st = p3d.lib.p3d_project_points(NULL, 0, 8, _cams(p3d, [(2.0, 2.0)]), 1, 4, 4, NULL, NULL,
                                    NULL, NULL, NULL, NULL)
    assert st == 0
    st = p3d.lib.p3d_bilinear_sample(FAKE, p3d.P3D_BF16, 1, 4, 4, 64, FAKE, NULL, 0, FAKE,
                                     p3d.P3D_BF16, NULL)
    assert st == 0


@pytest.mark.parametrize("args,status,needle", [
    (dict(fdt=0, odt=1), 3, "BF16 output needs a BF16 map"),
    (dict(fdt=5), 3, "feat_dtype"),
    (dict(C=20), 4, "multiple of 8"),
    (dict(n=-2), 1, "n must be"),
    (dict(feat=FAKE + 2), 4, "aligned"),
    (dict(B=0), 1, "map shape"),
])
def test_bilinear_sample_validation(p3d, args, status, needle):
    a = dict(feat=FAKE, fdt=1, B=1, H=4, W=4, C=64, grid=FAKE, bidx=NULL, n=10, out=FAKE, odt=1)
    a.update(args)
    st = p3d.lib.p3d_bilinear_sample(a["feat"], a["fdt"], a["B"], a["H"], a["W"], a["C"],
                                     a["grid"], a["bidx"], a["n"], a["out"], a["odt"], NULL)
    assert st == status
    assert needle in p3d.p3d_last_error()


def test_project_points_validation(p3d):
    st = p3d.lib.p3d_project_points(FAKE, 10, 8, NULL, 1, 4, 4, NULL, NULL, NULL, NULL, NULL,
                                    NULL)
    assert st == 1 and "cams is NULL" in p3d.p3d_last_error()
    st = p3d.lib.p3d_project_points(FAKE, 10, 8, _cams(p3d, [(2.0, 2.0)]), 1, 4, 4, FAKE + 4,
                                    NULL, NULL, NULL, NULL, NULL)
    assert st == 4 and "8-byte aligned" in p3d.p3d_last_error()


# ------------------------------------------- grid nodes, requantization, maps
@pytest.mark.parametrize("args,status,needle", [
    (dict(n=-1), 1, "n must be"),
    (dict(mode=5), 1, "ROUND_NODES or FLOOR_CELLS"),
    (dict(grid=1), 1, "grid >= 2"),
    (dict(src_res=0), 1, "src_resolution and grid"),
    (dict(grid=(1 << 20) + 1), 1, "src_resolution and grid"),
    (dict(src=FAKE + 4), 4, "16-byte aligned"),
], ids=lambda v: str(v)[:30])
def test_requantize_validation(p3d, args, status, needle):
    a = dict(src=FAKE, n=10, src_res=512, grid=64, mode=0, dst=FAKE)
    a.update(args)
    st = p3d.lib.p3d_requantize_coords(a["src"], a["n"], a["src_res"], a["grid"], a["mode"],
                                       a["dst"], NULL)
    assert st == status, p3d.p3d_last_error()
    assert needle in p3d.p3d_last_error()


def test_requantize_zero_tokens_is_ok(p3d):
    assert p3d.lib.p3d_requantize_coords(NULL, 0, 512, 64, 0, NULL, NULL) == 0
    assert p3d.lib.p3d_requantize_coords(NULL, 0, 512, 1, 1, NULL, NULL) == 0


def test_project_points_ex_validation(p3d):
    cams = _cams(p3d, [(2.0, 2.0)])
    st = p3d.lib.p3d_project_points_ex(FAKE, 8, 1, 1, cams, 1, 4, 4, NULL, NULL, NULL, NULL,
                                       NULL, NULL)
    assert st == 1 and "resolution >= 2" in p3d.p3d_last_error()
    st = p3d.lib.p3d_project_points_ex(FAKE, 8, 8, 3, cams, 1, 4, 4, NULL, NULL, NULL, NULL,
                                       NULL, NULL)
    assert st == 1 and "CELL_CENTRES or GRID_NODES" in p3d.p3d_last_error()


def _pcx(p3d, maps, **kw):
    arr = (p3d.p3d_map * max(1, len(maps)))()
    for i, (f, h, w, c) in enumerate(maps):
        arr[i].feat, arr[i].height, arr[i].width, arr[i].channels = f, h, w, c
    a = dict(coords=FAKE, n=16, R=8, points=0, cams=_cams(p3d, [(2.0, 2.0)]), batch=1,
             dtype=p3d.P3D_BF16, n_maps=len(maps), weight=FAKE, D=64, Cw=128, bias=NULL,
             n_null=0, out=FAKE, mask=NULL)
    a.update(kw)
    st = p3d.lib.p3d_proj_cond_ex(a["coords"], a["n"], a["R"], a["points"], a["cams"],
                                  a["batch"], a["dtype"], arr, a["n_maps"], a["weight"], a["D"],
                                  a["Cw"], a["bias"], a["n_null"], a["out"], a["mask"], NULL)
    return st, p3d.p3d_last_error()


def test_proj_cond_ex_validation(p3d):
    two = [(FAKE, 4, 4, 64), (FAKE, 8, 8, 64)]
    st, msg = _pcx(p3d, two, n_maps=3)
    assert st == 1 and "1 or 2 maps" in msg
    st, msg = _pcx(p3d, [(FAKE, 4, 4, 72), (FAKE, 8, 8, 64)], Cw=136)
    assert st == 4 and "multiple of 64" in msg
    st, msg = _pcx(p3d, [(FAKE, 4, 4, 64), (FAKE, 8, 8, 60)], Cw=124)
    assert st == 4 and "maps[1] channels" in msg
    st, msg = _pcx(p3d, [(FAKE, 4, 4, 64), (FAKE, 0, 8, 64)])
    assert st == 1 and "maps[1] height/width" in msg
    st, msg = _pcx(p3d, two, Cw=96)
    assert st == 2 and "[64, 96]" in msg and "[1, 4, 4, 64]" in msg and "[1, 8, 8, 64]" in msg
    st, msg = _pcx(p3d, [(FAKE + 8, 4, 4, 64), (FAKE, 8, 8, 64)])
    assert st == 4 and "maps[0] feat must be 16-byte aligned" in msg
    st, msg = _pcx(p3d, two, points=1, R=1)
    assert st == 1 and "resolution >= 2" in msg
    st, msg = _pcx(p3d, two, n=0, coords=NULL)
    assert st == 0, msg


def test_projection_stats_validation(p3d):
    cams = _cams(p3d, [(2.0, 2.0)])

    def call(maps, stats=FAKE, n=16, dtype=1, n_maps=None):
        arr = (p3d.p3d_map * max(1, len(maps)))()
        for i, (f, h, w, c) in enumerate(maps):
            arr[i].feat, arr[i].height, arr[i].width, arr[i].channels = f, h, w, c
        st = p3d.lib.p3d_projection_stats(FAKE, n, 8, 0, cams, 1, dtype, arr,
                                          len(maps) if n_maps is None else n_maps, stats, NULL)
        return st, p3d.p3d_last_error()

    st, msg = call([(FAKE, 4, 4, 64)], stats=NULL)
    assert st == 1 and "stats is NULL" in msg
    st, msg = call([(FAKE, 4, 4, 64)], stats=FAKE + 4)
    assert st == 4 and "8-byte aligned" in msg
    st, msg = call([(FAKE, 4, 4, 60)])
    assert st == 4 and "multiple of 8" in msg
    st, msg = call([(FAKE, 4, 4, 64), (FAKE, 4, 4, 64)], n_maps=3)
    assert st == 1 and "1 or 2 maps" in msg
    st, msg = call([(FAKE, 4, 4, 64)], dtype=4)
    assert st == 3 and "dtype" in msg
    st, msg = call([(NULL, 4, 4, 64)])
    assert st == 1 and "feat is NULL" in msg


def test_proj_linear_grouped_validation(p3d):
    def call(**kw):
        a = dict(S=FAKE, n=100, K=64, dtype=1, G=2, D=64, acc=0, weights=[FAKE, FAKE],
                 biases=None, outs=[FAKE, FAKE])
        a.update(kw)
        vp = ctypes.c_void_p
        w = (vp * max(1, len(a["weights"])))(*a["weights"]) if a["weights"] is not None else None
        o = (vp * max(1, len(a["outs"])))(*a["outs"]) if a["outs"] is not None else None
        b = (vp * len(a["biases"]))(*a["biases"]) if a["biases"] is not None else None
        st = p3d.lib.p3d_proj_linear_grouped(a["S"], a["n"], a["K"], a["dtype"], a["G"], w, b,
                                             a["D"], o, a["acc"], NULL)
        return st, p3d.p3d_last_error()

    assert call(dtype=0) == (4, call(dtype=0)[1]) and "only BF16" in call(dtype=0)[1]
    st, msg = call(G=0)
    assert st == 1 and "groups must be in [1, 64]" in msg
    st, msg = call(G=65)
    assert st == 1 and "groups" in msg
    st, msg = call(K=60)
    assert st == 4 and "K must be" in msg
    st, msg = call(D=100)
    assert st == 4 and "out_dim must be" in msg
    st, msg = call(weights=None)
    assert st == 1 and "host arrays" in msg
    st, msg = call(weights=[FAKE, NULL])
    assert st == 1 and "weights[1]" in msg
    st, msg = call(outs=[FAKE + 8, FAKE])
    assert st == 4 and "16-byte aligned" in msg
    st, msg = call(biases=[NULL, FAKE + 2])
    assert st == 4 and "biases[1]" in msg
    st, msg = call(n=-1)
    assert st == 1
    assert call(n=0, S=NULL)[0] == 0


def test_proj_sample_validation(p3d):
    cams = _cams(p3d, [(2.0, 2.0)])
    arr = (p3d.p3d_map * 2)()
    for i, (h, w, c) in enumerate([(4, 4, 64), (8, 8, 72)]):
        arr[i].feat, arr[i].height, arr[i].width, arr[i].channels = FAKE, h, w, c
    st = p3d.lib.p3d_proj_sample(FAKE, 16, 8, 0, cams, 1, 1, arr, 2, FAKE + 8, NULL, NULL)
    assert st == 4 and "S must be 16-byte aligned" in p3d.p3d_last_error()
    st = p3d.lib.p3d_proj_sample(FAKE, 16, 8, 0, cams, 1, 1, arr, 2, NULL, NULL, NULL)
    assert st == 1 and "S is NULL" in p3d.p3d_last_error()
    arr[1].channels = 70
    st = p3d.lib.p3d_proj_sample(FAKE, 16, 8, 0, cams, 1, 1, arr, 2, FAKE, NULL, NULL)
    assert st == 4 and "maps[1] channels" in p3d.p3d_last_error()
    assert p3d.lib.p3d_proj_sample(NULL, 0, 8, 0, cams, 1, 1, arr, 1, NULL, NULL, NULL) == 0


def _maps(p3d, shapes):
    arr = (p3d.p3d_map * len(shapes))()
    for i, (h, w, c) in enumerate(shapes):
        arr[i].feat = None
        arr[i].height, arr[i].width, arr[i].channels = h, w, c
    return arr


def test_proj_cond_workspace_size(p3d):
    lib = p3d.lib
    one = _maps(p3d, [(512, 512, 2048)])
    size = lib.p3d_proj_cond_workspace_size(100000, 1, one, 1)
    # sort keys and the order itself (4 bytes per token each) plus two bin
    # tables, every part 256-byte aligned
    assert size % 256 == 0 and 800000 <= size < 800000 + 2 * 4 * 16384 + 4 * 256, size
    assert lib.p3d_proj_cond_workspace_size(0, 1, one, 1) > 0
    two = _maps(p3d, [(64, 64, 1024), (512, 512, 1024)])
    assert lib.p3d_proj_cond_workspace_size(100000, 1, two, 2) == size
    for args in [(-1, 1, one, 1), (10, 0, one, 1), (10, 1, one, 3), (10, 1, None, 1),
                 (10, 1, _maps(p3d, [(0, 4, 8)]), 1)]:
        assert lib.p3d_proj_cond_workspace_size(*args) == 0, args
        assert p3d.p3d_last_error().startswith("p3d_proj_cond_workspace_size")


def test_proj_cond_ws_validation(p3d):
    """Argument checks run before anything is enqueued: a short workspace
    names both sizes; the shared checks name the ws entry point."""
    lib = p3d.lib
    cams = p3d.make_cameras([(2.0, 2.0)])
    one = _maps(p3d, [(8, 8, 16)])
    one[0].feat = 4096
    need = lib.p3d_proj_cond_workspace_size(40, 1, one, 1)
    st = lib.p3d_proj_cond_ws(4096, 40, 8, 0, cams, 1, p3d.P3D_BF16, one, 1, 4096, 32, 16, None,
                              0, 8192, None, 4096, need - 256, None)
    assert st == p3d.P3D_ERR_INVALID_ARG
    msg = p3d.p3d_last_error()
    assert msg.startswith("p3d_proj_cond_ws") and str(need) in msg and str(need - 256) in msg
    st = lib.p3d_proj_cond_ws(4096, 40, 8, 0, cams, 1, p3d.P3D_BF16, one, 1, 4096, 32, 24, None,
                              0, 8192, None, 4096, need, None)
    assert st == p3d.P3D_ERR_SHAPE and "[32, 24]" in p3d.p3d_last_error()
    st = lib.p3d_proj_cond_ws(4096, 40, 8, 0, cams, 1, p3d.P3D_BF16, one, 1, 4096, 32, 16, None,
                              0, 8192, None, 4100, need, None)
    assert st == p3d.P3D_ERR_UNSUPPORTED and "256-byte" in p3d.p3d_last_error()
    # nothing to do: no workspace needed
    assert lib.p3d_proj_cond_ws(None, 0, 8, 0, cams, 1, p3d.P3D_BF16, one, 1, 4096, 32, 16,
                                None, 0, 8192, None, None, 0, None) == p3d.P3D_OK


@pytest.mark.parametrize("n,D,cus,want", [
    # 782 x 3 = 2346 tiles = 9 rounds of 256 + 42: 4 x 42 <= 256, quarters
    (100000, 1536, 256, dict(tile_rows=128, token_tiles=782, feature_tiles=3,
                             whole_tiles=2304, part_rows=32, parts=168)),
    # 1563 x 3 = 4689 = 18 x 256 + 81: 4 x 81 > 256 >= 2 x 81, halves
    (200000, 1536, 256, dict(tile_rows=128, token_tiles=1563, feature_tiles=3,
                             whole_tiles=4608, part_rows=64, parts=162)),
    # 55 x 3 = 165 tiles: no split fits; 73 x 3 = 219 tiles of 96 tokens do
    (7000, 1536, 256, dict(tile_rows=96, token_tiles=73, feature_tiles=3,
                           whole_tiles=219, part_rows=0, parts=0)),
    # 192 tiles -> exactly 256 of 96; one token more -> 257, so 193 whole
    (24576, 512, 256, dict(tile_rows=96, token_tiles=256, feature_tiles=1,
                           whole_tiles=256, part_rows=0, parts=0)),
    (24577, 512, 256, dict(tile_rows=128, token_tiles=193, feature_tiles=1,
                           whole_tiles=193, part_rows=0, parts=0)),
    # whole rounds only; one token (a single tile as four parts); no tokens
    (32768, 512, 256, dict(tile_rows=128, token_tiles=256, feature_tiles=1,
                           whole_tiles=256, part_rows=0, parts=0)),
    (1, 8, 256, dict(tile_rows=128, token_tiles=1, feature_tiles=1,
                     whole_tiles=0, part_rows=32, parts=4)),
    (0, 1000, 256, dict(tile_rows=128, token_tiles=0, feature_tiles=2,
                        whole_tiles=0, part_rows=0, parts=0)),
    # one CU: every tile count is a whole number of rounds
    (1000, 8, 1, dict(tile_rows=128, token_tiles=8, feature_tiles=1,
                      whole_tiles=8, part_rows=0, parts=0)),
])
def test_proj_cond_plan(p3d, n, D, cus, want):
    """The documented tiling rule, worked by hand for each case."""
    assert p3d.p3d_proj_cond_plan(n, D, cus) == want


def test_proj_cond_plan_refusals(p3d):
    for args, status, needle in (((-1, 8, 256), 1, "n must be"), (((1 << 30) + 1, 8, 256), 1, "n must be"),
                                 ((10, 0, 256), 1, "out_dim"), ((10, (1 << 20) + 1, 256), 1, "out_dim"),
                                 ((10, 8, 0), 1, "compute_units"),
                                 ((1 << 30, 1 << 20, 256), 4, "tiles")):
        with pytest.raises(p3d.P3DError) as e:
            p3d.p3d_proj_cond_plan(*args)
        assert e.value.status == status and needle in p3d.p3d_last_error(), args
    assert p3d.lib.p3d_proj_cond_plan(10, 8, 256, None) == p3d.P3D_ERR_INVALID_ARG


def test_stats_figures_closed_forms(p3d):
    """p3d_stats_figures is host code: the figures of hand-made sums. Map 0:
    4 tokens x 2 channels of values {1, 3} (mean 2, std 1); map 1: values
    all 5 (std 0, sum_sq - N mean^2 rounds to 0); 3 of 4 tokens inside;
    cosines summing to 1.5 over 2 tokens."""
    raw = dict(tokens=4.0, inside=3.0, sum0=16.0, sum1=40.0, sum_sq0=40.0, sum_sq1=200.0,
               cos_sum=1.5, cos_count=2.0)
    f = p3d.p3d_stats_figures(raw, [2, 2])
    assert f == dict(coverage=0.75, mean0=2.0, std0=1.0, mean1=5.0, std1=0.0, cosine=0.75)
    f = p3d.p3d_stats_figures(dict(raw, cos_count=0.0, cos_sum=0.0), [2])
    assert f["mean1"] is None and f["std1"] is None and f["cosine"] is None
    assert p3d.p3d_stats_figures(dict.fromkeys(p3d.STAT_FIELDS, 0.0), [8]) == dict(
        coverage=None, mean0=None, std0=None, mean1=None, std1=None, cosine=None)
    # E[x^2] a hair below mean^2 after rounding: std is 0, not NaN
    f = p3d.p3d_stats_figures(dict(raw, sum0=0.3 * 8, sum_sq0=0.09 * 8 * (1 - 1e-16)), [2, 2])
    assert f["std0"] == 0.0
    for channels in ([0], [2, 2, 2], [2, -1]):
        with pytest.raises(p3d.P3DError) as e:
            p3d.p3d_stats_figures(raw, channels)
        assert e.value.status == p3d.P3D_ERR_INVALID_ARG


def test_token_order_workspace_size(p3d):
    """Sort keys (4 bytes per token) plus two bin tables of at most 16384
    counters, each part 256-byte aligned; refusals name the call."""
    lib = p3d.lib
    size = lib.p3d_token_order_workspace_size(100000, 1, 512, 512)
    assert size % 256 == 0 and 400000 <= size <= 400128 + 2 * 4 * 16384 + 2 * 256, size
    # 128 x 128 blocks of 4 texels per 512 x 512 item: 16384 bins for one
    # item; 16 items take 16-texel blocks (1024 bins each), 32 items
    # 32-texel blocks (256 bins each)
    assert size == 400128 + 2 * 4 * 16384
    assert lib.p3d_token_order_workspace_size(100000, 16, 512, 512) == 400128 + 2 * 4 * 16384
    assert lib.p3d_token_order_workspace_size(100000, 32, 512, 512) == 400128 + 2 * 4 * 8192
    for args in [(-1, 1, 8, 8), (10, 0, 8, 8), (10, 1, 0, 8), (10, 1, 8, 0)]:
        assert lib.p3d_token_order_workspace_size(*args) == 0, args
        assert p3d.p3d_last_error().startswith("p3d_token_order_workspace_size")


def test_token_order_validation(p3d):
    lib = p3d.lib
    cams = p3d.make_cameras([(2.0, 2.0)])
    need = lib.p3d_token_order_workspace_size(40, 1, 8, 8)
    st = lib.p3d_token_order(4096, 40, 8, 0, cams, 1, 8, 8, 4096, 4096, need - 256, None)
    assert st == p3d.P3D_ERR_INVALID_ARG
    msg = p3d.p3d_last_error()
    assert msg.startswith("p3d_token_order") and str(need) in msg
    st = lib.p3d_token_order(4096, 40, 8, 0, cams, 1, 8, 8, None, 4096, need, None)
    assert st == p3d.P3D_ERR_INVALID_ARG and "order" in p3d.p3d_last_error()
    st = lib.p3d_token_order(4096, 40, 8, 0, cams, 1, 8, 8, 4096, 4100, need, None)
    assert st == p3d.P3D_ERR_UNSUPPORTED and "256-byte" in p3d.p3d_last_error()
    st = lib.p3d_token_order(4096, 40, 8, 0, cams, 1, 0, 8, 4096, 4096, need, None)
    assert st != p3d.P3D_OK and p3d.p3d_last_error().startswith("p3d_token_order")
    st = lib.p3d_token_order(4096, 40, 8, 0, cams, 2, 8, 8, 4096, 4096, need, None)
    assert st != p3d.P3D_OK            # two batch items, one camera
    assert lib.p3d_token_order(None, 0, 8, 0, cams, 1, 8, 8, None, None, 0, None) == p3d.P3D_OK


def test_ordered_stats_and_sample_validation(p3d):
    """The ordered variants run the checks of the plain calls under their own
    names, and refuse a misaligned order."""
    lib = p3d.lib
    cams = p3d.make_cameras([(2.0, 2.0)])
    one = _maps(p3d, [(8, 8, 16)])
    one[0].feat = 4096
    st = lib.p3d_projection_stats_ordered(4096, 40, 8, 0, cams, 1, p3d.P3D_BF16, one, 1, 4098,
                                          4096, None)
    assert st == p3d.P3D_ERR_UNSUPPORTED
    assert p3d.p3d_last_error().startswith("p3d_projection_stats_ordered")
    st = lib.p3d_projection_stats_ordered(4096, 40, 8, 0, cams, 1, p3d.P3D_BF16, one, 1, 4096,
                                          None, None)
    assert st == p3d.P3D_ERR_INVALID_ARG and "stats" in p3d.p3d_last_error()
    st = lib.p3d_proj_sample_ordered(4096, 40, 8, 0, cams, 1, p3d.P3D_BF16, one, 1, 4098, 4096,
                                     None, None)
    assert st == p3d.P3D_ERR_UNSUPPORTED
    assert p3d.p3d_last_error().startswith("p3d_proj_sample_ordered")
    st = lib.p3d_proj_sample_ordered(4096, 40, 8, 0, cams, 1, p3d.P3D_BF16, one, 1, 4096, None,
                                     None, None)
    assert st == p3d.P3D_ERR_INVALID_ARG and "S is NULL" in p3d.p3d_last_error()


def test_proj_cond_ordered_validation(p3d):
    lib = p3d.lib
    cams = p3d.make_cameras([(2.0, 2.0)])
    one = _maps(p3d, [(8, 8, 16)])
    one[0].feat = 4096
    args = (4096, 40, 8, 0, cams, 1, p3d.P3D_BF16, one, 1, 4096, 32, 16, None, 0, 8192, None)
    assert lib.p3d_proj_cond_ordered(*args, 4098, None) == p3d.P3D_ERR_UNSUPPORTED
    assert p3d.p3d_last_error().startswith("p3d_proj_cond_ordered")
    assert lib.p3d_proj_cond_ordered(*args, None, None) == p3d.P3D_ERR_INVALID_ARG
    assert "order is NULL" in p3d.p3d_last_error()
    bad = (4096, 40, 8, 0, cams, 1, p3d.P3D_BF16, one, 1, 4096, 32, 24, None, 0, 8192, None)
    assert lib.p3d_proj_cond_ordered(*bad, 4096, None) == p3d.P3D_ERR_SHAPE
    assert lib.p3d_proj_cond_ordered(None, 0, 8, 0, cams, 1, p3d.P3D_BF16, one, 1, 4096, 32, 16,
                                     None, 0, 8192, None, None, None) == p3d.P3D_OK


def test_stream_copy_validation(p3d):
    lib = p3d.lib
    assert lib.p3d_stream_copy(None, None, 0, None) == p3d.P3D_OK
    assert lib.p3d_stream_copy(4096, 8192, -16, None) == p3d.P3D_ERR_INVALID_ARG
    assert lib.p3d_stream_copy(4096, 8192, 24, None) == p3d.P3D_ERR_UNSUPPORTED
    assert "multiple of 16" in p3d.p3d_last_error()
    assert lib.p3d_stream_copy(None, 8192, 32, None) == p3d.P3D_ERR_INVALID_ARG
    assert lib.p3d_stream_copy(4100, 8192, 32, None) == p3d.P3D_ERR_UNSUPPORTED
    assert p3d.p3d_last_error().startswith("p3d_stream_copy")


def test_bilinear_sample_ordered_validation(p3d):
    lib = p3d.lib
    st = lib.p3d_bilinear_sample_ordered(4096, p3d.P3D_BF16, 1, 8, 8, 16, 4096, None, 10, 4098,
                                         8192, p3d.P3D_BF16, None)
    assert st == p3d.P3D_ERR_UNSUPPORTED
    assert p3d.p3d_last_error().startswith("p3d_bilinear_sample_ordered")
    st = lib.p3d_bilinear_sample_ordered(4096, p3d.P3D_BF16, 1, 8, 8, 12, 4096, None, 10, 4096,
                                         8192, p3d.P3D_BF16, None)
    assert st == p3d.P3D_ERR_UNSUPPORTED and "multiple of 8" in p3d.p3d_last_error()
