// api.hip -- the extern "C" entry points of libp3d: validation of every
// argument before anything is enqueued, the host-side camera helpers, and
// dispatch to the kernels. Error messages follow the stage-wiring and lin()
// width-check commits of trellis.cpp PR #38: name the argument and give both
// the expected and the actual value or shape.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>

#include "p3d_internal.h"

using namespace p3d;

namespace {

thread_local std::string g_err;

constexpr int64_t kMaxTokens = int64_t(1) << 30;   // keeps tile counts in int32
constexpr int32_t kMaxOutDim = 1 << 20;            // keeps a tile's offsets in int32
constexpr int32_t kMaxGrid = 1 << 20;              // requantization grids

p3d_status fail(p3d_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

p3d_status ok() {
    g_err.clear();
    return P3D_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

const char* dtype_name(p3d_dtype d) {
    return d == P3D_F32 ? "F32" : d == P3D_BF16 ? "BF16" : "unknown";
}

p3d_status hip_fail(const char* what, hipError_t e) {
    return fail(P3D_ERR_HIP, "%s: HIP launch failed: %s", what, hipGetErrorString(e));
}

// Size of one feature map of the call's batch.
p3d_status check_map_size(const char* fn, const char* what, int32_t batch, int32_t H,
                          int32_t W) {
    if (H < 1 || W < 1)
        return fail(P3D_ERR_INVALID_ARG, "%s: %s height/width must be >= 1, got %dx%d", fn, what,
                    H, W);
    if ((int64_t)batch * H * W > INT32_MAX)
        return fail(P3D_ERR_UNSUPPORTED,
                    "%s: %s batch*height*width must be < 2^31 (row indices are int32), got %lld",
                    fn, what, (long long)((int64_t)batch * H * W));
    return P3D_OK;
}

// Shared checks of the token / camera arguments.
p3d_status check_tokens(const char* fn, const int32_t* coords, int64_t n, int32_t R,
                        p3d_points points, const p3d_camera* cams, int32_t batch,
                        CamTable* tab) {
    if (n < 0) return fail(P3D_ERR_INVALID_ARG, "%s: n must be >= 0, got %lld", fn, (long long)n);
    if (n > kMaxTokens)
        return fail(P3D_ERR_UNSUPPORTED, "%s: n must be <= %lld, got %lld", fn,
                    (long long)kMaxTokens, (long long)n);
    if (R < 1) return fail(P3D_ERR_INVALID_ARG, "%s: resolution must be >= 1, got %d", fn, R);
    if (points != P3D_POINTS_CELL_CENTRES && points != P3D_POINTS_GRID_NODES)
        return fail(P3D_ERR_INVALID_ARG, "%s: points must be CELL_CENTRES or GRID_NODES, got %d",
                    fn, (int)points);
    if (points == P3D_POINTS_GRID_NODES && R < 2)
        return fail(P3D_ERR_INVALID_ARG,
                    "%s: grid-node points need resolution >= 2 (linspace end points), got %d",
                    fn, R);
    if (batch < 1 || batch > P3D_MAX_BATCH)
        return fail(P3D_ERR_INVALID_ARG, "%s: batch must be in [1, %d], got %d", fn,
                    P3D_MAX_BATCH, batch);
    if (!coords) {
        const int64_t r3 = (int64_t)R * R * R;
        if (n > 0 && (R > 1290 || r3 * batch != n))   // 1290^3 * 256 still fits int64
            return fail(P3D_ERR_SHAPE,
                        "%s: dense grid (coords == NULL) needs n == batch*R^3 = %d*%d^3 = %lld, "
                        "got n = %lld", fn, batch, R, (long long)(r3 * batch), (long long)n);
    } else if (!aligned(coords, 16)) {
        return fail(P3D_ERR_UNSUPPORTED, "%s: coords must be 16-byte aligned ([n,4] int32 rows)",
                    fn);
    }
    if (!cams) return fail(P3D_ERR_INVALID_ARG, "%s: cams is NULL (host array [batch])", fn);
    for (int32_t b = 0; b < batch; ++b) {
        const float f = cams[b].focal, d = cams[b].distance;
        if (!(isfinite(f) && f > 0.0f))
            return fail(P3D_ERR_INVALID_ARG, "%s: cams[%d].focal must be finite and > 0, got %g",
                        fn, b, (double)f);
        if (!(isfinite(d) && d > 0.0f))
            return fail(P3D_ERR_INVALID_ARG,
                        "%s: cams[%d].distance must be finite and > 0, got %g", fn, b, (double)d);
        tab->cam[b] = cams[b];
    }
    for (int32_t b = batch; b < P3D_MAX_BATCH; ++b) tab->cam[b] = cams[batch - 1];
    return P3D_OK;
}

// Every check of the fused call; on P3D_OK, *a and *tab describe the launch
// (*nothing set to true when there is no work).
p3d_status prepare_proj_cond(const char* fn, const int32_t* coords, int64_t n,
                             int32_t resolution, p3d_points points, const p3d_camera* cams,
                             int32_t batch, p3d_dtype dtype, const p3d_map* maps,
                             int32_t n_maps, const void* weight, int32_t out_dim,
                             int32_t weight_in, const void* bias, int64_t n_null, void* out,
                             uint8_t* mask, ProjCondArgs* args, CamTable* tab_out,
                             bool* nothing) {
    CamTable& tab = *tab_out;
    *nothing = false;
    p3d_status st = check_tokens(fn, coords, n, resolution, points, cams, batch, &tab);
    if (st != P3D_OK) return st;
    if (!maps || n_maps < 1 || n_maps > 2)
        return fail(P3D_ERR_INVALID_ARG, "%s: maps must be a host array of 1 or 2 maps, got %d",
                    fn, maps ? n_maps : 0);
    if (dtype != P3D_F32 && dtype != P3D_BF16)
        return fail(P3D_ERR_DTYPE, "%s: dtype must be F32 or BF16, got %d", fn, (int)dtype);
    const int epv = dtype == P3D_BF16 ? 8 : 4;
    int64_t channels = 0;
    for (int32_t m = 0; m < n_maps; ++m) {
        char what[32];
        snprintf(what, sizeof what, n_maps > 1 ? "maps[%d]" : "feature map", m);
        st = check_map_size(fn, what, batch, maps[m].height, maps[m].width);
        if (st != P3D_OK) return st;
        if (maps[m].channels < 1)
            return fail(P3D_ERR_INVALID_ARG, "%s: %s channels must be >= 1, got %d", fn, what,
                        maps[m].channels);
        if (maps[m].channels % epv)
            return fail(P3D_ERR_UNSUPPORTED,
                        "%s: %s channels must be a multiple of %d for %s (16-byte rows), got %d",
                        fn, what, epv, dtype_name(dtype), maps[m].channels);
        if (!aligned(maps[m].feat, 16))
            return fail(P3D_ERR_UNSUPPORTED, "%s: %s feat must be 16-byte aligned", fn, what);
        channels += maps[m].channels;
    }
    if (n_maps == 2 && maps[0].channels % 64)
        return fail(P3D_ERR_UNSUPPORTED,
                    "%s: with two maps, maps[0].channels must be a multiple of 64, got %d", fn,
                    maps[0].channels);
    if (channels > INT32_MAX / 2)
        return fail(P3D_ERR_UNSUPPORTED, "%s: too many channels (%lld)", fn,
                    (long long)channels);
    if (n_null < 0 || n_null > kMaxTokens)
        return fail(P3D_ERR_INVALID_ARG, "%s: n_null must be in [0, %lld], got %lld", fn,
                    (long long)kMaxTokens, (long long)n_null);
    if (out_dim < 1)
        return fail(P3D_ERR_INVALID_ARG, "%s: out_dim must be >= 1, got %d", fn, out_dim);
    if (out_dim > kMaxOutDim)
        return fail(P3D_ERR_UNSUPPORTED, "%s: out_dim must be <= %d, got %d", fn, kMaxOutDim,
                    out_dim);
    {
        // tile counts are int32 in the launches: 128-token tiles of 512
        // (BF16) or 128 (F32) features
        const int64_t fw = dtype == P3D_BF16 ? 512 : 128;
        const int64_t tiles = ((n + 127) / 128) * ((out_dim + fw - 1) / fw);
        if (tiles >= ((int64_t)1 << 31))
            return fail(P3D_ERR_UNSUPPORTED,
                        "%s: %lld tokens x %d features make %lld tiles; the limit is 2^31 - 1",
                        fn, (long long)n, out_dim, (long long)tiles);
    }
    if (weight_in != channels) {
        const p3d_map& m0 = maps[0];
        if (n_maps == 1)
            return fail(P3D_ERR_SHAPE,
                        "%s: proj_linear weight is [%d, %d] but the feature map [%d, %d, %d, %d] "
                        "has %d channels: the weight's input width must equal the map's channels",
                        fn, out_dim, weight_in, batch, m0.height, m0.width, m0.channels,
                        m0.channels);
        const p3d_map& m1 = maps[1];
        return fail(P3D_ERR_SHAPE,
                    "%s: proj_linear weight is [%d, %d] but the feature maps [%d, %d, %d, %d] and "
                    "[%d, %d, %d, %d] concatenate to %lld channels: the weight's input width must "
                    "equal the summed channels",
                    fn, out_dim, weight_in, batch, m0.height, m0.width, m0.channels, batch,
                    m1.height, m1.width, m1.channels, (long long)channels);
    }
    if (out_dim % epv)
        return fail(P3D_ERR_UNSUPPORTED,
                    "%s: out_dim must be a multiple of %d for %s (16-byte rows), got %d", fn, epv,
                    dtype_name(dtype), out_dim);
    if (!aligned(weight, 16) || !aligned(out, 16) || !aligned(bias, 16))
        return fail(P3D_ERR_UNSUPPORTED, "%s: feat, weight, bias and out must be 16-byte aligned",
                    fn);
    if (n == 0 && n_null == 0) {
        *nothing = true;
        return P3D_OK;
    }
    if (!out) return fail(P3D_ERR_INVALID_ARG, "%s: out is NULL", fn);
    if (n > 0 && (!maps[0].feat || (n_maps == 2 && !maps[1].feat) || !weight))
        return fail(P3D_ERR_INVALID_ARG, "%s: feat and weight must be non-NULL", fn);
    ProjCondArgs& a = *args;
    a = ProjCondArgs{};
    a.coords = coords;
    a.n = n;
    a.R = resolution;
    a.points = (int32_t)points;
    a.batch = batch;
    a.feat = maps[0].feat;
    a.H = maps[0].height;
    a.W = maps[0].width;
    a.C = maps[0].channels;
    if (n_maps == 2) {
        a.feat1 = maps[1].feat;
        a.H1 = maps[1].height;
        a.W1 = maps[1].width;
        a.C1 = maps[1].channels;
    }
    a.weight = weight;
    a.bias = bias;
    a.D = out_dim;
    a.n_null = n_null;
    a.out = out;
    a.mask = mask;
    return P3D_OK;
}

// Key map of the image-space order: the map with the most texels.
void key_map(const p3d_map* maps, int32_t n_maps, int32_t* H, int32_t* W) {
    *H = maps[0].height;
    *W = maps[0].width;
    if (n_maps == 2 && (int64_t)maps[1].height * maps[1].width > (int64_t)*H * *W) {
        *H = maps[1].height;
        *W = maps[1].width;
    }
}

// Bytes of the ordered path's scratch for n tokens: the sort (bins, counts)
// and the order itself.
size_t ordered_bytes(int64_t n, int32_t batch, const p3d_map* maps, int32_t n_maps,
                     OrderBufs* ob, void* base) {
    int32_t kH, kW;
    key_map(maps, n_maps, &kH, &kW);
    return order_layout(n, batch, kH, kW, base, ob) + (((size_t)n * 4 + 255) & ~(size_t)255);
}

// The launches of p3d_proj_cond_ws once the arguments are checked: BF16
// calls with tokens sort them in `base` (bytes long) and run the fused kernel
// through that order; other calls run p3d_proj_cond_ex's kernels.
p3d_status run_ordered(const char* fn, ProjCondArgs a, const CamTable& tab, p3d_dtype dtype,
                       const p3d_map* maps, int32_t n_maps, void* base, size_t bytes,
                       hipStream_t s) {
    if (dtype == P3D_BF16 && a.n > 0) {
        OrderBufs ob;
        const size_t need = ordered_bytes(a.n, a.batch, maps, n_maps, &ob, base);
        if (!base || bytes < need)
            return fail(P3D_ERR_INVALID_ARG,
                        "%s: workspace must be a device buffer of at least %zu bytes "
                        "(p3d_proj_cond_workspace_size), got %zu bytes at %p",
                        fn, need, bytes, base);
        if (!aligned(base, 256))
            return fail(P3D_ERR_UNSUPPORTED, "%s: workspace must be 256-byte aligned", fn);
        int32_t* order = reinterpret_cast<int32_t*>(static_cast<char*>(base) + need -
                                                    (((size_t)a.n * 4 + 255) & ~(size_t)255));
        const OrderArgs oa{a.coords, a.n, a.R, a.points, a.batch};
        hipError_t e = launch_order(oa, tab, ob, order, s);
        if (e != hipSuccess) return hip_fail(fn, e);
        a.order = order;
    }
    hipError_t e = launch_proj_cond(a, dtype, tab, s);
    if (e != hipSuccess) return hip_fail(fn, e);
    return ok();
}

// Scratch of p3d_proj_cond_noalloc, for callers that cannot allocate: the
// sort of up to P3D_NOALLOC_MAX_TOKENS tokens (bins, bin counts, order),
// 8.25 MB that every GPU the library runs on holds until the process ends.
// Host code never uses this name as an address (on the host it is only a
// stand-in for the device variable): scratch_address() looks up the device
// address once per device, with that device current, and the launches take
// that pointer. The bin counts are cleared by a kernel on every call; every
// other byte is written before it is read. Calls that overlap on one GPU
// share the array and race.
constexpr size_t kScratchBytes = (size_t)P3D_NOALLOC_MAX_TOKENS * 8 + 2 * 65536 + 1024;
static __device__ __align__(256) char scratch[kScratchBytes];

p3d_status scratch_address(const char* fn, void** out) {
    static std::mutex lock;
    static void* addr[64] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= 64)
        return fail(P3D_ERR_HIP, "%s: no current device (%s)", fn,
                    e != hipSuccess ? hipGetErrorString(e) : "device index out of range");
    std::lock_guard<std::mutex> g(lock);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(P3D_ERR_HIP, "%s: hipGetSymbolAddress of the scratch array failed: %s",
                        fn, hipGetErrorString(e));
        addr[dev] = p;
    }
    *out = addr[dev];
    return P3D_OK;
}

}  // namespace

extern "C" {

const char* p3d_version(void) { return "p3d 1.0.0 gfx950"; }

p3d_status p3d_stream_copy(const void* src, void* dst, int64_t bytes, void* stream) {
    const char* fn = "p3d_stream_copy";
    if (bytes < 0) return fail(P3D_ERR_INVALID_ARG, "%s: bytes must be >= 0, got %lld", fn,
                               (long long)bytes);
    if (bytes % 16)
        return fail(P3D_ERR_UNSUPPORTED, "%s: bytes must be a multiple of 16, got %lld", fn,
                    (long long)bytes);
    if (bytes == 0) return ok();
    if (!src || !dst) return fail(P3D_ERR_INVALID_ARG, "%s: src and dst must be non-NULL", fn);
    if (!aligned(src, 16) || !aligned(dst, 16))
        return fail(P3D_ERR_UNSUPPORTED, "%s: src and dst must be 16-byte aligned", fn);
    hipError_t e = launch_stream_copy(src, dst, bytes / 16, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(fn, e);
    return ok();
}

const char* p3d_status_string(p3d_status s) {
    switch (s) {
        case P3D_OK: return "P3D_OK";
        case P3D_ERR_INVALID_ARG: return "P3D_ERR_INVALID_ARG";
        case P3D_ERR_SHAPE: return "P3D_ERR_SHAPE";
        case P3D_ERR_DTYPE: return "P3D_ERR_DTYPE";
        case P3D_ERR_UNSUPPORTED: return "P3D_ERR_UNSUPPORTED";
        case P3D_ERR_HIP: return "P3D_ERR_HIP";
    }
    return "P3D_ERR_UNKNOWN";
}

const char* p3d_last_error(void) { return g_err.c_str(); }

double p3d_distance_from_fov(double fov_deg, int32_t image_size, int32_t extend_px) {
    if (!(fov_deg > 0.0 && fov_deg < 180.0)) {
        fail(P3D_ERR_INVALID_ARG, "p3d_distance_from_fov: fov_deg must be in (0, 180), got %g",
             fov_deg);
        return NAN;
    }
    if (image_size < 1) {
        fail(P3D_ERR_INVALID_ARG, "p3d_distance_from_fov: image_size must be >= 1, got %d",
             image_size);
        return NAN;
    }
    const double half = 0.5 * (double)image_size;
    if (!(half + (double)extend_px > 0.0)) {
        fail(P3D_ERR_INVALID_ARG,
             "p3d_distance_from_fov: image_size/2 + extend_px must be > 0, got %g + %d", half,
             extend_px);
        return NAN;
    }
    g_err.clear();
    const double tan_half = tan(fov_deg * M_PI / 360.0);
    return 0.5 / tan_half * half / (half + (double)extend_px);
}

p3d_status p3d_make_camera(double fov_deg, double distance, p3d_camera* out) {
    if (!out) return fail(P3D_ERR_INVALID_ARG, "p3d_make_camera: out is NULL");
    if (!(fov_deg > 0.0 && fov_deg < 180.0))
        return fail(P3D_ERR_INVALID_ARG, "p3d_make_camera: fov_deg must be in (0, 180), got %g",
                    fov_deg);
    if (!(isfinite(distance) && distance > 0.0))
        return fail(P3D_ERR_INVALID_ARG,
                    "p3d_make_camera: distance must be finite and > 0, got %g", distance);
    out->focal = (float)(1.0 / tan(fov_deg * M_PI / 360.0));
    out->distance = (float)distance;
    return ok();
}

p3d_status p3d_project_points_ex(const int32_t* coords, int64_t n, int32_t resolution,
                                 p3d_points points, const p3d_camera* cams, int32_t batch,
                                 int32_t height, int32_t width, float* grid, int32_t* pixel,
                                 float* frac, float* depth, uint8_t* mask, void* stream) {
    const char* fn = "p3d_project_points";
    CamTable tab;
    p3d_status st = check_tokens(fn, coords, n, resolution, points, cams, batch, &tab);
    if (st != P3D_OK) return st;
    st = check_map_size(fn, "feature map", batch, height, width);
    if (st != P3D_OK) return st;
    if (!aligned(grid, 8) || !aligned(pixel, 8) || !aligned(frac, 8))
        return fail(P3D_ERR_UNSUPPORTED, "%s: grid, pixel and frac must be 8-byte aligned", fn);
    if (n == 0) return ok();
    ProjectArgs a{coords, n,     resolution, (int32_t)points, batch, height, width,
                  grid,   pixel, frac,       depth,           mask};
    hipError_t e = launch_project(a, tab, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(fn, e);
    return ok();
}

p3d_status p3d_project_points(const int32_t* coords, int64_t n, int32_t resolution,
                              const p3d_camera* cams, int32_t batch, int32_t height,
                              int32_t width, float* grid, int32_t* pixel, float* frac,
                              float* depth, uint8_t* mask, void* stream) {
    return p3d_project_points_ex(coords, n, resolution, P3D_POINTS_CELL_CENTRES, cams, batch,
                                 height, width, grid, pixel, frac, depth, mask, stream);
}

p3d_status p3d_requantize_coords(const int32_t* src, int64_t n, int32_t src_resolution,
                                 int32_t grid, p3d_requant mode, int32_t* dst, void* stream) {
    const char* fn = "p3d_requantize_coords";
    if (n < 0) return fail(P3D_ERR_INVALID_ARG, "%s: n must be >= 0, got %lld", fn, (long long)n);
    if (n > kMaxTokens)
        return fail(P3D_ERR_UNSUPPORTED, "%s: n must be <= %lld, got %lld", fn,
                    (long long)kMaxTokens, (long long)n);
    if (mode != P3D_REQUANT_ROUND_NODES && mode != P3D_REQUANT_FLOOR_CELLS)
        return fail(P3D_ERR_INVALID_ARG, "%s: mode must be ROUND_NODES or FLOOR_CELLS, got %d",
                    fn, (int)mode);
    if (src_resolution < 1 || src_resolution > kMaxGrid || grid < 1 || grid > kMaxGrid)
        return fail(P3D_ERR_INVALID_ARG,
                    "%s: src_resolution and grid must be in [1, %d], got %d and %d", fn,
                    kMaxGrid, src_resolution, grid);
    if (mode == P3D_REQUANT_ROUND_NODES && grid < 2)
        return fail(P3D_ERR_INVALID_ARG, "%s: nearest-node rounding needs grid >= 2, got %d", fn,
                    grid);
    if (!aligned(src, 16) || !aligned(dst, 16))
        return fail(P3D_ERR_UNSUPPORTED, "%s: src and dst must be 16-byte aligned ([n,4] int32)",
                    fn);
    if (n == 0) return ok();
    if (!src || !dst) return fail(P3D_ERR_INVALID_ARG, "%s: src and dst must be non-NULL", fn);
    RequantArgs a{src, dst, n, src_resolution, grid, (int32_t)mode};
    hipError_t e = launch_requantize(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(fn, e);
    return ok();
}

p3d_status p3d_bilinear_sample_ordered(const void* feat, p3d_dtype feat_dtype, int32_t batch,
                                       int32_t height, int32_t width, int32_t channels,
                                       const float* grid, const int32_t* batch_index, int64_t n,
                                       const int32_t* order, void* out, p3d_dtype out_dtype,
                                       void* stream) {
    const char* fn = order ? "p3d_bilinear_sample_ordered" : "p3d_bilinear_sample";
    if (!aligned(order, 4)) return fail(P3D_ERR_UNSUPPORTED, "%s: order must be 4-byte aligned", fn);
    if (n < 0) return fail(P3D_ERR_INVALID_ARG, "%s: n must be >= 0, got %lld", fn, (long long)n);
    if (n > kMaxTokens)
        return fail(P3D_ERR_UNSUPPORTED, "%s: n must be <= %lld, got %lld", fn,
                    (long long)kMaxTokens, (long long)n);
    if (feat_dtype != P3D_F32 && feat_dtype != P3D_BF16)
        return fail(P3D_ERR_DTYPE, "%s: feat_dtype must be F32 or BF16, got %d", fn,
                    (int)feat_dtype);
    if (out_dtype != P3D_F32 && out_dtype != P3D_BF16)
        return fail(P3D_ERR_DTYPE, "%s: out_dtype must be F32 or BF16, got %d", fn,
                    (int)out_dtype);
    if (feat_dtype == P3D_F32 && out_dtype == P3D_BF16)
        return fail(P3D_ERR_DTYPE, "%s: a BF16 output needs a BF16 map (feat F32, out BF16)", fn);
    if (batch < 1 || height < 1 || width < 1 || channels < 1)
        return fail(P3D_ERR_INVALID_ARG,
                    "%s: map shape must be positive, got [batch=%d, H=%d, W=%d, C=%d]", fn,
                    batch, height, width, channels);
    if ((int64_t)batch * height * width > INT32_MAX)
        return fail(P3D_ERR_UNSUPPORTED, "%s: batch*height*width must be < 2^31, got %lld", fn,
                    (long long)((int64_t)batch * height * width));
    const int epv = feat_dtype == P3D_BF16 ? 8 : 4;
    if (channels % epv)
        return fail(P3D_ERR_UNSUPPORTED,
                    "%s: channels must be a multiple of %d for a %s map (16-byte rows), got %d",
                    fn, epv, dtype_name(feat_dtype), channels);
    if (!aligned(feat, 16) || !aligned(out, 16) || !aligned(grid, 8))
        return fail(P3D_ERR_UNSUPPORTED, "%s: feat and out must be 16-byte aligned, grid 8-byte",
                    fn);
    if (n == 0) return ok();
    if (!feat || !grid || !out)
        return fail(P3D_ERR_INVALID_ARG, "%s: feat, grid and out must be non-NULL", fn);
    SampleArgs a{};
    a.feat = feat;
    a.batch = batch;
    a.H = height;
    a.W = width;
    a.C = channels;
    a.grid = grid;
    a.bidx = batch_index;
    a.n = n;
    a.out = out;
    a.out_stride = channels;
    a.order = order;
    static const CamTable no_cams{};
    hipError_t e = launch_sample(a, feat_dtype, out_dtype, no_cams,
                                 static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(fn, e);
    return ok();
}

p3d_status p3d_bilinear_sample(const void* feat, p3d_dtype feat_dtype, int32_t batch,
                               int32_t height, int32_t width, int32_t channels,
                               const float* grid, const int32_t* batch_index, int64_t n,
                               void* out, p3d_dtype out_dtype, void* stream) {
    return p3d_bilinear_sample_ordered(feat, feat_dtype, batch, height, width, channels, grid,
                                       batch_index, n, nullptr, out, out_dtype, stream);
}

p3d_status p3d_proj_cond_ex(const int32_t* coords, int64_t n, int32_t resolution,
                            p3d_points points, const p3d_camera* cams, int32_t batch,
                            p3d_dtype dtype, const p3d_map* maps, int32_t n_maps,
                            const void* weight, int32_t out_dim, int32_t weight_in,
                            const void* bias, int64_t n_null, void* out, uint8_t* mask,
                            void* stream) {
    const char* fn = "p3d_proj_cond";
    ProjCondArgs a;
    CamTable tab;
    bool nothing;
    p3d_status st = prepare_proj_cond(fn, coords, n, resolution, points, cams, batch, dtype, maps,
                                      n_maps, weight, out_dim, weight_in, bias, n_null, out, mask,
                                      &a, &tab, &nothing);
    if (st != P3D_OK) return st;
    if (nothing) return ok();
    hipError_t e = launch_proj_cond(a, dtype, tab, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(fn, e);
    return ok();
}

p3d_status p3d_proj_cond_ordered(const int32_t* coords, int64_t n, int32_t resolution,
                                 p3d_points points, const p3d_camera* cams, int32_t batch,
                                 p3d_dtype dtype, const p3d_map* maps, int32_t n_maps,
                                 const void* weight, int32_t out_dim, int32_t weight_in,
                                 const void* bias, int64_t n_null, void* out, uint8_t* mask,
                                 const int32_t* order, void* stream) {
    const char* fn = "p3d_proj_cond_ordered";
    if (!aligned(order, 4)) return fail(P3D_ERR_UNSUPPORTED, "%s: order must be 4-byte aligned", fn);
    ProjCondArgs a;
    CamTable tab;
    bool nothing;
    p3d_status st = prepare_proj_cond(fn, coords, n, resolution, points, cams, batch, dtype, maps,
                                      n_maps, weight, out_dim, weight_in, bias, n_null, out, mask,
                                      &a, &tab, &nothing);
    if (st != P3D_OK) return st;
    if (nothing) return ok();
    if (n > 0 && !order) return fail(P3D_ERR_INVALID_ARG, "%s: order is NULL", fn);
    if (dtype == P3D_BF16) a.order = order;
    hipError_t e = launch_proj_cond(a, dtype, tab, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(fn, e);
    return ok();
}

size_t p3d_proj_cond_workspace_size(int64_t n, int32_t batch, const p3d_map* maps,
                                    int32_t n_maps) {
    const char* fn = "p3d_proj_cond_workspace_size";
    if (n < 0 || n > kMaxTokens || batch < 1 || batch > P3D_MAX_BATCH || !maps || n_maps < 1 ||
        n_maps > 2) {
        fail(P3D_ERR_INVALID_ARG,
             "%s: needs 0 <= n <= %lld, 1 <= batch <= %d and a host array of 1 or 2 maps, "
             "got n = %lld, batch = %d, %d maps",
             fn, (long long)kMaxTokens, P3D_MAX_BATCH, (long long)n, batch, maps ? n_maps : 0);
        return 0;
    }
    for (int32_t m = 0; m < n_maps; ++m) {
        if (maps[m].height < 1 || maps[m].width < 1) {
            fail(P3D_ERR_INVALID_ARG, "%s: maps[%d] height/width must be >= 1, got %dx%d", fn, m,
                 maps[m].height, maps[m].width);
            return 0;
        }
    }
    g_err.clear();
    return ordered_bytes(n, batch, maps, n_maps, nullptr, nullptr);
}

p3d_status p3d_proj_cond_ws(const int32_t* coords, int64_t n, int32_t resolution,
                            p3d_points points, const p3d_camera* cams, int32_t batch,
                            p3d_dtype dtype, const p3d_map* maps, int32_t n_maps,
                            const void* weight, int32_t out_dim, int32_t weight_in,
                            const void* bias, int64_t n_null, void* out, uint8_t* mask,
                            void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "p3d_proj_cond_ws";
    ProjCondArgs a;
    CamTable tab;
    bool nothing;
    p3d_status st = prepare_proj_cond(fn, coords, n, resolution, points, cams, batch, dtype, maps,
                                      n_maps, weight, out_dim, weight_in, bias, n_null, out, mask,
                                      &a, &tab, &nothing);
    if (st != P3D_OK) return st;
    if (nothing) return ok();
    return run_ordered(fn, a, tab, dtype, maps, n_maps, workspace, workspace_bytes,
                       static_cast<hipStream_t>(stream));
}

// The allocation-free variant of p3d_proj_cond_ws: the same launches, with
// the sort's scratch in this file's `scratch` array (see its comment).
p3d_status p3d_proj_cond_noalloc(const int32_t* coords, int64_t n, int32_t resolution,
                                 p3d_points points, const p3d_camera* cams, int32_t batch,
                                 p3d_dtype dtype, const p3d_map* maps, int32_t n_maps,
                                 const void* weight, int32_t out_dim, int32_t weight_in,
                                 const void* bias, int64_t n_null, void* out, uint8_t* mask,
                                 void* stream) {
    const char* fn = "p3d_proj_cond_noalloc";
    ProjCondArgs a;
    CamTable tab;
    bool nothing;
    p3d_status st = prepare_proj_cond(fn, coords, n, resolution, points, cams, batch, dtype, maps,
                                      n_maps, weight, out_dim, weight_in, bias, n_null, out, mask,
                                      &a, &tab, &nothing);
    if (st != P3D_OK) return st;
    if (n > P3D_NOALLOC_MAX_TOKENS)
        return fail(P3D_ERR_UNSUPPORTED,
                    "%s: n must be <= %d (P3D_NOALLOC_MAX_TOKENS, the size of the library's "
                    "scratch), got %lld; use p3d_proj_cond_ws with a workspace",
                    fn, P3D_NOALLOC_MAX_TOKENS, (long long)n);
    if (nothing) return ok();
    void* base = nullptr;
    st = scratch_address(fn, &base);
    if (st != P3D_OK) return st;
    return run_ordered(fn, a, tab, dtype, maps, n_maps, base, kScratchBytes,
                       static_cast<hipStream_t>(stream));
}

p3d_status p3d_projection_stats_ordered(const int32_t* coords, int64_t n, int32_t resolution,
                                        p3d_points points, const p3d_camera* cams, int32_t batch,
                                        p3d_dtype dtype, const p3d_map* maps, int32_t n_maps,
                                        const int32_t* order, p3d_proj_stats* stats,
                                        void* stream) {
    const char* fn = order ? "p3d_projection_stats_ordered" : "p3d_projection_stats";
    if (!aligned(order, 4)) return fail(P3D_ERR_UNSUPPORTED, "%s: order must be 4-byte aligned", fn);
    CamTable tab;
    p3d_status st = check_tokens(fn, coords, n, resolution, points, cams, batch, &tab);
    if (st != P3D_OK) return st;
    if (!maps || n_maps < 1 || n_maps > 2)
        return fail(P3D_ERR_INVALID_ARG, "%s: maps must be a host array of 1 or 2 maps, got %d",
                    fn, maps ? n_maps : 0);
    if (dtype != P3D_F32 && dtype != P3D_BF16)
        return fail(P3D_ERR_DTYPE, "%s: dtype must be F32 or BF16, got %d", fn, (int)dtype);
    const int epv = dtype == P3D_BF16 ? 8 : 4;
    for (int32_t m = 0; m < n_maps; ++m) {
        char what[32];
        snprintf(what, sizeof what, n_maps > 1 ? "maps[%d]" : "feature map", m);
        st = check_map_size(fn, what, batch, maps[m].height, maps[m].width);
        if (st != P3D_OK) return st;
        if (maps[m].channels < 1 || maps[m].channels % epv)
            return fail(P3D_ERR_UNSUPPORTED,
                        "%s: %s channels must be a positive multiple of %d for %s, got %d", fn,
                        what, epv, dtype_name(dtype), maps[m].channels);
        if (!aligned(maps[m].feat, 16))
            return fail(P3D_ERR_UNSUPPORTED, "%s: %s feat must be 16-byte aligned", fn, what);
        if (n > 0 && !maps[m].feat)
            return fail(P3D_ERR_INVALID_ARG, "%s: %s feat is NULL", fn, what);
    }
    if (!stats) return fail(P3D_ERR_INVALID_ARG, "%s: stats is NULL", fn);
    if (!aligned(stats, 8))
        return fail(P3D_ERR_UNSUPPORTED, "%s: stats must be 8-byte aligned", fn);
    StatsArgs a{};
    a.coords = coords;
    a.n = n;
    a.R = resolution;
    a.points = (int32_t)points;
    a.batch = batch;
    a.feat0 = maps[0].feat;
    a.H0 = maps[0].height;
    a.W0 = maps[0].width;
    a.C0 = maps[0].channels;
    if (n_maps == 2) {
        a.feat1 = maps[1].feat;
        a.H1 = maps[1].height;
        a.W1 = maps[1].width;
        a.C1 = maps[1].channels;
    }
    a.stats = stats;
    a.order = order;
    hipError_t e = launch_stats(a, dtype == P3D_BF16, tab, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(fn, e);
    return ok();
}

p3d_status p3d_projection_stats(const int32_t* coords, int64_t n, int32_t resolution,
                                p3d_points points, const p3d_camera* cams, int32_t batch,
                                p3d_dtype dtype, const p3d_map* maps, int32_t n_maps,
                                p3d_proj_stats* stats, void* stream) {
    return p3d_projection_stats_ordered(coords, n, resolution, points, cams, batch, dtype, maps,
                                        n_maps, nullptr, stats, stream);
}

p3d_status p3d_stats_figures(const p3d_proj_stats* stats, const int32_t* channels,
                             int32_t n_maps, p3d_stats_fig* out) {
    const char* fn = "p3d_stats_figures";
    if (!stats || !out || !channels)
        return fail(P3D_ERR_INVALID_ARG, "%s: stats, channels and out must be non-NULL", fn);
    if (n_maps < 1 || n_maps > 2)
        return fail(P3D_ERR_INVALID_ARG, "%s: n_maps must be 1 or 2, got %d", fn, n_maps);
    for (int32_t h = 0; h < n_maps; ++h)
        if (channels[h] < 1)
            return fail(P3D_ERR_INVALID_ARG, "%s: channels[%d] must be >= 1, got %d", fn, h,
                        channels[h]);
    const double t = stats->tokens;
    out->coverage = t > 0.0 ? stats->inside / t : NAN;
    for (int32_t h = 0; h < 2; ++h) {
        out->mean[h] = NAN;
        out->std[h] = NAN;
        const double cnt = h < n_maps ? t * (double)channels[h] : 0.0;
        if (cnt > 0.0) {
            const double m = stats->sum[h] / cnt;
            const double m2 = stats->sum_sq[h] / cnt;     // E[x^2]
            out->mean[h] = m;
            out->std[h] = sqrt(fmax(m2 - m * m, 0.0));  // rounding may dip below 0
        }
    }
    out->cosine = stats->cos_count > 0.0 ? stats->cos_sum / stats->cos_count : NAN;
    return ok();
}

p3d_status p3d_proj_cond_plan(int64_t n, int32_t out_dim, int32_t compute_units,
                              p3d_tile_plan* plan) {
    const char* fn = "p3d_proj_cond_plan";
    if (!plan) return fail(P3D_ERR_INVALID_ARG, "%s: plan is NULL", fn);
    if (n < 0 || n > kMaxTokens)
        return fail(P3D_ERR_INVALID_ARG, "%s: n must be in [0, %lld], got %lld", fn,
                    (long long)kMaxTokens, (long long)n);
    if (out_dim < 1 || out_dim > kMaxOutDim)
        return fail(P3D_ERR_INVALID_ARG, "%s: out_dim must be in [1, %d], got %d", fn,
                    kMaxOutDim, out_dim);
    if (compute_units < 1)
        return fail(P3D_ERR_INVALID_ARG, "%s: compute_units must be >= 1, got %d", fn,
                    compute_units);
    const int64_t tiles = ((n + 127) / 128) * (((int64_t)out_dim + 511) / 512);
    if (tiles >= ((int64_t)1 << 31))
        return fail(P3D_ERR_UNSUPPORTED,
                    "%s: %lld tokens x %d features make %lld tiles; the limit is 2^31 - 1", fn,
                    (long long)n, out_dim, (long long)tiles);
    *plan = plan_proj_cond_bf16(n, out_dim, compute_units);
    return ok();
}

p3d_status p3d_proj_sample_ordered(const int32_t* coords, int64_t n, int32_t resolution,
                                   p3d_points points, const p3d_camera* cams, int32_t batch,
                                   p3d_dtype dtype, const p3d_map* maps, int32_t n_maps,
                                   const int32_t* order, void* S, uint8_t* mask, void* stream) {
    const char* fn = order ? "p3d_proj_sample_ordered" : "p3d_proj_sample";
    if (!aligned(order, 4)) return fail(P3D_ERR_UNSUPPORTED, "%s: order must be 4-byte aligned", fn);
    CamTable tab;
    p3d_status st = check_tokens(fn, coords, n, resolution, points, cams, batch, &tab);
    if (st != P3D_OK) return st;
    if (!maps || n_maps < 1 || n_maps > 2)
        return fail(P3D_ERR_INVALID_ARG, "%s: maps must be a host array of 1 or 2 maps, got %d",
                    fn, maps ? n_maps : 0);
    if (dtype != P3D_F32 && dtype != P3D_BF16)
        return fail(P3D_ERR_DTYPE, "%s: dtype must be F32 or BF16, got %d", fn, (int)dtype);
    const int epv = dtype == P3D_BF16 ? 8 : 4;
    int64_t channels = 0;
    for (int32_t m = 0; m < n_maps; ++m) {
        char what[32];
        snprintf(what, sizeof what, n_maps > 1 ? "maps[%d]" : "feature map", m);
        st = check_map_size(fn, what, batch, maps[m].height, maps[m].width);
        if (st != P3D_OK) return st;
        if (maps[m].channels < 1 || maps[m].channels % epv)
            return fail(P3D_ERR_UNSUPPORTED,
                        "%s: %s channels must be a positive multiple of %d for %s, got %d", fn,
                        what, epv, dtype_name(dtype), maps[m].channels);
        if (!aligned(maps[m].feat, 16))
            return fail(P3D_ERR_UNSUPPORTED, "%s: %s feat must be 16-byte aligned", fn, what);
        if (n > 0 && !maps[m].feat)
            return fail(P3D_ERR_INVALID_ARG, "%s: %s feat is NULL", fn, what);
        channels += maps[m].channels;
    }
    if (!aligned(S, 16)) return fail(P3D_ERR_UNSUPPORTED, "%s: S must be 16-byte aligned", fn);
    if (n == 0) return ok();
    if (!S) return fail(P3D_ERR_INVALID_ARG, "%s: S is NULL", fn);
    // both maps in one launch: map 1's samples follow map 0's in each S row
    SampleArgs a{};
    a.feat = maps[0].feat;
    a.batch = batch;
    a.H = maps[0].height;
    a.W = maps[0].width;
    a.C = maps[0].channels;
    if (n_maps == 2) {
        a.feat1 = maps[1].feat;
        a.H1 = maps[1].height;
        a.W1 = maps[1].width;
        a.C1 = maps[1].channels;
    }
    a.coords = coords;
    a.R = resolution;
    a.points = (int32_t)points;
    a.project = true;
    a.n = n;
    a.out = S;
    a.out_stride = channels;
    a.out_col = 0;
    a.mask = mask;
    a.order = order;
    hipError_t e = launch_sample(a, dtype, dtype, tab, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(fn, e);
    return ok();
}

p3d_status p3d_proj_sample(const int32_t* coords, int64_t n, int32_t resolution,
                           p3d_points points, const p3d_camera* cams, int32_t batch,
                           p3d_dtype dtype, const p3d_map* maps, int32_t n_maps, void* S,
                           uint8_t* mask, void* stream) {
    return p3d_proj_sample_ordered(coords, n, resolution, points, cams, batch, dtype, maps,
                                   n_maps, nullptr, S, mask, stream);
}

size_t p3d_token_order_workspace_size(int64_t n, int32_t batch, int32_t key_height,
                                      int32_t key_width) {
    if (n < 0 || n > kMaxTokens || batch < 1 || batch > P3D_MAX_BATCH || key_height < 1 ||
        key_width < 1) {
        fail(P3D_ERR_INVALID_ARG,
             "p3d_token_order_workspace_size: needs 0 <= n <= %lld, 1 <= batch <= %d and a "
             "key map of at least 1x1, got n = %lld, batch = %d, %dx%d",
             (long long)kMaxTokens, P3D_MAX_BATCH, (long long)n, batch, key_height, key_width);
        return 0;
    }
    g_err.clear();
    return order_layout(n, batch, key_height, key_width, nullptr, nullptr);
}

p3d_status p3d_token_order(const int32_t* coords, int64_t n, int32_t resolution,
                           p3d_points points, const p3d_camera* cams, int32_t batch,
                           int32_t key_height, int32_t key_width, int32_t* order,
                           void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "p3d_token_order";
    CamTable tab;
    p3d_status st = check_tokens(fn, coords, n, resolution, points, cams, batch, &tab);
    if (st != P3D_OK) return st;
    st = check_map_size(fn, "key map", batch, key_height, key_width);
    if (st != P3D_OK) return st;
    if (n == 0) return ok();
    if (!order || !aligned(order, 4))
        return fail(P3D_ERR_INVALID_ARG, "%s: order must be a 4-byte aligned device array [n]",
                    fn);
    OrderBufs ob;
    const size_t need = order_layout(n, batch, key_height, key_width, workspace, &ob);
    if (!workspace || workspace_bytes < need)
        return fail(P3D_ERR_INVALID_ARG,
                    "%s: workspace must be a device buffer of at least %zu bytes "
                    "(p3d_token_order_workspace_size), got %zu bytes at %p",
                    fn, need, workspace_bytes, workspace);
    if (!aligned(workspace, 256))
        return fail(P3D_ERR_UNSUPPORTED, "%s: workspace must be 256-byte aligned", fn);
    const OrderArgs oa{coords, n, resolution, (int32_t)points, batch};
    hipError_t e = launch_order(oa, tab, ob, order, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(fn, e);
    return ok();
}

p3d_status p3d_proj_linear_grouped(const void* S, int64_t n, int32_t K, p3d_dtype dtype,
                                   int32_t groups, const void* const* weights,
                                   const void* const* biases, int32_t out_dim,
                                   void* const* outs, int32_t accumulate, void* stream) {
    const char* fn = "p3d_proj_linear_grouped";
    if (n < 0) return fail(P3D_ERR_INVALID_ARG, "%s: n must be >= 0, got %lld", fn, (long long)n);
    if (n > kMaxTokens)
        return fail(P3D_ERR_UNSUPPORTED, "%s: n must be <= %lld, got %lld", fn,
                    (long long)kMaxTokens, (long long)n);
    if (dtype != P3D_BF16)
        return fail(P3D_ERR_UNSUPPORTED, "%s: only BF16 S and weights are supported, got %s", fn,
                    dtype_name(dtype));
    if (groups < 1 || groups > P3D_MAX_GROUPS)
        return fail(P3D_ERR_INVALID_ARG, "%s: groups must be in [1, %d], got %d", fn,
                    P3D_MAX_GROUPS, groups);
    if (K < 8 || K % 8)
        return fail(P3D_ERR_UNSUPPORTED, "%s: K must be a positive multiple of 8, got %d", fn, K);
    if (out_dim < 8 || out_dim % 8 || out_dim > kMaxOutDim)
        return fail(P3D_ERR_UNSUPPORTED,
                    "%s: out_dim must be a positive multiple of 8 up to %d, got %d", fn,
                    kMaxOutDim, out_dim);
    if (!weights || !outs)
        return fail(P3D_ERR_INVALID_ARG, "%s: weights and outs must be host arrays [%d]", fn,
                    groups);
    if (!aligned(S, 16)) return fail(P3D_ERR_UNSUPPORTED, "%s: S must be 16-byte aligned", fn);
    GroupedArgs a{};
    for (int32_t g = 0; g < groups; ++g) {
        if (!weights[g] || !outs[g])
            return fail(P3D_ERR_INVALID_ARG, "%s: weights[%d] and outs[%d] must be non-NULL", fn,
                        g, g);
        const void* b = biases ? biases[g] : nullptr;
        if (!aligned(weights[g], 16) || !aligned(outs[g], 16) || !aligned(b, 16))
            return fail(P3D_ERR_UNSUPPORTED,
                        "%s: weights[%d], biases[%d] and outs[%d] must be 16-byte aligned", fn, g,
                        g, g);
        a.W[g] = weights[g];
        a.bias[g] = b;
        a.out[g] = outs[g];
    }
    if (n == 0) return ok();
    if (!S) return fail(P3D_ERR_INVALID_ARG, "%s: S is NULL", fn);
    a.S = S;
    a.n = n;
    a.K = K;
    a.G = groups;
    a.D = out_dim;
    hipError_t e = launch_grouped(a, accumulate != 0, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(fn, e);
    return ok();
}

p3d_status p3d_proj_cond(const int32_t* coords, int64_t n, int32_t resolution,
                         const p3d_camera* cams, int32_t batch, const void* feat,
                         p3d_dtype dtype, int32_t height, int32_t width, int32_t channels,
                         const void* weight, int32_t out_dim, int32_t weight_in,
                         const void* bias, int64_t n_null, void* out, uint8_t* mask,
                         void* stream) {
    const p3d_map map{feat, height, width, channels};
    return p3d_proj_cond_ex(coords, n, resolution, P3D_POINTS_CELL_CENTRES, cams, batch, dtype,
                            &map, 1, weight, out_dim, weight_in, bias, n_null, out, mask, stream);
}

}  // extern "C"
