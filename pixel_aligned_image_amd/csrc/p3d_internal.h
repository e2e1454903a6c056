// p3d_internal.h -- device-side building blocks and launch interfaces of
// libp3d (gfx950). Not installed; the public interface is include/p3d.h.
//
// Every translation unit is compiled with -ffp-contract=off: the projection
// and index mapping below must round once per operation, in the written
// order, so that pixel indices and masks are reproducible bit for bit. Where
// a fused multiply-add is wanted (the bilinear blend, never an index
// decision) it is written explicitly with fmaf.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "p3d.h"

namespace p3d {

struct CamTable {
    p3d_camera cam[P3D_MAX_BATCH];
};

// ---------------------------------------------------------------------------
// Projection (pixel-aligned head commit: project_points; pixal3d.cpp commit:
// fixed frontal camera on +Z looking down -Z, full-angle focal).
// ---------------------------------------------------------------------------

// Integer cell of token t: explicit coords (b, x, y, z), or the dense
// enumeration t = ((b*R + x)*R + y)*R + z.
__device__ __forceinline__ void token_cell(const int32_t* __restrict__ coords, int64_t t,
                                           int32_t R, int32_t& b, int32_t& x, int32_t& y,
                                           int32_t& z) {
    if (coords) {
        const int4 c = *reinterpret_cast<const int4*>(coords + 4 * t);
        b = c.x; x = c.y; y = c.z; z = c.w;
    } else {
        const int64_t r = R;
        z = (int32_t)(t % r);
        const int64_t q = t / r;
        y = (int32_t)(q % r);
        const int64_t q2 = q / r;
        x = (int32_t)(q2 % r);
        b = (int32_t)(q2 / r);
    }
}

// The token at position t of an image-space order (order.hip), or t itself
// without one. An order entry outside [0, n) (a caller contract violation)
// is clamped into it, so no access leaves the coords or output rows.
__device__ __forceinline__ int64_t ordered_token(const int32_t* __restrict__ order, int64_t t,
                                                int64_t n) {
    if (!order) return t;
    const int64_t k = order[t];
    return k < 0 ? 0 : (k >= n ? n - 1 : k);
}

// Cell centre in the unit cube [-1/2, 1/2]: (c + 1/2)/R - 1/2, binary32.
__device__ __forceinline__ float cell_centre(int32_t c, int32_t R) {
    return ((float)c + 0.5f) / (float)R - 0.5f;
}

// Node c of the endpoint-inclusive projection grid linspace(-1, 1, R) at half
// scale (cascade requantization commit): c/(R - 1) - 1/2, binary32; R >= 2.
__device__ __forceinline__ float grid_node(int32_t c, int32_t R) {
    return (float)c / (float)(R - 1) - 0.5f;
}

// World coordinate of integer position c: cell centre or grid node
// (p3d_points; uniform across a launch).
__device__ __forceinline__ float token_point(int32_t c, int32_t R, int32_t points) {
    return points == P3D_POINTS_GRID_NODES ? grid_node(c, R) : cell_centre(c, R);
}

struct Projected {
    float gx, gy, depth;
    int32_t b;      // batch item after clamping into [0, batch)
    uint8_t mask;
};

__device__ __forceinline__ Projected project_cell(int32_t b, int32_t cx, int32_t cy, int32_t cz,
                                                  int32_t R, int32_t points,
                                                  const CamTable& cams, int32_t batch) {
    Projected p;
    const bool valid = (b >= 0) && (b < batch);
    b = b < 0 ? 0 : (b >= batch ? batch - 1 : b);
    const float px = token_point(cx, R, points);
    const float py = token_point(cy, R, points);
    const float pz = token_point(cz, R, points);
    const float f = cams.cam[b].focal;
    const float depth = cams.cam[b].distance - pz;
    const float gx = (f * px) / depth;
    const float gy = -((f * py) / depth);
    p.gx = gx;
    p.gy = gy;
    p.depth = depth;
    p.b = b;
    p.mask = (uint8_t)(valid && depth > 0.0f && gx >= -1.0f && gx <= 1.0f &&
                       gy >= -1.0f && gy <= 1.0f);
    return p;
}

// grid_sample(align_corners=False, padding_mode='border') source index: the
// normalised g maps to ((g+1)*size - 1)/2, which is clamped to [0, size-1]
// (NaN -> 0) BEFORE the two neighbouring texels are chosen.
struct SrcIdx {
    int32_t i0, i1;
    float t;
};

__device__ __forceinline__ SrcIdx source_index(float g, int32_t size) {
    float ix = ((g + 1.0f) * (float)size - 1.0f) / 2.0f;
    ix = fminf(fmaxf(ix, 0.0f), (float)(size - 1));
    const float fl = floorf(ix);
    SrcIdx s;
    s.i0 = (int32_t)fl;
    s.t = ix - fl;
    s.i1 = (s.i0 + 1 < size) ? s.i0 + 1 : size - 1;
    return s;
}

// Corner rows (in units of map rows of C channels) and bilinear weights of
// one sampling point.
struct Corners {
    int32_t r00, r01, r10, r11;
    float w00, w01, w10, w11;
};

__device__ __forceinline__ Corners corners_of(float gx, float gy, int32_t b, int32_t H,
                                              int32_t W) {
    const SrcIdx sx = source_index(gx, W);
    const SrcIdx sy = source_index(gy, H);
    Corners c;
    const int32_t base = b * H;
    c.r00 = (base + sy.i0) * W + sx.i0;
    c.r01 = (base + sy.i0) * W + sx.i1;
    c.r10 = (base + sy.i1) * W + sx.i0;
    c.r11 = (base + sy.i1) * W + sx.i1;
    c.w00 = (1.0f - sx.t) * (1.0f - sy.t);
    c.w01 = sx.t * (1.0f - sy.t);
    c.w10 = (1.0f - sx.t) * sy.t;
    c.w11 = sx.t * sy.t;
    return c;
}

// ---------------------------------------------------------------------------
// bf16 helpers. Widening is a shift; narrowing uses the gfx950 packed
// convert (round to nearest even, NaN stays NaN).
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte store that bypasses the caches' allocate-on-write (streamed output).
__device__ __forceinline__ void store_nt16(void* p, uint4 v) {
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, v), reinterpret_cast<u32x4_t*>(p));
}

__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------------------
// Launch interfaces (each returns the hipError_t of its launch).
// ---------------------------------------------------------------------------
struct ProjectArgs {
    const int32_t* coords;
    int64_t n;
    int32_t R, points, batch, H, W;
    float* grid;
    int32_t* pixel;
    float* frac;
    float* depth;
    uint8_t* mask;
};

struct SampleArgs {
    const void* feat;
    int32_t batch, H, W, C;
    const float* grid;            // points (grid mode), or
    const int32_t* bidx;
    const int32_t* coords;        // tokens to project (project mode)
    int32_t R, points;
    bool project;
    int64_t n;
    void* out;                    // row t, columns [out_col, out_col + C)
    int64_t out_stride;           // elements per output row
    int32_t out_col;
    uint8_t* mask;                // project mode: in-image mask, or NULL
    const int32_t* order;         // point (token) of each position, or NULL
    const void* feat1;            // project mode: a second map [batch, H1, W1, C1]
    int32_t H1, W1, C1;           // (C1 == 0: none); its samples follow map 0's
};

struct ProjCondArgs {
    const int32_t* coords;
    int64_t n;
    int32_t R, points, batch;
    const void* feat;             // map 0 [batch, H, W, C]
    int32_t H, W, C;
    const void* feat1;            // map 1 [batch, H1, W1, C1], or C1 == 0
    int32_t H1, W1, C1;           // K = C + C1; C % 64 == 0 when C1 > 0
    const void* weight;
    const void* bias;
    int32_t D;
    int64_t n_null;
    void* out;
    uint8_t* mask;
    const int32_t* order;         // token of each processed position, or NULL (identity)
};

struct RequantArgs {
    const int32_t* src;
    int32_t* dst;
    int64_t n;
    int32_t src_res, grid, mode;
};

struct StatsArgs {
    const int32_t* coords;
    int64_t n;
    int32_t R, points, batch;
    const void* feat0;
    int32_t H0, W0, C0;
    const void* feat1;            // or C1 == 0
    int32_t H1, W1, C1;
    p3d_proj_stats* stats;
    const int32_t* order;         // token of each position, or NULL
};

struct GroupedArgs {
    const void* S;                // [n, K] bf16
    int64_t n;
    int32_t K, G, D;
    const void* W[P3D_MAX_GROUPS];      // [D, K] bf16 each
    const void* bias[P3D_MAX_GROUPS];   // [D] bf16 or NULL
    void* out[P3D_MAX_GROUPS];          // [n, D] bf16
};

// Image-space token order (order.hip): a counting sort of the tokens by the
// texel block their top-left corner projects to on the key map.
struct OrderArgs {
    const int32_t* coords;
    int64_t n;
    int32_t R, points, batch;
};
struct OrderBufs {
    uint32_t* bins;               // [n] bin of every token
    uint32_t* hist;               // [nbins] tokens per bin
    uint32_t* cursor;             // [nbins] next sorted position of each bin
    int32_t kH, kW, shift;        // key map; texel -> block shift
    uint32_t per_item;            // bins per batch item
    int32_t nbins;
};
// Workspace layout of the sort for n tokens (pointers relative to `base`,
// which may be NULL to size it); returns the byte count, a multiple of 256.
size_t order_layout(int64_t n, int32_t batch, int32_t kH, int32_t kW, void* base,
                    OrderBufs* ob);
// order[i] = the token at sorted position i (a permutation of [0, n)).
hipError_t launch_order(const OrderArgs& a, const CamTable& cams, const OrderBufs& ob,
                        int32_t* order, hipStream_t s);

hipError_t launch_project(const ProjectArgs& a, const CamTable& cams, hipStream_t s);
hipError_t launch_stream_copy(const void* src, void* dst, int64_t vectors, hipStream_t s);
hipError_t launch_grouped(const GroupedArgs& a, bool accumulate, hipStream_t s);
hipError_t launch_stats(const StatsArgs& a, bool bf16, const CamTable& cams, hipStream_t s);
hipError_t launch_requantize(const RequantArgs& a, hipStream_t s);
hipError_t launch_sample(const SampleArgs& a, p3d_dtype in, p3d_dtype out, const CamTable& cams,
                         hipStream_t s);
hipError_t launch_proj_cond(const ProjCondArgs& a, p3d_dtype dt, const CamTable& cams,
                            hipStream_t s);
// bf16 fused kernel; writes the null rows too when a.n > 0
hipError_t launch_proj_cond_bf16(const ProjCondArgs& a, const CamTable& cams, hipStream_t s);
// how that kernel cuts n tokens x D features into tiles on `cus` CUs (the
// rule p3d_proj_cond_plan documents); host-only
p3d_tile_plan plan_proj_cond_bf16(int64_t n, int32_t D, int32_t cus);

}  // namespace p3d
