// sample.hip -- p3d_bilinear_sample: grid_sample(bilinear,
// align_corners=False, padding_mode='border') on a channels-last map
// (pixel-aligned head commit, pixal3d_mrp_mlx: bilinear_sample).
//
// HBM-bound gather. A workgroup owns a run of TOK consecutive points; their
// four corner rows are read as 16-byte vectors spread across the lanes
// (eight consecutive lanes cover 128 contiguous bytes of one corner row, so
// every wave request is made of whole 128-byte segments), blended in
// binary32 and written with non-temporal 16-byte stores. Consecutive point
// runs share most corner rows; tiles are mapped so that each XCD walks a
// contiguous range of runs and those shared rows hit its own L2.
// Rows are read in channel slices of 1 KB (64 vectors), the slice being the
// slowest tile index: an XCD has thousands of points in flight, and with
// whole rows (4 KB at 2048 bf16 channels) their footprint is far larger
// than its 4 MB L2, so rows shared by neighbouring points were fetched
// again; a slice pass has a quarter of that footprint (11 % faster on the
// 1024^3 shell workload, same bytes requested).
//
// The same kernel serves p3d_proj_sample (project mode): the points come from
// projecting the tokens, and each map's samples go to their columns of a
// wider S row. Two maps share one launch: the slice index runs over map 0's
// slices, then map 1's, so the launch covers whole S rows and the XCDs work
// on both maps at once (a small map's slices are read from the L2 while a
// large map's come from HBM; on the texture stage's 64 x 64 + 512 x 512
// maps about 4 % faster than a launch per map, and 20 % faster than giving
// each XCD one slice as the one-map mapping does).
#include "p3d_internal.h"

namespace p3d {

namespace {

constexpr int kThreads = 256;
constexpr int kTok = 16;        // points per workgroup
// 16-byte items in flight per thread per step: 4 for the standalone gather,
// 3 for the projected gather (swept on the 1024^3 shell gather and the
// texture stage's two maps: 2 / 3 / 4 / 8 items gave 0.206 / 0.204 / 0.202 /
// 0.248 ms and 0.165 / 0.165 / 0.169 / 0.210 ms)
template <bool Project>
constexpr int unroll_items() { return Project ? 3 : 4; }
constexpr int kSlice = 64;      // 16-byte vectors per channel slice (1 KB)

// One 16-byte input vector -> values (8 for bf16, 4 for f32).
__device__ __forceinline__ void widen(const uint4& q, float* v, bool bf16) {
    if (bf16) {
        v[0] = bf16lo(q.x); v[1] = bf16hi(q.x);
        v[2] = bf16lo(q.y); v[3] = bf16hi(q.y);
        v[4] = bf16lo(q.z); v[5] = bf16hi(q.z);
        v[6] = bf16lo(q.w); v[7] = bf16hi(q.w);
    } else {
        v[0] = __uint_as_float(q.x); v[1] = __uint_as_float(q.y);
        v[2] = __uint_as_float(q.z); v[3] = __uint_as_float(q.w);
    }
}

template <bool InBf16, bool OutBf16, bool Project>
__global__ __launch_bounds__(kThreads) void sample_kernel(SampleArgs a, CamTable cams,
                                                          int64_t tiles, int64_t per_xcd) {
    // XCD-aware order: workgroup g runs on XCD g % 8 as that XCD's (g / 8)-th.
    //  - one map: XCD x owns the contiguous range [x per_xcd, (x + 1) per_xcd)
    //    of the (slice, tile) pairs, slice slowest, so that each XCD sweeps a
    //    run of neighbouring points in one slice and their shared rows hit
    //    its L2;
    //  - two maps: the slices differ in cost (a small map is read from the
    //    L2, a large one from HBM), so XCD x instead owns the tile range
    //    [x per_xcd, (x + 1) per_xcd) and walks it once per slice, starting
    //    at slice x (mod the slice count): every XCD covers every slice of
    //    both maps, and at any time the XCDs read and write different slices.
    const int64_t g = blockIdx.x;
    const int64_t j = g >> 3;
    const int xcd = (int)(g & 7);
    constexpr int SLICE = kSlice;
    constexpr int kEpv = InBf16 ? 8 : 4;          // elements per 16-byte vector
    const int n_slices0 = (a.C / kEpv + SLICE - 1) / SLICE;
    const int n_slices = n_slices0 + (a.C1 / kEpv + SLICE - 1) / SLICE;
    int slice_all;
    int64_t tile;
    if (a.C1 == 0) {
        const int64_t tile_all = xcd * per_xcd + j;
        if (tile_all >= tiles * n_slices) return;
        slice_all = (int)(tile_all / tiles);
        tile = tile_all - (int64_t)slice_all * tiles;
    } else {
        const int pass = (int)(j / per_xcd);
        if (pass >= n_slices) return;
        slice_all = (pass + xcd) % n_slices;
        tile = xcd * per_xcd + (j - (int64_t)pass * per_xcd);
        if (tile >= tiles) return;
    }
    // the map this slice belongs to
    const bool second = slice_all >= n_slices0;
    const int slice = second ? slice_all - n_slices0 : slice_all;
    const void* const map = second ? a.feat1 : a.feat;
    const int32_t H = second ? a.H1 : a.H, W = second ? a.W1 : a.W;
    const int32_t C = second ? a.C1 : a.C;
    const int64_t col = (int64_t)a.out_col + (second ? a.C : 0);

    __shared__ int32_t s_row[kTok][4];
    __shared__ float s_w[kTok][4];
    __shared__ int64_t s_out[kTok];        // output row of each point

    const int64_t t0 = tile * kTok;
    const int ntok = (int)((a.n - t0) < kTok ? (a.n - t0) : kTok);
    if (threadIdx.x < ntok) {
        const int64_t t = t0 + threadIdx.x;
        float2 gp;
        int32_t b;
        if constexpr (Project) {
            const int64_t tk = ordered_token(a.order, t, a.n);
            s_out[threadIdx.x] = tk;
            int32_t x, y, z;
            token_cell(a.coords, tk, a.R, b, x, y, z);
            const Projected p = project_cell(b, x, y, z, a.R, a.points, cams, a.batch);
            gp = make_float2(p.gx, p.gy);
            b = p.b;
            if (a.mask && slice_all == 0) a.mask[tk] = p.mask;
        } else {
            const int64_t tk = ordered_token(a.order, t, a.n);
            s_out[threadIdx.x] = tk;
            gp = reinterpret_cast<const float2*>(a.grid)[tk];
            b = a.bidx ? a.bidx[tk] : 0;
            b = b < 0 ? 0 : (b >= a.batch ? a.batch - 1 : b);
        }
        const Corners c = corners_of(gp.x, gp.y, b, H, W);
        s_row[threadIdx.x][0] = c.r00; s_row[threadIdx.x][1] = c.r01;
        s_row[threadIdx.x][2] = c.r10; s_row[threadIdx.x][3] = c.r11;
        s_w[threadIdx.x][0] = c.w00; s_w[threadIdx.x][1] = c.w01;
        s_w[threadIdx.x][2] = c.w10; s_w[threadIdx.x][3] = c.w11;
    }
    __syncthreads();

    const int vpr = C / kEpv;                      // vectors per map row
    const int v0 = slice * SLICE;
    const int svpr = (vpr - v0) < SLICE ? (vpr - v0) : SLICE;
    const int items = ntok * svpr;
    const uint4* __restrict__ feat = reinterpret_cast<const uint4*>(map);

    constexpr int kUnroll = unroll_items<Project>();
    for (int base = threadIdx.x; base < items; base += kThreads * kUnroll) {
        uint4 q[kUnroll][4];
        int tok[kUnroll], vec[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int i = base + u * kThreads;
            tok[u] = i < items ? i / svpr : 0;
            vec[u] = i < items ? v0 + (i - tok[u] * svpr) : 0;
            if (i < items) {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    q[u][k] = feat[(int64_t)s_row[tok[u]][k] * vpr + vec[u]];
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int i = base + u * kThreads;
            if (i >= items) break;
            const float w0 = s_w[tok[u]][0], w1 = s_w[tok[u]][1];
            const float w2 = s_w[tok[u]][2], w3 = s_w[tok[u]][3];
            float f0[8], f1[8], f2[8], f3[8], r[8];
            widen(q[u][0], f0, InBf16);
            widen(q[u][1], f1, InBf16);
            widen(q[u][2], f2, InBf16);
            widen(q[u][3], f3, InBf16);
#pragma unroll
            for (int e = 0; e < kEpv; ++e)
                r[e] = fmaf(w3, f3[e], fmaf(w2, f2[e], fmaf(w1, f1[e], w0 * f0[e])));
            const int64_t t = s_out[tok[u]];
            if (OutBf16) {
                uint4 o;
                o.x = pack_bf16x2(r[0], r[1]);
                o.y = pack_bf16x2(r[2], r[3]);
                o.z = pack_bf16x2(r[4], r[5]);
                o.w = pack_bf16x2(r[6], r[7]);
                uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.out) +
                                                      t * a.out_stride + col) + vec[u];
                store_nt16(dst, o);
            } else {
                float4* dst = reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) +
                                                        t * a.out_stride + col +
                                                        (int64_t)vec[u] * kEpv);
                store_nt16(dst, make_uint4(__float_as_uint(r[0]), __float_as_uint(r[1]),
                                           __float_as_uint(r[2]), __float_as_uint(r[3])));
                if (kEpv == 8)
                    store_nt16(dst + 1, make_uint4(__float_as_uint(r[4]), __float_as_uint(r[5]),
                                                   __float_as_uint(r[6]), __float_as_uint(r[7])));
            }
        }
    }
}

}  // namespace

hipError_t launch_sample(const SampleArgs& a, p3d_dtype in, p3d_dtype out, const CamTable& cams,
                         hipStream_t s) {
    const int64_t tiles = (a.n + kTok - 1) / kTok;
    const int64_t epv = in == P3D_BF16 ? 8 : 4;
    const int64_t n_slices = (a.C / epv + kSlice - 1) / kSlice + (a.C1 / epv + kSlice - 1) / kSlice;
    // one map: (slice, tile) pairs per XCD; two maps: tiles per XCD, once per
    // slice (the kernel's mapping comment)
    const int64_t per_xcd = a.C1 == 0 ? (tiles * n_slices + 7) / 8 : (tiles + 7) / 8;
    const int64_t blocks = a.C1 == 0 ? per_xcd * 8 : per_xcd * 8 * n_slices;
    SampleArgs args = a;
    CamTable tab = cams;
    int64_t t = tiles, p = per_xcd;
    void* params[] = {&args, &tab, &t, &p};
    const void* fn;
    if (a.project)
        fn = in == P3D_BF16 ? reinterpret_cast<const void*>(&sample_kernel<true, true, true>)
                            : reinterpret_cast<const void*>(&sample_kernel<false, false, true>);
    else if (in == P3D_BF16 && out == P3D_BF16)
        fn = reinterpret_cast<const void*>(&sample_kernel<true, true, false>);
    else if (in == P3D_BF16)
        fn = reinterpret_cast<const void*>(&sample_kernel<true, false, false>);
    else
        fn = reinterpret_cast<const void*>(&sample_kernel<false, false, false>);
    return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kThreads), params, 0, s);
}

}  // namespace p3d
