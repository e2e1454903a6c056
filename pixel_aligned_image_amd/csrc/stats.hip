// stats.hip -- p3d_projection_stats: projection diagnostics (trellis.cpp
// PR #38, commits adding the per-stage projection statistics and the
// cross-resolution agreement): coverage, per-map sums and sums of squares of
// the samples, and the per-token cosine between two maps' samples.
//
// An HBM-bound gather with a reduction instead of a store. Tokens go to the
// waves as quads of 4 consecutive tokens: each XCD owns a contiguous range,
// and its waves take its quads round-robin, so that at any time an XCD's
// waves sample one window of consecutive tokens, whose corner rows overlap,
// in the same L2. Lanes project 16 quads at a time; then each 16-lane row of
// the wave takes one token of a quad: the row's lanes walk that token's
// channels 16 vectors (of 16 bytes) apart, map 0 and map 1 at the same
// channel offset in the same lane, with the corner loads of several vectors
// issued before any is blended. The cosine's dot product and norms stay
// per-lane partial sums until one 16-lane reduction per token (four DPP
// steps, no LDS). Samples are blended and rounded exactly as the fused
// kernel feeds them to proj_linear. For bf16 maps a token's per-lane partial
// sums are binary32 (C / 16 products of bf16-rounded values each: 64 for 1024
// channels, 128 for 2048) and are carried in binary64 from there on; fp32
// maps accumulate in binary64 throughout. Sums are reduced over the workgroup in LDS and added to the
// result with one device atomic per figure per workgroup.
#include <type_traits>

#include "p3d_internal.h"

namespace p3d {

namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerCU = 8;     // target residency (at most 256 registers per lane)

// Corner metadata of token t on an H x W map (top-left row, 0/1 steps right
// and down, fractions); the same construction as the fused kernel's.
struct Meta {
    int32_t r00, steps;
    float tx, ty;
};

__device__ __forceinline__ Meta meta_of(const Projected& p, int32_t H, int32_t W) {
    const SrcIdx sx = source_index(p.gx, W);
    const SrcIdx sy = source_index(p.gy, H);
    Meta m;
    m.r00 = (p.b * H + sy.i0) * W + sx.i0;
    m.steps = (sx.i1 - sx.i0) | ((sy.i1 - sy.i0) << 1);
    m.tx = sx.t;
    m.ty = sy.t;
    return m;
}

// A token's four corner rows on one map (vector pointers) and bilinear
// weights.
struct Tok {
    const uint4* row[4];
    float w[4];
};

__device__ __forceinline__ Tok tok_of(const uint4* __restrict__ feat, int vpr, const Meta& m,
                                      int W) {
    const int32_t dx = m.steps & 1, dyw = (m.steps & 2) ? W : 0;
    Tok t;
    t.row[0] = feat + (int64_t)m.r00 * vpr;
    t.row[1] = feat + (int64_t)(m.r00 + dx) * vpr;
    t.row[2] = feat + (int64_t)(m.r00 + dyw) * vpr;
    t.row[3] = feat + (int64_t)(m.r00 + dyw + dx) * vpr;
    t.w[0] = (1.0f - m.tx) * (1.0f - m.ty);
    t.w[1] = m.tx * (1.0f - m.ty);
    t.w[2] = (1.0f - m.tx) * m.ty;
    t.w[3] = m.tx * m.ty;
    return t;
}

__device__ __forceinline__ void load_corners(const Tok& t, int v, uint4 (&q)[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) q[k] = t.row[k][v];
}

// The blended samples of one 16-byte vector of a bf16 map: 8 values rounded
// to bf16 (as proj_linear receives them), as 4 packed pairs.
__device__ __forceinline__ void blend_bf16(const uint4 (&q)[4], const Tok& t, uint32_t (&r)[4]) {
    const uint32_t* pa = reinterpret_cast<const uint32_t*>(&q[0]);
    const uint32_t* pb = reinterpret_cast<const uint32_t*>(&q[1]);
    const uint32_t* pc = reinterpret_cast<const uint32_t*>(&q[2]);
    const uint32_t* pd = reinterpret_cast<const uint32_t*>(&q[3]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float lo = fmaf(t.w[3], bf16lo(pd[e]), fmaf(t.w[2], bf16lo(pc[e]),
                              fmaf(t.w[1], bf16lo(pb[e]), t.w[0] * bf16lo(pa[e]))));
        const float hi = fmaf(t.w[3], bf16hi(pd[e]), fmaf(t.w[2], bf16hi(pc[e]),
                              fmaf(t.w[1], bf16hi(pb[e]), t.w[0] * bf16hi(pa[e]))));
        r[e] = pack_bf16x2(lo, hi);
    }
}

// The blended samples of one 16-byte vector of an fp32 map: 4 values.
__device__ __forceinline__ void blend_f32(const uint4 (&q)[4], const Tok& t, float (&o)[4]) {
    const uint32_t* pa = reinterpret_cast<const uint32_t*>(&q[0]);
    const uint32_t* pb = reinterpret_cast<const uint32_t*>(&q[1]);
    const uint32_t* pc = reinterpret_cast<const uint32_t*>(&q[2]);
    const uint32_t* pd = reinterpret_cast<const uint32_t*>(&q[3]);
#pragma unroll
    for (int e = 0; e < 4; ++e)
        o[e] = fmaf(t.w[3], __uint_as_float(pd[e]), fmaf(t.w[2], __uint_as_float(pc[e]),
                    fmaf(t.w[1], __uint_as_float(pb[e]), t.w[0] * __uint_as_float(pa[e]))));
}

// a.lo * b.lo + a.hi * b.hi + c for packed bf16 pairs (each product is exact
// in binary32; the sums round as binary32 additions do).
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}
constexpr uint32_t kOnePair = 0x3F803F80u;   // (1.0, 1.0) in bf16

// Per-lane partial sums of one token on one or two maps: the row's lanes
// take vectors rl, rl + 16, ...; U vectors (of each map) are loaded before
// any is blended, so that 4 U (one map) or 8 U (two maps) loads are in
// flight; the last vectors of a ragged row go one at a time. bf16 samples
// are summed as packed pairs (sum: dot with (1, 1); squares and the two-map
// dot product: dot of the pairs); a sample is non-zero when its magnitude
// bits are.
template <bool Bf16, bool Two, typename Acc>
struct Partial {
    Acc su = 0, sw = 0, d = 0, x = 0, y = 0;
    uint32_t or0 = 0, or1 = 0;         // bf16: OR of the packed samples
    bool nz0 = false, nz1 = false;     // fp32

    __device__ __forceinline__ void step(const uint4 (&qa)[4], const uint4 (&qb)[4],
                                         const Tok& ta, const Tok& tb) {
        if constexpr (Bf16) {
            uint32_t ru[4], rw[4];
            blend_bf16(qa, ta, ru);
            if constexpr (Two) blend_bf16(qb, tb, rw);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                su = dot2(ru[e], kOnePair, su);
                x = dot2(ru[e], ru[e], x);
                or0 |= ru[e];
                if constexpr (Two) {
                    sw = dot2(rw[e], kOnePair, sw);
                    y = dot2(rw[e], rw[e], y);
                    d = dot2(ru[e], rw[e], d);
                    or1 |= rw[e];
                }
            }
        } else {
            float u[4], w[4];
            blend_f32(qa, ta, u);
            if constexpr (Two) blend_f32(qb, tb, w);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const Acc uu = u[e];
                nz0 |= u[e] != 0.0f;
                su += uu;
                x = fma(uu, uu, x);
                if constexpr (Two) {
                    const Acc ww = w[e];
                    nz1 |= w[e] != 0.0f;
                    sw += ww;
                    d = fma(uu, ww, d);
                    y = fma(ww, ww, y);
                }
            }
        }
    }

    __device__ __forceinline__ bool nonzero0() const {
        return Bf16 ? (or0 & 0x7FFF7FFFu) != 0 : nz0;
    }
    __device__ __forceinline__ bool nonzero1() const {
        return Bf16 ? (or1 & 0x7FFF7FFFu) != 0 : nz1;
    }

    __device__ __forceinline__ void run(const Tok& ta, const Tok& tb, int rl, int vpr) {
        constexpr int U = Two ? 4 : 8;
        int v0 = rl;
#pragma unroll 1
        for (; v0 + 16 * (U - 1) < vpr; v0 += 16 * U) {
            uint4 qa[U][4], qb[Two ? U : 1][4];
#pragma unroll
            for (int j = 0; j < U; ++j) {
                load_corners(ta, v0 + 16 * j, qa[j]);
                if constexpr (Two) load_corners(tb, v0 + 16 * j, qb[j]);
            }
#pragma unroll
            for (int j = 0; j < U; ++j) step(qa[j], qb[Two ? j : 0], ta, tb);
        }
#pragma unroll 1
        for (; v0 < vpr; v0 += 16) {
            uint4 qa[4], qb[4];
            load_corners(ta, v0, qa);
            if constexpr (Two) load_corners(tb, v0, qb);
            step(qa, qb, ta, tb);
        }
    }
};

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// Lane value of a DPP permutation within each 16-lane row.
template <int Ctrl>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), Ctrl, 0xF, 0xF, false));
}
template <int Ctrl>
__device__ __forceinline__ double dpp_d(double x) {
    const int64_t v = __double_as_longlong(x);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)v, Ctrl, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(v >> 32), Ctrl, 0xF, 0xF, false);
    return __longlong_as_double(((int64_t)hi << 32) | (uint32_t)lo);
}

// Sum over each 16-lane row, in every lane of the row: partners at xor 1 and
// xor 2 (quad permutations), then the other quad of the half row (half
// mirror), then the other half (mirror). Every lane adds the same pairs, so
// all lanes of a row hold the same bits.
template <typename T>
__device__ __forceinline__ T row_sum(T x) {
    if constexpr (std::is_same<T, float>::value) {
        x += dpp_f<0xB1>(x);      // quad_perm [1, 0, 3, 2]
        x += dpp_f<0x4E>(x);      // quad_perm [2, 3, 0, 1]
        x += dpp_f<0x141>(x);     // row_half_mirror
        x += dpp_f<0x140>(x);     // row_mirror
    } else {
        x += dpp_d<0xB1>(x);
        x += dpp_d<0x4E>(x);
        x += dpp_d<0x141>(x);
        x += dpp_d<0x140>(x);
    }
    return x;
}

__global__ __launch_bounds__(64) void stats_zero_kernel(p3d_proj_stats* s) {
    if (threadIdx.x < sizeof(p3d_proj_stats) / sizeof(double))
        reinterpret_cast<double*>(s)[threadIdx.x] = 0.0;
}

__device__ __forceinline__ Meta shfl_meta(const Meta& m, int src) {
    Meta r;
    r.r00 = __shfl(m.r00, src);
    r.steps = __shfl(m.steps, src);
    r.tx = __shfl(m.tx, src);
    r.ty = __shfl(m.ty, src);
    return r;
}

// Workgroup g runs on XCD g % 8 as that XCD's (g / 8)-th. XCD x owns the
// tokens [x Wx per_wave, (x + 1) Wx per_wave), Wx = 4 per_xcd waves, as
// quads of 4 consecutive tokens; the XCD's wave j takes quads j, j + Wx,
// j + 2 Wx, ... (per_wave / 4 of them). The XCD's waves thus sweep one
// window of consecutive tokens together, and neighbouring tokens, which
// share corner rows, are sampled at about the same time in the same L2.
template <bool Bf16>
__global__ __launch_bounds__(kThreads, kWavesPerCU / (kThreads / 64)) void stats_kernel(StatsArgs a, CamTable cams,
                                                         int64_t per_wave, int64_t per_xcd) {
    constexpr int EPV = Bf16 ? 8 : 4;
    using Acc = typename std::conditional<Bf16, float, double>::type;
    const int lane = threadIdx.x & 63;
    const int row = lane >> 4, rl = lane & 15;
    const int64_t wx = (int64_t)(blockIdx.x >> 3) * (kThreads / 64) + (threadIdx.x >> 6);
    const int64_t Wx = per_xcd * (kThreads / 64);
    const int64_t xcd_t0 = (int64_t)(blockIdx.x & 7) * Wx * per_wave;
    const int64_t quads = per_wave / 4;
    const uint4* __restrict__ f0 = reinterpret_cast<const uint4*>(a.feat0);
    const uint4* __restrict__ f1 = reinterpret_cast<const uint4*>(a.feat1);
    const int vpr0 = a.C0 / EPV, vpr1 = a.C1 / EPV;
    const bool two = a.C1 > 0;
    const bool cosine = two && a.C0 == a.C1;

    double s0 = 0.0, q0 = 0.0, s1 = 0.0, q1 = 0.0;   // per lane
    double cos_sum = 0.0, cos_cnt = 0.0;             // per lane (row leaders add)
    double inside = 0.0, tokens = 0.0;               // wave-uniform

    for (int64_t k0 = 0; k0 < quads; k0 += 16) {
        // ---- lane l projects token l % 4 of this wave's quad k0 + l / 4
        const int64_t k = k0 + (lane >> 2);
        const int64_t t = xcd_t0 + 4 * (wx + k * Wx) + (lane & 3);
        const bool valid = k < quads && t < a.n;
        Meta m0{0, 0, 0.0f, 0.0f}, m1{0, 0, 0.0f, 0.0f};
        int in = 0;
        if (valid) {
            int32_t b, x, y, z;
            token_cell(a.coords, ordered_token(a.order, t, a.n), a.R, b, x, y, z);
            const Projected p = project_cell(b, x, y, z, a.R, a.points, cams, a.batch);
            m0 = meta_of(p, a.H0, a.W0);
            if (two) m1 = meta_of(p, a.H1, a.W1);
            in = p.mask;
        }
        const uint64_t vmask = __ballot(valid);
        if (vmask == 0) break;                       // past the tokens: so are later quads
        inside += (double)__builtin_popcountll(__ballot(in));
        tokens += (double)__builtin_popcountll(vmask);
        const int nq = quads - k0 < 16 ? (int)(quads - k0) : 16;
        // ---- row r takes token r of each quad
        for (int q = 0; q < nq; ++q) {
            const int src = 4 * q + row;
            const Meta a0 = shfl_meta(m0, src);
            const Meta a1 = shfl_meta(m1, src);
            const bool live = (vmask >> src) & 1;
            const Tok ta = tok_of(f0, vpr0, a0, a.W0);
            if (cosine) {
                // map 0 and map 1 at the same channels, in the same lanes
                const Tok tb = tok_of(f1, vpr1, a1, a.W1);
                Partial<Bf16, true, Acc> pt;
                if (live) pt.run(ta, tb, rl, vpr0);
                s0 += (double)pt.su;
                s1 += (double)pt.sw;
                q0 += (double)pt.x;
                q1 += (double)pt.y;
                const Acc dr = row_sum(pt.d), xr = row_sum(pt.x), yr = row_sum(pt.y);
                // both samples non-zero somewhere in the row: exact, whatever
                // the binary32 norms do
                const uint64_t b0 = __ballot(pt.nonzero0()), b1 = __ballot(pt.nonzero1());
                const bool both = ((b0 >> (16 * row)) & 0xFFFF) && ((b1 >> (16 * row)) & 0xFFFF);
                if (live && rl == 0 && both) {
                    cos_sum += (double)dr / (sqrt((double)xr) * sqrt((double)yr));
                    cos_cnt += 1.0;
                }
            } else if (live) {
                Partial<Bf16, false, Acc> p0;
                p0.run(ta, ta, rl, vpr0);
                s0 += (double)p0.su;
                q0 += (double)p0.x;
                if (two) {
                    const Tok tb = tok_of(f1, vpr1, a1, a.W1);
                    Partial<Bf16, false, Acc> p1;
                    p1.run(tb, tb, rl, vpr1);
                    s1 += (double)p1.su;
                    q1 += (double)p1.x;
                }
            }
        }
    }
    // ---- workgroup reduction, then one atomic per figure
    __shared__ double part[kThreads / 64][8];
    const double fig[8] = {tokens, inside, wave_sum(s0), wave_sum(s1), wave_sum(q0),
                           wave_sum(q1), wave_sum(cos_sum), wave_sum(cos_cnt)};
    if (lane == 0)
#pragma unroll
        for (int k = 0; k < 8; ++k) part[threadIdx.x >> 6][k] = fig[k];
    __syncthreads();
    if (threadIdx.x < 8) {
        double v = 0.0;
#pragma unroll
        for (int w = 0; w < kThreads / 64; ++w) v += part[w][threadIdx.x];
        // figures a launch does not produce stay exactly 0 (zeroed first)
        if (v != 0.0) unsafeAtomicAdd(reinterpret_cast<double*>(a.stats) + threadIdx.x, v);
    }
}

// Compute units of the current device.
int stats_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        return 256;
    return cus;
}

}  // namespace

hipError_t launch_stats(const StatsArgs& a, bool bf16, const CamTable& cams, hipStream_t s) {
    StatsArgs args = a;
    {
        p3d_proj_stats* st = a.stats;
        void* params[] = {&st};
        hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&stats_zero_kernel), dim3(1),
                                       dim3(64), params, 0, s);
        if (e != hipSuccess || a.n == 0) return e;
    }
    // an equal share of the tokens per wave, for a full residency of waves
    const int64_t max_waves = (int64_t)stats_cus() * kWavesPerCU;
    int64_t per_wave = (a.n + max_waves - 1) / max_waves;
    per_wave = (per_wave + 3) & ~(int64_t)3;
    const int64_t waves = (a.n + per_wave - 1) / per_wave;
    const int64_t blocks_needed = (waves + kThreads / 64 - 1) / (kThreads / 64);
    int64_t per_xcd = (blocks_needed + 7) / 8;
    const int64_t blocks = per_xcd * 8;             // the last XCD's tail runs empty
    CamTable tab = cams;
    void* params[] = {&args, &tab, &per_wave, &per_xcd};
    const void* fn = bf16 ? reinterpret_cast<const void*>(&stats_kernel<true>)
                          : reinterpret_cast<const void*>(&stats_kernel<false>);
    return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kThreads), params, 0, s);
}

}  // namespace p3d
