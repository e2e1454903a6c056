// stats.hip -- p3d_projection_stats: projection diagnostics (trellis.cpp
// PR #38, commits adding the per-stage projection statistics and the
// cross-resolution agreement): coverage, per-map sums and sums of squares of
// the samples, and the per-token cosine between two maps' samples.
//
// An HBM-bound gather with a reduction instead of a store. A wave takes TPW
// tokens at a time: lanes 0..TPW-1 project one each, then the wave walks the
// TPW tokens, broadcasting each token's corner metadata from its lane
// (readlane) and gathering its corner rows with the lanes spread over the
// channels (16-byte vectors, 64 lanes = 1 KB of a row per instruction), two
// tokens at a time so that both tokens' loads are in flight together. Map 0
// and map 1 vectors at the same channel offset sit in the same lane, so the
// cosine's dot product and norms need no shuffles until the per-token wave
// reduction. Samples are blended and rounded exactly as the fused kernel
// feeds them to proj_linear; sums are binary64, reduced over the workgroup
// in LDS and added to the result with one device atomic per figure per
// workgroup (atomics on eight addresses serialise, so their count is kept to
// a few thousand).
#include "p3d_internal.h"

namespace p3d {

namespace {

constexpr int kThreads = 256;
// Tokens per wave and step. Each token keeps a whole wave's loads in flight
// (16 per lane for two 1024-channel bf16 maps), so concurrency comes from the
// number of waves: 16 tokens per wave gives 100k tokens ~6000 waves.
constexpr int TPW = 16;
constexpr int kMaxBlocks = 1024;   // 16 waves per CU; atomics: 8 per block

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

// The token's meta broadcast from lane j (uniform values).
__device__ __forceinline__ Meta lane_meta(const Meta& m, int j) {
    Meta r;
    r.r00 = __builtin_amdgcn_readlane(m.r00, j);
    r.steps = __builtin_amdgcn_readlane(m.steps, j);
    r.tx = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m.tx), j));
    r.ty = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m.ty), j));
    return r;
}

// Vector v of the blended sample of one token: 8 bf16 values (rounded to
// bf16, as proj_linear receives them) or 4 binary32 values.
template <bool Bf16>
__device__ __forceinline__ void sample_vec(const uint4* __restrict__ feat, int vpr,
                                           const Meta& m, int W, int v, float* out) {
    const int32_t dx = m.steps & 1, dyw = (m.steps & 2) ? W : 0;
    const uint4 a = feat[(int64_t)m.r00 * vpr + v];
    const uint4 b = feat[(int64_t)(m.r00 + dx) * vpr + v];
    const uint4 c = feat[(int64_t)(m.r00 + dyw) * vpr + v];
    const uint4 d = feat[(int64_t)(m.r00 + dyw + dx) * vpr + v];
    const float w0 = (1.0f - m.tx) * (1.0f - m.ty), w1 = m.tx * (1.0f - m.ty);
    const float w2 = (1.0f - m.tx) * m.ty, w3 = m.tx * m.ty;
    const uint32_t* pa = reinterpret_cast<const uint32_t*>(&a);
    const uint32_t* pb = reinterpret_cast<const uint32_t*>(&b);
    const uint32_t* pc = reinterpret_cast<const uint32_t*>(&c);
    const uint32_t* pd = reinterpret_cast<const uint32_t*>(&d);
    if constexpr (Bf16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float lo = fmaf(w3, bf16lo(pd[e]), fmaf(w2, bf16lo(pc[e]),
                                  fmaf(w1, bf16lo(pb[e]), w0 * bf16lo(pa[e]))));
            const float hi = fmaf(w3, bf16hi(pd[e]), fmaf(w2, bf16hi(pc[e]),
                                  fmaf(w1, bf16hi(pb[e]), w0 * bf16hi(pa[e]))));
            const uint32_t q = pack_bf16x2(lo, hi);
            out[2 * e] = bf16lo(q);
            out[2 * e + 1] = bf16hi(q);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            out[e] = fmaf(w3, __uint_as_float(pd[e]), fmaf(w2, __uint_as_float(pc[e]),
                          fmaf(w1, __uint_as_float(pb[e]), w0 * __uint_as_float(pa[e]))));
    }
}

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

__global__ __launch_bounds__(64) void stats_zero_kernel(p3d_proj_stats* s) {
    if (threadIdx.x < sizeof(p3d_proj_stats) / sizeof(double))
        reinterpret_cast<double*>(s)[threadIdx.x] = 0.0;
}

template <bool Bf16>
__global__ __launch_bounds__(kThreads) void stats_kernel(StatsArgs a, CamTable cams) {
    constexpr int EPV = Bf16 ? 8 : 4;
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
    const int64_t waves = ((int64_t)gridDim.x * kThreads) >> 6;
    const uint4* __restrict__ f0 = reinterpret_cast<const uint4*>(a.feat0);
    const uint4* __restrict__ f1 = reinterpret_cast<const uint4*>(a.feat1);
    const int vpr0 = a.C0 / EPV, vpr1 = a.C1 / EPV;
    const bool two = a.C1 > 0;
    const bool cosine = two && a.C0 == a.C1;

    double s0 = 0.0, q0 = 0.0, s1 = 0.0, q1 = 0.0;   // per lane
    double cos_sum = 0.0, cos_cnt = 0.0, inside = 0.0, tokens = 0.0;   // wave-uniform

    for (int64_t base = wave * TPW; base < a.n; base += waves * TPW) {
        // ---- lane j < TPW projects token base + j
        const int64_t t = base + lane;
        Meta m0{0, 0, 0.0f, 0.0f}, m1{0, 0, 0.0f, 0.0f};
        int in = 0;
        if (lane < TPW && t < a.n) {
            int32_t b, x, y, z;
            token_cell(a.coords, t, a.R, b, x, y, z);
            const Projected p = project_cell(b, x, y, z, a.R, a.points, cams, a.batch);
            m0 = meta_of(p, a.H0, a.W0);
            if (two) m1 = meta_of(p, a.H1, a.W1);
            in = p.mask;
        }
        const int64_t cnt = a.n - base < TPW ? a.n - base : TPW;
        inside += (double)__builtin_popcountll(__ballot(in));
        tokens += (double)cnt;
        // ---- the wave walks its tokens two at a time: both tokens' corner
        // loads are in flight together and their reductions interleave
        int j = 0;
        for (; j + 1 < (int)cnt; j += 2) {
            const Meta a0 = lane_meta(m0, j), b0 = lane_meta(m0, j + 1);
            const Meta a1 = lane_meta(m1, j), b1 = lane_meta(m1, j + 1);
            double dA = 0.0, xA = 0.0, yA = 0.0, dB = 0.0, xB = 0.0, yB = 0.0;
            for (int v = lane; v < vpr0; v += 64) {
                float pa[EPV], pb[EPV];
                sample_vec<Bf16>(f0, vpr0, a0, a.W0, v, pa);
                sample_vec<Bf16>(f0, vpr0, b0, a.W0, v, pb);
                if (cosine) {
                    float qa[EPV], qb[EPV];
                    sample_vec<Bf16>(f1, vpr1, a1, a.W1, v, qa);
                    sample_vec<Bf16>(f1, vpr1, b1, a.W1, v, qb);
#pragma unroll
                    for (int e = 0; e < EPV; ++e) {
                        const double u = pa[e], w = qa[e], u2 = pb[e], w2 = qb[e];
                        s0 += u + u2;
                        s1 += w + w2;
                        dA = fma(u, w, dA);
                        xA = fma(u, u, xA);
                        yA = fma(w, w, yA);
                        dB = fma(u2, w2, dB);
                        xB = fma(u2, u2, xB);
                        yB = fma(w2, w2, yB);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < EPV; ++e) {
                        const double u = pa[e], u2 = pb[e];
                        s0 += u + u2;
                        q0 = fma(u, u, fma(u2, u2, q0));
                    }
                }
            }
            if (cosine) {
                q0 += xA + xB;
                q1 += yA + yB;
                dA = wave_sum(dA);
                dB = wave_sum(dB);
                xA = wave_sum(xA);
                xB = wave_sum(xB);
                yA = wave_sum(yA);
                yB = wave_sum(yB);
                if (xA > 0.0 && yA > 0.0) {
                    cos_sum += dA / (sqrt(xA) * sqrt(yA));
                    cos_cnt += 1.0;
                }
                if (xB > 0.0 && yB > 0.0) {
                    cos_sum += dB / (sqrt(xB) * sqrt(yB));
                    cos_cnt += 1.0;
                }
            } else if (two) {
                for (int v = lane; v < vpr1; v += 64) {
                    float qa[EPV], qb[EPV];
                    sample_vec<Bf16>(f1, vpr1, a1, a.W1, v, qa);
                    sample_vec<Bf16>(f1, vpr1, b1, a.W1, v, qb);
#pragma unroll
                    for (int e = 0; e < EPV; ++e) {
                        const double w = qa[e], w2 = qb[e];
                        s1 += w + w2;
                        q1 = fma(w, w, fma(w2, w2, q1));
                    }
                }
            }
        }
        // ---- an odd last token alone
        if (j < (int)cnt) {
            const Meta t0 = lane_meta(m0, j);
            double dot = 0.0, n0 = 0.0, n1 = 0.0;
            for (int v = lane; v < vpr0; v += 64) {
                float x0[EPV];
                sample_vec<Bf16>(f0, vpr0, t0, a.W0, v, x0);
                if (cosine) {
                    const Meta t1 = lane_meta(m1, j);
                    float x1[EPV];
                    sample_vec<Bf16>(f1, vpr1, t1, a.W1, v, x1);
#pragma unroll
                    for (int e = 0; e < EPV; ++e) {
                        const double u = x0[e], w = x1[e];
                        s0 += u;
                        s1 += w;
                        dot = fma(u, w, dot);
                        n0 = fma(u, u, n0);
                        n1 = fma(w, w, n1);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < EPV; ++e) {
                        const double u = x0[e];
                        s0 += u;
                        q0 = fma(u, u, q0);
                    }
                }
            }
            if (cosine) {
                q0 += n0;
                q1 += n1;
                dot = wave_sum(dot);
                n0 = wave_sum(n0);
                n1 = wave_sum(n1);
                if (n0 > 0.0 && n1 > 0.0) {
                    cos_sum += dot / (sqrt(n0) * sqrt(n1));
                    cos_cnt += 1.0;
                }
            } else if (two) {
                const Meta t1 = lane_meta(m1, j);
                for (int v = lane; v < vpr1; v += 64) {
                    float x1[EPV];
                    sample_vec<Bf16>(f1, vpr1, t1, a.W1, v, x1);
#pragma unroll
                    for (int e = 0; e < EPV; ++e) {
                        const double w = x1[e];
                        s1 += w;
                        q1 = fma(w, w, q1);
                    }
                }
            }
        }
    }
    // ---- workgroup reduction, then one atomic per figure
    __shared__ double part[kThreads / 64][8];
    const double fig[8] = {tokens, inside, wave_sum(s0), wave_sum(s1), wave_sum(q0),
                           wave_sum(q1), cos_sum, cos_cnt};
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
    // one step of TPW tokens per wave where the grid allows; larger inputs
    // loop (grid-stride)
    const int64_t per_block = (int64_t)TPW * (kThreads / 64);
    const int64_t blocks_needed = (a.n + per_block - 1) / per_block;
    int64_t blocks = blocks_needed < kMaxBlocks ? blocks_needed : kMaxBlocks;
    CamTable tab = cams;
    void* params[] = {&args, &tab};
    const void* fn = bf16 ? reinterpret_cast<const void*>(&stats_kernel<true>)
                          : reinterpret_cast<const void*>(&stats_kernel<false>);
    return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kThreads), params, 0, s);
}

}  // namespace p3d
