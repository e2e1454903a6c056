// order.hip -- image-space token order for the fused, sampling and
// diagnostics kernels (p3d_token_order, and the *_ws entry points that
// compute it in their workspace).
//
// Why: the kernels take tokens in runs (tiles of 128 in the fused kernel,
// windows of consecutive tokens in the sampler and the diagnostics). In the
// caller's order -- sparse voxels sorted by (x, y, z) -- a run's corner reads
// scatter over the image: on the 1024^3 shell workload a 128-token run
// touches about 420 distinct map rows for its 512 corner reads, and
// neighbouring runs share little. Grouped by the texel block they project to,
// a run touches about 210, and rows that neighbouring runs share are read
// while they are still in the L2 and the L1.
//
// A counting sort by block, all on the caller's stream:
//   1. clear_kernel: zero the block histogram;
//   2. bin_kernel: project every token (the same binary32 steps as every
//      other kernel: pixel-aligned head commit of pixal3d_mrp_mlx) onto the
//      key map -- the one with the most texels -- and give it the bin (batch
//      item, Morton index of the 4 x 4-texel block holding its top-left
//      corner texel); blocks are coarser when the bins would exceed 16384.
//      (On the 1024^3 shell workload, 4 x 4 blocks left the fused kernel
//      1.8 % faster than 16 x 16 ones, 8 x 8 1.4 %; 32 x 32 1.2 % slower: a
//      128-token tile covers about 13 x 13 texels, and inside a block the
//      order is arbitrary.)
//      Counts go to LDS first, then one device atomic per bin and workgroup;
//   3. scan_kernel: exclusive prefix sum of the counts;
//   4. scatter_kernel: every token takes the next position of its bin. The
//      order inside a bin follows the atomics and may change between runs.
//      No output depends on it: every output row and mask byte is computed
//      from its own token alone, and rows are written at the token's index.
#include "p3d_internal.h"

namespace p3d {

namespace {

constexpr int kThreads = 256;
constexpr int kBinTokens = 1024;         // tokens per bin / scatter workgroup
constexpr int kMaxBins = 1 << 14;        // LDS counters of one workgroup
constexpr int kScanThreads = 1024;

// Interleave the low 16 bits of v with zeros (bit i -> bit 2i).
__device__ __forceinline__ uint32_t spread_bits(uint32_t v) {
    v &= 0xffffu;
    v = (v | (v << 8)) & 0x00FF00FFu;
    v = (v | (v << 4)) & 0x0F0F0F0Fu;
    v = (v | (v << 2)) & 0x33333333u;
    v = (v | (v << 1)) & 0x55555555u;
    return v;
}

// Zero the first nbins LDS counters, rounded up to whole 16-byte vectors
// (kMaxBins, the array's size, is a multiple of 4).
__device__ __forceinline__ void zero_counts(uint32_t* cnt, int nbins, int tid) {
    uint4* c4 = reinterpret_cast<uint4*>(cnt);
    for (int i = tid; i < (nbins + 3) / 4; i += kThreads) c4[i] = make_uint4(0, 0, 0, 0);
}

// For every non-zero LDS counter c[i] (i < nbins): old = atomicAdd(&dst[i], c[i]);
// with Return, c[i] becomes old. Sixteen counters per thread and step (four
// runs of four), their atomics all issued before any result is used.
template <bool Return>
__device__ __forceinline__ void flush_counts(uint32_t* cnt, uint32_t* __restrict__ dst, int nbins,
                                             int tid) {
    constexpr int kPer = 16;                  // counters per thread and step
    for (int i0 = tid * 4; i0 < nbins; i0 += kThreads * kPer) {
        uint32_t c[kPer], r[kPer];
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int i = i0 + (k / 4) * kThreads * 4 + (k % 4);
            c[k] = i < nbins ? cnt[i] : 0u;
        }
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int i = i0 + (k / 4) * kThreads * 4 + (k % 4);
            r[k] = 0u;
            if (c[k]) {
                if constexpr (Return) r[k] = atomicAdd(&dst[i], c[k]);
                else atomicAdd(&dst[i], c[k]);
            }
        }
        if constexpr (Return) {
#pragma unroll
            for (int k = 0; k < kPer; ++k) {
                const int i = i0 + (k / 4) * kThreads * 4 + (k % 4);
                if (c[k]) cnt[i] = r[k];
            }
        }
    }
}

__global__ __launch_bounds__(kThreads) void clear_kernel(uint32_t* __restrict__ hist,
                                                         int32_t nbins) {
    const int i = blockIdx.x * kThreads + threadIdx.x;
    if (i < nbins) hist[i] = 0;
}

// Workgroup w bins tokens [kBinTokens w, kBinTokens (w + 1)).
__global__ __launch_bounds__(kThreads) void bin_kernel(OrderArgs a, CamTable cams,
                                                       OrderBufs ob) {
    __shared__ __align__(16) uint32_t cnt[kMaxBins];
    const int tid = threadIdx.x;
    zero_counts(cnt, ob.nbins, tid);
    __syncthreads();
    const int64_t t0 = (int64_t)blockIdx.x * kBinTokens;
    for (int i = tid; i < kBinTokens; i += kThreads) {
        const int64_t t = t0 + i;
        if (t >= a.n) break;
        int32_t b, x, y, z;
        token_cell(a.coords, t, a.R, b, x, y, z);
        const Projected p = project_cell(b, x, y, z, a.R, a.points, cams, a.batch);
        const SrcIdx sx = source_index(p.gx, ob.kW);
        const SrcIdx sy = source_index(p.gy, ob.kH);
        const uint32_t bin = (uint32_t)p.b * ob.per_item +
                             (spread_bits((uint32_t)sx.i0 >> ob.shift) |
                              (spread_bits((uint32_t)sy.i0 >> ob.shift) << 1));
        ob.bins[t] = bin;
        atomicAdd(&cnt[bin], 1u);
    }
    __syncthreads();
    flush_counts<false>(cnt, ob.hist, ob.nbins, tid);
}

// Exclusive prefix sum of hist[0, nbins) into cursor, in one workgroup. The
// counts are taken as rows of kScanThreads (row r: bins r kScanThreads ..):
// every thread loads its column of all rows first (coalesced, all loads in
// flight together: one workgroup alone is latency-bound), then each row is
// scanned across the workgroup (wave scans with shuffles, then the wave
// totals) and offset by the total of the rows before it.
__global__ __launch_bounds__(kScanThreads) void scan_kernel(OrderBufs ob) {
    constexpr int kRows = kMaxBins / kScanThreads;
    constexpr int kWaves = kScanThreads / 64;
    __shared__ uint32_t wsum[kRows][kWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t c[kRows], v[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        const int i = r * kScanThreads + tid;
        c[r] = i < ob.nbins ? ob.hist[i] : 0u;
    }
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        v[r] = c[r];
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {           // inclusive scan in the wave
            const uint32_t u = __shfl_up(v[r], d);
            if (lane >= d) v[r] += u;
        }
        if (lane == 63) wsum[r][wave] = v[r];
    }
    __syncthreads();
    // wave 0: exclusive scan of the kRows x kWaves totals in (row, wave)
    // order, four per lane, back into wsum
    static_assert(kRows * kWaves == 4 * 64, "four totals per lane");
    if (wave == 0) {
        uint32_t* flat = &wsum[0][0];
        uint32_t t[4], sum = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            t[k] = flat[4 * lane + k];
            sum += t[k];
        }
        uint32_t incl = sum;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const uint32_t u = __shfl_up(incl, d);
            if (lane >= d) incl += u;
        }
        uint32_t run = incl - sum;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            flat[4 * lane + k] = run;
            run += t[k];
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        const int i = r * kScanThreads + tid;
        if (i < ob.nbins) ob.cursor[i] = wsum[r][wave] + v[r] - c[r];
    }
}

// The token ranges of bin_kernel: ranks inside the workgroup from LDS
// counters, one device atomic per bin reserves the workgroup's run of
// positions, then every token lands at run start + rank.
__global__ __launch_bounds__(kThreads) void scatter_kernel(int64_t n, OrderBufs ob,
                                                           int32_t* __restrict__ order) {
    __shared__ __align__(16) uint32_t cnt[kMaxBins];
    constexpr int PER = kBinTokens / kThreads;
    const int tid = threadIdx.x;
    zero_counts(cnt, ob.nbins, tid);
    __syncthreads();
    const int64_t t0 = (int64_t)blockIdx.x * kBinTokens;
    uint32_t bin[PER], rank[PER];
#pragma unroll
    for (int r = 0; r < PER; ++r) {
        const int64_t t = t0 + tid + (int64_t)r * kThreads;
        bin[r] = t < n ? ob.bins[t] : 0u;
        rank[r] = t < n ? atomicAdd(&cnt[bin[r]], 1u) : 0u;
    }
    __syncthreads();
    flush_counts<true>(cnt, ob.cursor, ob.nbins, tid);
    __syncthreads();
#pragma unroll
    for (int r = 0; r < PER; ++r) {
        const int64_t t = t0 + tid + (int64_t)r * kThreads;
        if (t < n) order[cnt[bin[r]] + rank[r]] = (int32_t)t;
    }
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t order_layout(int64_t n, int32_t batch, int32_t kH, int32_t kW, void* base,
                    OrderBufs* ob) {
    OrderBufs o{};
    o.kH = kH;
    o.kW = kW;
    // 4 x 4-texel blocks, coarser until batch * P^2 <= kMaxBins (P: blocks
    // per axis, rounded up to a power of 2 for the Morton index)
    const int32_t side = kH > kW ? kH : kW;
    for (o.shift = 2;; ++o.shift) {
        int64_t P = 1;
        while (P * ((int64_t)1 << o.shift) < side) P <<= 1;
        if ((int64_t)batch * P * P <= kMaxBins || o.shift >= 30) {
            o.per_item = (uint32_t)(P * P);
            o.nbins = (int32_t)(batch * P * P);
            break;
        }
    }
    char* c = static_cast<char*>(base);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* q = c ? c + off : nullptr;
        off += align_up(bytes);
        return q;
    };
    o.bins = reinterpret_cast<uint32_t*>(take((size_t)n * 4));
    o.hist = reinterpret_cast<uint32_t*>(take((size_t)o.nbins * 4));
    o.cursor = reinterpret_cast<uint32_t*>(take((size_t)o.nbins * 4));
    if (ob) *ob = o;
    return off;
}

hipError_t launch_order(const OrderArgs& a, const CamTable& cams, const OrderBufs& ob,
                        int32_t* order, hipStream_t s) {
    OrderArgs args = a;
    CamTable tab = cams;
    OrderBufs o = ob;
    hipError_t e;
    {
        uint32_t* hist = o.hist;
        int32_t nbins = o.nbins;
        void* params[] = {&hist, &nbins};
        e = hipLaunchKernel(reinterpret_cast<const void*>(&clear_kernel),
                            dim3((unsigned)((nbins + kThreads - 1) / kThreads)), dim3(kThreads),
                            params, 0, s);
        if (e != hipSuccess) return e;
    }
    const unsigned blocks = (unsigned)((a.n + kBinTokens - 1) / kBinTokens);
    {
        void* params[] = {&args, &tab, &o};
        e = hipLaunchKernel(reinterpret_cast<const void*>(&bin_kernel), dim3(blocks),
                            dim3(kThreads), params, 0, s);
        if (e != hipSuccess) return e;
    }
    {
        void* params[] = {&o};
        e = hipLaunchKernel(reinterpret_cast<const void*>(&scan_kernel), dim3(1),
                            dim3(kScanThreads), params, 0, s);
        if (e != hipSuccess) return e;
    }
    {
        int64_t n = a.n;
        int32_t* ord = order;
        void* params[] = {&n, &o, &ord};
        e = hipLaunchKernel(reinterpret_cast<const void*>(&scatter_kernel), dim3(blocks),
                            dim3(kThreads), params, 0, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace p3d
