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
//      item, Morton index of the 16 x 16-texel block holding its top-left
//      corner texel); blocks are coarser when the bins would exceed 16384.
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

__global__ __launch_bounds__(kThreads) void clear_kernel(uint32_t* __restrict__ hist,
                                                         int32_t nbins) {
    const int i = blockIdx.x * kThreads + threadIdx.x;
    if (i < nbins) hist[i] = 0;
}

// Workgroup w bins tokens [kBinTokens w, kBinTokens (w + 1)).
__global__ __launch_bounds__(kThreads) void bin_kernel(OrderArgs a, CamTable cams,
                                                       OrderBufs ob) {
    __shared__ uint32_t cnt[kMaxBins];
    const int tid = threadIdx.x;
    for (int i = tid; i < ob.nbins; i += kThreads) cnt[i] = 0;
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
    for (int i = tid; i < ob.nbins; i += kThreads)
        if (cnt[i]) atomicAdd(&ob.hist[i], cnt[i]);
}

// Exclusive prefix sum of hist[0, nbins) into cursor, in one workgroup:
// thread i sums its run of nbins / kScanThreads counts, the run totals are
// scanned in LDS, then each thread writes its run's prefixes.
__global__ __launch_bounds__(kScanThreads) void scan_kernel(OrderBufs ob) {
    __shared__ uint32_t part[kScanThreads];
    const int tid = threadIdx.x;
    const int per = (ob.nbins + kScanThreads - 1) / kScanThreads;
    const int lo = tid * per, hi = min(lo + per, ob.nbins);
    uint32_t sum = 0;
    for (int i = lo; i < hi; ++i) sum += ob.hist[i];
    part[tid] = sum;
    __syncthreads();
    for (int d = 1; d < kScanThreads; d <<= 1) {     // inclusive Hillis-Steele scan
        const uint32_t v = tid >= d ? part[tid - d] : 0u;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    uint32_t run = part[tid] - sum;
    for (int i = lo; i < hi; ++i) {
        ob.cursor[i] = run;
        run += ob.hist[i];
    }
}

// The token ranges of bin_kernel: ranks inside the workgroup from LDS
// counters, one device atomic per bin reserves the workgroup's run of
// positions, then every token lands at run start + rank.
__global__ __launch_bounds__(kThreads) void scatter_kernel(int64_t n, OrderBufs ob,
                                                           int32_t* __restrict__ order) {
    __shared__ uint32_t cnt[kMaxBins];
    constexpr int PER = kBinTokens / kThreads;
    const int tid = threadIdx.x;
    for (int i = tid; i < ob.nbins; i += kThreads) cnt[i] = 0;
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
    for (int i = tid; i < ob.nbins; i += kThreads)
        if (cnt[i]) cnt[i] = atomicAdd(&ob.cursor[i], cnt[i]);
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
    // 16 x 16-texel blocks, coarser until batch * P^2 <= kMaxBins (P: blocks
    // per axis, rounded up to a power of 2 for the Morton index)
    const int32_t side = kH > kW ? kH : kW;
    for (o.shift = 4;; ++o.shift) {
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
