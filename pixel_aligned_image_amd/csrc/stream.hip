// stream.hip -- p3d_stream_copy: a device-to-device streaming copy, the
// achievable HBM rate that the measurements set beside the datasheet figure.
// Not a step of the method.
//
// 16-byte non-temporal loads and stores, four per thread in flight, in a
// grid-stride loop over 16384 workgroups (the configuration that measured
// fastest among 1024 .. 16384 workgroups, two or four 16-byte vectors in
// flight and ordinary or non-temporal accesses: 5.5-5.8 TB/s on 2 GiB,
// against 4.9 TB/s for the runtime's own device-to-device copy).
#include "p3d_internal.h"

namespace p3d {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr long kMaxBlocks = 16384;

__global__ __launch_bounds__(kThreads) void stream_copy_kernel(const u32x4_t* __restrict__ src,
                                                               u32x4_t* __restrict__ dst,
                                                               int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * kThreads * kUnroll;
    for (int64_t i = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; i < n; i += stride) {
        u32x4_t v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t j = i + (int64_t)u * kThreads;
            v[u] = j < n ? __builtin_nontemporal_load(src + j) : u32x4_t{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t j = i + (int64_t)u * kThreads;
            if (j < n) __builtin_nontemporal_store(v[u], dst + j);
        }
    }
}

}  // namespace

hipError_t launch_stream_copy(const void* src, void* dst, int64_t vectors, hipStream_t s) {
    const int64_t per_block = (int64_t)kThreads * kUnroll;
    int64_t blocks = (vectors + per_block - 1) / per_block;
    if (blocks > kMaxBlocks) blocks = kMaxBlocks;
    const u32x4_t* a = static_cast<const u32x4_t*>(src);
    u32x4_t* b = static_cast<u32x4_t*>(dst);
    int64_t n = vectors;
    void* params[] = {&a, &b, &n};
    return hipLaunchKernel(reinterpret_cast<const void*>(&stream_copy_kernel), dim3((unsigned)blocks),
                           dim3(kThreads), params, 0, s);
}

}  // namespace p3d
