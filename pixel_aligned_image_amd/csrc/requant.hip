// requant.hip -- p3d_requantize_coords: cascade requantization of sparse
// coords onto the high-resolution token grid (trellis.cpp PR #38, cascade
// requantization commit).
//
// Per axis, u = (c + 1/2)/R_src. Pixal3D's rule takes the nearest node of
// the G-node projection grid, round(u (G - 1)); TRELLIS.2's takes the cell
// floor(u G). Both are ratios of integers, (2c + 1)(G - 1) / (2 R_src) and
// (2c + 1) G / (2 R_src), so they are evaluated exactly in 64-bit integers
// (round: to nearest, ties to even). One thread per token, one 16-byte load
// and one 16-byte store: bound by HBM, 32 bytes per token.
#include "p3d_internal.h"

namespace p3d {

namespace {

__device__ __forceinline__ int32_t requant_axis(int32_t c, int32_t src_res, int32_t grid,
                                                int32_t mode) {
    c = c < 0 ? 0 : (c > src_res - 1 ? src_res - 1 : c);
    const int64_t den = 2 * (int64_t)src_res;
    const int64_t odd = 2 * (int64_t)c + 1;
    if (mode == P3D_REQUANT_FLOOR_CELLS) return (int32_t)(odd * grid / den);
    const int64_t num = odd * (int64_t)(grid - 1);
    int64_t q = num / den;
    const int64_t twice_rem = 2 * (num - q * den);
    q += (twice_rem > den || (twice_rem == den && (q & 1))) ? 1 : 0;
    return (int32_t)q;
}

__global__ __launch_bounds__(256) void requant_kernel(RequantArgs a) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < a.n; t += stride) {
        const int4 c = reinterpret_cast<const int4*>(a.src)[t];
        int4 o;
        o.x = c.x;
        o.y = requant_axis(c.y, a.src_res, a.grid, a.mode);
        o.z = requant_axis(c.z, a.src_res, a.grid, a.mode);
        o.w = requant_axis(c.w, a.src_res, a.grid, a.mode);
        reinterpret_cast<int4*>(a.dst)[t] = o;
    }
}

}  // namespace

hipError_t launch_requantize(const RequantArgs& a, hipStream_t s) {
    int64_t blocks = (a.n + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    RequantArgs args = a;
    void* params[] = {&args};
    return hipLaunchKernel(reinterpret_cast<const void*>(&requant_kernel), dim3((unsigned)blocks),
                           dim3(256), params, 0, s);
}

}  // namespace p3d
