// project.hip -- p3d_project_points: one thread per token.
//
// project_points of the pixel-aligned head commit (pixal3d_mrp_mlx): cell
// centre -> frontal pinhole on +Z looking down -Z -> normalised image
// coordinates, depth and in-image mask, plus the border-clamped
// align_corners=False source index (corner pixel and fraction) that the
// sampler uses. Pure ALU work on 16 bytes of input per token; bound by the
// output writes (up to 33 bytes per token).
#include "p3d_internal.h"

namespace p3d {

__global__ __launch_bounds__(256) void project_kernel(ProjectArgs a, CamTable cams) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < a.n; t += stride) {
        int32_t b, x, y, z;
        token_cell(a.coords, t, a.R, b, x, y, z);
        const Projected p = project_cell(b, x, y, z, a.R, a.points, cams, a.batch);
        if (a.grid) reinterpret_cast<float2*>(a.grid)[t] = make_float2(p.gx, p.gy);
        if (a.depth) a.depth[t] = p.depth;
        if (a.mask) a.mask[t] = p.mask;
        if (a.pixel || a.frac) {
            const SrcIdx sx = source_index(p.gx, a.W);
            const SrcIdx sy = source_index(p.gy, a.H);
            if (a.pixel) reinterpret_cast<int2*>(a.pixel)[t] = make_int2(sx.i0, sy.i0);
            if (a.frac) reinterpret_cast<float2*>(a.frac)[t] = make_float2(sx.t, sy.t);
        }
    }
}

hipError_t launch_project(const ProjectArgs& a, const CamTable& cams, hipStream_t s) {
    const int threads = 256;
    int64_t blocks = (a.n + threads - 1) / threads;
    if (blocks > 65536) blocks = 65536;
    ProjectArgs args = a;
    CamTable tab = cams;
    void* params[] = {&args, &tab};
    return hipLaunchKernel(reinterpret_cast<const void*>(&project_kernel), dim3((unsigned)blocks),
                           dim3(threads), params, 0, s);
}

}  // namespace p3d
