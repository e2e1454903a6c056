// proj_cond.hip -- p3d_proj_cond for binary32 maps (projection -> bilinear
// gather -> proj_linear on the matrix cores, fused), the CFG null-branch
// fill, and the dispatch between this path and the bf16 kernel.
//
// Sources: pixal3d_mrp_mlx tests/ history, pixel-aligned head commit
// (project_points, bilinear_sample); trellis.cpp PR #38 "Initial support for
// Pixal3D", FlowCond commit (proj_linear maps the per-token view-aligned
// feature into model space; the null proj is zeroed on the device, so the
// null rows are proj_linear(0) = bias).
//
// GEMM view: Y[M=n, N=D] = S[M, K=C] * W[N, K]^T + bias, where the A operand
// S is never stored: each workgroup projects its BM tokens, then for every
// K chunk gathers the four corner rows of each token (16-byte vectors,
// eight lanes per 128-byte corner segment), blends them in binary32 and
// writes the chunk into LDS next to the matching chunk of W; the matrix
// cores (v_mfma_f32_16x16x4_f32) accumulate in binary32. Eight waves, two
// per SIMD, each own a 64 x 32 block of the 128 x 128 tile, so that one
// wave's blend and barrier wait run under the other's MFMAs; the chunks
// alternate between two LDS stages (one barrier per chunk), and the next
// chunk's global loads are issued before the current chunk's MFMAs. Tiles are
// mapped so that the D-tiles of one token tile run on the same XCD and share
// its gathered corner rows in that XCD's L2. With a second map (NAF commit:
// the DINOv3 map and its upsampled version, concatenated along K) the tokens
// are projected once and the corners of both maps are kept in LDS; the K
// chunks past map 0's channels read map 1.
#include "p3d_internal.h"

namespace p3d {

namespace {

constexpr int WAVES_M = 2, WAVES_N = 4;         // 8 waves, two per SIMD
constexpr int kThreads = 64 * WAVES_M * WAVES_N;
constexpr int BM = 128, BN = 128, BK = 32;       // K chunk: 32 floats = 128 bytes
constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;   // wave tile
constexpr int MI = WM / 16, NJ = WN / 16;        // 16x16 blocks per wave
constexpr int A_ITEMS = BM * 8 / kThreads;       // gathered vectors per thread
constexpr int B_ITEMS = BN * 8 / kThreads;       // weight vectors per thread

// Tile rows in LDS are BK elements = 128 bytes = 8 vectors of 16 bytes; the
// vector index is XOR-swizzled with the row so that 16 lanes reading one
// column of vectors from 16 consecutive rows spread over the banks.
__device__ __forceinline__ int swz(int row, int v) { return row * 8 + (v ^ (row & 7)); }

// Bilinear blend of four 4-float vectors, binary32, corner order 00, 01, 10, 11.
__device__ __forceinline__ uint4 blend4(const uint4 (&q)[4], float w0, float w1, float w2,
                                        float w3) {
    const float* a = reinterpret_cast<const float*>(&q[0]);
    const float* b = reinterpret_cast<const float*>(&q[1]);
    const float* c = reinterpret_cast<const float*>(&q[2]);
    const float* d = reinterpret_cast<const float*>(&q[3]);
    uint4 o;
    float* r = reinterpret_cast<float*>(&o);
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = fmaf(w3, d[e], fmaf(w2, c[e], fmaf(w1, b[e], w0 * a[e])));
    return o;
}

__global__ __launch_bounds__(kThreads) void proj_cond_kernel(ProjCondArgs a, CamTable cams,
                                                             int32_t m_tiles, int32_t n_tiles,
                                                             int32_t per_xcd) {
    __shared__ int32_t s_row[2][BM][4];    // corner rows per map
    __shared__ float s_w[2][BM][4];
    __shared__ uint4 s_a[2][BM * 8];      // two stages: chunk kc uses stage kc % 2
    __shared__ uint4 s_b[2][BN * 8];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave % WAVES_M, wn = wave / WAVES_M;

    const int32_t g = blockIdx.x;
    const int32_t tile = (g & 7) * per_xcd + (g >> 3);
    if (tile >= m_tiles * n_tiles) return;
    const int32_t mt = tile / n_tiles, nt = tile - mt * n_tiles;
    const int64_t m0 = (int64_t)mt * BM;
    const int32_t n0 = nt * BN;

    // ---- project the tile's tokens: corner rows + weights of each map
    if (tid < BM) {
        const int64_t t = m0 + tid;
        for (int m = 0; m < (a.C1 > 0 ? 2 : 1); ++m) {
            if (t < a.n) {
                int32_t b, x, y, z;
                token_cell(a.coords, t, a.R, b, x, y, z);
                const Projected p = project_cell(b, x, y, z, a.R, a.points, cams, a.batch);
                const Corners c = m ? corners_of(p.gx, p.gy, p.b, a.H1, a.W1)
                                    : corners_of(p.gx, p.gy, p.b, a.H, a.W);
                s_row[m][tid][0] = c.r00; s_row[m][tid][1] = c.r01;
                s_row[m][tid][2] = c.r10; s_row[m][tid][3] = c.r11;
                s_w[m][tid][0] = c.w00; s_w[m][tid][1] = c.w01;
                s_w[m][tid][2] = c.w10; s_w[m][tid][3] = c.w11;
                if (m == 0 && a.mask && nt == 0) a.mask[t] = p.mask;
            } else {
                s_row[m][tid][0] = s_row[m][tid][1] = s_row[m][tid][2] = s_row[m][tid][3] = 0;
                s_w[m][tid][0] = s_w[m][tid][1] = s_w[m][tid][2] = s_w[m][tid][3] = 0.0f;
            }
        }
    }
    __syncthreads();

    const uint4* __restrict__ feat0 = reinterpret_cast<const uint4*>(a.feat);
    const uint4* __restrict__ feat1 = reinterpret_cast<const uint4*>(a.feat1);
    const uint4* __restrict__ wgt = reinterpret_cast<const uint4*>(a.weight);
    const int vpr0 = a.C / 4, vpr1 = a.C1 / 4;       // vectors per map row
    const int vprw = vpr0 + vpr1;                    // vectors per weight row
    const int k1 = a.C1 > 0 ? a.C / BK : 1 << 30;    // first chunk of map 1
    const int nk = (a.C + a.C1 + BK - 1) / BK;

    uint4 qa[A_ITEMS][4];
    uint4 qb[B_ITEMS];

    auto issue_loads = [&](int kc) {
        const int mp = kc >= k1 ? 1 : 0;                 // map of this chunk (uniform)
        const uint4* __restrict__ feat = mp ? feat1 : feat0;
        const int vpr = mp ? vpr1 : vpr0;
        const int kl = mp ? kc - k1 : kc;                // chunk within the map
#pragma unroll
        for (int u = 0; u < A_ITEMS; ++u) {
            const int i = tid + u * kThreads;
            const int m = i >> 3, v = i & 7;
            const int kv = kl * 8 + v;
            if (kv < vpr) {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    qa[u][k] = feat[(int64_t)s_row[mp][m][k] * vpr + kv];
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) qa[u][k] = make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int u = 0; u < B_ITEMS; ++u) {
            const int i = tid + u * kThreads;
            const int j = i >> 3, v = i & 7;
            const int kv = kc * 8 + v;
            qb[u] = (kv < vprw && n0 + j < a.D) ? wgt[(int64_t)(n0 + j) * vprw + kv]
                                                : make_uint4(0, 0, 0, 0);
        }
    };

    f32x4_t acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    issue_loads(0);
    for (int kc = 0; kc < nk; ++kc) {
        uint4 av[A_ITEMS];
        const int mp = kc >= k1 ? 1 : 0;
#pragma unroll
        for (int u = 0; u < A_ITEMS; ++u) {
            const int m = (tid + u * kThreads) >> 3;
            av[u] = blend4(qa[u], s_w[mp][m][0], s_w[mp][m][1], s_w[mp][m][2], s_w[mp][m][3]);
        }
        // stage kc % 2 was last read by the MFMAs of chunk kc - 2, which
        // every wave finished before the barrier of chunk kc - 1
        uint4* __restrict__ sa = s_a[kc & 1];
        uint4* __restrict__ sb = s_b[kc & 1];
#pragma unroll
        for (int u = 0; u < A_ITEMS; ++u) {
            const int i = tid + u * kThreads;
            sa[swz(i >> 3, i & 7)] = av[u];
        }
#pragma unroll
        for (int u = 0; u < B_ITEMS; ++u) {
            const int i = tid + u * kThreads;
            sb[swz(i >> 3, i & 7)] = qb[u];
        }
        __syncthreads();
        if (kc + 1 < nk) issue_loads(kc + 1);

        // v_mfma_f32_16x16x4_f32: lane l supplies A[l%16][l/16] and
        // B[l/16][l%16]; the four K quarters of a 16-byte vector are four
        // MFMAs (K order within the chunk is permuted identically on both
        // operands, which leaves the dot products unchanged).
#pragma unroll
        for (int kq = 0; kq < BK / 16; ++kq) {
            const int v = kq * 4 + (lane >> 4);
            float4 af[MI], bfr[NJ];
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const int row = wm * WM + i * 16 + (lane & 15);
                af[i] = __builtin_bit_cast(float4, sa[swz(row, v)]);
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int row = wn * WN + j * 16 + (lane & 15);
                bfr[j] = __builtin_bit_cast(float4, sb[swz(row, v)]);
            }
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i].x, bfr[j].x,
                                                                    acc[i][j], 0, 0, 0);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i].y, bfr[j].y,
                                                                    acc[i][j], 0, 0, 0);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i].z, bfr[j].z,
                                                                    acc[i][j], 0, 0, 0);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i].w, bfr[j].w,
                                                                    acc[i][j], 0, 0, 0);
                }
        }
    }

    // ---- epilogue: + bias, stage 16 rows at a time through LDS for
    // coalesced 16-byte row stores. A 16x16 block's lane l holds rows
    // 4*(l/16) + r (r = 0..3) of column l % 16.
    float bias_v[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int col = n0 + wn * WN + j * 16 + (lane & 15);
        bias_v[j] = (a.bias && col < a.D) ? reinterpret_cast<const float*>(a.bias)[col] : 0.0f;
    }
    constexpr int STAGE_VEC = 16 * WN / 4;           // 16-byte vectors per wave stage
    constexpr int ROW_VEC = WN / 4;                  // vectors per staged row
    float* stage = reinterpret_cast<float*>(s_a[0]) + wave * (16 * WN);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
        __syncthreads();
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * (lane >> 4) + r;
                const int col = j * 16 + (lane & 15);
                stage[row * WN + col] = acc[i][j][r] + bias_v[j];
            }
        __syncthreads();
        const uint4* st4 = reinterpret_cast<const uint4*>(stage);
#pragma unroll
        for (int rep = 0; rep < STAGE_VEC / 64; ++rep) {
            const int q = rep * 64 + lane;
            const int row = q / ROW_VEC, cv = q - row * ROW_VEC;
            const int64_t t = m0 + wm * WM + i * 16 + row;
            const int col = n0 + wn * WN + cv * 4;
            if (t < a.n && col < a.D)
                *reinterpret_cast<uint4*>(reinterpret_cast<float*>(a.out) + t * a.D + col) =
                    st4[q];
        }
    }
}

// Null rows [n, n + n_null): the bias (or +0) broadcast, 16-byte stores.
template <bool Bf16>
__global__ __launch_bounds__(256) void null_fill_kernel(const void* bias, int32_t D, int64_t n,
                                                        int64_t n_null, void* out) {
    constexpr int EPV = Bf16 ? 8 : 4;
    const int vpr = D / EPV;
    const int64_t total = n_null * vpr;
    uint4* o = reinterpret_cast<uint4*>(out) + n * vpr;
    const uint4* b = reinterpret_cast<const uint4*>(bias);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total; q += stride) {
        const int v = (int)(q % vpr);
        const uint4 val = b ? b[v] : make_uint4(0, 0, 0, 0);
        store_nt16(o + q, val);
    }
}

}  // namespace

hipError_t launch_proj_cond(const ProjCondArgs& a, p3d_dtype dt, const CamTable& cams,
                            hipStream_t s) {
    const bool bf16 = dt == P3D_BF16;
    if (bf16 && a.n > 0) return launch_proj_cond_bf16(a, cams, s);   // null rows included
    if (a.n > 0) {
        int32_t m_tiles = (int32_t)((a.n + BM - 1) / BM);
        int32_t n_tiles = (a.D + BN - 1) / BN;
        int32_t per_xcd = (int32_t)(((int64_t)m_tiles * n_tiles + 7) / 8);
        ProjCondArgs args = a;
        CamTable tab = cams;
        void* params[] = {&args, &tab, &m_tiles, &n_tiles, &per_xcd};
        hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&proj_cond_kernel),
                                       dim3((unsigned)per_xcd * 8), dim3(kThreads), params, 0, s);
        if (e != hipSuccess) return e;
    }
    if (a.n_null > 0) {
        const void* bias = a.bias;
        int32_t D = a.D;
        int64_t n = a.n, nn = a.n_null;
        void* out = a.out;
        void* params[] = {&bias, &D, &n, &nn, &out};
        const int64_t vec = a.n_null * (a.D / (bf16 ? 8 : 4));
        int64_t blocks = (vec + 255) / 256;
        if (blocks > 8192) blocks = 8192;
        const void* fn = bf16 ? reinterpret_cast<const void*>(&null_fill_kernel<true>)
                              : reinterpret_cast<const void*>(&null_fill_kernel<false>);
        hipError_t e = hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(256), params, 0, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace p3d
