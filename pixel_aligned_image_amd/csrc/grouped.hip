// grouped.hip -- p3d_proj_linear_grouped: the per-block proj_linear of the
// DiT over one stage-constant projection (trellis.cpp PR #38, commit adding
// proj mode: every block carries its own proj_linear, whose output is added
// into that block's residual). S is gathered once per stage
// (p3d_proj_sample); every denoising step then applies, for each block g,
//   Y_g = W_g S + b_g        or, as a residual add,   Y_g += W_g S + b_g.
//
// One launch covers all blocks. The workgroup is the 128 x 512 tile of the
// fused kernel (bf16_tile.h): 8 consumer waves on the matrix cores, 4
// producer waves that here load dense S rows (one 16-byte vector per item,
// a chunk ahead in registers, no gather, no blend) and stream W_g through
// LDS with direct loads. Tiles run feature tile fastest, then token tile,
// then block; each XCD walks a contiguous range, so the feature tiles of a
// token tile share its S rows in that XCD's L2 and a block's W stays hot
// while its token tiles stream by.
#include "bf16_tile.h"

namespace p3d {

namespace {

using namespace tile;

constexpr int S_ITEMS = BM * (BK / 8) / kProdThreads;   // S vectors per producer thread

struct DenseProducer {
    const uint4* S;
    int vprs, ptid, gv;
    int64_t m0, last;               // first token of the tile, last valid token
    const char* sbase;              // row m0 of S (uniform)
    uint32_t off[S_ITEMS];          // per item: (row - m0) * row bytes + 16 gv
    bool off32;                     // the tile's rows of S span under 2 GiB
    WLoader wl;

    // Rows past the last token repeat it (their outputs are never stored).
    __device__ __forceinline__ void set_items() {
        sbase = reinterpret_cast<const char*>(S) + m0 * (int64_t)vprs * 16;
        off32 = (int64_t)BM * vprs * 16 < ((int64_t)1 << 31);
#pragma unroll
        for (int u = 0; u < S_ITEMS; ++u) {
            int64_t row = m0 + ((ptid + u * kProdThreads) >> 3);
            row = row < last ? row : last;
            off[u] = (uint32_t)((row - m0) * vprs * 16 + gv * 16);
        }
    }

    // Queue S vector gv of chunk kc for the thread's items: a uniform base
    // plus the items' 32-bit offsets. A K tail clamps the vector index and
    // commit() zeroes the value (zeroing here would make the loads'
    // registers wait).
    __device__ __forceinline__ void s_issue(uint4 (&q)[S_ITEMS], int kc) const {
        if (off32 && (kc + 1) * 8 <= vprs) {
            const char* b = sbase + kc * 128;
#pragma unroll
            for (int u = 0; u < S_ITEMS; ++u) q[u] = *reinterpret_cast<const uint4*>(b + off[u]);
            return;
        }
        const int kv = min(kc * 8 + gv, vprs - 1);
#pragma unroll
        for (int u = 0; u < S_ITEMS; ++u) {
            int64_t row = m0 + ((ptid + u * kProdThreads) >> 3);
            row = row < last ? row : last;
            q[u] = S[row * vprs + kv];
        }
    }

    __device__ __forceinline__ void commit(const uint4 (&q)[S_ITEMS], int kc,
                                           uint4* __restrict__ sa) const {
        const bool dead = kc * 8 + gv >= vprs;
#pragma unroll
        for (int u = 0; u < S_ITEMS; ++u)
            sa[slot((ptid + u * kProdThreads) >> 3, gv)] = dead ? make_uint4(0, 0, 0, 0) : q[u];
    }
};

// One producer iteration (see the fused kernel): W of chunk kc+1, S of chunk
// kc+1 into LDS, S of chunk kc+2 queued, this wave's W landed, barrier.
__device__ __forceinline__ void produce(const DenseProducer& p, int kc, int nk2,
                                        uint4 (&q)[S_ITEMS], uint4* __restrict__ sa_n,
                                        uint4* __restrict__ sw_n) {
    if (kc + 1 < nk2) {
        // W first: with no blend to overlap, waiting for S before queueing W
        // only delays the W loads
        p.wl.issue(sw_n, kc + 1);
        p.commit(q, kc + 1, sa_n);
        if (kc + 2 < nk2) {
            p.s_issue(q, kc + 2);
            wait_vmcnt<S_ITEMS>();                   // the queued S may stay in flight
        } else {
            wait_vmcnt<0>();
        }
    }
    lds_barrier();
}

template <bool Accumulate>
__global__ __launch_bounds__(kThreads) void grouped_kernel(GroupedArgs a, int32_t m_tiles,
                                                           int32_t n_tiles, int64_t per_xcd) {
    __shared__ uint4 sW0[BN * 8], sW1[BN * 8];     // 2 x 64 KB
    __shared__ uint4 sA0[BM * 8], sA1[BM * 8];     // 2 x 16 KB

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    const int64_t g = blockIdx.x;
    const int64_t tile = (g & 7) * per_xcd + (g >> 3);
    const int64_t per_group = (int64_t)m_tiles * n_tiles;
    if (tile >= per_group * a.G) return;
    const int32_t grp = (int32_t)(tile / per_group);
    const int64_t r = tile - grp * per_group;
    const int32_t mt = (int32_t)(r / n_tiles), nt = (int32_t)(r - (int64_t)mt * n_tiles);
    const int64_t m0 = (int64_t)mt * BM;
    const int32_t n0 = nt * BN;
    const int nk = (a.K + BK - 1) / BK;
    const int nk2 = (nk + 1) & ~1;                    // even chunk count: two stages per round

    if (wave >= N_CONS) {
        DenseProducer p;
        p.S = reinterpret_cast<const uint4*>(a.S);
        p.vprs = a.K >> 3;
        p.ptid = tid - N_CONS * 64;
        p.gv = p.ptid & 7;
        p.m0 = m0;
        p.last = a.n - 1;
        p.set_items();
        p.wl.init(a.W[grp], a.K >> 3, a.D, n0, __builtin_amdgcn_readfirstlane(wave - N_CONS),
                  lane);
        uint4 q[S_ITEMS];
        p.s_issue(q, 0);
        p.wl.issue(sW0, 0);
        p.commit(q, 0, sA0);
        p.s_issue(q, 1);
        wait_vmcnt<S_ITEMS>();
        lds_barrier();                                            // B_0
        for (int kc = 0; kc < nk2; kc += 2) {
            produce(p, kc, nk2, q, sA1, sW1);
            produce(p, kc + 1, nk2, q, sA0, sW0);
        }
        __syncthreads();                                          // consumers staged
        return;
    }

    const int cw = wave;
    f32x4_t acc[FJ][TI];
#pragma unroll
    for (int j = 0; j < FJ; ++j)
#pragma unroll
        for (int i = 0; i < TI; ++i) acc[j][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    lds_barrier();                                                // B_0
    for (int kc = 0; kc < nk2; kc += 2) {
        consume(acc, lane, cw, sA0, sW0);
        consume(acc, lane, cw, sA1, sW1);
    }
    store_tile<Accumulate>(acc, lane, cw, n0, m0, a.n, a.D,
                           reinterpret_cast<const uint16_t*>(a.bias[grp]), a.out[grp], sW0, sW1);
}

}  // namespace

hipError_t launch_grouped(const GroupedArgs& a, bool accumulate, hipStream_t s) {
    int32_t m_tiles = (int32_t)((a.n + BM - 1) / BM);
    int32_t n_tiles = (a.D + BN - 1) / BN;
    int64_t per_xcd = ((int64_t)m_tiles * n_tiles * a.G + 7) / 8;
    GroupedArgs args = a;
    void* params[] = {&args, &m_tiles, &n_tiles, &per_xcd};
    const void* fn = accumulate ? reinterpret_cast<const void*>(&grouped_kernel<true>)
                                : reinterpret_cast<const void*>(&grouped_kernel<false>);
    return hipLaunchKernel(fn, dim3((unsigned)(per_xcd * 8)), dim3(kThreads), params, 0, s);
}

}  // namespace p3d
