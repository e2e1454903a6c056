// bf16_tile.h -- the 128 x 512 bf16 MFMA tile shared by the fused
// projection-conditioning kernel and the per-block (grouped) proj_linear:
// workgroup shape, LDS layout and swizzle, the direct-to-LDS W stream, the
// consumer MFMA loop and the epilogue. Device code only; included by the .hip
// files that build the kernels.
//
// Workgroup: 128 tokens x 512 output features, one workgroup per CU (160 KB
// of LDS), 12 waves: 8 consumer waves (two per SIMD) only issue
// v_mfma_f32_16x16x32_bf16 -- consumer c owns features [64c, 64c + 64) of all
// 128 tokens in 4 x 8 blocks (128 accumulator registers), W the row operand,
// S the column operand; 4 producer waves fill the LDS stages. K advances in
// 64-channel chunks through two stages of S (128 x 128 bytes) and W
// (512 x 128 bytes).
#pragma once

#include "p3d_internal.h"

namespace p3d {
namespace tile {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int N_CONS = 8, N_PROD = 4;
constexpr int kThreads = 64 * (N_CONS + N_PROD);
constexpr int kProdThreads = 64 * N_PROD;
constexpr int BM = 128, BN = 512, BK = 64;
constexpr int WN = BN / N_CONS;     // features per consumer wave
constexpr int TI = BM / 16;         // token blocks per consumer wave
constexpr int FJ = WN / 16;         // feature blocks per consumer wave
constexpr int W_ROWS = BN / N_PROD;                     // W rows loaded per producer wave
constexpr int W_INSTR = W_ROWS * (BK / 8) / 64;         // direct W loads per producer lane

// s_waitcnt vmcnt(n), expcnt and lgkmcnt left at their maxima (gfx9 layout:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier for LDS hand-offs only: this wave's LDS accesses have
// completed, then s_barrier. Unlike __syncthreads() it does not wait for
// outstanding global loads (that fence drains vmcnt), so the gather queued
// for a later chunk stays in flight across it; whoever hands over data that
// arrived by direct-to-LDS loads waits for those explicitly first.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// LDS slot of 16-byte vector v (0..7) of tile row `row` (128-byte rows).
// Sixteen lanes reading vector v of sixteen consecutive rows then hit
// sixteen distinct 16-byte slots of a 256-byte bank window (64 banks).
__device__ __forceinline__ int slot(int row, int v) { return row * 8 + (v ^ ((row >> 1) & 7)); }

// A producer wave's share of the tile's W stream: rows row0 .. row0+127
// (row0 = n0 + pw*W_ROWS), one 64-channel chunk at a time, into the LDS
// stage. Load q moves rows q*8 .. q*8+7 (lane l: row q*8 + l/8) with
// global_load_lds_dwordx4; lane l lands in LDS slot l%8 of its row, which
// holds logical vector (l%8) ^ ((row/2) % 8), a swizzle that only depends on
// the parity of q.
// Fast path (every row below D, the chunk inside K): the address is a
// uniform base (row0, chunk kc, load q: scalar registers) plus one of two
// per-lane 32-bit offsets fixed for the tile, so a load costs no vector
// instructions. Otherwise rows past D repeat row D-1 (their outputs are never
// stored) and the vector index is clamped to the row (the matching S values
// are zero).
struct WLoader {
    const uint4* wgt;
    const char* base;                // row row0 of W (uniform)
    uint32_t voff_even, voff_odd;    // per lane: row lane/8, swizzled vector
    int row_bytes, vprw, D, row0, pw, lane;
    bool full;                       // rows row0 .. row0 + W_ROWS - 1 all below D

    __device__ __forceinline__ void init(const void* w, int vprw_, int D_, int n0, int pw_,
                                         int lane_) {
        wgt = reinterpret_cast<const uint4*>(w);
        vprw = vprw_;
        D = D_;
        pw = pw_;
        lane = lane_;
        row0 = n0 + pw * W_ROWS;
        row_bytes = vprw * 16;
        base = reinterpret_cast<const char*>(w) + (int64_t)row0 * row_bytes;
        // every offset must fit 32 bits: W_ROWS rows of W
        full = row0 + W_ROWS <= D && (int64_t)W_ROWS * row_bytes < ((int64_t)1 << 31);
        const int wv_even = (lane & 7) ^ ((lane >> 4) & 7);
        const int wv_odd = (lane & 7) ^ ((4 + (lane >> 4)) & 7);
        voff_even = (uint32_t)((lane >> 3) * row_bytes + wv_even * 16);
        voff_odd = (uint32_t)((lane >> 3) * row_bytes + wv_odd * 16);
    }

    __device__ __forceinline__ void issue(uint4* __restrict__ sw, int kc) const {
        uint4* dst = sw + pw * W_ROWS * 8;
        if (full && (kc + 1) * 8 <= vprw) {
            const char* b = base + kc * 128;
#pragma unroll
            for (int q = 0; q < W_INSTR; ++q) {
                const char* bq = b + (int64_t)q * 8 * row_bytes;
                __builtin_amdgcn_global_load_lds(
                    reinterpret_cast<const void*>(bq + ((q & 1) ? voff_odd : voff_even)),
                    (lds_void*)(dst + q * 64), 16, 0, 0);
            }
        } else {
            // the lane index is opaque here, so that the clamped row
            // addresses are formed per load rather than hoisted out of the K
            // loop (where they would take registers the producers need)
            int l = lane;
            asm volatile("" : "+v"(l));
            const int wv_even = (l & 7) ^ ((l >> 4) & 7);
            const int wv_odd = (l & 7) ^ ((4 + (l >> 4)) & 7);
#pragma unroll
            for (int q = 0; q < W_INSTR; ++q) {
                const int col = min(row0 + q * 8 + (l >> 3), D - 1);
                const int kv = min(kc * 8 + ((q & 1) ? wv_odd : wv_even), vprw - 1);
                __builtin_amdgcn_global_load_lds(
                    reinterpret_cast<const void*>(wgt + (int64_t)col * vprw + kv),
                    (lds_void*)(dst + q * 64), 16, 0, 0);
            }
        }
    }
};

// Consumer: the chunk's 2 x TIt x 4 MFMAs over the first 16 TIt tokens of
// the stage (TIt = TI for a full tile). The S fragment of token block i + 1
// is read before the MFMAs of block i are issued (the scheduling barriers
// keep that order), so its LDS latency runs under them; the other consumer
// wave on the SIMD covers the rest.
template <int TIt = TI>
__device__ __forceinline__ void consume(f32x4_t (&acc)[FJ][TIt], int lane, int cw,
                                        const uint4* __restrict__ sa,
                                        const uint4* __restrict__ sw) {
    const int n = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int s = 0; s < BK / 32; ++s) {
        const int v = s * 4 + g4;
        bf16x8_t wf[FJ];
#pragma unroll
        for (int j = 0; j < FJ; ++j)
            wf[j] = __builtin_bit_cast(bf16x8_t, sw[slot(cw * WN + j * 16 + n, v)]);
        bf16x8_t sf = __builtin_bit_cast(bf16x8_t, sa[slot(n, v)]);
#pragma unroll
        for (int i = 0; i < TIt; ++i) {
            bf16x8_t nxt = sf;
            if (i + 1 < TIt) nxt = __builtin_bit_cast(bf16x8_t, sa[slot((i + 1) * 16 + n, v)]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < FJ; ++j)
                acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[j], sf, acc[j][i], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            sf = nxt;
        }
    }
    lds_barrier();
}

// Epilogue: + bias (bf16 parameters), optionally + the value already in
// `out` (Accumulate: a residual add, rounded once), round to bf16, stage the
// wave's 16 TIt x 64 block in the free W stages (token-major 128-byte rows,
// the same slot swizzle) and write 16-byte row pieces with non-temporal
// stores (the output is not read back here). Lane l of block (j, i)
// holds features 4*(l/16) + r of token l % 16. out is [n, D] bf16; tile row
// t goes to output row m0 + t, or to rows[t] when an LDS table `rows` is
// given (-1: not stored); rows at or past n are not touched.
constexpr int OLD_BATCH = 4;        // residual loads in flight together (registers)
static_assert(TI % OLD_BATCH == 0, "residual batches");

template <bool Accumulate, int TIt = TI>
__device__ __forceinline__ void store_tile(const f32x4_t (&acc)[FJ][TIt], int lane, int cw,
                                           int32_t n0, int64_t m0, int64_t n, int32_t D,
                                           const uint16_t* bias16, void* out,
                                           uint4* __restrict__ sW0, uint4* __restrict__ sW1,
                                           const int32_t* rows = nullptr) {
    constexpr int BATCH = TIt % OLD_BATCH == 0 ? OLD_BATCH : (TIt % 2 == 0 ? 2 : 1);
    static_assert(TIt % BATCH == 0, "residual batches");
    const int fbase = n0 + cw * WN;
    const int dv = D >> 3;                            // 16-byte vectors per output row
    uint4* stage4 = (cw < N_CONS / 2 ? sW0 : sW1) + (cw % (N_CONS / 2)) * (BM * 8);
    uint2* stage2 = reinterpret_cast<uint2*>(stage4);
    const uint16_t* out16 = reinterpret_cast<const uint16_t*>(out);
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
        // D is a multiple of 8, so a lane's four features are all below D or
        // all past it. The loads are unconditional, from clamped addresses,
        // with the values selected afterwards: a batch of loads then goes out
        // together and shares one wait (conditional loads each wait alone).
        const int f0 = fbase + j * 16 + 4 * (lane >> 4);
        const bool fin = f0 < D;
        const int fc = fin ? f0 : D - 4;
        uint2 b2 = make_uint2(0, 0);
        if (bias16) b2 = *reinterpret_cast<const uint2*>(bias16 + fc);
        if (!fin) b2 = make_uint2(0, 0);
        const float bv[4] = {bf16lo(b2.x), bf16hi(b2.x), bf16lo(b2.y), bf16hi(b2.y)};
        uint2 old[TIt];
#pragma unroll
        for (int i = 0; i < TIt; ++i) {
            if (Accumulate && i % BATCH == 0) {
                // the residual values of the next BATCH token blocks
#pragma unroll
                for (int u = i; u < i + BATCH; ++u) {
                    const int64_t tok = m0 + u * 16 + (lane & 15);
                    old[u] = *reinterpret_cast<const uint2*>(out16 + (tok < n ? tok : n - 1) * D + fc);
                }
            }
            const int t = i * 16 + (lane & 15);
            const int f = j * 16 + 4 * (lane >> 4);
            float y[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) y[r] = acc[j][i][r] + bv[r];
            if constexpr (Accumulate) {
                // rows past n and features past D are never stored
                y[0] += bf16lo(old[i].x);
                y[1] += bf16hi(old[i].x);
                y[2] += bf16lo(old[i].y);
                y[3] += bf16hi(old[i].y);
            }
            uint2 pk;
            pk.x = pack_bf16x2(y[0], y[1]);
            pk.y = pack_bf16x2(y[2], y[3]);
            stage2[slot(t, f >> 3) * 2 + ((f >> 2) & 1)] = pk;
        }
    }
    __syncthreads();                                              // consumers staged
    uint4* out4 = reinterpret_cast<uint4*>(out);
#pragma unroll
    for (int r = 0; r < TIt * 16 * 8 / 64; ++r) {
        const int q = r * 64 + lane;
        const int t = q >> 3, cv = q & 7;
        const int64_t tok = rows ? (int64_t)rows[t] : (m0 + t < n ? m0 + t : -1);
        const int colv = (fbase >> 3) + cv;
        if (tok >= 0 && colv < dv) store_nt16(out4 + tok * dv + colv, stage4[slot(t, cv)]);
    }
}

}  // namespace tile
}  // namespace p3d
