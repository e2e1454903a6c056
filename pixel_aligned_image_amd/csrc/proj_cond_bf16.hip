// proj_cond_bf16.hip -- the fused projection -> gather -> proj_linear kernel
// for bf16 maps and weights (fp32 accumulation on the matrix cores), plus the
// CFG null-branch rows in the same launch.
//
// Sources: pixal3d_mrp_mlx tests/ history, pixel-aligned head commit
// (project_points, bilinear_sample with grid_sample's align_corners=False,
// border padding); trellis.cpp PR #38 "Initial support for Pixal3D",
// FlowCond commit (proj_linear; the null proj is zeroed on the device, so its
// rows are proj_linear(0) = bias).
//
// GEMM view: Y[M=n, N=D] = S[M, K=C] W[N, K]^T + b, S never stored.
//
// Workgroup: 128 tokens x 512 output features, one workgroup per CU (all 160
// KB of LDS), 12 waves in two roles, three waves per SIMD:
//   8 consumer waves (two per SIMD) only run the matrix cores: consumer c
//     owns features [64c, 64c + 64) for all 128 tokens, 4 x 8 blocks of
//     v_mfma_f32_16x16x32_bf16 (128 accumulator registers), W as the row
//     operand and S as the column operand (a lane ends up with four
//     consecutive features of one token);
//   4 producer waves (one per SIMD) do everything else: project the tokens,
//     keep the corner-row gather a chunk ahead in registers, blend and
//     round the samples into the LDS S tile, stream W through LDS with
//     direct loads, and write the tile's share of the null rows, one
//     16-byte store per lane per K chunk.
// A wave issuing MFMAs is held at each one until the matrix core takes it,
// so a wave's own VALU work does not overlap its MFMAs; a producer on the
// same SIMD fills those issue slots instead.
//
// Per 64-channel K chunk k (barrier B_k before it):
//   consumers: MFMA on S stage k%2 and W stage k%2;
//   producers: wait for the corner rows of chunk k+1 (queued a chunk ago),
//     queue W of chunk k+1 into W stage (k+1)%2 (freed at B_k), blend chunk
//     k+1 into S stage (k+1)%2, queue the corner rows of chunk k+2, then wait
//     for their own W loads;
//   B_{k+1}.
// Tile start: the producers queue W of chunk 0, project the tokens into LDS,
// then queue the corner rows of chunk 1; meanwhile the consumers, whose
// accumulators are not live yet, gather and blend chunk 0 into S stage 0,
// so the first two round trips to memory overlap; B_0.
// Per tile, each producer item keeps its corner rows' offsets and its
// bilinear weights (Producer), so a chunk's gather and W loads need no
// vector address arithmetic.
// W tile (512 rows x 128 bytes) arrives through global_load_lds_dwordx4,
// eight full 128-byte rows per wave instruction (16 rows x 64 bytes, which
// is what loading MFMA fragments straight from a row-major W would do, moves
// about a third of the bytes per clock); the LDS slot of each 16-byte vector
// is swizzled through the source address, since the destination of a direct
// load is fixed by the lane number.
// Why 128 x 512: every N tile repeats the gather (four corner reads and a
// blend per token and channel), every M tile re-reads W; with 64K fp32
// accumulators per CU, 128 x 512 minimises the sum.
// Two maps (NAF commit: the DINOv3 map and its upsampled version,
// concatenated along K): the chunks past map 0's channels read map 1. The
// producers keep one set of per-token corner metadata; after blending the
// last map-0 chunk and before queueing the first map-1 chunk they recompute
// it for map 1's size from the token coords (projection costs a few ALU
// operations; a second set would not fit in the registers).
// Tile order: workgroup g runs on XCD g % 8; each XCD walks a contiguous
// range of (token tile, N tile) pairs, N fastest, so the N tiles of a token
// tile and its neighbours share corner rows in that XCD's L2.
// Tail: with one workgroup per CU the tiles run in rounds of one per CU.
// When the tiles past the last full round fit one round four times over,
// each of them runs as four 32-token parts (the same code with two token
// blocks per consumer and one gathered vector per producer thread), else,
// when they fit twice over, as two 64-token parts (four token blocks, two
// vectors); the parts are queued after every whole tile. A launch of fewer
// tiles than CUs that neither split fits runs as 96-token tiles when those
// still fit one round.
#include <atomic>
#include <type_traits>

#include "bf16_tile.h"

namespace p3d {

namespace {

using namespace tile;

// Tail sub-tiles: 32 tokens (TI_QUARTER token blocks) or 64 tokens
// (TI_HALF) of a 128-token tile.
constexpr int TI_QUARTER = 2;
constexpr int TI_HALF = 4;
// A launch whose 128-token tiles fill less than one round, too many to split
// into parts: 96-token tiles throughout (TI_ROUND token blocks), when they
// still fit one round.
constexpr int TI_ROUND = 6;

// Gathered vectors per producer thread for a tile of TIt token blocks.
template <int TIt>
constexpr int g_items() { return TIt * 16 * (BK / 8) / kProdThreads; }

__device__ __forceinline__ uint4 blend_bf16(const uint4 (&q)[4], const float (&w)[4]) {
    const uint32_t* a = reinterpret_cast<const uint32_t*>(&q[0]);
    const uint32_t* b = reinterpret_cast<const uint32_t*>(&q[1]);
    const uint32_t* c = reinterpret_cast<const uint32_t*>(&q[2]);
    const uint32_t* d = reinterpret_cast<const uint32_t*>(&q[3]);
    uint4 o;
    uint32_t* r = reinterpret_cast<uint32_t*>(&o);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float lo = fmaf(w[3], bf16lo(d[e]), fmaf(w[2], bf16lo(c[e]),
                              fmaf(w[1], bf16lo(b[e]), w[0] * bf16lo(a[e]))));
        const float hi = fmaf(w[3], bf16hi(d[e]), fmaf(w[2], bf16hi(c[e]),
                              fmaf(w[1], bf16hi(b[e]), w[0] * bf16hi(a[e]))));
        r[e] = pack_bf16x2(lo, hi);
    }
    return o;
}

template <int G>
using Gq = uint4[G][4];

// Corner metadata of the token at position t on an H x W map: (top-left
// corner row, the 0/1 row steps to the right and lower corners, x fraction,
// y fraction); a position past the end gets weight 0 everywhere (flag 4 in
// the steps). Position t holds token a.order[t] (t itself without an order);
// *mask receives its in-image flag.
__device__ __forceinline__ int4 token_entry(const ProjCondArgs& a, const CamTable& cams,
                                            int64_t t, int32_t H, int32_t W, uint8_t* mask) {
    int4 e = make_int4(0, 4, 0, 0);
    if (t < a.n) {
        const int64_t tok = ordered_token(a.order, t, a.n);
        int32_t b, x, y, z;
        token_cell(a.coords, tok, a.R, b, x, y, z);
        const Projected pr = project_cell(b, x, y, z, a.R, a.points, cams, a.batch);
        const SrcIdx sx = source_index(pr.gx, W);
        const SrcIdx sy = source_index(pr.gy, H);
        e.x = (pr.b * H + sy.i0) * W + sx.i0;
        e.y = (sx.i1 - sx.i0) | ((sy.i1 - sy.i0) << 1);
        e.z = __float_as_int(sx.t);
        e.w = __float_as_int(sy.t);
        if (mask) *mask = pr.mask;
    }
    return e;
}

// Gather state of one thread: a producer's items of every chunk past the
// first, or a consumer's items of chunk 0. TwoMaps: the gather
// switches to map 1 part-way through K (kbase, vpr, W and the metadata
// change); with one map they are constants of the launch. Off32: every map
// is under 4 GiB, so a corner vector's byte offset in its map fits 32 bits.
// Per tile (and again at the map switch) each item keeps its four corner
// offsets and its four bilinear weights; a chunk's gather is then a uniform
// base (map, chunk: scalar registers) plus those offsets, with no vector
// address arithmetic, and the blend reuses the weights.
template <bool TwoMaps, bool Off32, int G>
struct Producer {
    const uint4* feat;               // map of the chunks being gathered
    int vpr;                         // 16-byte vectors per row of that map
    int kbase;                       // first K chunk of that map
    int W;                           // that map's width (row step between image rows)
    int vfirst, vstride;             // item u is vector vfirst + u vstride of a chunk
    int gv;                          // vector of each gathered 128-byte segment
    int4 gt[G];                      // token_entry of each item (used without Off32)
    uint32_t off[G][4];              // corner rows' byte offsets + 16 gv (Off32)
    __amdgpu_buffer_rsrc_t rsrc;     // the map as a buffer resource (Off32)
    float wt[G][4];                  // bilinear weights, 0 for a padding token
    WLoader wl;

    // Tile row (token) of item u.
    __device__ __forceinline__ int row(int u) const { return (vfirst + u * vstride) >> 3; }

    // Offsets and weights of the items from their corner metadata gt.
    __device__ __forceinline__ void set_items() {
        if constexpr (Off32)
            rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(feat), (short)0,
                                                     (int)0xffffffffu, 0x00020000);
#pragma unroll
        for (int u = 0; u < G; ++u) {
            const int32_t r00 = gt[u].x, steps = gt[u].y;
            const int32_t dx = steps & 1, dyw = (steps & 2) ? W : 0;
            const int32_t rows[4] = {r00, r00 + dx, r00 + dyw, r00 + dyw + dx};
            if constexpr (Off32) {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    off[u][k] = (uint32_t)rows[k] * (uint32_t)(vpr * 16) + (uint32_t)(gv * 16);
            }
            const float tx = __int_as_float(gt[u].z), ty = __int_as_float(gt[u].w);
            wt[u][0] = (1.0f - tx) * (1.0f - ty);
            wt[u][1] = tx * (1.0f - ty);
            wt[u][2] = (1.0f - tx) * ty;
            wt[u][3] = tx * ty;
            if (steps & 4) wt[u][0] = 0.0f;           // padding token: all weights 0
        }
    }

    // Switch the gather to map 1: its base, row length, width and the
    // items' corner metadata on its grid.
    __device__ __forceinline__ void to_map1(const ProjCondArgs& a, const CamTable& cams,
                                            int64_t m0, int k1) {
        feat = reinterpret_cast<const uint4*>(a.feat1);
        vpr = a.C1 >> 3;
        kbase = k1;
        W = a.W1;
#pragma unroll
        for (int u = 0; u < G; ++u)
            gt[u] = token_entry(a, cams, m0 + row(u), a.H1, a.W1, nullptr);
        set_items();
    }

    // Queue the four corner vectors of every item of chunk kc. A K tail (the
    // map's channels not a multiple of 64, or the padding chunk) clamps the
    // address; commit() zeroes those values (zeroing here would make the
    // loads' registers wait).
    __device__ __forceinline__ void gather_issue(Gq<G>& gq, int kc) const {
        const int kl = TwoMaps ? kc - kbase : kc;
        if constexpr (Off32) {
            if ((kl + 1) * 8 <= vpr) {
                // buffer loads: map base in a resource, the chunk as the scalar
                // offset, the item's 32-bit offset as is
#pragma unroll
                for (int u = 0; u < G; ++u)
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        gq[u][k] = __builtin_bit_cast(
                            uint4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off[u][k], kl * 128, 0));
            } else {
                // K tail: the vector index kv clamped to the row, from the map
                // base. off - 16 gv is the row's byte offset, and adding 16 kv
                // stays inside the map (under 4 GiB): neither step wraps
                const char* f = reinterpret_cast<const char*>(feat);
                const uint32_t kv16 = (uint32_t)min(kl * 8 + gv, vpr - 1) * 16u;
                const uint32_t gv16 = (uint32_t)gv * 16u;
#pragma unroll
                for (int u = 0; u < G; ++u)
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        gq[u][k] = *reinterpret_cast<const uint4*>(f + (off[u][k] - gv16 + kv16));
            }
            return;
        }
        const int kv = min(kl * 8 + gv, vpr - 1);
#pragma unroll
        for (int u = 0; u < G; ++u) {
            // the 32-bit row index stays live, not four hoisted 64-bit
            // addresses (those would not fit in the registers)
            int32_t r00 = gt[u].x, steps = gt[u].y;
            asm volatile("" : "+v"(r00), "+v"(steps));
            const int32_t dx = steps & 1, dyw = (steps & 2) ? W : 0;
            const int32_t rows[4] = {r00, r00 + dx, r00 + dyw, r00 + dyw + dx};
#pragma unroll
            for (int k = 0; k < 4; ++k) gq[u][k] = feat[(int64_t)rows[k] * vpr + kv];
        }
    }

    // Blend the queued vectors of chunk kc (bilinear weights computed as in
    // the standalone sampler) and store the bf16 S chunk into sa; vectors
    // past the map's channels store zeros.
    __device__ __forceinline__ void commit(const Gq<G>& gq, int kc, uint4* __restrict__ sa) const {
        const int kl = TwoMaps ? kc - kbase : kc;
        const bool dead = kl * 8 + gv >= vpr;
#pragma unroll
        for (int u = 0; u < G; ++u) {
            const uint4 v = blend_bf16(gq[u], wt[u]);
            sa[slot(row(u), gv)] = dead ? make_uint4(0, 0, 0, 0) : v;
        }
    }
};

// A producer lane's share of its tile's null rows, written a few vectors per
// K chunk (the bias rows would otherwise all go out at the tile's end, when
// the consumers store the tile's output through the same load/store path).
// The lane owns column vector colv (fixed for the tile) of rows
// row0 + 4 i (i < ipt) of every null block q = mt, mt + m_tiles, ...; item
// j is block j / ipt, row i = j % ipt. Everything but colv and the bias
// value is uniform over the wave.
struct NullWriter {
    uint4* out4;
    int64_t row0;                    // first row of this wave's share of block mt
    int64_t q_rows;                  // rows between blocks q and q + m_tiles
    int64_t n_end;                   // n + n_null
    int dv, colv, ipt;
    int j, total, per;               // next item, items, items per chunk
    uint4 val;                       // bias vector colv (or zeros)

    __device__ __forceinline__ void issue() {
        for (int s = 0; s < per && j < total; ++s, ++j) {
            const int qi = j / ipt, i = j - qi * ipt;
            const int64_t row = row0 + qi * q_rows + 4 * i;
            if (row < n_end && colv < dv) store_nt16(out4 + row * dv + colv, val);
        }
    }
};

// One producer iteration: W of chunk kc+1, S of chunk kc+1 (its corner rows
// were queued one chunk ago), corner rows of chunk kc+2 (from map 1 from
// chunk k1 on), then this wave's W loads must have landed before the
// barrier. The LDS stages are restrict parameters so that the compiler can
// tell the direct W loads apart from the S stores.
template <bool TwoMaps, bool Off32, int G>
__device__ __forceinline__ void produce(Producer<TwoMaps, Off32, G>& p, NullWriter& nw,
                                        const ProjCondArgs& a, const CamTable& cams, int64_t m0,
                                        int k1, int kc, int nk2, Gq<G>& gq,
                                        uint4* __restrict__ sa_n, uint4* __restrict__ sw_n) {
    if (kc + 1 < nk2) {
        // Only this chunk's corners are in flight here: wait for them
        // explicitly, then queue W, then blend. Without the explicit wait the
        // compiler waits before the blend, for the W loads queued just before
        // it as well. This chunk's null-row stores go first, so that they
        // have the whole chunk to complete before the next chunk's wait for
        // everything in flight.
        wait_vmcnt<0>();
        nw.issue();
        p.wl.issue(sw_n, kc + 1);
        p.commit(gq, kc + 1, sa_n);
        if constexpr (TwoMaps) {
            if (kc + 2 == k1) p.to_map1(a, cams, m0, k1);
        }
        if (kc + 2 < nk2) {
            p.gather_issue(gq, kc + 2);
            wait_vmcnt<G * 4>();               // the queued gather may stay in flight
        } else {
            wait_vmcnt<0>();
        }
    }
    lds_barrier();
}

// One tile: 16 TIt tokens starting at token m0 = MRows mt + 16 TIt sub,
// features n0 .. n0 + 511. MRows is the height the launch numbers its token
// tiles by: 128 (TIt = TI: a whole tile; TIt = TI_QUARTER or TI_HALF:
// sub-tile `sub` of tile mt), or 96 for the 96-token tiles (TIt = TI_ROUND,
// sub 0).
// The tile also writes its share of the null rows: rows m0 - MRows mt ..
// m0 - MRows mt + 16 TIt - 1 of every MRows-row null block q = mt,
// mt + m_tiles, ..., for the same features.
//
// Kernel tags the instantiation with the kernel's part size: two kernels that
// inline one shared instantiation of the whole tile both spill registers to
// scratch (hipcc of ROCm 7.2), while a copy per kernel does not.
template <bool TwoMaps, bool Off32, int TIt, int MRows, int Kernel>
__device__ __forceinline__ void run_tile(const ProjCondArgs& a, const CamTable& cams,
                                         int32_t mt, int32_t nt, int sub, int32_t m_tiles,
                                         int32_t null_tiles, uint4* __restrict__ sW0,
                                         uint4* __restrict__ sW1, uint4* __restrict__ sA0,
                                         uint4* __restrict__ sA1) {
    constexpr int BMt = TIt * 16;
    constexpr int G = g_items<TIt>();
    constexpr int NULL_VEC = BMt * BN / 8;                // 16-byte vectors of a null share
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const bool producer = wave >= N_CONS;

    const int32_t r0 = sub * BMt;                          // first row within the MRows-row tile
    const int64_t m0 = (int64_t)mt * MRows + r0;
    const int32_t n0 = nt * BN;
    const int nk = (a.C + a.C1 + BK - 1) / BK;
    const int k1 = a.C1 > 0 ? a.C / BK : 1 << 30;     // first chunk of map 1
    const int nk2 = (nk + 1) & ~1;                    // even chunk count: two stages per round
    uint4* out4 = reinterpret_cast<uint4*>(a.out);
    const int dv = a.D >> 3;                          // 16-byte vectors per output row

    if (producer) {
        const int ptid = tid - N_CONS * 64;
        // ---- this tile's share of the null blocks q = mt, mt + m_tiles, ...
        // (written inside the K loop); the lane's bias vector first, so that
        // its load has landed long before the first store
        NullWriter nw;
        nw.out4 = out4;
        nw.dv = dv;
        nw.colv = (n0 >> 3) + (ptid & 63);                    // 64 vectors per 512-wide row
        nw.ipt = NULL_VEC / kProdThreads;
        nw.row0 = a.n + (int64_t)mt * MRows + r0 + (ptid >> 6);
        nw.q_rows = (int64_t)m_tiles * MRows;
        nw.n_end = a.n + a.n_null;
        nw.j = 0;
        nw.total = mt < null_tiles ? ((null_tiles - 1 - mt) / m_tiles + 1) * nw.ipt : 0;
        nw.per = (nw.total + nk2 - 2) / (nk2 - 1);             // over the nk2 - 1 loaded chunks
        nw.val = make_uint4(0, 0, 0, 0);
        if (a.bias && nw.total > 0 && nw.colv < dv)
            nw.val = reinterpret_cast<const uint4*>(a.bias)[nw.colv];
        Producer<TwoMaps, Off32, G> p;
        p.wl.init(a.weight, (a.C + a.C1) >> 3, a.D, n0,
                  __builtin_amdgcn_readfirstlane(wave - N_CONS), lane);
        // W of chunk 0 does not depend on the tokens: queue it before
        // projecting them, so that its latency overlaps the projection and
        // the first gather
        p.wl.issue(sW0, 0);
        // ---- project the tile's tokens; per token park (top-left row, the
        // row steps to the right / lower corner, the two fractions) in sA1.
        // sA1 is next written after B_0, which every wave (producers and the
        // consumers gathering chunk 0) passes only once its reads of this
        // table have completed.
        int4* s_tok = reinterpret_cast<int4*>(sA1);            // [BMt]
        if (ptid < BMt) {
            const int64_t t = m0 + ptid;
            uint8_t mk = 0;
            s_tok[ptid] = token_entry(a, cams, t, a.H, a.W, &mk);
            if (a.mask && nt == 0 && t < a.n) a.mask[ordered_token(a.order, t, a.n)] = mk;
        }
        lds_barrier();                                            // tokens parked

        p.feat = reinterpret_cast<const uint4*>(a.feat);
        p.vpr = a.C >> 3;
        p.kbase = 0;
        p.W = a.W;
        p.vfirst = ptid;
        p.vstride = kProdThreads;
        p.gv = ptid & 7;
#pragma unroll
        for (int u = 0; u < G; ++u) p.gt[u] = s_tok[p.row(u)];
        p.set_items();
        // chunk 0 is gathered and blended by the consumers (below); the
        // producers queue chunk 1 at once, so the two round trips overlap
        Gq<G> gq;
        if constexpr (TwoMaps) {
            if (k1 == 1) p.to_map1(a, cams, m0, k1);
        }
        p.gather_issue(gq, 1);
        wait_vmcnt<G * 4>();                                      // W of chunk 0 (older)
        lds_barrier();                                            // B_0
        for (int kc = 0; kc < nk2; kc += 2) {
            produce(p, nw, a, cams, m0, k1, kc, nk2, gq, sA1, sW1);
            produce(p, nw, a, cams, m0, k1, kc + 1, nk2, gq, sA0, sW0);
        }
        // with a token order, the output row of each tile row, for the
        // consumers' stores (S stage 0 is free after the last chunk)
        if (a.order) {
            int32_t* s_rows = reinterpret_cast<int32_t*>(sA0);
            if (ptid < BMt)
                s_rows[ptid] = m0 + ptid < a.n ? (int32_t)ordered_token(a.order, m0 + ptid, a.n) : -1;
        }
        __syncthreads();                                          // consumers staged
        return;
    }

    // ---------------------------------------------------------- consumers
    const int cw = wave;
    lds_barrier();                                                // tokens parked
    {
        // chunk 0's samples: gathered and blended here (the accumulators are
        // not live yet), while the producers queue chunk 1. Vector v of the
        // chunk goes to consumer thread v % 512; a 32-token part has 256
        // vectors, so only the first four waves take one, a 64-token part
        // one per thread; of a 96-token tile's 768 vectors the first four
        // waves take two, the others one (their second item is a padding
        // token: weight 0 on row 0, stored to a tile row past the tokens,
        // which no consumer reads).
        constexpr int NV = TIt * 16 * (BK / 8);
        constexpr int CT = N_CONS * 64;
        constexpr int GC = (NV + CT - 1) / CT;
        static_assert(NV % 64 == 0, "whole waves");
        if (NV >= CT || tid < NV) {
            const int4* s_tok = reinterpret_cast<const int4*>(sA1);
            Producer<TwoMaps, Off32, GC> c;
            c.feat = reinterpret_cast<const uint4*>(a.feat);
            c.vpr = a.C >> 3;
            c.kbase = 0;
            c.W = a.W;
            c.vfirst = tid;
            c.vstride = CT;
            c.gv = tid & 7;
#pragma unroll
            for (int u = 0; u < GC; ++u) {
                if constexpr (NV % CT == 0) {
                    c.gt[u] = s_tok[c.row(u)];
                } else {
                    c.gt[u] = c.vfirst + u * c.vstride < NV ? s_tok[c.row(u)]
                                                            : make_int4(0, 4, 0, 0);
                }
            }
            c.set_items();
            Gq<GC> gq;
            c.gather_issue(gq, 0);
            wait_vmcnt<0>();
            c.commit(gq, 0, sA0);
        }
    }
    f32x4_t acc[FJ][TIt];
#pragma unroll
    for (int j = 0; j < FJ; ++j)
#pragma unroll
        for (int i = 0; i < TIt; ++i) acc[j][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    lds_barrier();                                                // B_0
    for (int kc = 0; kc < nk2; kc += 2) {
        consume<TIt>(acc, lane, cw, sA0, sW0);
        consume<TIt>(acc, lane, cw, sA1, sW1);
    }

    store_tile<false, TIt>(acc, lane, cw, n0, m0, a.n, a.D,
                           reinterpret_cast<const uint16_t*>(a.bias), a.out, sW0, sW1,
                           a.order ? reinterpret_cast<const int32_t*>(sA0) : nullptr);
}

// Work of workgroup g, which runs on XCD x = g % 8 as its (g / 8)-th:
// whole tiles x * big_per_xcd .. x * big_per_xcd + big_per_xcd - 1 (below
// n_big), then tail sub-tiles x * small_per_xcd + ... (below n_small): tile
// n_big + s / split, part s % split, of 16 TIp tokens (split = TI / TIp).
// Tiles are numbered token tile major, N tile fastest. The part size is a
// template parameter, so that each kernel holds only two tile shapes (a
// third would raise its register pressure).
template <bool TwoMaps, bool Off32, int TIp>
__global__ __launch_bounds__(kThreads) void proj_cond_bf16_kernel(
    ProjCondArgs a, CamTable cams, int32_t m_tiles, int32_t n_tiles, int32_t n_big,
    int32_t big_per_xcd, int32_t n_small, int32_t small_per_xcd, int32_t null_tiles) {
    constexpr int split = TI / TIp;
    __shared__ uint4 sW0[BN * 8], sW1[BN * 8];     // 2 x 64 KB
    __shared__ uint4 sA0[BM * 8], sA1[BM * 8];     // 2 x 16 KB

    const int32_t g = blockIdx.x;
    const int32_t x = g & 7, i = g >> 3;
    if (i < big_per_xcd) {
        const int32_t tile = x * big_per_xcd + i;
        if (tile >= n_big) return;
        const int32_t mt = tile / n_tiles;
        run_tile<TwoMaps, Off32, TI, BM, TIp>(a, cams, mt, tile - mt * n_tiles, 0, m_tiles,
                                              null_tiles, sW0, sW1, sA0, sA1);
    } else {
        const int32_t st = x * small_per_xcd + (i - big_per_xcd);
        if (st >= n_small) return;
        const int32_t tile = n_big + st / split;
        const int32_t mt = tile / n_tiles;
        run_tile<TwoMaps, Off32, TIp, BM, TIp>(a, cams, mt, tile - mt * n_tiles, st % split,
                                               m_tiles, null_tiles, sW0, sW1, sA0, sA1);
    }
}

// A launch of one round of 96-token tiles: workgroup g runs on XCD x = g % 8
// as its (g / 8)-th and takes tile x * per_xcd + g / 8 (below `tiles`),
// numbered as above with 96-token tiles.
template <bool TwoMaps, bool Off32>
__global__ __launch_bounds__(kThreads) void proj_cond_bf16_round_kernel(
    ProjCondArgs a, CamTable cams, int32_t m_tiles, int32_t n_tiles, int32_t tiles,
    int32_t per_xcd, int32_t null_tiles) {
    __shared__ uint4 sW0[BN * 8], sW1[BN * 8];     // 2 x 64 KB
    __shared__ uint4 sA0[BM * 8], sA1[BM * 8];     // 2 x 16 KB

    const int32_t g = blockIdx.x;
    const int32_t tile = (g & 7) * per_xcd + (g >> 3);
    if (tile >= tiles) return;
    const int32_t mt = tile / n_tiles;
    run_tile<TwoMaps, Off32, TI_ROUND, 16 * TI_ROUND, TI_ROUND>(
        a, cams, mt, tile - mt * n_tiles, 0, m_tiles, null_tiles, sW0, sW1, sA0, sA1);
}

// Compute units of the current device (queried once per device).
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        return 256;
    if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

}  // namespace

// Tail split: one workgroup per CU, so T tiles take ceil(T / CUs) rounds and
// the last round may leave most CUs idle. When the R tiles past the last
// full round fit one round as 32-token sub-tiles (4 R <= CUs), or else as
// 64-token sub-tiles (2 R <= CUs), they run as sub-tiles instead: each
// moves the full W stream of its N tile and a quarter or half of the
// gather, so it takes well under a whole tile's time.
// A launch of fewer tiles than CUs that neither split fits (more than
// CUs / 2 tiles) takes one tile's time however many CUs it leaves idle: it
// runs as 96-token tiles when those still fit one round, each with three
// quarters of a tile's gather and products (and the same W stream).
p3d_tile_plan plan_proj_cond_bf16(int64_t n, int32_t D, int32_t cus) {
    p3d_tile_plan p{};
    p.tile_rows = BM;
    p.feature_tiles = (D + BN - 1) / BN;
    p.token_tiles = (int32_t)((n + BM - 1) / BM);
    if (n == 0) return p;                          // no tiles
    const int32_t tiles = p.token_tiles * p.feature_tiles;
    const int32_t rem = tiles % cus;
    int32_t split = 0;
    if (rem > 0 && rem * (TI / TI_QUARTER) <= cus) split = TI / TI_QUARTER;
    else if (rem > 0 && rem * (TI / TI_HALF) <= cus) split = TI / TI_HALF;
    constexpr int RM = 16 * TI_ROUND;
    const int32_t round_tiles = (int32_t)((n + RM - 1) / RM) * p.feature_tiles;
    if (split == 0 && tiles < cus && round_tiles <= cus) {
        p.tile_rows = RM;
        p.token_tiles = (int32_t)((n + RM - 1) / RM);
        p.whole_tiles = round_tiles;
        return p;
    }
    p.whole_tiles = split ? tiles - rem : tiles;
    p.part_rows = split ? BM / split : 0;
    p.parts = split ? rem * split : 0;
    return p;
}

hipError_t launch_proj_cond_bf16(const ProjCondArgs& a, const CamTable& cams, hipStream_t s) {
    const p3d_tile_plan plan = plan_proj_cond_bf16(a.n, a.D, device_cus());
    int32_t m_tiles = plan.token_tiles;
    int32_t n_tiles = plan.feature_tiles;
    int32_t null_tiles = (int32_t)((a.n_null + plan.tile_rows - 1) / plan.tile_rows);
    // corner offsets fit 32 bits when every map is under 4 GiB
    const auto map_bytes = [&](int32_t H, int32_t W, int32_t C) {
        return (uint64_t)a.batch * (uint64_t)H * (uint64_t)W * (uint64_t)C * 2u;
    };
    const bool off32 = map_bytes(a.H, a.W, a.C) < ((uint64_t)1 << 32) &&
                       (a.C1 == 0 || map_bytes(a.H1, a.W1, a.C1) < ((uint64_t)1 << 32));
    using yes = std::true_type;
    using no = std::false_type;
    ProjCondArgs args = a;
    CamTable tab = cams;
    if (plan.tile_rows != BM) {
        // one round of 96-token tiles
        int32_t tiles = plan.whole_tiles;
        int32_t per_xcd = (tiles + 7) / 8;
        void* params[] = {&args, &tab, &m_tiles, &n_tiles, &tiles, &per_xcd, &null_tiles};
        const auto pick = [&](auto two_maps, auto o32) -> const void* {
            constexpr bool T = decltype(two_maps)::value, O = decltype(o32)::value;
            return reinterpret_cast<const void*>(&proj_cond_bf16_round_kernel<T, O>);
        };
        const void* fn = a.C1 > 0 ? (off32 ? pick(yes{}, yes{}) : pick(yes{}, no{}))
                                  : (off32 ? pick(no{}, yes{}) : pick(no{}, no{}));
        return hipLaunchKernel(fn, dim3((unsigned)per_xcd * 8), dim3(kThreads), params, 0, s);
    }
    int32_t n_big = plan.whole_tiles;
    int32_t n_small = plan.parts;
    int32_t big_per_xcd = (n_big + 7) / 8;
    int32_t small_per_xcd = (n_small + 7) / 8;
    void* params[] = {&args,    &tab,        &m_tiles,       &n_tiles,   &n_big,
                      &big_per_xcd, &n_small, &small_per_xcd, &null_tiles};
    const bool half = plan.part_rows == 16 * TI_HALF;
    const auto pick = [&](auto two_maps, auto o32) -> const void* {
        constexpr bool T = decltype(two_maps)::value, O = decltype(o32)::value;
        return half ? reinterpret_cast<const void*>(&proj_cond_bf16_kernel<T, O, TI_HALF>)
                    : reinterpret_cast<const void*>(&proj_cond_bf16_kernel<T, O, TI_QUARTER>);
    };
    const void* fn = a.C1 > 0 ? (off32 ? pick(yes{}, yes{}) : pick(yes{}, no{}))
                              : (off32 ? pick(no{}, yes{}) : pick(no{}, no{}));
    return hipLaunchKernel(fn, dim3((unsigned)(big_per_xcd + small_per_xcd) * 8), dim3(kThreads),
                           params, 0, s);
}

}  // namespace p3d
