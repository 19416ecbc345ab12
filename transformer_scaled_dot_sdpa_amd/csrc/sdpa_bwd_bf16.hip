// Backward of the fused bf16 attention for gfx950 (CDNA4) matrix cores.
//
// For a loss L with dL/dO = dO, and P = softmax(S), S = Q K^T / sqrt(d)
// (eq. (1) of "Aufmerksamkeit ist alles, was Sie brauchen", section 3.2.1),
// the proof section (証明) of the formula page "トランスフォーマーの注意機構"
// gives everything needed:
//   output display  O = P V          ->  dV = P^T dO,   dP = dO V^T
//   Jacobian display da_j/ds_l = a_j (delta_jl - a_l)
//                                    ->  dS = P o (dP - D),  D_i = sum_j P_ij dP_ij
//                                                               = sum_t dO_it O_it
//   score display   s = q.k / sqrt(d) ->  dQ = dS K / sqrt(d), dK = dS^T Q / sqrt(d)
// P is recomputed from S and the forward's log-sum-exp (P = exp(S - lse)),
// so no score matrix is stored.
//
// Two kernels:
//   bwd_dq      per block of 128 query rows (32 per wavefront): first
//               D = rowsum(dO o O) of the wavefront's rows (fp32, also
//               written out for the next kernel), then stream K and V tiles
//               of 64 keys through LDS and accumulate
//               dQ^T += K^T dS^T  after  S^T = K Q^T, dP^T = V dO^T;
//   bwd_dkdv    per block of 128 keys (32 per wavefront): stream Q and dO
//               tiles of 64 query rows through LDS and accumulate
//               dV^T += dO^T P  and  dK^T += Q^T dS  after  S = Q K^T,
//               dP = dO V^T.  K and V of the wavefront's keys stay in
//               registers; one wavefront per SIMD holds all four products.
// All products are v_mfma_f32_32x32x16_bf16 with fp32 accumulation; P and dS
// are rounded to bf16 (RNE) as MFMA operands.  Every LDS tile has its rows
// permuted as the forward kernel's K tiles (bits 2 and 3 swapped inside each
// 32-row block) and its 16-byte chunks XOR-swizzled (t_swz): read with
// ds_read_b128 it is the row operand of S / dP, and the permutation puts the
// result of those products directly in the operand layout of the next one;
// read with ds_read_b64_tr_b16 it is the transposed operand (K^T, Q^T, dO^T).
#include "sdpa_internal.h"
#include "bf16_common.h"

#include <math.h>

namespace sdpa {
namespace {

using namespace bf16k;

struct BParams {
    const uint16_t* __restrict__ q;
    const uint16_t* __restrict__ k;
    const uint16_t* __restrict__ v;
    const uint16_t* __restrict__ o;
    const uint16_t* __restrict__ dout;
    const float* __restrict__ lse;
    float* __restrict__ delta;
    uint16_t* __restrict__ dq;
    uint16_t* __restrict__ dk;
    uint16_t* __restrict__ dv;
    const int32_t* __restrict__ key_lens;
    int H, Lq, Lk;
    int num_blocks;    // row blocks per (b, h): query blocks (dq) or key blocks (dkdv)
    int num_items;
    int upi;
    int num_units;
    int cu_pairs;      // compute units per XCD when units are renumbered in compute-unit pairs, else 0
    float scale;       // 1 / sqrt(d)
    float scale_log2;  // log2(e) / sqrt(d)
};

constexpr float kLog2e = 1.44269504088896340736f;
// dK and dV in two passes (bwd_dkdv_kernel MODE 1 and 2) rather than one
// when the single pass needs more registers than two wavefronts per SIMD
// allow (d = 128; at d = 64 the single pass already runs two per SIMD and
// is faster)
template <int D>
constexpr bool kSplitDkDv = D == 128;

// XOR swizzle of the 16-byte chunk index inside an LDS row of a backward
// tile.  Tiles here are read both ways: ds_read_b128 of one chunk from 16
// consecutive rows, and ds_read_b64_tr_b16 of 64 bytes from each of 4
// consecutive rows (aligned to 4).  The swizzle is a bijection of the row's
// low bits (rows 0..15 for D = 128; row pairs for D = 64, whose rows are half
// the 256-byte bank width), so the first pattern covers all banks; and rows
// 4m .. 4m + 3 get different values in bits 2..3 of it (D = 128; bit 2 for
// the two rows of one parity when D = 64), which moves their 64-byte pieces
// to different quarters of the banks.  It depends only on row bits 0..3.
template <int D>
__device__ __forceinline__ int t_swz(int row) {
    if (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
    const int u = (row >> 1) & 7;
    return ((u & 1) << 2) | (u >> 1);
}

// Per-lane offsets shared by both kernels (elements inside a 64-row tile:
// rows permuted as the forward's K tiles, chunks swizzled by t_swz).
template <int D>
struct TileOffsets {
    static constexpr int NKS = D / 16;
    static constexpr int NDT = D / 32;
    int rd[NKS];       // row operand: row n (physical), chunk 2ks + h
    int tr_lo[NDT];    // transposed operand, logical rows 16s + 8h + 0..3 of a 32-row block
    int tr_hi[NDT];    // logical rows 16s + 8h + 4..7
    __device__ __forceinline__ void init(int lane) {
        const int n = lane & 31, h = lane >> 5, li = lane & 15;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) rd[ks] = n * D + (((2 * ks + h) ^ t_swz<D>(n)) << 3);
        // logical row 16s + 8h + c sits at physical row 16s + 4h + c (c < 4)
        // or 16s + 8 + 4h + (c - 4); the swizzle only depends on row bits
        // below 4, so the 16s and 32-row block offsets are plain additions
        const int rr = li >> 2;
        const int colg = 16 * ((lane >> 4) & 1) + 4 * (li & 3);
        const int plo = 4 * h + rr, phi = 8 + 4 * h + rr;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const int col = dt * 32 + colg;
            tr_lo[dt] = plo * D + (((col >> 3) ^ t_swz<D>(plo)) << 3) + (col & 7);
            tr_hi[dt] = phi * D + (((col >> 3) ^ t_swz<D>(phi)) << 3) + (col & 7);
        }
    }
};

// transposed operand of rows [32 kt + 16 s, +16) of a tile, output column
// block dt: lane (n, h) gets rows 16s + 8h + 0..7 (logical) of column
// 32 dt + n
template <int D>
__device__ __forceinline__ bf16x8 read_tr(const uint16_t* T, const TileOffsets<D>& off, int kt,
                                          int s, int dt) {
    const uint16_t* base = T + (32 * kt + 16 * s) * D;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + off.tr_lo[dt]));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + off.tr_hi[dt]));
    return __builtin_bit_cast(bf16x8, i16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
}

// DMA slot offsets of the tile layout for this thread's KCH loads
template <int D, int KCH>
__device__ __forceinline__ void dma_offsets(int wave, int lane, uint32_t* boff) {
    constexpr int CPR = D / 8;
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
        const int s = (wave * KCH + u) * 64 + lane;
        const int row = s / CPR, pc = s % CPR;
        boff[u] = (k_lds_row(row) * D + ((pc ^ t_swz<D>(row)) << 3)) * 2;
    }
}

// ---------------------------------------------------------------- dQ
template <int D, bool CAUSAL, bool LENS>
__global__ void __launch_bounds__(256, 2) bwd_dq_kernel(BParams p) {
    constexpr int BC = 64, NT = 256, BR = 128;
    constexpr int CPR = D / 8;
    constexpr int KCH = BC * CPR / NT;
    constexpr int TILE = BC * D;
    constexpr int NDT = D / 32;
    constexpr int NKS = D / 16;

    __shared__ __align__(16) uint16_t k_lds0[TILE], k_lds1[TILE], v_lds0[TILE], v_lds1[TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31;
    const int h = lane >> 5;
    uint32_t boff[KCH];
    dma_offsets<D, KCH>(wave, lane, boff);
    TileOffsets<D> off;
    off.init(lane);

    int unit = workgroup_unit();
    if (CAUSAL && p.cu_pairs > 0) unit = cu_pair_unit(p.cu_pairs, unit);
    for (int item = unit * p.upi; item < min(unit * p.upi + p.upi, p.num_items); ++item) {
    int bh, qb;
    item_block<CAUSAL>(item, p.num_blocks, &bh, &qb);
    const int b = bh / p.H;
    const int q0 = qb * BR;
    int kv_len = p.Lk;
    if (LENS) {
        int L = p.key_lens[b];
        L = L < 0 ? 0 : L;
        kv_len = L < kv_len ? L : kv_len;
    }
    const int kv_end = CAUSAL ? min(kv_len, q0 + BR) : kv_len;
    const int ntiles = (kv_end + BC - 1) / BC;
    const int q0w = q0 + wave * 32;
    const int qrow = q0w + n;
    const int wave_kv_end = CAUSAL ? min(kv_len, q0w + 32) : kv_len;
    const size_t q_base = (size_t)bh * p.Lq * D;
    const uint16_t* kg = p.k + (size_t)bh * p.Lk * D;
    const uint16_t* vg = p.v + (size_t)bh * p.Lk * D;
    const uint32_t kv_bytes = (uint32_t)kv_len * D * 2;

    // Q and dO of the wavefront's rows as B operands (rows past Lq load the
    // last row; their results are never stored)
    const int qr = qrow < p.Lq ? qrow : p.Lq - 1;
    bf16x8 qf[NKS], df[NKS];
    {
        const i16x8* sq = reinterpret_cast<const i16x8*>(p.q + q_base + (size_t)qr * D + 8 * h);
        const i16x8* sd = reinterpret_cast<const i16x8*>(p.dout + q_base + (size_t)qr * D + 8 * h);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            qf[ks] = __builtin_bit_cast(bf16x8, sq[2 * ks]);
            df[ks] = __builtin_bit_cast(bf16x8, sd[2 * ks]);
        }
    }
    const float lse2 = p.lse[(size_t)bh * p.Lq + qr] * kLog2e;
    const bool row_ok = qrow < p.Lq;
    // D = dO . O of the row, in fp32: this lane holds half of the row's dO
    // (the B-operand chunks) and reads the matching half of O; a bf16 value
    // widens to fp32 by placing its bits in the high half.  Written out for
    // the dK/dV kernels, which run after this one.
    float dl;
    {
        const uint4* so = reinterpret_cast<const uint4*>(p.o + q_base + (size_t)qr * D + 8 * h);
        float part = 0.f;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const uint4 a = so[2 * ks];
            const uint4 g = __builtin_bit_cast(uint4, df[ks]);
            const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, gw[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                part = fmaf(__uint_as_float(aw[e] << 16), __uint_as_float(gw[e] << 16), part);
                part = fmaf(__uint_as_float(aw[e] & 0xffff0000u), __uint_as_float(gw[e] & 0xffff0000u), part);
            }
        }
        dl = sum_across_halves(part);
        if (row_ok && h == 0) p.delta[(size_t)bh * p.Lq + qrow] = dl;
    }

    auto issue_loads = [&](int t, uint16_t* kb, uint16_t* vb) __attribute__((always_inline)) {
        const uint32_t toff = (uint32_t)(t * BC) * D * 2;
#pragma unroll
        for (int u = 0; u < KCH; ++u) {
            buffer_load_lds16(kg, kv_bytes, (lds_void*)(kb + (wave * KCH + u) * 64 * 8), boff[u], toff);
            buffer_load_lds16(vg, kv_bytes, (lds_void*)(vb + (wave * KCH + u) * 64 * 8), boff[u], toff);
        }
    };

    f32x16 acc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;

    auto tile = [&](int t, const uint16_t* Ks, const uint16_t* Vs) __attribute__((always_inline)) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            const int kbase = t * BC + 32 * kt;
            if (kbase >= wave_kv_end) continue;
            f32x16 s, dp;
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Ks + kt * 32 * D + off.rd[ks]);
                const bf16x8 va = *reinterpret_cast<const bf16x8*>(Vs + kt * 32 * D + off.rd[ks]);
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, df[ks], dp, 0, 0, 0);
            }
            // dS^T = P^T o (dP^T - D): accumulator r of lane (n, h) is key
            // kbase + 16(r/8) + 8h + r%8 of query row n
            // weights; the masks (rows past Lq, keys past the key length,
            // the causal diagonal) run as one block, only on sub-tiles that
            // cross a boundary (a masked weight is replaced, never used, so
            // the infinite exponential of a row without keys does no harm)
            const bool full = q0w + 32 <= p.Lq && kbase + 32 <= kv_len && (!CAUSAL || kbase + 31 <= q0w);
            float pv[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) pv[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], p.scale_log2, -lse2));
            if (!full) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kbase + 16 * (r >> 3) + 8 * h + (r & 7);
                    bool ok = row_ok && key < kv_len;
                    if (CAUSAL) ok = ok && key <= qrow;
                    pv[r] = ok ? pv[r] : 0.f;
                }
            }
            bf16x8 pb[2];
#pragma unroll
            for (int r = 0; r < 16; ++r) pb[r >> 3][r & 7] = (__bf16)(pv[r] * (dp[r] - dl));
            // dQ^T += K^T dS^T
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
                    acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_tr<D>(Ks, off, kt, st, dt), pb[st],
                                                                      acc[dt], 0, 0, 0);
        }
    };

    if (ntiles > 0) {
        issue_loads(0, k_lds0, v_lds0);
        for (int t = 0; t < ntiles; t += 2) {
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            __syncthreads();
            if (t + 1 < ntiles) issue_loads(t + 1, k_lds1, v_lds1);
            tile(t, k_lds0, v_lds0);
            if (t + 1 >= ntiles) break;
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            __syncthreads();
            if (t + 2 < ntiles) issue_loads(t + 2, k_lds0, v_lds0);
            tile(t + 1, k_lds1, v_lds1);
        }
    }

    // dQ = (dS K) / sqrt(d), stored as whole rows through the K buffers
    // (two wavefronts' 32 x D blocks each), free once every wavefront has
    // passed the barrier
    __syncthreads();
    store_rows_bf16<D>(acc, p.scale, (lds_u16*)((wave >> 1) ? k_lds1 : k_lds0) + (wave & 1) * 32 * D,
                       p.dq + q_base + (size_t)q0w * D, D, p.Lq - q0w, lane);
    __syncthreads();
    }
}

// ---------------------------------------------------------------- dK, dV
// MODE 0: dK and dV in one pass (all four products; one wavefront per SIMD).
// MODE 1: dV only (S, P, dV).  MODE 2: dK only (S, dP, dS, dK).  The two
// single passes recompute S once more but need half the registers each, so
// two wavefronts share every SIMD.
template <int D, bool CAUSAL, bool LENS, int MODE>
__global__ void __launch_bounds__(256, MODE == 0 ? 1 : 2) bwd_dkdv_kernel(BParams p) {
    constexpr bool DO_DV = MODE != 2, DO_DK = MODE != 1;
    constexpr int BQ = 64, NT = 256, BK = 128;
    constexpr int CPR = D / 8;
    constexpr int KCH = BQ * CPR / NT;
    constexpr int TILE = BQ * D;
    constexpr int NDT = D / 32;
    constexpr int NKS = D / 16;

    __shared__ __align__(16) uint16_t q_lds0[TILE], q_lds1[TILE], g_lds0[TILE], g_lds1[TILE];
    __shared__ __align__(16) float st_lds[2][2][BQ];   // [buffer][lse*log2e, D][row]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31;
    const int h = lane >> 5;
    uint32_t boff[KCH];
    dma_offsets<D, KCH>(wave, lane, boff);
    TileOffsets<D> off;
    off.init(lane);

    int unit = workgroup_unit();
    if (CAUSAL && p.cu_pairs > 0) unit = cu_pair_unit(p.cu_pairs, unit);
    for (int item = unit * p.upi; item < min(unit * p.upi + p.upi, p.num_items); ++item) {
    int bh, kb;
    item_block<CAUSAL>(item, p.num_blocks, &bh, &kb);
    // causal: the lowest key blocks see the most query rows
    if (CAUSAL) kb = p.num_blocks - 1 - kb;
    const int b = bh / p.H;
    const int k0 = kb * BK;
    int kv_len = p.Lk;
    if (LENS) {
        int L = p.key_lens[b];
        L = L < 0 ? 0 : L;
        kv_len = L < kv_len ? L : kv_len;
    }
    const int k0w = k0 + wave * 32;
    const int key = k0w + n;
    // query tiles that can see a key of this block: causal queries i >= k0
    const int ntq = (p.Lq + BQ - 1) / BQ;
    const int t0 = CAUSAL ? k0 / BQ : 0;
    const int t_end = k0 < kv_len ? ntq : t0;   // no valid key in the block: nothing to do
    const size_t q_base = (size_t)bh * p.Lq * D;
    const size_t kv_base = (size_t)bh * p.Lk * D;
    const uint16_t* qg = p.q + q_base;
    const uint16_t* gg = p.dout + q_base;
    const uint32_t q_bytes = (uint32_t)p.Lq * D * 2;
    const float* lse_g = p.lse + (size_t)bh * p.Lq;
    const float* dl_g = p.delta + (size_t)bh * p.Lq;

    const int kr = key < p.Lk ? key : p.Lk - 1;
    bf16x8 kf[NKS], vf[NKS];
    {
        const i16x8* sk = reinterpret_cast<const i16x8*>(p.k + kv_base + (size_t)kr * D + 8 * h);
        const i16x8* sv = reinterpret_cast<const i16x8*>(p.v + kv_base + (size_t)kr * D + 8 * h);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            kf[ks] = __builtin_bit_cast(bf16x8, sk[2 * ks]);
            if constexpr (DO_DK) vf[ks] = __builtin_bit_cast(bf16x8, sv[2 * ks]);
        }
    }
    const bool key_ok = key < kv_len;

    // per-row statistics of a query tile, loaded by the first 128 threads
    // into registers and stored to LDS before the barrier that opens the
    // tile: the lse and D.  With dK (S_START) the lse is stored as
    // -lse / scale (raw score units) and is the starting value of the S
    // product, so that the accumulator over the scale is the exponent of P
    // and the registers of a separate lse vector stay free for the dK pass;
    // the dV-only pass stores lse in exp2 units and subtracts it, which
    // keeps the LDS read off the path to its first product.  dP starts from
    // zero and D is subtracted afterwards: with one valid key dP and D are
    // then the same fp32 dot product and dS is exactly zero.  The load is
    // consumed only at the store: any arithmetic on it right after the load
    // would make the wavefront wait for all its loads in flight, the next
    // tile's included.
    constexpr bool S_START = DO_DK;
    float stat = 0.f;
    const float stat_mul = tid < BQ ? (S_START ? -1.f / p.scale : kLog2e) : 1.f;
    auto stat_load = [&](int t) __attribute__((always_inline)) {
        if (tid < 2 * BQ) {
            int row = t * BQ + (tid & (BQ - 1));
            row = row < p.Lq ? row : p.Lq - 1;
            stat = tid < BQ ? lse_g[row] : dl_g[row];
        }
    };
    auto stat_store = [&](int buf) __attribute__((always_inline)) {
        if (tid < 2 * BQ) st_lds[buf][tid / BQ][tid & (BQ - 1)] = stat * stat_mul;
    };
    auto issue_loads = [&](int t, uint16_t* qb, uint16_t* gb) __attribute__((always_inline)) {
        const uint32_t toff = (uint32_t)(t * BQ) * D * 2;
#pragma unroll
        for (int u = 0; u < KCH; ++u) {
            buffer_load_lds16(qg, q_bytes, (lds_void*)(qb + (wave * KCH + u) * 64 * 8), boff[u], toff);
            buffer_load_lds16(gg, q_bytes, (lds_void*)(gb + (wave * KCH + u) * 64 * 8), boff[u], toff);
        }
    };

    f32x16 dka[NDT], dva[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) dka[dt][r] = dva[dt][r] = 0.f;

    auto tile = [&](int t, const uint16_t* Qs, const uint16_t* Gs, int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            const int qbase = t * BQ + 32 * qt;
            // causal: rows of this sub-tile all before the wavefront's first key
            if (CAUSAL && qbase + 31 < k0w) continue;
            if (qbase >= p.Lq) continue;
            // accumulator r of lane (n, h) is query row qbase + 16(r/8) + 8h +
            // r%8 against key `key`; the row statistics of rows 16j + 8h +
            // 0..7 are read as vectors
            f32x16 s, dp;
            float lsv[16];
            auto read_lse = [&](float* dst) __attribute__((always_inline)) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const float4* s0 = reinterpret_cast<const float4*>(&st_lds[buf][0][32 * qt + 16 * j + 8 * h]);
                    const float4 u0 = s0[0], u1 = s0[1];
                    const float uu[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) dst[8 * j + e] = uu[e];
                }
            };
            if constexpr (S_START) {
                float st[16];
                read_lse(st);
#pragma unroll
                for (int r = 0; r < 16; ++r) s[r] = st[r];
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if constexpr (!S_START) s[r] = 0.f;
                dp[r] = 0.f;
            }
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const bf16x8 qa = *reinterpret_cast<const bf16x8*>(Qs + qt * 32 * D + off.rd[ks]);
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[ks], s, 0, 0, 0);
                if constexpr (DO_DK) {
                    const bf16x8 ga = *reinterpret_cast<const bf16x8*>(Gs + qt * 32 * D + off.rd[ks]);
                    dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, vf[ks], dp, 0, 0, 0);
                }
            }
            // (the dV-only pass reads the lse here, after its products)
            if constexpr (!S_START) read_lse(lsv);
            // D of the same rows, read as vectors before any use so that no
            // load sits under a mask
            float dlv[16];
            if constexpr (DO_DK) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const float4* s1 = reinterpret_cast<const float4*>(&st_lds[buf][1][32 * qt + 16 * j + 8 * h]);
                    const float4 w0 = s1[0], w1 = s1[1];
                    const float ww[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) dlv[8 * j + e] = ww[e];
                }
            }
            // every (row, key) pair of the sub-tile valid: no masking
            const bool full = qbase + 32 <= p.Lq && k0w + 32 <= kv_len && (!CAUSAL || qbase >= k0w + 31);
            // the masks run as one block after the exponentials, only on
            // sub-tiles that cross a boundary
            float pv[16];
#pragma unroll
            for (int r = 0; r < 16; ++r)
                pv[r] = __builtin_amdgcn_exp2f(S_START ? s[r] * p.scale_log2
                                                       : __builtin_fmaf(s[r], p.scale_log2, -lsv[r]));
            if (!full) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int qrow = qbase + 16 * (r >> 3) + 8 * h + (r & 7);
                    bool ok = key_ok && qrow < p.Lq;
                    if (CAUSAL) ok = ok && key <= qrow;
                    pv[r] = ok ? pv[r] : 0.f;
                }
            }
            bf16x8 pb[2], sb[2];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if constexpr (DO_DV) pb[r >> 3][r & 7] = (__bf16)pv[r];
                if constexpr (DO_DK) sb[r >> 3][r & 7] = (__bf16)(pv[r] * (dp[r] - dlv[r]));
            }
            // dV^T += dO^T P,  dK^T += Q^T dS
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    if constexpr (DO_DV)
                        dva[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_tr<D>(Gs, off, qt, st, dt),
                                                                          pb[st], dva[dt], 0, 0, 0);
                    if constexpr (DO_DK)
                        dka[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_tr<D>(Qs, off, qt, st, dt),
                                                                          sb[st], dka[dt], 0, 0, 0);
                }
        }
    };

    if (t0 < t_end) {
        issue_loads(t0, q_lds0, g_lds0);
        stat_load(t0);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        stat_store(0);
        for (int t = t0; t < t_end; t += 2) {
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            __syncthreads();
            if (t + 1 < t_end) {
                issue_loads(t + 1, q_lds1, g_lds1);
                stat_load(t + 1);
            }
            tile(t, q_lds0, g_lds0, 0);
            if (t + 1 >= t_end) break;
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            stat_store(1);
            __syncthreads();
            if (t + 2 < t_end) {
                issue_loads(t + 2, q_lds0, g_lds0);
                stat_load(t + 2);
            }
            tile(t + 1, q_lds1, g_lds1, 1);
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            stat_store(0);
        }
    }

    // dK = dS^T Q / sqrt(d) and dV = P^T dO, stored as whole rows (keys)
    // through the Q buffers (dK) and the dO buffers (dV), two wavefronts'
    // 32 x D blocks each, free once every wavefront has passed the barrier
    __syncthreads();
    if constexpr (DO_DK)
        store_rows_bf16<D>(dka, p.scale, (lds_u16*)((wave >> 1) ? q_lds1 : q_lds0) + (wave & 1) * 32 * D,
                           p.dk + kv_base + (size_t)k0w * D, D, p.Lk - k0w, lane);
    if constexpr (DO_DV)
        store_rows_bf16<D>(dva, 1.f, (lds_u16*)((wave >> 1) ? g_lds1 : g_lds0) + (wave & 1) * 32 * D,
                           p.dv + kv_base + (size_t)k0w * D, D, p.Lk - k0w, lane);
    __syncthreads();
    }
}

template <int D, bool CAUSAL, bool LENS>
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
    BParams p;
    p.q = static_cast<const uint16_t*>(a.q);
    p.k = static_cast<const uint16_t*>(a.k);
    p.v = static_cast<const uint16_t*>(a.v);
    p.o = static_cast<const uint16_t*>(a.out);
    p.dout = static_cast<const uint16_t*>(a.dout);
    p.lse = a.lse;
    p.delta = a.delta;
    p.dq = static_cast<uint16_t*>(a.dq);
    p.dk = static_cast<uint16_t*>(a.dk);
    p.dv = static_cast<uint16_t*>(a.dv);
    p.key_lens = a.key_lens;
    p.H = a.H;
    p.Lq = a.Lq;
    p.Lk = a.Lk;
    p.scale = (float)(1.0 / sqrt((double)D));
    p.scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));

    // causal work runs as long/short pairs of items once the items
    // outnumber the resident workgroups (2 per CU), except below 1.25 slots'
    // worth of items, where pairs would leave slots idle
    // (causal_items_per_unit); a smaller problem takes one item per
    // workgroup so that every item starts at once, renumbered so that a
    // compute unit holding two runs a long and a short one (cu_pair_unit;
    // the query or key blocks of a slice alternate long and short, and an
    // even count keeps the alternation aligned)
    const int cus = a.num_cus > 0 ? a.num_cus : 256;
    const long long slots = (long long)cus * 2;
    const long long single_max = (5 * slots - 1) / 4;
    auto cu_pairs_for = [&](long long items) {
        return (CAUSAL && p.upi == 1 && items <= slots && items > cus && p.num_blocks % 2 == 0 && cus % 8 == 0)
                   ? cus / 8 : 0;
    };
    {
        p.num_blocks = (a.Lq + 127) / 128;
        const long long items = (long long)p.num_blocks * a.B * a.H;
        if (items > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        p.num_items = (int)items;
        p.upi = CAUSAL ? causal_items_per_unit(items, slots, single_max, 0, 0) : 1;
        p.num_units = (int)((items + p.upi - 1) / p.upi);
        p.cu_pairs = cu_pairs_for(items);
        hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, LENS>), dim3((unsigned)p.num_units), dim3(256), 0,
                           stream, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    {
        p.num_blocks = (a.Lk + 127) / 128;
        const long long items = (long long)p.num_blocks * a.B * a.H;
        if (items > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        p.num_items = (int)items;
        p.upi = CAUSAL ? causal_items_per_unit(items, slots, single_max, 0, 0) : 1;
        p.num_units = (int)((items + p.upi - 1) / p.upi);
        p.cu_pairs = cu_pairs_for(items);
        if constexpr (kSplitDkDv<D>) {
            hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, LENS, 1>), dim3((unsigned)p.num_units), dim3(256), 0,
                               stream, p);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, LENS, 2>), dim3((unsigned)p.num_units), dim3(256), 0,
                               stream, p);
        } else {
            hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, LENS, 0>), dim3((unsigned)p.num_units), dim3(256), 0,
                               stream, p);
        }
        return hipGetLastError();
    }
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t s) {
    const bool lens = a.key_lens != nullptr;
    if (a.causal) return lens ? launch_bwd<D, true, true>(a, s) : launch_bwd<D, true, false>(a, s);
    return lens ? launch_bwd<D, false, true>(a, s) : launch_bwd<D, false, false>(a, s);
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t s) {
    if (a.d == 128) return launch_bwd_d<128>(a, s);
    if (a.d == 64) return launch_bwd_d<64>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace sdpa
