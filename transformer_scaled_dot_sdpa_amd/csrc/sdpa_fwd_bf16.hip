// Fused scaled dot-product attention forward, bf16 in / fp32 accumulate,
// for gfx950 (CDNA4) matrix cores.
//
// Computes, for every (batch, head) slice, eq. (1) of "Aufmerksamkeit ist
// alles, was Sie brauchen", section 3.2.1:  O = softmax(Q K^T / sqrt(d)) V,
// without ever writing the score matrix to memory.  Keys are streamed in
// tiles of BC; per query row a running maximum m and running sum l of the
// exponentials are kept, which is exact because softmax weights depend only
// on score differences (formula page "トランスフォーマーの注意機構", section
// 証明, the ratio identity a_j / a_i = e^{s_j - s_i}).
//
// Work decomposition
//   * one workgroup = NW wavefronts = BR = 32*NW query rows of one (b, h);
//     every wavefront owns 32 consecutive query rows;
//   * the workgroup streams K and V tiles of BC keys into LDS with direct
//     global->LDS 16-byte loads (no register staging), double buffered with
//     one barrier per tile; the loads of tile t+1 overlap the math of tile t;
//   * per tile and wavefront:
//       S^T (BC x 32)  = K_tile (BC x d) . Q_w^T (d x 32)   32x32x16 bf16 MFMA
//       online softmax over the keys (column of S^T = one query, so all of
//       a query's scores live in two lanes: n and n + 32)
//       O^T (d x 32)  += V_tile^T (d x BC) . P^T (BC x 32)  32x32x16 bf16 MFMA
//     Computing the transposed products keeps each query's running max/sum
//     and its whole output column inside one lane pair, so the rescale of O
//     is a per-lane multiply and the row reductions need one cross-lane swap.
//   * key split (KS = 2): the workgroup holds two groups of NW wavefronts
//     over the same query rows; group g takes key tiles g, g + 2, g + 4, ...
//     with K/V buffers of its own, and at the end group 1 hands its (O, m, l)
//     to group 0 through LDS, which merges them as
//       m = max(m0, m1), O = 2^(m0-m) O0 + 2^(m1-m) O1, l likewise
//     (exact by the same ratio identity).  When a problem has too few query
//     blocks to fill the GPU but long key ranges (few heads, long
//     sequences), its workgroups then finish in half the tile steps.
//   * masking (causal: key j > query i; padding: j >= key length; ragged
//     tails) only runs on tiles that cross a boundary; tiles entirely above
//     the causal diagonal are neither loaded nor computed.  K/V come in with
//     buffer loads bounded at the valid key length: rows past it arrive as
//     zeros (and are masked), so padded memory is never read.
//
// MFMA operand layouts (32x32x16 bf16, lane l = n + 32*h, n < 32, h < 2):
//   A (32 x 16): lane holds A[n][8h .. 8h+7];  B (16 x 32): lane holds
//   B[8h .. 8h+7][n];  C/D (32 x 32): lane holds D[8*(r/4) + 4h + r%4][n],
//   r = 0..15.  To feed the S^T result straight back as the B operand of the
//   P.V product, the K rows are stored in LDS with bits 2 and 3 of the key
//   index swapped inside each 32-key block: then accumulator r of lane
//   (n, h) holds key 16*(r/8) + 8h + r%8, exactly the eight consecutive keys
//   the B operand wants.  V stays row-major in LDS and is read transposed
//   with ds_read_b64_tr_b16 (four keys x one column per lane and read).
#include "sdpa_internal.h"
#include "bf16_common.h"

#include <math.h>

#include <type_traits>

namespace sdpa {
namespace {

using namespace bf16k;

// D: width of queries and keys; DV: width of values and outputs.  MASK adds
// an fp32 bias to the scaled scores.  Tensor rows are addressed through the
// strides in KParams (contiguous or head-interleaved layouts alike).
// Tile configurations run two wavefronts per SIMD (the second
// __launch_bounds__ argument, which caps a wavefront at 256 registers),
// except the d64 key split and d64 8-wavefront tiles, which fit four (128
// registers, V operands read one key step ahead): 4 * waves-per-SIMD /
// (NW * KS) workgroups per compute unit, at least one.
template <int D, int NW, int KS>
constexpr int fwd_waves_per_simd() {
    return (D == 64 && (KS == 2 || NW == 8)) ? 4 : 2;
}
template <int D, int NW, int KS>
constexpr int fwd_blocks_per_cu() {
    return 4 * fwd_waves_per_simd<D, NW, KS>() / (NW * KS) > 0 ? 4 * fwd_waves_per_simd<D, NW, KS>() / (NW * KS)
                                                                 : 1;
}

template <int D, int DV, int BC, int NW, int KS, bool CAUSAL, bool LENS, bool MASK>
__global__ void __launch_bounds__(NW * KS * 64, (fwd_waves_per_simd<D, NW, KS>()))
fwd_bf16_kernel(KParams p) {
    static_assert(KS == 1 || KS == 2, "key split of 1 or 2 groups");
    constexpr int NT = NW * 64;                // threads of one group
    constexpr int BR = NW * 32;
    constexpr int CPR = D / 8;                 // 16-byte chunks per key row
    constexpr int CPRV = DV / 8;               // 16-byte chunks per value row
    constexpr int KCH = BC * CPR / NT;         // 16-byte K loads per thread per tile
    constexpr int KCHV = BC * CPRV / NT;       // 16-byte V loads per thread per tile
    constexpr int TILE = BC * D;               // elements per K tile
    constexpr int TILEV = BC * DV;             // elements per V tile
    constexpr int NKT = BC / 32;               // 32-key sub-tiles
    constexpr int NDT = DV / 32;               // 32-wide output column tiles
    constexpr int NKS = D / 16;                // k-steps of the Q.K^T product
    static_assert((BC * CPR) % NT == 0 && (BC * CPRV) % NT == 0, "tile must split evenly over threads");
    static_assert(BC % 32 == 0, "BC must be a multiple of 32");

    // K and V tiles, double buffered (one pair of buffers per key-split
    // group).  Four separate arrays rather than one: the compiler can then
    // tell that the direct-to-LDS loads into one buffer never alias the
    // reads of the other, and does not make those reads wait for the loads
    // in flight (the tile barrier provides the real ordering).
    __shared__ __align__(16) uint16_t k_lds0[KS * TILE], k_lds1[KS * TILE], v_lds0[KS * TILEV],
        v_lds1[KS * TILEV];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave indices are uniform: keep them in scalar registers.  grp: key-split
    // group; wave: wavefront inside the group (its 32 query rows).
    const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = KS == 1 ? 0 : __builtin_amdgcn_readfirstlane(wave_all / NW);
    const int wave = KS == 1 ? wave_all : __builtin_amdgcn_readfirstlane(wave_all - grp * NW);
    // this group's K/V buffers
    uint16_t* const kb0 = k_lds0 + grp * TILE;
    uint16_t* const kb1 = k_lds1 + grp * TILE;
    uint16_t* const vb0 = v_lds0 + grp * TILEV;
    uint16_t* const vb1 = v_lds1 + grp * TILEV;
    const int n = lane & 31;   // query column inside the wave
    const int h = lane >> 5;   // which half of the 16-wide k slice

    // ---- direct global -> LDS loads.  Load u of this thread fills LDS slot
    // s = (wave*KCH + u)*64 + lane of the tile (16 bytes each).  The slot's
    // (row, physical chunk) is fixed; the global source is chosen so that the
    // swizzled / key-permuted layout comes out in LDS.  Buffer loads take the
    // tile offset in a scalar register and the per-lane offset from a fixed
    // register; the buffer ends at the valid key length, so rows past it
    // arrive as zeros without being read.
    uint32_t k_boff[KCH], v_boff[KCHV];
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
        const int s = (wave * KCH + u) * 64 + lane;
        const int row = s / CPR, pc = s % CPR;
        k_boff[u] = (k_lds_row(row) * p.k_sl + ((pc ^ k_swz<D>(row)) << 3)) * 2;
    }
#pragma unroll
    for (int u = 0; u < KCHV; ++u) {
        const int s = (wave * KCHV + u) * 64 + lane;
        const int row = s / CPRV, pc = s % CPRV;
        v_boff[u] = (row * p.v_sl + ((pc ^ v_swz<DV>(row)) << 3)) * 2;
    }
    // ---- per-lane LDS read offsets (elements) inside a tile
    // K operand: row kt*32 + n, chunk (2ks + h) ^ swz  -> one base per ks,
    // kt adds 32 rows.
    int k_rd[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) k_rd[ks] = n * D + (((2 * ks + h) ^ k_swz<D>(n)) << 3);
    // V operand (transposed read): rows kt*32 + 16ksl + 8h + 4r + li/4, column
    // dt*32 + 16*((lane>>4)&1) + 4*(li&3).  The swizzle depends on row & 3,
    // which the kt / ksl / r steps (multiples of 4) leave unchanged, so one
    // base per dt suffices.
    const int li = lane & 15;
    int v_rd[NDT];
    {
        const int row = 8 * h + (li >> 2);
        const int colg = 16 * ((lane >> 4) & 1) + 4 * (li & 3);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const int col = dt * 32 + colg;
            v_rd[dt] = row * DV + (((col >> 3) ^ v_swz<DV>(row)) << 3) + (col & 7);
        }
    }

    // ---- key-length pairs: rank the batches by clamped key length (longest
    // first, ties by index) in LDS; position r of the order holds batch
    // s_order[r].  Every workgroup ranks the (few) lengths itself.
    __shared__ int s_len[LENS ? kMaxPairBatches : 1], s_order[LENS ? kMaxPairBatches : 1];
    if (LENS && p.lens_pairs) {
        for (int i = tid; i < p.B; i += NT * KS) {
            const int L = p.key_lens[i];
            s_len[i] = L < 0 ? 0 : (L > p.Lk ? p.Lk : L);
        }
        __syncthreads();
        for (int i = tid; i < p.B; i += NT * KS) {
            const int li = s_len[i];
            int r = 0;
            for (int j = 0; j < p.B; ++j) r += (s_len[j] > li) || (s_len[j] == li && j < i);
            s_order[r] = i;
        }
        __syncthreads();
    }

    // ---- the workgroup's work items, one after the other (see
    // workgroup_unit and item_block for the schedule and the order)
    int unit = workgroup_unit();
    if (p.cu_pairs > 0) unit = cu_pair_unit(p.cu_pairs, unit);
    for (int k_item = 0; k_item < p.upi; ++k_item) {
    int item;
    if (LENS && p.lens_pairs == 1) {
        // items u and num_items - 1 - u: a long one and a short one
        item = k_item == 0 ? unit : p.num_items - 1 - unit;
        if (k_item == 1 && item <= unit) break;   // the middle item of an odd count runs once
    } else if (LENS && p.lens_pairs == 2) {
        // one item per unit, in length-rank order interleaved from both
        // ends: units 2k and 2k + 1 (one compute unit, see cu_pair_unit)
        // take the k-th longest and the k-th shortest item
        item = (unit & 1) ? p.num_items - 1 - (unit >> 1) : (unit >> 1);
    } else {
        item = unit * p.upi + k_item;
        if (item >= p.num_items) break;
    }
    int bh, qb;
    if (LENS && p.lens_pairs) {
        // item = position in the length ranking: batch s_order[r]
        const int per_b = p.H * p.num_qb;
        const int r = item / per_b, rem = item - r * per_b;
        const int hq = rem / p.num_qb;
        bh = s_order[r] * p.H + hq;
        qb = rem - hq * p.num_qb;
    } else {
        item_block<CAUSAL>(item, p.num_qb, &bh, &qb);
    }
    const int b = bh / p.H;
    const int hh = bh - b * p.H;
    const int q0 = qb * BR;

    int kv_len = p.Lk;
    if (LENS && p.lens_pairs) {
        kv_len = s_len[b];   // already clamped, and in LDS: no second trip to memory
    } else if (LENS) {
        int L = p.key_lens[b];
        L = L < 0 ? 0 : L;
        kv_len = L < kv_len ? L : kv_len;
    }
    const int kv_end = CAUSAL ? min(kv_len, q0 + BR) : kv_len;
    const int ntiles = (kv_end + BC - 1) / BC;
    // tile steps of the workgroup; in step r group g takes tile r * KS + g
    const int nsteps = (ntiles + KS - 1) / KS;

    const int q0w = q0 + wave * 32;
    const int qrow = q0w + n;
    const int wave_kv_end = CAUSAL ? min(kv_len, q0w + 32) : kv_len;

    const uint16_t* qg = p.q + b * p.q_sb + hh * p.q_sh;
    const uint16_t* kg = p.k + b * p.k_sb + hh * p.k_sh;
    const uint16_t* vg = p.v + b * p.v_sb + hh * p.v_sh;

    // ---- Q^T operand fragments, kept in registers for the whole loop.  Rows
    // past Lq load the last valid row; their results are never stored.
    bf16x8 qf[NKS];
    {
        const int qr = qrow < p.Lq ? qrow : p.Lq - 1;
        const i16x8* src = reinterpret_cast<const i16x8*>(qg + (size_t)qr * p.q_sl + 8 * h);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, src[2 * ks]);
    }

    // rows at or past kv_len start at or past these byte counts
    const uint32_t k_bytes = (uint32_t)kv_len * p.k_sl * 2;
    const uint32_t v_bytes = (uint32_t)kv_len * p.v_sl * 2;
    // Load u of K or V tile t into LDS buffer buf.  t < 0 asks for nothing:
    // the buffer then has zero length and the load only writes zeros into a
    // buffer no wavefront reads any more (so the instruction needs no branch
    // around it and the surrounding MFMA code stays one block).
    auto load_k = [&](int t, int buf, int u) __attribute__((always_inline)) {
        const uint32_t toff = (uint32_t)((t < 0 ? 0 : t) * BC) * p.k_sl * 2;
        lds_void* kd = (lds_void*)((buf ? kb1 : kb0) + (wave * KCH + u) * 64 * 8);
        buffer_load_lds16(kg, t < 0 ? 0u : k_bytes, kd, k_boff[u], toff);
    };
    auto load_v = [&](int t, int buf, int u) __attribute__((always_inline)) {
        const uint32_t toff = (uint32_t)((t < 0 ? 0 : t) * BC) * p.v_sl * 2;
        lds_void* vd = (lds_void*)((buf ? vb1 : vb0) + (wave * KCHV + u) * 64 * 8);
        buffer_load_lds16(vg, t < 0 ? 0u : v_bytes, vd, v_boff[u], toff);
    };
    auto issue_loads = [&](int t, int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < KCH; ++u) load_k(t, buf, u);
#pragma unroll
        for (int u = 0; u < KCHV; ++u) load_v(t, buf, u);
    };

    // additive mask of this slice: a buffer over rows [0, Lq) (row qrow, or
    // the last row for rows past Lq); reads past its end return zeros, and
    // keys past kv_len are masked anyway
    const float* mg = MASK ? p.mask + b * p.m_sb + hh * p.m_sh : nullptr;
    const uint32_t m_bytes = MASK ? (uint32_t)(((long long)(p.Lq - 1) * p.m_sl + p.Lk) * 4) : 0u;
    const __amdgpu_buffer_rsrc_t mrsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(mg), (short)0, (int)m_bytes, 0x00020000);
    const uint32_t m_row_off = MASK ? (uint32_t)(qrow < p.Lq ? qrow : p.Lq - 1) * p.m_sl * 4 : 0u;
    // this lane's mask values for one tile: 16 keys per 32-key sub-tile
    // (two runs of 8 consecutive keys).  The first sub-tile's values are
    // loaded one tile ahead, between the softmax and the P.V products, so
    // that they arrive under those products and the tile barrier; the
    // others at the start of their tile, under the first sub-tile's S
    // products.  (All of them one tile ahead needs 32 more registers than
    // two wavefronts per SIMD leave, and the spills cost more than the
    // latency saved: measured on MI355X.)  The mask kernels also read V
    // operands one key step ahead instead of two, for the same registers.
    constexpr int MPF = 1;   // sub-tiles whose mask values are loaded a tile ahead
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    f32x4 mb[MASK ? NKT : 1][4];
    auto load_mask = [&](int t, int kt) __attribute__((always_inline)) {
        if constexpr (MASK) {
            const int ts = t * BC;
            if (p.mask_vec) {   // 16-byte aligned rows: one 16-byte load per 4 keys
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int key = ts + kt * 32 + 16 * (j >> 1) + 8 * h + 4 * (j & 1);
                    mb[kt][j] = __builtin_bit_cast(
                        f32x4, __builtin_amdgcn_raw_buffer_load_b128(mrsrc, m_row_off + key * 4, 0, 0));
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int key = ts + kt * 32 + 16 * (j >> 1) + 8 * h + 4 * (j & 1) + e;
                        mb[kt][j][e] = __builtin_bit_cast(
                            float, __builtin_amdgcn_raw_buffer_load_b32(mrsrc, m_row_off + key * 4, 0, 0));
                    }
            }
        }
    };
    // the next tile's K/V loads and mask loads, for a tile this wavefront skips
    auto skip_tile = [&](int lt, int lb) __attribute__((always_inline)) {
        issue_loads(lt, lb);
#pragma unroll
        for (int kt = 0; kt < (MPF < NKT ? MPF : NKT); ++kt) load_mask(lt, kt);
    };

    f32x16 o[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
    float m_run = -INFINITY;  // reference maximum, exp2 units
    float l_run = 0.f;        // this lane's partial sum of weights
    bool big = false;         // a fixed-reference tile's weights reached 2^64
    const float sl = p.scale_log2;

    // One tile of 64 keys.  FAST (std::true_type) takes the exponentials
    // against the fixed reference m_run and only records, per lane, whether
    // the tile's weights reached 2^64 (or were not finite); the exact path
    // (std::false_type) maintains the running maximum as usual.
    // The loads of the next tile (lt, into buffer lb; lt < 0: none) are
    // spread over the tile's MFMAs -- K loads among the S products, V loads
    // among the P.V products -- so that no wavefront stalls on a full
    // memory-request queue, as it does when all of them issue at once.
    auto tile_math = [&](auto FAST, int t, const uint16_t* Ks, const uint16_t* Vs, int lt,
                         int lb) __attribute__((always_inline)) {
        // Without the causal mask every tile is a full one: the backend's
        // MFMA / LDS-read interleave strategy 0 measured 1-3% faster on long
        // key ranges there (d128 L4096 1.6-2.7%, d64 L2048 1%), and 0.7%
        // slower on the causal workload, which therefore keeps the default
        // schedule.
        if constexpr (!CAUSAL) __builtin_amdgcn_iglp_opt(0);
        const int ts = t * BC;
        if constexpr (MASK) {
#pragma unroll
            for (int kt = (MPF < NKT ? MPF : NKT); kt < NKT; ++kt) load_mask(t, kt);
        }
        // S^T = K Q^T, one 32-key sub-tile after the other so the softmax of
        // the first can start under the MFMAs of the second; operand reads
        // run one k-step ahead.
        f32x16 s[NKT];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kt][r] = 0.f;
            bf16x8 ka[2];
            ka[0] = *reinterpret_cast<const bf16x8*>(Ks + kt * 32 * D + k_rd[0]);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                if (ks + 1 < NKS)
                    ka[(ks + 1) & 1] = *reinterpret_cast<const bf16x8*>(Ks + kt * 32 * D + k_rd[ks + 1]);
                s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks & 1], qf[ks], s[kt], 0, 0, 0);
                // K loads u in [i*KCH/NM, (i+1)*KCH/NM) after MFMA i of NM
                constexpr int NM = NKT * NKS;
                const int i = kt * NKS + ks;
#pragma unroll
                for (int u = i * KCH / NM; u < (i + 1) * KCH / NM; ++u) load_k(lt, lb, u);
            }
            // additive mask, in raw-score units (the weights take s * sl);
            // added per sub-tile, so that its registers free up early
            if constexpr (MASK) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    s[kt][r] = __builtin_fmaf(mb[kt][r >> 2][r & 3], p.inv_scale, s[kt][r]);
            }
        }
        // masks: padding / ragged tail and the causal diagonal
        const bool need_mask = (ts + BC > kv_len) || (CAUSAL && ts + BC - 1 > q0w);
        if (need_mask) {
            // key ts + 8h + off is valid when off < lim: below kv_len and, with
            // the causal mask, at most qrow.  One bound per tile against
            // constant offsets (per-element key indices would otherwise be
            // kept in registers across the loop).
            const int lim = (CAUSAL ? min(kv_len, qrow + 1) : kv_len) - ts - 8 * h;
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int off = kt * 32 + 16 * (r >> 3) + (r & 7);
                    s[kt][r] = off < lim ? s[kt][r] : -INFINITY;
                }
        }

        // the transposed V reads of the first key steps go out before the
        // softmax, whose vector work covers their latency
        constexpr int NSTEP = 2 * NKT;
        // V operand reads run RA key steps ahead
        constexpr int RA = (MASK || fwd_waves_per_simd<D, NW, KS>() > 2) ? 1 : 2;
        constexpr int VA = RA + 1;
        i16x8 va[VA][NDT];
        auto read_v = [&](int step, i16x8* dst) __attribute__((always_inline)) {
            const int roff = (step * 16) * DV;   // step = 2*kt + ksl
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4*)(Vs + roff + v_rd[dt]));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4*)(Vs + roff + 4 * DV + v_rd[dt]));
                dst[dt] = i16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
        };
#pragma unroll
        for (int st = 0; st < RA; ++st) read_v(st, va[st]);

        bf16x8 pb[NKT][2];
        if constexpr (decltype(FAST)::value) {
            // fixed reference: weights 2^(s*sl - m_run), no maximum taken.  A
            // row whose earlier tiles were all masked (m_run still -inf: a
            // mask that drops its first keys) takes this tile's maximum as
            // its reference, exactly as the first tile does.
            if (__ballot(m_run == -INFINITY) != 0ull) {
                float mx = -INFINITY;
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
                mx = max_across_halves(mx);
                if (m_run == -INFINITY) m_run = mx * sl;
            }
            const float mref = (m_run == -INFINITY) ? 0.f : m_run;
            float lsum = 0.f;
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][r], sl, -mref));
                    lsum += pv;
                    pb[kt][r >> 3][r & 7] = (__bf16)pv;
                }
            l_run += lsum;
            big |= !(lsum < 0x1p64f);
        } else {
            // exact online softmax: running maximum, lazily raised
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
            mx = max_across_halves(mx);
            const float mt = mx * sl;
            if (__ballot(mt > m_run + kRescaleSlack) != 0ull) {
                const float mn = fmaxf(m_run, mt);
                const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - mn);
                l_run *= alpha;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
                m_run = mn;
            }
            const float mref = (m_run == -INFINITY) ? 0.f : m_run;
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    // fp32 weights feed the row sum (so lse follows the exact
                    // sum of exponentials); their bf16 roundings multiply V
                    const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][r], sl, -mref));
                    l_run += pv;
                    pb[kt][r >> 3][r & 7] = (__bf16)pv;
                }
        }

        // the next tile's mask values, now that the scores' registers are free
        if (MASK && lt >= 0) {
#pragma unroll
            for (int kt = 0; kt < (MPF < NKT ? MPF : NKT); ++kt) load_mask(lt, kt);
        }

        // O^T += V^T P^T over 2*NKT key steps of 16; the NDT output chains
        // interleave, the transposed V reads run two key steps ahead and the
        // V loads of the next tile are spread over the steps.
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) {
            if (st + RA < NSTEP) read_v(st + RA, va[(st + RA) % VA]);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
                o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, va[st % VA][dt]), pb[st >> 1][st & 1], o[dt], 0, 0, 0);
#pragma unroll
            for (int u = st * KCHV / NSTEP; u < (st + 1) * KCHV / NSTEP; ++u) load_v(lt, lb, u);
        }
    };

    // ---- main loop.  First pass: the first tile of each group sets the
    // reference maximum exactly, every later tile runs the branch-free
    // fixed-reference softmax.  If any of those tiles in the workgroup saw
    // weights >= 2^64 (scores that far above the reference), the whole
    // workgroup starts over with the exact online softmax on every tile.
    // Step r uses LDS buffer r & 1; loops are unrolled by two so the offsets
    // are constants.  In step r this group computes tile r * KS + grp (if it
    // exists and reaches this wavefront's rows) and loads tile (r+1) * KS +
    // grp (-1: none).
    auto tile_of = [&](int r) __attribute__((always_inline)) {
        const int t = r * KS + grp;
        return t < ntiles ? t : -1;
    };
    auto run_pass = [&](auto TAIL) __attribute__((always_inline)) {
        if (tile_of(0) >= 0) skip_tile(tile_of(0), 0);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        {
            const int t0 = tile_of(0);
            if (t0 >= 0 && t0 * BC < wave_kv_end)
                tile_math(std::false_type(), t0, kb0, vb0, tile_of(1), 1);
            else if (tile_of(1) >= 0) skip_tile(tile_of(1), 1);
        }
        for (int r = 1; r < nsteps; r += 2) {
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            __syncthreads();
            const int c0 = tile_of(r), l0 = r + 1 < nsteps ? tile_of(r + 1) : -1;
            if (c0 >= 0 && c0 * BC < wave_kv_end) tile_math(TAIL, c0, kb1, vb1, l0, 0);
            else if (l0 >= 0) skip_tile(l0, 0);
            if (r + 1 >= nsteps) break;
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            __syncthreads();
            const int c1 = tile_of(r + 1), l1 = r + 2 < nsteps ? tile_of(r + 2) : -1;
            if (c1 >= 0 && c1 * BC < wave_kv_end) tile_math(TAIL, c1, kb0, vb0, l1, 1);
            else if (l1 >= 0) skip_tile(l1, 1);
        }
        // zero-length loads of the last tile may still be in flight
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    };
    if (ntiles > 0) {
        run_pass(std::true_type());
        if (__syncthreads_or(big)) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
            m_run = -INFINITY;
            l_run = 0.f;
            run_pass(std::false_type());
        }
    }

    // ---- key split: group 1 hands (O, m, l) to group 0 through LDS (the
    // K/V buffers, free once every wavefront has passed the barrier below),
    // lane for lane: both groups hold the same rows in the same lanes.
    if constexpr (KS == 2) {
        constexpr int CHUNK = NW * 16 * 64;          // floats of one dt block of O
        constexpr int CAP_K = KS * TILE * 2 / (CHUNK * 4);
        constexpr int CAP_V = KS * TILEV * 2 / (CHUNK * 4);
        static_assert(2 * CAP_K + 2 * CAP_V >= NDT + 1, "LDS too small for the key-split exchange");
        // chunk c (c < NDT: O block dt = c; c = NDT: m and l) -> LDS address.
        // The pointers are typed as LDS (address space 3): through generic
        // pointers the compiler may lose the address space and emit global
        // accesses at LDS addresses.
        typedef __attribute__((address_space(3))) float lds_f32;
        auto xch = [&](int c) __attribute__((always_inline)) -> lds_f32* {
            return c < CAP_K             ? (lds_f32*)k_lds0 + c * CHUNK
                   : c < 2 * CAP_K         ? (lds_f32*)k_lds1 + (c - CAP_K) * CHUNK
                   : c < 2 * CAP_K + CAP_V ? (lds_f32*)v_lds0 + (c - 2 * CAP_K) * CHUNK
                                           : (lds_f32*)v_lds1 + (c - 2 * CAP_K - CAP_V) * CHUNK;
        };
        __syncthreads();
        const int li64 = wave * 16 * 64 + lane;
        if (grp == 1) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                lds_f32* dst = xch(dt);
#pragma unroll
                for (int r = 0; r < 16; ++r) dst[li64 + r * 64] = o[dt][r];
            }
            lds_f32* ml = xch(NDT);
            ml[wave * 128 + lane] = m_run;
            ml[wave * 128 + 64 + lane] = l_run;
        }
        __syncthreads();
        if (grp == 0) {
            const lds_f32* ml = xch(NDT);
            const float m1 = ml[wave * 128 + lane];
            const float l1 = ml[wave * 128 + 64 + lane];
            const float mn = fmaxf(m_run, m1);
            // a group that saw no valid key has m = -inf and weight 0
            const float a0 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mn);
            const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mn);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const lds_f32* src = xch(dt);
#pragma unroll
                for (int r = 0; r < 16; ++r) o[dt][r] = o[dt][r] * a0 + src[li64 + r * 64] * a1;
            }
            l_run = l_run * a0 + l1 * a1;
            m_run = mn;
        }
    }

    // ---- epilogue: O = O^T / l, lse = ln 2 * (m + log2 l).  Each
    // wavefront stages its 32 output rows in the K/V buffers (free after the
    // barrier below) and stores whole rows with non-temporal 16-byte stores
    // (store_rows_bf16).  Measured on MI355X against stores straight from
    // the accumulators (same machine, interleaved): encoder_d64 -12%,
    // decoder_causal_d64 -19%, cross_padded_d64 -14%, the large causal
    // workload -2.3%, with a shared additive bias -1.5%.
    const float l = sum_across_halves(l_run);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    {
        static_assert(NW <= 4 * KS || D == DV, "staging needs the K buffers");
        constexpr int PER = 2 * KS;   // wavefronts per staging buffer (32 rows x DV each)
        __syncthreads();              // every wavefront is done reading the last K/V tile
        if (grp == 0) {
            const int bi = wave / PER;
            lds_u16* stage = (lds_u16*)(bi == 0 ? v_lds0 : bi == 1 ? v_lds1 : bi == 2 ? k_lds0 : k_lds1) +
                             (wave % PER) * 32 * DV;
            store_rows_bf16<DV>(o, inv, stage, p.out + b * p.o_sb + hh * p.o_sh + (size_t)q0w * p.o_sl,
                                (size_t)p.o_sl, p.Lq - q0w, lane);
        }
    }
    if (grp == 0 && qrow < p.Lq && p.lse != nullptr && h == 0)
        p.lse[(size_t)bh * p.Lq + qrow] = l > 0.f ? (m_run + __log2f(l)) * kLn2 : -INFINITY;
    // every wavefront is done with the LDS buffers before the next item's
    // first loads overwrite them
    __syncthreads();
    }
}

template <int D, int DV, int BC, int NW, int KS, bool CAUSAL, bool LENS, bool MASK>
hipError_t launch_one(const FwdArgs& a, int sched, hipStream_t stream) {
    const bool pairs = sched == 1;
    constexpr int BR = NW * 32;
    auto kern = fwd_bf16_kernel<D, DV, BC, NW, KS, CAUSAL, LENS, MASK>;
    KParams p;
    p.q = static_cast<const uint16_t*>(a.q);
    p.k = static_cast<const uint16_t*>(a.k);
    p.v = static_cast<const uint16_t*>(a.v);
    p.out = static_cast<uint16_t*>(a.out);
    p.lse = a.lse;
    p.key_lens = a.key_lens;
    p.H = a.H;
    p.Lq = a.Lq;
    p.Lk = a.Lk;
    p.num_qb = (a.Lq + BR - 1) / BR;
    const double scale = a.scale > 0.f ? (double)a.scale : 1.0 / sqrt((double)D);
    p.scale_log2 = (float)(1.4426950408889634 * scale);
    p.inv_scale = (float)(1.0 / scale);
    p.q_sb = a.q_sb; p.q_sh = a.q_sh; p.q_sl = a.q_sl;
    p.k_sb = a.k_sb; p.k_sh = a.k_sh; p.k_sl = a.k_sl;
    p.v_sb = a.v_sb; p.v_sh = a.v_sh; p.v_sl = a.v_sl;
    p.o_sb = a.o_sb; p.o_sh = a.o_sh; p.o_sl = a.o_sl;
    p.mask = a.mask;
    p.m_sb = a.m_sb; p.m_sh = a.m_sh; p.m_sl = a.m_sl;
    p.mask_vec = a.mask != nullptr && reinterpret_cast<uintptr_t>(a.mask) % 16 == 0 && a.m_sb % 4 == 0 &&
                 a.m_sh % 4 == 0 && a.m_sl % 4 == 0;
    const long long items = (long long)p.num_qb * a.B * a.H;
    if (items <= 0 || items > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    p.num_items = (int)items;
    // one unit per workgroup: the hardware hands units to free slots as they
    // come, which balances better than a fixed assignment.  Causal units are
    // long/short pairs of equal length once there are more items than
    // resident workgroups, unless pairs would leave slots idle
    // (causal_items_per_unit: with two workgroups per CU up to 1.6 slots'
    // worth of items, and items of at most 8 key tiles); a smaller problem
    // takes one item per workgroup so that every item starts at once.
    const long long slots = (long long)(a.num_cus > 0 ? a.num_cus : 256) * fwd_blocks_per_cu<D, NW, KS>();
    p.upi = CAUSAL ? causal_items_per_unit(items, slots, fwd_blocks_per_cu<D, NW, KS>() == 2 ? 8 * slots / 5 : slots,
                                           ((a.Lq < a.Lk ? a.Lq : a.Lk) + 63) / 64, 8)
                   : 1;
    p.B = a.B;
    // Compute-unit pairs (default schedule): when every workgroup is
    // resident at once and some compute units hold two, renumber the units
    // so that each such compute unit runs a long item and a short one
    // (cu_pair_unit).  Causal query blocks already alternate long and short
    // (an even count per slice keeps the alternation aligned); with key
    // lengths the items are taken in length-rank order interleaved from both
    // ends (from 5 key tiles up: shorter key ranges measured no gain).
    p.lens_pairs = 0;
    p.cu_pairs = 0;
    const int cus = a.num_cus > 0 ? a.num_cus : 256;
    const bool cu_pairing = sched == 0 && items <= slots && items > cus && fwd_blocks_per_cu<D, NW, KS>() == 2 &&
                            cus % 8 == 0;
    if (LENS && !CAUSAL && pairs && a.B > 1 && a.B <= kMaxPairBatches) {
        p.lens_pairs = 1;
        p.upi = 2;
    } else if (LENS && !CAUSAL && cu_pairing && (a.Lk + 63) / 64 >= 5 && a.B > 1 && a.B <= kMaxPairBatches) {
        p.lens_pairs = 2;
        p.cu_pairs = cus / 8;
    } else if (CAUSAL && cu_pairing && p.upi == 1 && p.num_qb % 2 == 0 &&
               (D == 64 || (a.Lq < a.Lk ? a.Lq : a.Lk) > 4 * 64)) {
        // (d128 with at most 4 key tiles per row measured 8% slower paired)
        p.cu_pairs = cus / 8;
    }
    p.num_units = (int)((items + p.upi - 1) / p.upi);
    const long long nwg = p.num_units;
    hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(NW * KS * 64), 0, stream, p);
    return hipGetLastError();
}

template <int D, int DV, int BC, int NW, int KS, bool MASK>
hipError_t launch_d(const FwdArgs& a, int pairs, hipStream_t s) {
    const bool lens = a.key_lens != nullptr;
    if (a.causal)
        return lens ? launch_one<D, DV, BC, NW, KS, true, true, MASK>(a, pairs, s)
                    : launch_one<D, DV, BC, NW, KS, true, false, MASK>(a, pairs, s);
    return lens ? launch_one<D, DV, BC, NW, KS, false, true, MASK>(a, pairs, s)
                : launch_one<D, DV, BC, NW, KS, false, false, MASK>(a, pairs, s);
}

// default tiles (64 keys, 4 wavefronts, no key split) for every (d_k, d_v)
// pair, with and without the additive mask
template <int D, int DV>
hipError_t launch_default(const FwdArgs& a, int pairs, hipStream_t s) {
    return a.mask != nullptr ? launch_d<D, DV, 64, 4, 1, true>(a, pairs, s)
                             : launch_d<D, DV, 64, 4, 1, false>(a, pairs, s);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, const Bf16Tile& t, hipStream_t s) {
    if (t.d != a.d) return hipErrorInvalidValue;
    const int pairs = t.pairs;   // 0 (default, with compute-unit pairs) or 1 (key-length pairs)
    if (t.bc == 64 && t.waves == 4 && t.ks == 1) {
        if (a.d == 128 && a.dv == 128) return launch_default<128, 128>(a, pairs, s);
        if (a.d == 128 && a.dv == 64) return launch_default<128, 64>(a, pairs, s);
        if (a.d == 64 && a.dv == 64) return launch_default<64, 64>(a, pairs, s);
        if (a.d == 64 && a.dv == 128) return launch_default<64, 128>(a, pairs, s);
        return hipErrorInvalidValue;
    }
    // the other tiles: d_v = d_k, no mask
    if (a.dv != a.d || a.mask != nullptr) return hipErrorInvalidValue;
    if (t.d == 128 && t.bc == 64 && t.waves == 4 && t.ks == 2) return launch_d<128, 128, 64, 4, 2, false>(a, pairs, s);
    if (t.d == 128 && t.bc == 64 && t.waves == 8 && t.ks == 1) return launch_d<128, 128, 64, 8, 1, false>(a, pairs, s);
    if (t.d == 64 && t.bc == 64 && t.waves == 8 && t.ks == 1) return launch_d<64, 64, 64, 8, 1, false>(a, pairs, s);
    if (t.d == 64 && t.bc == 64 && t.waves == 4 && t.ks == 2) return launch_d<64, 64, 64, 4, 2, false>(a, pairs, s);
    return hipErrorInvalidValue;
}

}  // namespace sdpa
