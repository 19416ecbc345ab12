// Staggered variant of the fused bf16 attention forward for gfx950.
//
// Same mathematics, operand layouts, LDS layouts and masking as
// sdpa_fwd_bf16.hip: eq. (1) of "Aufmerksamkeit ist alles, was Sie
// brauchen", section 3.2.1, with the running maximum and sum justified by
// the ratio identity of the formula page "トランスフォーマーの注意機構",
// section 証明.  What differs is the order of the work inside a tile.
//
// With one tile barrier per 64 keys, two workgroups that share a CU were
// measured to start their tiles nearly in step, so the two wavefronts of a
// SIMD run their matrix products at the same time and their softmax at the
// same time.  Here one workgroup of 8 wavefronts (256 query rows, one per
// CU) holds both: wavefronts w and w + 4 share a SIMD, and the two groups
// order a tile differently:
//     group A (0..3):  S(t), softmax(t), P(t).V(t)
//     group B (4..7):  P(t-1).V(t-1), S(t), softmax(t)
// so after the tile barrier A's S products meet B's P.V products, then A's
// softmax meets B's S products and B's softmax meets A's P.V products.
// Query blocks of 32 rows alternate between the groups (A: 0, 2, 4, 6; B:
// 1, 3, 5, 7) to balance the causal diagonal.
//
// B reads V(t - 1) while A reads V(t), so V (and, for a uniform schedule,
// K) is triple buffered: tile t lives in buffer t % 3.  The loads of tile
// t + 1 go out right after the barrier that opens tile t and are waited
// for at the next one.
//
// Measured on the large causal d_k = 128 workload this variant is 7% slower
// than the default kernel: it takes more cycles, its wavefronts waiting
// longer at the tile barriers and on LDS operands (a wavefront alone does not
// keep the matrix core busy).  It stays selectable for comparison.
#include "sdpa_internal.h"
#include "bf16_common.h"

#include <math.h>

#include <type_traits>

namespace sdpa {
namespace {

using namespace bf16k;

template <int D, bool CAUSAL, bool LENS>
__global__ void __launch_bounds__(512, 1) fwd_bf16_mix_kernel(KParams p) {
    constexpr int NW = 8;
    constexpr int NT = NW * 64;
    constexpr int BR = NW * 32;                // 256 query rows
    constexpr int BC = 64;                     // keys per tile
    constexpr int CPR = D / 8;                 // 16-byte chunks per row
    constexpr int KCH = BC * CPR / NT;         // 16-byte loads per thread per K (or V) tile
    constexpr int TILE = BC * D;
    constexpr int NKT = BC / 32;
    constexpr int NDT = D / 32;
    constexpr int NKS = D / 16;
    static_assert((BC * CPR) % NT == 0, "tile must split evenly over threads");

    // three K and three V buffers (tile t in buffer t % 3), in separate
    // arrays so that the compiler sees the loads into one buffer never alias
    // the reads of another and adds no waits for them
    __shared__ __align__(16) uint16_t k_lds0[TILE], k_lds1[TILE], k_lds2[TILE];
    __shared__ __align__(16) uint16_t v_lds0[TILE], v_lds1[TILE], v_lds2[TILE];
    auto k_buf = [&](int i) __attribute__((always_inline)) { return i == 0 ? k_lds0 : i == 1 ? k_lds1 : k_lds2; };
    auto v_buf = [&](int i) __attribute__((always_inline)) { return i == 0 ? v_lds0 : i == 1 ? v_lds1 : v_lds2; };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int group = wave >> 2;               // 0: A; 1: B, P.V one tile late
    const int blk = 2 * (wave & 3) + group;    // this wavefront's 32-row block
    const int n = lane & 31;
    const int h = lane >> 5;

    // load u of this thread fills LDS slot (wave*KCH + u)*64 + lane of a tile
    uint32_t k_boff[KCH], v_boff[KCH];
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
        const int s = (wave * KCH + u) * 64 + lane;
        const int row = s / CPR, pc = s % CPR;
        k_boff[u] = (k_lds_row(row) * p.k_sl + ((pc ^ k_swz<D>(row)) << 3)) * 2;
        v_boff[u] = (row * p.v_sl + ((pc ^ v_swz<D>(row)) << 3)) * 2;
    }
    // per-lane LDS read offsets (elements), as in the main kernel
    int k_rd[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) k_rd[ks] = n * D + (((2 * ks + h) ^ k_swz<D>(n)) << 3);
    const int li = lane & 15;
    int v_rd[NDT];
    {
        const int row = 8 * h + (li >> 2);
        const int colg = 16 * ((lane >> 4) & 1) + 4 * (li & 3);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const int col = dt * 32 + colg;
            v_rd[dt] = row * D + (((col >> 3) ^ v_swz<D>(row)) << 3) + (col & 7);
        }
    }

    int unit_first, unit_step, unit_last;
    workgroup_units(p.num_units, &unit_first, &unit_step, &unit_last);
    for (int unit = unit_first; unit < unit_last; unit += unit_step)
    for (int item = unit * p.upi; item < min(unit * p.upi + p.upi, p.num_items); ++item) {
    int bh, qb;
    item_block<CAUSAL>(item, p.num_qb, &bh, &qb);
    const int b = bh / p.H;
    const int hh = bh - b * p.H;
    const int q0 = qb * BR;

    int kv_len = p.Lk;
    if (LENS) {
        int L = p.key_lens[b];
        L = L < 0 ? 0 : L;
        kv_len = L < kv_len ? L : kv_len;
    }
    const int kv_end = CAUSAL ? min(kv_len, q0 + BR) : kv_len;
    const int ntiles = (kv_end + BC - 1) / BC;

    const int q0w = q0 + blk * 32;
    const int qrow = q0w + n;
    const int wave_kv_end = CAUSAL ? min(kv_len, q0w + 32) : kv_len;

    const uint16_t* qg = p.q + b * p.q_sb + hh * p.q_sh;
    const uint16_t* kg = p.k + b * p.k_sb + hh * p.k_sh;
    const uint16_t* vg = p.v + b * p.v_sb + hh * p.v_sh;

    bf16x8 qf[NKS];
    {
        const int qr = qrow < p.Lq ? qrow : p.Lq - 1;
        const i16x8* src = reinterpret_cast<const i16x8*>(qg + (size_t)qr * p.q_sl + 8 * h);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, src[2 * ks]);
    }

    const uint32_t k_bytes = (uint32_t)kv_len * p.k_sl * 2;
    const uint32_t v_bytes = (uint32_t)kv_len * p.v_sl * 2;
    // loads of tile t into buffer buf; t < 0: zero-length loads (nothing is
    // read; zeros land in a buffer no wavefront reads any more)
    auto issue_k = [&](int t, int buf) __attribute__((always_inline)) {
        const uint32_t toff = (uint32_t)((t < 0 ? 0 : t) * BC) * p.k_sl * 2;
#pragma unroll
        for (int u = 0; u < KCH; ++u) {
            lds_void* dst = (lds_void*)(k_buf(buf) + (wave * KCH + u) * 64 * 8);
            buffer_load_lds16(kg, t < 0 ? 0u : k_bytes, dst, k_boff[u], toff);
        }
    };
    auto issue_v = [&](int t, int buf) __attribute__((always_inline)) {
        const uint32_t toff = (uint32_t)((t < 0 ? 0 : t) * BC) * p.v_sl * 2;
#pragma unroll
        for (int u = 0; u < KCH; ++u) {
            lds_void* dst = (lds_void*)(v_buf(buf) + (wave * KCH + u) * 64 * 8);
            buffer_load_lds16(vg, t < 0 ? 0u : v_bytes, dst, v_boff[u], toff);
        }
    };

    f32x16 o[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
    float m_run = -INFINITY;
    float l_run = 0.f;
    bool big = false;
    const float sl = p.scale_log2;
    f32x16 s[NKT];   // the scores of a tile, from its S step to its SMPV step

    // S(t): S^T = K Q^T, then the key-length and causal masks
    auto do_s = [&](int t, const uint16_t* Ks) __attribute__((always_inline)) {
        const int ts = t * BC;
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
            }
        }
        const bool need_mask = (ts + BC > kv_len) || (CAUSAL && ts + BC - 1 > q0w);
        if (need_mask) {
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = ts + kt * 32 + 16 * (r >> 3) + 8 * h + (r & 7);
                    bool ok = key < kv_len;
                    if (CAUSAL) ok = ok && key <= qrow;
                    s[kt][r] = ok ? s[kt][r] : -INFINITY;
                }
        }
    };

    bf16x8 pb[NKT][2];   // the bf16 weights of a tile, from its softmax to its P.V

    // SM(t): weights from the scores of S(t).  fast: exponentials against
    // the fixed reference m_run (set exactly by the first tile), recording
    // only whether a tile's weights reached 2^64; otherwise the exact running
    // maximum (rescaling O, which then holds the tiles before t only).
    auto do_sm = [&](bool fast) __attribute__((always_inline)) {
        if (fast) {
            float lsum = 0.f;
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][r], sl, -m_run));
                    lsum += pv;
                    pb[kt][r >> 3][r & 7] = (__bf16)pv;
                }
            l_run += lsum;
            big |= !(lsum < 0x1p64f);
        } else {
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
                    const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][r], sl, -mref));
                    l_run += pv;
                    pb[kt][r >> 3][r & 7] = (__bf16)pv;
                }
        }
    };

    // PV: O^T += V^T P^T with the weights of the last softmax; the
    // transposed V reads run one key step ahead
    auto do_pv = [&](const uint16_t* Vs) __attribute__((always_inline)) {
        constexpr int NSTEP = 2 * NKT;
        i16x8 va[2][NDT];
        auto read_v = [&](int step, i16x8* dst) __attribute__((always_inline)) {
            const int roff = (step * 16) * D;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4*)(Vs + roff + v_rd[dt]));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4*)(Vs + roff + 4 * D + v_rd[dt]));
                dst[dt] = i16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
        };
        read_v(0, va[0]);
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) {
            if (st + 1 < NSTEP) read_v(st + 1, va[(st + 1) & 1]);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
                o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, va[st & 1][dt]), pb[st >> 1][st & 1], o[dt], 0, 0, 0);
        }
    };

    // One pass over the tiles.  Tile t is in buffers t % 3; the loop is
    // unrolled by three tiles so that every buffer is a compile-time choice.
    // all_exact: the exact softmax on every tile (the re-run after an
    // overflow).
    auto run_pass = [&](bool all_exact) __attribute__((always_inline)) {
        auto tile = [&](int t) __attribute__((always_inline)) { return t < ntiles ? t : -1; };
        auto live = [&](int t) __attribute__((always_inline)) {
            return t >= 0 && t < ntiles && t * BC < wave_kv_end;
        };
        issue_k(0, 0);
        issue_v(0, 0);
        // tile t has landed everywhere; every wavefront is done with tile
        // t - 2, whose buffers take tile t + 1
        auto tile_barrier = [&]() __attribute__((always_inline)) {
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            __syncthreads();
        };
        // each group runs its own copy of the loop, so that B's weights,
        // live across the barrier, do not hold registers in A's copy
        if (group == 0) {
            for (int t0 = 0; t0 < ntiles; t0 += 3) {
#pragma unroll
                for (int j = 0; j < 3; ++j) {
                    const int t = t0 + j;
                    if (j > 0 && t >= ntiles) break;
                    tile_barrier();
                    issue_k(tile(t + 1), (j + 1) % 3);
                    issue_v(tile(t + 1), (j + 1) % 3);
                    if (live(t)) {
                        do_s(t, k_buf(j));
                        do_sm(!all_exact && t > 0);
                        do_pv(v_buf(j));
                    }
                }
            }
        } else {
            for (int t0 = 0; t0 < ntiles; t0 += 3) {
#pragma unroll
                for (int j = 0; j < 3; ++j) {
                    const int t = t0 + j;
                    if (j > 0 && t >= ntiles) break;
                    tile_barrier();
                    issue_k(tile(t + 1), (j + 1) % 3);
                    issue_v(tile(t + 1), (j + 1) % 3);
                    if (live(t - 1)) do_pv(v_buf((j + 2) % 3));
                    if (live(t)) {
                        do_s(t, k_buf(j));
                        do_sm(!all_exact && t > 0);
                    }
                }
            }
            // the last P.V: tile ntiles - 1 is in LDS and no load targets
            // its buffers
            if (live(ntiles - 1)) {
                const int jl = (ntiles - 1) % 3;
                do_pv(jl == 0 ? v_lds0 : jl == 1 ? v_lds1 : v_lds2);
            }
        }
        // zero-length loads past the last tile may still be in flight
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    };
    if (ntiles > 0) {
        run_pass(false);
        if (__syncthreads_or(big)) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
            m_run = -INFINITY;
            l_run = 0.f;
            run_pass(true);
        }
    }

    // ---- epilogue: O = O^T / l, lse = ln 2 * (m + log2 l)
    const float l = sum_across_halves(l_run);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (qrow < p.Lq) {
        uint16_t* dst = p.out + b * p.o_sb + hh * p.o_sh + (size_t)qrow * p.o_sl;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d0 = dt * 32 + 8 * g4 + 4 * h;
                __bf16 w[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) w[c] = (__bf16)(o[dt][4 * g4 + c] * inv);
                *reinterpret_cast<uint2*>(dst + d0) = __builtin_bit_cast(uint2, w);
            }
        if (p.lse != nullptr && h == 0)
            p.lse[(size_t)bh * p.Lq + qrow] = l > 0.f ? (m_run + __log2f(l)) * kLn2 : -INFINITY;
    }
    // every wavefront is done with both LDS buffers before the next item's
    // first loads overwrite them
    __syncthreads();
    }
}

template <int D, bool CAUSAL, bool LENS>
hipError_t launch_one(const FwdArgs& a, hipStream_t stream) {
    constexpr int BR = 256;
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
    p.mask = nullptr;
    p.m_sb = p.m_sh = 0;
    p.m_sl = 0;
    p.mask_vec = 0;
    const long long items = (long long)p.num_qb * a.B * a.H;
    if (items <= 0 || items > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    p.num_items = (int)items;
    // one workgroup per CU; causal long/short pairs once the items
    // outnumber the CUs
    const long long slots = a.num_cus > 0 ? a.num_cus : 256;
    p.upi = (CAUSAL && items > slots) ? 2 : 1;
    p.num_units = (int)((items + p.upi - 1) / p.upi);
    hipLaunchKernelGGL((fwd_bf16_mix_kernel<D, CAUSAL, LENS>), dim3((unsigned)p.num_units), dim3(512), 0,
                       stream, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t s) {
    const bool lens = a.key_lens != nullptr;
    if (a.causal)
        return lens ? launch_one<D, true, true>(a, s) : launch_one<D, true, false>(a, s);
    return lens ? launch_one<D, false, true>(a, s) : launch_one<D, false, false>(a, s);
}

}  // namespace

hipError_t launch_fwd_bf16_mix(const FwdArgs& a, const Bf16Tile& t, hipStream_t s) {
    if (t.d != a.d || a.dv != a.d || a.mask != nullptr) return hipErrorInvalidValue;
    if (t.d == 128) return launch_d<128>(a, s);
    if (t.d == 64) return launch_d<64>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace sdpa
