// Fused bf16 attention forward for gfx950 with 64 query rows per wavefront.
//
// Same mathematics, operand layouts, LDS layouts and masking rules as
// sdpa_fwd_bf16.hip (eq. (1) of "Aufmerksamkeit ist alles, was Sie
// brauchen", section 3.2.1, with the online softmax justified by the ratio
// identity of the formula page "トランスフォーマーの注意機構", section 証明),
// and the same software pipeline as sdpa_fwd_bf16_pipe.hip: block b issues
// S(b+2), the softmax of S(b+1) and P(b).V over 32-key sub-tiles, written
// step by step so that every MFMA has vector work beside it.
//
// What differs is the wavefront's share: two 32-row blocks of queries
// instead of one.  Every K fragment and every transposed V fragment read
// from LDS feeds two MFMAs (one per row block), which halves the LDS reads
// per MFMA, and a workgroup of four wavefronts covers 256 query rows, which
// halves the K/V traffic into LDS per MFMA.  The price is registers: the
// d = 128 accumulators of O (128 per lane) leave room for one wavefront per
// SIMD, so the kernel relies on its own interleaving rather than on a second
// wavefront to fill the gaps.
#include "sdpa_internal.h"
#include "bf16_common.h"

#include <math.h>

#include <type_traits>

namespace sdpa {
namespace {

using namespace bf16k;
template <int V>
using IC = std::integral_constant<int, V>;

template <int D, bool CAUSAL, bool LENS>
__global__ void __launch_bounds__(256, D == 64 ? 2 : 1) fwd_bf16_wide_kernel(KParams p) {
    constexpr int NW = 4;                      // wavefronts per workgroup
    constexpr int RB = 2;                      // 32-row blocks per wavefront
    constexpr int BC = 64;                     // keys per LDS tile
    constexpr int NT = NW * 64;
    constexpr int BR = NW * RB * 32;           // query rows per workgroup
    constexpr int CPR = D / 8;                 // 16-byte chunks per row
    constexpr int KCH = BC * CPR / NT;         // 16-byte loads per thread per tile
    constexpr int TILE = BC * D;               // elements per K or V tile
    constexpr int NDT = D / 32;                // 32-wide output column tiles
    constexpr int NKS = D / 16;                // k-steps of the Q.K^T product
    static_assert((BC * CPR) % NT == 0, "tile must split evenly over threads");

    __shared__ __align__(16) uint16_t k_lds0[TILE], k_lds1[TILE], v_lds0[TILE], v_lds1[TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31;
    const int h = lane >> 5;

    uint32_t k_boff[KCH], v_boff[KCH];
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
        const int s = (wave * KCH + u) * 64 + lane;
        const int row = s / CPR, pc = s % CPR;
        k_boff[u] = (k_lds_row(row) * D + ((pc ^ k_swz<D>(row)) << 3)) * 2;
        v_boff[u] = (row * D + ((pc ^ v_swz<D>(row)) << 3)) * 2;
    }
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
    const float sl = p.scale_log2;

    int unit_first, unit_step, unit_last;
    workgroup_units(p.num_units, &unit_first, &unit_step, &unit_last);
    for (int unit = unit_first; unit < unit_last; unit += unit_step)
    for (int item = unit * p.upi; item < min(unit * p.upi + p.upi, p.num_items); ++item) {
    int bh, qb;
    item_block<CAUSAL>(item, p.num_qb, &bh, &qb);
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
    const int q0w = q0 + wave * RB * 32;       // first row of this wavefront
    int qrow[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) qrow[rb] = q0w + 32 * rb + n;
    const int wave_kv_end = CAUSAL ? min(kv_len, q0w + RB * 32) : kv_len;
    const int nsub = wave_kv_end > 0 ? (wave_kv_end + 31) / 32 : 0;   // sub-tiles of this wave
    // whether some row of this wavefront may not see some key of sub-tile j
    auto needs_mask = [&](int j) { return (32 * j + 32 > kv_len) || (CAUSAL && 32 * j + 31 > q0w); };

    const size_t q_base = (size_t)bh * p.Lq * D;
    const uint16_t* kg = p.k + (size_t)bh * p.Lk * D;
    const uint16_t* vg = p.v + (size_t)bh * p.Lk * D;
    const uint32_t kv_bytes = (uint32_t)kv_len * D * 2;

    bf16x8 qf[RB][NKS];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int qr = qrow[rb] < p.Lq ? qrow[rb] : p.Lq - 1;
        const i16x8* src = reinterpret_cast<const i16x8*>(p.q + q_base + (size_t)qr * D + 8 * h);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qf[rb][ks] = __builtin_bit_cast(bf16x8, src[2 * ks]);
    }

    auto load_k = [&](int t, uint16_t* buf) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < KCH; ++u)
            buffer_load_lds16(kg, kv_bytes, (lds_void*)(buf + (wave * KCH + u) * 64 * 8), k_boff[u],
                              (uint32_t)(t * BC) * D * 2);
    };
    auto load_v = [&](int t, uint16_t* buf) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < KCH; ++u)
            buffer_load_lds16(vg, kv_bytes, (lds_void*)(buf + (wave * KCH + u) * 64 * 8), v_boff[u],
                              (uint32_t)(t * BC) * D * 2);
    };
    auto tile_barrier = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
    };

    f32x16 o[RB][NDT];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[rb][dt][r] = 0.f;
    float m_run[RB], l_run[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        m_run[rb] = -INFINITY;
        l_run[rb] = 0.f;
    }
    bool big = false;

    // ---- sub-tile steps (key order inside S and P as in the other kernels)
    auto s_sub = [&](int j, const uint16_t* Kt, f32x16* acc) __attribute__((always_inline)) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[rb][r] = 0.f;
        const uint16_t* base = Kt + (j & 1) * 32 * D;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const bf16x8 k = *reinterpret_cast<const bf16x8*>(base + k_rd[ks]);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k, qf[rb][ks], acc[rb], 0, 0, 0);
        }
    };
    auto mask_sub = [&](int j, f32x16* s) __attribute__((always_inline)) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = 32 * j + 16 * (r >> 3) + 8 * h + (r & 7);
                bool ok = key < kv_len;
                if (CAUSAL) ok = ok && key <= qrow[rb];
                s[rb][r] = ok ? s[rb][r] : -INFINITY;
            }
    };
    auto sm_exact = [&](const f32x16* s, bf16x8 (*pb)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            float mx = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[rb][r]);
            mx = max_across_halves(mx);
            const float mt = mx * sl;
            if (__ballot(mt > m_run[rb] + kRescaleSlack) != 0ull) {
                const float mn = fmaxf(m_run[rb], mt);
                const float alpha = (m_run[rb] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run[rb] - mn);
                l_run[rb] *= alpha;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[rb][dt][r] *= alpha;
                m_run[rb] = mn;
            }
            const float mref = (m_run[rb] == -INFINITY) ? 0.f : m_run[rb];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rb][r], sl, -mref));
                l_run[rb] += pv;
                pb[rb][r >> 3][r & 7] = (__bf16)pv;
            }
        }
    };
    auto read_v = [&](const uint16_t* Vt, int j, int ksl, int dt) __attribute__((always_inline)) {
        const uint16_t* a = Vt + ((j & 1) * 32 + 16 * ksl) * D + v_rd[dt];
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)a);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a + 4 * D));
        return __builtin_bit_cast(bf16x8, i16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
    };
    auto pv_sub = [&](int j, const uint16_t* Vt, bf16x8 (*pb)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int ksl = 0; ksl < 2; ++ksl)
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const bf16x8 v = read_v(Vt, j, ksl, dt);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    o[rb][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v, pb[rb][ksl], o[rb][dt], 0, 0, 0);
            }
    };

    // pipeline registers (see sdpa_fwd_bf16_pipe.hip): even blocks read set
    // A and write set B, odd blocks the other way round
    f32x16 sA[RB], sB[RB];
    bf16x8 pA[RB][2], pB[RB][2];

    auto block = [&](auto PAR, int bb, const uint16_t* Kt, const uint16_t* Vt) __attribute__((always_inline)) {
        f32x16* s_in = PAR.value ? sB : sA;
        f32x16* s_out = PAR.value ? sA : sB;
        bf16x8 (*p_in)[2] = PAR.value ? pB : pA;
        bf16x8 (*p_out)[2] = PAR.value ? pA : pB;
        // the softmax of the last sub-tiles, or of one past them, first
        // masks the keys a row may not see; a sub-tile past the wavefront's
        // keys is masked completely and S(b+2) of it reads unused LDS data
        if (needs_mask(bb + 1)) mask_sub(bb + 1, s_in);
        const uint16_t* kbase = Kt + ((bb + 2) & 1) * 32 * D;
        constexpr int PER = 16 / NKS;        // softmax values per row block and step
        constexpr int PVM = 2 * NDT / NKS;   // V operands per step
        constexpr int AHEAD = 2;
        f32x16 acc[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[rb][r] = 0.f;
        float part[RB][2];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) part[rb][0] = part[rb][1] = 0.f;
        bf16x8 kop[AHEAD + 1], vop[AHEAD + 1][PVM];
        auto read_ops = [&](int i, int slot) __attribute__((always_inline)) {
            kop[slot] = *reinterpret_cast<const bf16x8*>(kbase + k_rd[i]);
#pragma unroll
            for (int c = 0; c < PVM; ++c) {
                const int q = i * PVM + c;
                vop[slot][c] = read_v(Vt, bb, q / NDT, q % NDT);
            }
        };
        auto softmax_part = [&](int rb, int r0, int r1) __attribute__((always_inline)) {
#pragma unroll
            for (int r = r0; r < r1; ++r) {
                const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s_in[rb][r], sl, -m_run[rb]));
                part[rb][r & 1] += pv;
                p_out[rb][r >> 3][r & 7] = (__bf16)pv;
            }
        };
#pragma unroll
        for (int i = 0; i < AHEAD && i < NKS; ++i) read_ops(i, i);
#pragma unroll
        for (int i = 0; i < NKS; ++i) {
            if (i + AHEAD < NKS) read_ops(i + AHEAD, (i + AHEAD) % (AHEAD + 1));
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[i % (AHEAD + 1)], qf[rb][i], acc[rb],
                                                                   0, 0, 0);
                softmax_part(rb, i * PER, i * PER + PER / 2);
            }
#pragma unroll
            for (int c = 0; c < PVM; ++c) {
                const int q = i * PVM + c;
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    o[rb][q % NDT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        vop[i % (AHEAD + 1)][c], p_in[rb][q / NDT], o[rb][q % NDT], 0, 0, 0);
                    softmax_part(rb, i * PER + PER / 2, (i + 1) * PER);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const float lsum = part[rb][0] + part[rb][1];
            l_run[rb] += lsum;
            big |= !(lsum < 0x1p64f);
            s_out[rb] = acc[rb];
        }
    };
    auto pair = [&](int T, const uint16_t* Kt, const uint16_t* Vt) __attribute__((always_inline)) {
        const int b0 = 2 * T;
        if (b0 < nsub) block(IC<0>(), b0, Kt, Vt);
        if (b0 + 1 < nsub) block(IC<1>(), b0 + 1, Kt, Vt);
    };

    if (ntiles > 0) {
        // prologue: K(0), V(0), K(1); S(0), S(1) and the exact softmax of
        // sub-tile 0, which fixes each row's reference maximum
        load_k(0, k_lds0);
        load_v(0, v_lds0);
        if (1 < ntiles) load_k(1, k_lds1);
        tile_barrier();
        if (nsub > 0) {
            f32x16 s0[RB];
            s_sub(0, k_lds0, s0);
            if (needs_mask(0)) mask_sub(0, s0);
            s_sub(1, k_lds0, sA);   // masked in block 0 if past the keys
            sm_exact(s0, pA);
        }
        for (int T = 0; T < ntiles; T += 2) {
            tile_barrier();
            if (T + 2 < ntiles) load_k(T + 2, k_lds0);
            if (T + 1 < ntiles) load_v(T + 1, v_lds1);
            pair(T, k_lds1, v_lds0);
            if (T + 1 >= ntiles) break;
            tile_barrier();
            if (T + 3 < ntiles) load_k(T + 3, k_lds1);
            if (T + 2 < ntiles) load_v(T + 2, v_lds0);
            pair(T + 1, k_lds0, v_lds1);
        }

        // a fixed-reference sum reached 2^64 somewhere: exact pass, one
        // sub-tile after the other, K(T) and V(T) both in buffer T & 1
        if (__syncthreads_or(big)) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[rb][dt][r] = 0.f;
                m_run[rb] = -INFINITY;
                l_run[rb] = 0.f;
            }
            auto exact_tile = [&](int T, const uint16_t* Kt,
                                  const uint16_t* Vt) __attribute__((always_inline)) {
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    const int j = 2 * T + jj;
                    if (j < nsub) {
                        f32x16 s[RB];
                        s_sub(j, Kt, s);
                        if (needs_mask(j)) mask_sub(j, s);
                        bf16x8 pb[RB][2];
                        sm_exact(s, pb);
                        pv_sub(j, Vt, pb);
                    }
                }
            };
            load_k(0, k_lds0);
            load_v(0, v_lds0);
            for (int T = 0; T < ntiles; T += 2) {
                tile_barrier();
                if (T + 1 < ntiles) {
                    load_k(T + 1, k_lds1);
                    load_v(T + 1, v_lds1);
                }
                exact_tile(T, k_lds0, v_lds0);
                if (T + 1 >= ntiles) break;
                tile_barrier();
                if (T + 2 < ntiles) {
                    load_k(T + 2, k_lds0);
                    load_v(T + 2, v_lds0);
                }
                exact_tile(T + 1, k_lds1, v_lds1);
            }
        }
    }

    // ---- epilogue: O = O^T / l, lse = ln 2 * (m + log2 l)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const float l = sum_across_halves(l_run[rb]);
        const float inv = l > 0.f ? 1.f / l : 0.f;
        if (qrow[rb] < p.Lq) {
            uint16_t* dst = p.out + q_base + (size_t)qrow[rb] * D;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int d0 = dt * 32 + 8 * g4 + 4 * h;
                    __bf16 w[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c) w[c] = (__bf16)(o[rb][dt][4 * g4 + c] * inv);
                    *reinterpret_cast<uint2*>(dst + d0) = __builtin_bit_cast(uint2, w);
                }
            if (p.lse != nullptr && h == 0)
                p.lse[(size_t)bh * p.Lq + qrow[rb]] = l > 0.f ? (m_run[rb] + __log2f(l)) * kLn2 : -INFINITY;
        }
    }
    // both LDS buffers are free before the next item's first loads
    __syncthreads();
    }
}

template <int D, bool CAUSAL, bool LENS>
hipError_t launch_one(const FwdArgs& a, hipStream_t stream) {
    constexpr int BR = 256;
    auto kern = fwd_bf16_wide_kernel<D, CAUSAL, LENS>;
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
    p.scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    const long long items = (long long)p.num_qb * a.B * a.H;
    if (items <= 0 || items > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    p.num_items = (int)items;
    p.upi = CAUSAL ? 2 : 1;
    p.num_units = (int)((items + p.upi - 1) / p.upi);
    hipLaunchKernelGGL(kern, dim3((unsigned)p.num_units), dim3(256), 0, stream, p);
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

hipError_t launch_fwd_bf16_wide(const FwdArgs& a, const Bf16Tile& t, hipStream_t s) {
    if (t.d == 128) return launch_d<128>(a, s);
    if (t.d == 64) return launch_d<64>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace sdpa
