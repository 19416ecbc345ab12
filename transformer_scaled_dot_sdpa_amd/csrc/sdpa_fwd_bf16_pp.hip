// Ping-pong variant of the fused bf16 attention forward for gfx950.
//
// Same mathematics, layouts and masking as sdpa_fwd_bf16.hip (eq. (1) of
// "Aufmerksamkeit ist alles, was Sie brauchen", section 3.2.1, with the
// online softmax justified by the ratio identity of the formula page
// "トランスフォーマーの注意機構", section 証明).  What differs is how the two
// wavefronts that share a SIMD are phased.
//
// A workgroup has 8 wavefronts (256 query rows); wavefronts w and w + 4 run
// on the same SIMD.  Group A (waves 0..3) and group B (waves 4..7) do the
// same per-tile work -- S = K Q^T on the matrix cores, then the softmax on
// the vector ALU and O += P V on the matrix cores -- but B runs one phase
// behind A, phases being separated by workgroup barriers:
//
//     phase 2t   : A computes S(t)                B does softmax + P.V (t-1)
//     phase 2t+1 : A does softmax + P.V (t)       B computes S(t)
//
// so in every phase one wave of each SIMD keeps the matrix cores busy while
// the other one's vector work runs beside it.  Query blocks of 32 rows
// alternate between the groups (A: 0, 2, 4, 6; B: 1, 3, 5, 7), so on a causal
// diagonal both groups stop at about the same tile.
//
// Both groups run the same sequence -- S(t), barrier, softmax + P.V (t),
// barrier -- and B enters it through one extra barrier (A leaves through
// one at the end), which puts B exactly one phase behind A.
//
// LDS: K and V tiles of 64 keys, two buffers each (64 KiB).  Group A issues
// all loads: K(t+1) as it starts S(t), V(t+1) as it starts softmax + P.V (t);
// at each barrier A waits for every batch but the one it issued in that
// phase, so a batch has two phases to arrive.
#include "sdpa_internal.h"
#include "bf16_common.h"

#include <math.h>

namespace sdpa {
namespace {

using namespace bf16k;

// s_waitcnt immediates: vmcnt = N, expcnt and lgkmcnt at max (no wait).
template <int N>
constexpr int wait_vmcnt() {
    return (N & 0xF) | ((N >> 4) << 14) | 0x0F70;
}

template <int D, bool CAUSAL, bool LENS>
__global__ void __launch_bounds__(512, 1) fwd_bf16_pp_kernel(KParams p) {
    constexpr int NW = 8;
    constexpr int BC = 64;
    constexpr int NT = NW * 64;
    constexpr int BR = NW * 32;
    constexpr int CPR = D / 8;
    constexpr int KCH = BC * CPR / (NT / 2);   // 16-byte loads per group-A thread per tile
    constexpr int TILE = BC * D;
    constexpr int NKT = BC / 32;
    constexpr int NDT = D / 32;
    constexpr int NKS = D / 16;
    static_assert((BC * CPR) % (NT / 2) == 0, "tile must split evenly over group A");

    extern __shared__ __align__(16) uint16_t smem[];  // K[0], K[1], V[0], V[1]

    int bh, qb;
    map_workgroup<CAUSAL>(p.num_qb, &bh, &qb);
    const int b = bh / p.H;
    const int q0 = qb * BR;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int group = wave >> 2;                        // 0 = A, 1 = B
    const int blk = 2 * (wave & 3) + group;             // 32-row block of this wave
    const int n = lane & 31;
    const int h = lane >> 5;

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

    const size_t q_base = (size_t)bh * p.Lq * D;
    const uint16_t* kg = p.k + (size_t)bh * p.Lk * D;
    const uint16_t* vg = p.v + (size_t)bh * p.Lk * D;

    bf16x8 qf[NKS];
    {
        const int qr = qrow < p.Lq ? qrow : p.Lq - 1;
        const i16x8* src = reinterpret_cast<const i16x8*>(p.q + q_base + (size_t)qr * D + 8 * h);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, src[2 * ks]);
    }

    // direct global -> LDS loads by group A (layout as in sdpa_fwd_bf16.hip)
    const int wl = wave & 3;
    uint32_t k_boff[KCH], v_boff[KCH];
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
        const int s = (wl * KCH + u) * 64 + lane;
        const int row = s / CPR, pc = s % CPR;
        k_boff[u] = (k_lds_row(row) * D + ((pc ^ k_swz<D>(row)) << 3)) * 2;
        v_boff[u] = (row * D + ((pc ^ v_swz<D>(row)) << 3)) * 2;
    }
    // returns whether loads were issued
    auto issue = [&](const uint16_t* gbase, const uint32_t* boff, int t,
                     uint16_t* lds_tile) __attribute__((always_inline)) -> bool {
        if (t >= ntiles) return false;
        const int ts = t * BC;
        const char* src = reinterpret_cast<const char*>(gbase + (size_t)ts * D);
        lds_void* dst = (lds_void*)(lds_tile + wl * KCH * 64 * 8);
        if (ts + BC <= kv_len) {
#pragma unroll
            for (int u = 0; u < KCH; ++u)
                __builtin_amdgcn_global_load_lds((const void*)(src + boff[u]),
                                                 (lds_void*)((char*)dst + u * 1024), 16, 0, 0);
        } else {
            const int last = kv_len - 1 - ts;
#pragma unroll
            for (int u = 0; u < KCH; ++u) {
                const int r = (int)boff[u] / (2 * D), c = (int)boff[u] - r * 2 * D;
                const uint32_t off = (uint32_t)((r < last ? r : last) * 2 * D + c);
                __builtin_amdgcn_global_load_lds((const void*)(src + off),
                                                 (lds_void*)((char*)dst + u * 1024), 16, 0, 0);
            }
        }
        return true;
    };
    // phase barrier.  Group A first waits for all of its loads except the
    // batch it issued in this phase (if it issued one); B only synchronises.
    auto phase_barrier = [&](bool issued_now) __attribute__((always_inline)) {
        if (group == 0) {
            if (issued_now)
                __builtin_amdgcn_s_waitcnt(wait_vmcnt<KCH>());
            else
                __builtin_amdgcn_s_waitcnt(wait_vmcnt<0>());
        }
        __syncthreads();
    };
    uint16_t* const Kb[2] = {smem, smem + TILE};
    uint16_t* const Vb[2] = {smem + 2 * TILE, smem + 3 * TILE};

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

    f32x16 o[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
    f32x16 s[NKT];
    float m_run = -INFINITY;
    float l_run = 0.f;
    const float sl = p.scale_log2;

    // S^T = K Q^T for the whole 64-key tile (k-steps outermost, operand
    // reads one k-step ahead)
    auto s_phase = [&](const uint16_t* Ks) __attribute__((always_inline)) {
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kt][r] = 0.f;
        bf16x8 ka[2][NKT];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
            ka[0][kt] = *reinterpret_cast<const bf16x8*>(Ks + kt * 32 * D + k_rd[0]);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            if (ks + 1 < NKS) {
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt)
                    ka[(ks + 1) & 1][kt] =
                        *reinterpret_cast<const bf16x8*>(Ks + kt * 32 * D + k_rd[ks + 1]);
            }
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
                s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks & 1][kt], qf[ks], s[kt], 0, 0, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, NKT, 0);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            if (ks + 1 < NKS) __builtin_amdgcn_sched_group_barrier(0x100, NKT, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, NKT, 0);
        }
    };

    // masks, online softmax and O^T += V^T P^T for tile t
    auto smpv_phase = [&](int t, const uint16_t* Vs) __attribute__((always_inline)) {
        const int ts = t * BC;
        if ((ts + BC > kv_len) || (CAUSAL && ts + BC - 1 > q0w)) {
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
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
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
        bf16x8 pb[NKT][2];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][r], sl, -mref));
                l_run += pv;
                pb[kt][r >> 3][r & 7] = (__bf16)pv;
            }
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
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * NDT, 1);
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) {
            if (st + 1 < NSTEP) __builtin_amdgcn_sched_group_barrier(0x100, 2 * NDT, 1);
            __builtin_amdgcn_sched_group_barrier(0x008, NDT, 1);
        }
    };

    // phase work of this wave: S(t) from K buffer t&1, or softmax + P.V (t)
    // from V buffer t&1 -- only for tiles that hold keys of this wave
    auto do_s = [&](int t, const uint16_t* Ks) __attribute__((always_inline)) {
        if (t >= 0 && t < ntiles && t * BC < wave_kv_end) s_phase(Ks);
    };
    auto do_smpv = [&](int t, const uint16_t* Vs) __attribute__((always_inline)) {
        if (t >= 0 && t < ntiles && t * BC < wave_kv_end) smpv_phase(t, Vs);
    };

    if (ntiles > 0) {
        const bool isA = group == 0;
        if (isA) {
            issue(kg, k_boff, 0, Kb[0]);
            issue(vg, v_boff, 0, Vb[0]);
        }
        __builtin_amdgcn_s_waitcnt(wait_vmcnt<0>());
        __syncthreads();
        if (!isA) __syncthreads();   // B runs one phase behind A
        bool iss;
        for (int t = 0;; t += 2) {
            // tile t: buffers 0
            iss = isA && issue(kg, k_boff, t + 1, Kb[1]);
            do_s(t, Kb[0]);
            phase_barrier(iss);
            iss = isA && issue(vg, v_boff, t + 1, Vb[1]);
            do_smpv(t, Vb[0]);
            if (t + 1 >= ntiles) break;
            phase_barrier(iss);
            // tile t + 1: buffers 1
            iss = isA && issue(kg, k_boff, t + 2, Kb[0]);
            do_s(t + 1, Kb[1]);
            phase_barrier(iss);
            iss = isA && issue(vg, v_boff, t + 2, Vb[0]);
            do_smpv(t + 1, Vb[1]);
            if (t + 2 >= ntiles) break;
            phase_barrier(iss);
        }
        if (isA) __syncthreads();    // pairs with B's extra barrier
    }

    // ---- epilogue: O = O^T / l, lse = ln 2 * (m + log2 l)
    const float l = l_run + __shfl_xor(l_run, 32);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (qrow < p.Lq) {
        uint16_t* dst = p.out + q_base + (size_t)qrow * D;
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
}

template <int D, bool CAUSAL, bool LENS>
hipError_t launch_one(const FwdArgs& a, hipStream_t stream) {
    constexpr int BR = 256;
    const size_t lds = 4 * (size_t)64 * D * sizeof(uint16_t);
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
    const long long nwg = (long long)p.num_qb * a.B * a.H;
    if (nwg <= 0 || nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((fwd_bf16_pp_kernel<D, CAUSAL, LENS>), dim3((unsigned)nwg), dim3(512), lds,
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

hipError_t launch_fwd_bf16_pp(const FwdArgs& a, const Bf16Tile& t, hipStream_t s) {
    if (t.d == 128) return launch_d<128>(a, s);
    if (t.d == 64) return launch_d<64>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace sdpa
