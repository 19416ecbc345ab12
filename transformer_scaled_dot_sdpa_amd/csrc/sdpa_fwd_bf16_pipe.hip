// Software-pipelined variant of the fused bf16 attention forward for gfx950.
//
// Same mathematics, layouts and masking as sdpa_fwd_bf16.hip (eq. (1) of
// "Aufmerksamkeit ist alles, was Sie brauchen", section 3.2.1, with the
// online softmax justified by the ratio identity of the formula page
// "トランスフォーマーの注意機構", section 証明).  What differs is the order of
// work inside a wavefront: keys are processed in 32-key sub-tiles j, and the
// block of instructions for sub-tile j issues
//     the MFMAs of S(j+1) = K_{j+1} Q^T        (matrix cores)
//     the MFMAs of O += V_{j-1}^T P(j-1)^T     (matrix cores)
//     the softmax of S(j): max, exp2, sum, bf16 pack   (vector ALU)
// with no data dependence between the three, so the scheduler interleaves
// vector work under the MFMAs of the same wavefront instead of relying on a
// second wavefront being in the opposite phase.
//
// Rescaling.  softmax(j) may raise the reference maximum (lazily, when the
// sub-tile maximum exceeds it by more than 2^8).  P(j-1), accumulated into O
// in the same block, was formed with the old maximum, so the factor
// alpha = 2^(m_old - m_new) is applied to O at the end of the block, after
// that MFMA, and to the running sum before adding the new weights.
//
// LDS.  K and V tiles of 64 keys, two buffers each (64 KiB per workgroup).
// Block j reads K of sub-tile j+1 and V of sub-tile j-1; after every
// even block both the K tile and the V tile that were just read for the
// last time are free, so one barrier per tile lets the next K tile (two
// tiles ahead) and the next V tile (one tile ahead) stream in.
#include "sdpa_internal.h"
#include "bf16_common.h"

#include <math.h>

#include <type_traits>

namespace sdpa {
namespace {

using namespace bf16k;
template <int V>
using IC = std::integral_constant<int, V>;

template <int D, int NW, bool CAUSAL, bool LENS>
__global__ void __launch_bounds__(NW * 64, 1) fwd_bf16_pipe_kernel(KParams p) {
    constexpr int BC = 64;                     // keys per LDS tile
    constexpr int NT = NW * 64;
    constexpr int BR = NW * 32;
    constexpr int CPR = D / 8;                 // 16-byte chunks per row
    constexpr int KCH = BC * CPR / NT;         // 16-byte loads per thread per tile
    constexpr int TILE = BC * D;               // elements per K or V tile
    constexpr int NDT = D / 32;                // 32-wide output column tiles
    constexpr int NKS = D / 16;                // k-steps of the Q.K^T product
    static_assert((BC * CPR) % NT == 0, "tile must split evenly over threads");

    extern __shared__ __align__(16) uint16_t smem[];  // K[0], K[1], V[0], V[1]

    int bh, qb;
    map_workgroup<CAUSAL>(p.num_qb, &bh, &qb);
    const int b = bh / p.H;
    const int q0 = qb * BR;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

    const int q0w = q0 + wave * 32;
    const int qrow = q0w + n;
    const int wave_kv_end = CAUSAL ? min(kv_len, q0w + 32) : kv_len;
    const int nsub = (wave_kv_end + 31) / 32;   // sub-tiles this wave computes

    const size_t q_base = (size_t)bh * p.Lq * D;
    const uint16_t* kg = p.k + (size_t)bh * p.Lk * D;
    const uint16_t* vg = p.v + (size_t)bh * p.Lk * D;

    // Q^T operand fragments (rows past Lq load the last valid row; never stored)
    bf16x8 qf[NKS];
    {
        const int qr = qrow < p.Lq ? qrow : p.Lq - 1;
        const i16x8* src = reinterpret_cast<const i16x8*>(p.q + q_base + (size_t)qr * D + 8 * h);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, src[2 * ks]);
    }

    // direct global -> LDS loads (see sdpa_fwd_bf16.hip for the layout)
    uint32_t k_boff[KCH], v_boff[KCH];
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
        const int s = (wave * KCH + u) * 64 + lane;
        const int row = s / CPR, pc = s % CPR;
        k_boff[u] = (k_lds_row(row) * D + ((pc ^ k_swz<D>(row)) << 3)) * 2;
        v_boff[u] = (row * D + ((pc ^ v_swz<D>(row)) << 3)) * 2;
    }
    auto issue = [&](const uint16_t* gbase, const uint32_t* boff, int t,
                     uint16_t* lds_tile) __attribute__((always_inline)) {
        if (t >= ntiles) return;
        const int ts = t * BC;
        const char* src = reinterpret_cast<const char*>(gbase + (size_t)ts * D);
        lds_void* dst = (lds_void*)(lds_tile + wave * KCH * 64 * 8);
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
    };
    uint16_t* const Kbuf0 = smem;
    uint16_t* const Kbuf1 = smem + TILE;
    uint16_t* const Vbuf0 = smem + 2 * TILE;
    uint16_t* const Vbuf1 = smem + 3 * TILE;

    // per-lane LDS read offsets (elements); see sdpa_fwd_bf16.hip
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
    f32x16 sacc[2];
    bf16x8 pb[2][2];
    float m_run = -INFINITY;   // reference maximum, exp2 units
    float l_run = 0.f;         // this lane's partial sum of weights
    const float sl = p.scale_log2;

    // S^T of one 32-key sub-tile (position kt in the K tile at Ks)
    auto s_product = [&](f32x16& acc, const uint16_t* Ks, int kt) __attribute__((always_inline)) {
        bf16x8 ka[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            ka[ks] = *reinterpret_cast<const bf16x8*>(Ks + kt * 32 * D + k_rd[ks]);
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qf[ks], acc, 0, 0, 0);
    };

    // One pipeline block for sub-tile j (see file header).  PAR = j & 1
    // selects the register buffers; the K and V tiles are passed in.  Every
    // block runs the same straight-line code: at the ends of the sequence
    // the extra work is harmless (S of a sub-tile past the end is never
    // used, a sub-tile past the wave's keys is fully masked, and P before
    // the first sub-tile is zero against a zero-filled V buffer).
    auto block = [&](auto PAR, const uint16_t* Ks, const uint16_t* Vs,
                     int j) __attribute__((always_inline)) {
        constexpr int par = decltype(PAR)::value;
        constexpr int nxt = par ^ 1;
        constexpr int kt = par ^ 1;   // position of sub-tiles j+1 and j-1 in their tiles
        const int js = 32 * j;
        if ((js + 32 > kv_len) || (CAUSAL && js + 31 > q0w)) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = js + 16 * (r >> 3) + 8 * h + (r & 7);
                bool ok = key < kv_len;
                if (CAUSAL) ok = ok && key <= qrow;
                sacc[par][r] = ok ? sacc[par][r] : -INFINITY;
            }
        }
        // softmax of S(j) (vector ALU)
        float mx = sacc[par][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[par][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mt = mx * sl;
        const bool raise = mt > m_run + kRescaleSlack;   // false when mt = -inf
        const float mn = raise ? mt : m_run;
        const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - mt) : 1.f;  // 0 if m_run = -inf
        const float mref = (mn == -INFINITY) ? 0.f : mn;
        m_run = mn;
        float lsum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[par][r], sl, -mref));
            lsum += pv;
            pb[par][r >> 3][r & 7] = (__bf16)pv;
        }
        l_run = __builtin_fmaf(l_run, alpha, lsum);
        // matrix cores: S(j+1) and O += V(j-1)^T P(j-1)^T, interleaved; each
        // operand is read from LDS next to its MFMA (the scheduler hoists the
        // reads as far as registers allow)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[nxt][r] = 0.f;
#pragma unroll
        for (int i = 0; i < NKS; ++i) {
            const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Ks + kt * 32 * D + k_rd[i]);
            sacc[nxt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[i], sacc[nxt], 0, 0, 0);
            if (i < 2 * NDT) {
                const int ksl = i / NDT, dt = i % NDT;
                const int roff = (kt * 32 + 16 * ksl) * D;
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4*)(Vs + roff + v_rd[dt]));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4*)(Vs + roff + 4 * D + v_rd[dt]));
                const i16x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, va), pb[nxt][ksl], o[dt], 0, 0, 0);
            }
        }
        // rescale O (rare) once P(j-1) has been accumulated; the empty asm
        // keeps the compiler from executing the multiplies unconditionally
        if (__ballot(alpha != 1.f) != 0ull) {
            asm volatile("" ::: "memory");
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
        }
    };

    if (ntiles > 0) {
        // ---- prologue: K(0), V(0), K(1) in flight; zero V buffer 1 (read by
        // the empty P.V of block 0); P starts at zero; then S(0)
        issue(kg, k_boff, 0, Kbuf0);
        issue(vg, v_boff, 0, Vbuf0);
        issue(kg, k_boff, 1, Kbuf1);
#pragma unroll
        for (int i = tid; i < TILE / 8; i += NT)
            reinterpret_cast<i16x8*>(Vbuf1)[i] = i16x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int y = 0; y < 2; ++y)
                pb[x][y] = __builtin_bit_cast(bf16x8, i16x8{0, 0, 0, 0, 0, 0, 0, 0});
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        s_product(sacc[0], Kbuf0, 0);

        // ---- blocks j = 0 .. nblocks (the last one drains P.V of the final
        // sub-tile); four per trip so every buffer index is a constant.
        // A wave skips the blocks past j = nsub (nothing left for it).
        const int nblocks = 2 * ntiles;
        for (int J = 0;; J += 4) {
            const int T = J / 2;
            if (J <= nsub) block(IC<0>(), Kbuf0, Vbuf1, J);   // S: tile T kt1; PV: tile T-1 kt1
            if (J == nblocks) break;
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            __syncthreads();
            issue(kg, k_boff, T + 2, Kbuf0);
            issue(vg, v_boff, T + 1, Vbuf1);
            if (J + 1 <= nsub) block(IC<1>(), Kbuf1, Vbuf0, J + 1);   // S: tile T+1 kt0; PV: tile T kt0
            if (J + 2 <= nsub) block(IC<0>(), Kbuf1, Vbuf0, J + 2);   // S: tile T+1 kt1; PV: tile T kt1
            if (J + 2 == nblocks) break;
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            __syncthreads();
            issue(kg, k_boff, T + 3, Kbuf1);
            issue(vg, v_boff, T + 2, Vbuf0);
            if (J + 3 <= nsub) block(IC<1>(), Kbuf0, Vbuf1, J + 3);   // S: tile T+2 kt0; PV: tile T+1 kt0
        }
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

template <int D, int NW, bool CAUSAL, bool LENS>
hipError_t launch_one(const FwdArgs& a, hipStream_t stream) {
    constexpr int BR = NW * 32;
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
    hipLaunchKernelGGL((fwd_bf16_pipe_kernel<D, NW, CAUSAL, LENS>), dim3((unsigned)nwg),
                       dim3(NW * 64), lds, stream, p);
    return hipGetLastError();
}

template <int D, int NW>
hipError_t launch_d(const FwdArgs& a, hipStream_t s) {
    const bool lens = a.key_lens != nullptr;
    if (a.causal)
        return lens ? launch_one<D, NW, true, true>(a, s) : launch_one<D, NW, true, false>(a, s);
    return lens ? launch_one<D, NW, false, true>(a, s) : launch_one<D, NW, false, false>(a, s);
}

}  // namespace

hipError_t launch_fwd_bf16_pipe(const FwdArgs& a, const Bf16Tile& t, hipStream_t s) {
    if (t.d == 128 && t.waves == 4) return launch_d<128, 4>(a, s);
    if (t.d == 64 && t.waves == 4) return launch_d<64, 4>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace sdpa
