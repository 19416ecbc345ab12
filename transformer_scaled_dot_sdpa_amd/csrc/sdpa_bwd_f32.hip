// Attention backward in fp32 for any head size 1..256.
//
// The gradients follow from the proof section (証明) of the formula page
// "トランスフォーマーの注意機構": with a_j the softmax weights of one query row,
// o = sum_j a_j v_j and da_j/ds_l = a_j (delta_jl - a_l),
//   dL/ds_j = a_j (dO . v_j - D),   D = sum_l a_l (dO . v_l) = dO . o,
//   dq = sum_j dL/ds_j k_j / sqrt(d),  dk_j += dL/ds_j q / sqrt(d),
//   dv_j += a_j dO.
// The weights are recomputed from the scores and the forward's log-sum-exp,
// a_j = e^{s_j - lse}.  Plain fp32 arithmetic, not tuned: this path serves
// fp32 and odd head sizes; bf16 uses the matrix-core kernels.
//
// bwd_f32_delta  one wavefront per query row: D = dO . O.
// bwd_f32_dq     one wavefront per query row, 64 keys at a time (one per lane).
// bwd_f32_dkdv   one wavefront per key, 64 query rows at a time (one per lane).
#include "sdpa_internal.h"

#include <math.h>

namespace sdpa {
namespace {

constexpr int kWaves = 4;
constexpr int kMaxD = 256;

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

// number of valid keys of query row i (mask rules of the forward)
__device__ __forceinline__ int valid_keys(const int32_t* key_lens, int b, int i, int Lk, int causal) {
    int n = Lk;
    if (key_lens != nullptr) {
        int L = key_lens[b];
        L = L < 0 ? 0 : L;
        n = L < n ? L : n;
    }
    if (causal && i + 1 < n) n = i + 1;
    return n;
}

__global__ void __launch_bounds__(kWaves * 64) bwd_f32_delta(const float* __restrict__ o,
                                                             const float* __restrict__ dout,
                                                             float* __restrict__ delta,
                                                             long long nrows, int d) {
    const int lane = threadIdx.x & 63;
    const long long row = (long long)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (row >= nrows) return;
    float acc = 0.f;
    for (int t = lane; t < d; t += 64) acc = fmaf(o[(size_t)row * d + t], dout[(size_t)row * d + t], acc);
    acc = wave_sum(acc);
    if (lane == 0) delta[row] = acc;
}

__global__ void __launch_bounds__(kWaves * 64) bwd_f32_dq(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    float* __restrict__ dq, const int32_t* __restrict__ key_lens, long long nrows, int H, int Lq,
    int Lk, int d, int causal, float scale) {
    __shared__ float qs[kWaves][kMaxD];
    __shared__ float gs[kWaves][kMaxD];
    __shared__ float ws[kWaves][64];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const long long row = (long long)blockIdx.x * kWaves + wave;  // flat (b, h, i)
    const bool live = row < nrows;
    const int i = live ? (int)(row % Lq) : 0;
    const long long bh = live ? row / Lq : 0;
    const int n_valid = live ? valid_keys(key_lens, (int)(bh / H), i, Lk, causal) : 0;
    if (live)
        for (int t = lane; t < d; t += 64) {
            qs[wave][t] = q[(size_t)row * d + t];
            gs[wave][t] = dout[(size_t)row * d + t];
        }
    __syncthreads();
    const float L = live ? lse[row] : 0.f;
    const float Dr = live ? delta[row] : 0.f;
    const float* kb = k + (size_t)bh * Lk * d;
    const float* vb = v + (size_t)bh * Lk * d;

    float acc[kMaxD / 64];
#pragma unroll
    for (int r = 0; r < kMaxD / 64; ++r) acc[r] = 0.f;
    for (int j0 = 0; j0 < n_valid; j0 += 64) {
        const int j = j0 + lane;
        float ds = 0.f;
        if (j < n_valid) {
            float z = 0.f, g = 0.f;
            for (int t = 0; t < d; ++t) {
                z = fmaf(qs[wave][t], kb[(size_t)j * d + t], z);
                g = fmaf(gs[wave][t], vb[(size_t)j * d + t], g);
            }
            const float a = expf(z * scale - L);
            ds = a * (g - Dr);
        }
        ws[wave][lane] = ds;
        __builtin_amdgcn_wave_barrier();
        const int cnt = min(64, n_valid - j0);
#pragma unroll
        for (int r = 0; r < kMaxD / 64; ++r) {
            const int t = lane + 64 * r;
            if (t < d) {
                float x = acc[r];
                for (int jj = 0; jj < cnt; ++jj) x = fmaf(ws[wave][jj], kb[(size_t)(j0 + jj) * d + t], x);
                acc[r] = x;
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
    if (live)
#pragma unroll
        for (int r = 0; r < kMaxD / 64; ++r) {
            const int t = lane + 64 * r;
            if (t < d) dq[(size_t)row * d + t] = acc[r] * scale;
        }
}

__global__ void __launch_bounds__(kWaves * 64) bwd_f32_dkdv(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    float* __restrict__ dk, float* __restrict__ dv, const int32_t* __restrict__ key_lens,
    long long nkeys, int H, int Lq, int Lk, int d, int causal, float scale) {
    __shared__ float ks[kWaves][kMaxD];
    __shared__ float vs[kWaves][kMaxD];
    __shared__ float wa[kWaves][64];
    __shared__ float wd[kWaves][64];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const long long krow = (long long)blockIdx.x * kWaves + wave;  // flat (b, h, j)
    const bool live = krow < nkeys;
    const int j = live ? (int)(krow % Lk) : 0;
    const long long bh = live ? krow / Lk : 0;
    // key j is seen by query rows i >= i0 (causal) whose valid length covers it
    bool key_ok = live;
    if (live && key_lens != nullptr) {
        int Lb = key_lens[(int)(bh / H)];
        Lb = Lb < 0 ? 0 : Lb;
        key_ok = j < Lb;
    }
    const int i0 = causal ? j : 0;
    if (live)
        for (int t = lane; t < d; t += 64) {
            ks[wave][t] = k[(size_t)krow * d + t];
            vs[wave][t] = v[(size_t)krow * d + t];
        }
    __syncthreads();
    const float* qb = q + (size_t)bh * Lq * d;
    const float* gb = dout + (size_t)bh * Lq * d;
    const float* lb = lse + (size_t)bh * Lq;
    const float* db = delta + (size_t)bh * Lq;

    float acck[kMaxD / 64], accv[kMaxD / 64];
#pragma unroll
    for (int r = 0; r < kMaxD / 64; ++r) acck[r] = accv[r] = 0.f;
    const int i_end = key_ok ? Lq : i0;
    for (int ib = i0; ib < i_end; ib += 64) {
        const int i = ib + lane;
        float a = 0.f, ds = 0.f;
        if (i < Lq) {
            float z = 0.f, g = 0.f;
            for (int t = 0; t < d; ++t) {
                z = fmaf(qb[(size_t)i * d + t], ks[wave][t], z);
                g = fmaf(gb[(size_t)i * d + t], vs[wave][t], g);
            }
            a = expf(z * scale - lb[i]);
            ds = a * (g - db[i]);
        }
        wa[wave][lane] = a;
        wd[wave][lane] = ds;
        __builtin_amdgcn_wave_barrier();
        const int cnt = min(64, i_end - ib);
#pragma unroll
        for (int r = 0; r < kMaxD / 64; ++r) {
            const int t = lane + 64 * r;
            if (t < d) {
                float xk = acck[r], xv = accv[r];
                for (int ii = 0; ii < cnt; ++ii) {
                    xk = fmaf(wd[wave][ii], qb[(size_t)(ib + ii) * d + t], xk);
                    xv = fmaf(wa[wave][ii], gb[(size_t)(ib + ii) * d + t], xv);
                }
                acck[r] = xk;
                accv[r] = xv;
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
    if (live)
#pragma unroll
        for (int r = 0; r < kMaxD / 64; ++r) {
            const int t = lane + 64 * r;
            if (t < d) {
                dk[(size_t)krow * d + t] = acck[r] * scale;
                dv[(size_t)krow * d + t] = accv[r];
            }
        }
}

}  // namespace

hipError_t launch_bwd_f32(const BwdArgs& a, hipStream_t s) {
    if (a.d < 1 || a.d > kMaxD) return hipErrorInvalidValue;
    const long long rows = (long long)a.B * a.H * a.Lq;
    const long long keys = (long long)a.B * a.H * a.Lk;
    const long long qblocks = (rows + kWaves - 1) / kWaves;
    const long long kblocks = (keys + kWaves - 1) / kWaves;
    if (qblocks < 1 || kblocks < 1 || qblocks > 0x7fffffffLL || kblocks > 0x7fffffffLL)
        return hipErrorInvalidConfiguration;
    const float scale = (float)(1.0 / sqrt((double)a.d));
    const float* q = static_cast<const float*>(a.q);
    const float* k = static_cast<const float*>(a.k);
    const float* v = static_cast<const float*>(a.v);
    const float* dout = static_cast<const float*>(a.dout);
    hipLaunchKernelGGL(bwd_f32_delta, dim3((unsigned)qblocks), dim3(kWaves * 64), 0, s,
                       static_cast<const float*>(a.out), dout, a.delta, rows, a.d);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_f32_dq, dim3((unsigned)qblocks), dim3(kWaves * 64), 0, s, q, k, v, dout,
                       a.lse, a.delta, static_cast<float*>(a.dq), a.key_lens, rows, a.H, a.Lq, a.Lk,
                       a.d, a.causal, scale);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_f32_dkdv, dim3((unsigned)kblocks), dim3(kWaves * 64), 0, s, q, k, v, dout,
                       a.lse, a.delta, static_cast<float*>(a.dk), static_cast<float*>(a.dv),
                       a.key_lens, keys, a.H, a.Lq, a.Lk, a.d, a.causal, scale);
    return hipGetLastError();
}

}  // namespace sdpa
