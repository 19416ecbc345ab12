// Scaled dot-product attention forward in fp32 for any head size 1..256.
//
// O = softmax(Q K^T / sqrt(d)) V per (batch, head) slice ("Aufmerksamkeit ist
// alles, was Sie brauchen", section 3.2.1, eq. (1)).  This path serves small
// and fp32 problems (e.g. the toy model's d = 3 heads from the cookipedia
// article's "トイモデル" section); it favours plain fp32 arithmetic over speed.
//
// One wavefront per query row.  Keys are processed 64 at a time, one key per
// lane: the lane forms the dot product, the wavefront reduces the chunk's
// maximum and sum, and the running output (each lane owns columns lane,
// lane + 64, ...) is rescaled by e^{m_old - m_new} -- exact because weights
// depend only on score differences (formula page "トランスフォーマーの注意機構",
// section 証明, ratio identity).
#include "sdpa_internal.h"

#include <math.h>

namespace sdpa {
namespace {

constexpr int kWaves = 4;
constexpr int kMaxD = 256;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

__global__ void __launch_bounds__(kWaves * 64) fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ out, float* __restrict__ lse, const int32_t* __restrict__ key_lens,
    long long nrows, int H, int Lq, int Lk, int d, int causal, float inv_sqrt_d) {
    __shared__ float qs[kWaves][kMaxD];
    __shared__ float ps[kWaves][64];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const long long row = (long long)blockIdx.x * kWaves + wave;  // flat (b, h, i)
    const bool live = row < nrows;
    const int i = live ? (int)(row % Lq) : 0;
    const long long bh = live ? row / Lq : 0;
    const int b = (int)(bh / H);

    int n_valid = 0;
    if (live) {
        n_valid = Lk;
        if (key_lens != nullptr) {
            int L = key_lens[b];
            L = L < 0 ? 0 : L;
            n_valid = L < n_valid ? L : n_valid;
        }
        if (causal && i + 1 < n_valid) n_valid = i + 1;
        for (int t = lane; t < d; t += 64) qs[wave][t] = q[(size_t)row * d + t];
    }
    __syncthreads();

    const float* kb = k + (size_t)bh * Lk * d;
    const float* vb = v + (size_t)bh * Lk * d;
    float m = -INFINITY, l = 0.f;
    float o[kMaxD / 64];
#pragma unroll
    for (int r = 0; r < kMaxD / 64; ++r) o[r] = 0.f;

    for (int j0 = 0; j0 < n_valid; j0 += 64) {
        const int j = j0 + lane;
        float s = -INFINITY;
        if (j < n_valid) {
            const float* kr = kb + (size_t)j * d;
            float z = 0.f;
            for (int t = 0; t < d; ++t) z = fmaf(qs[wave][t], kr[t], z);
            s = z * inv_sqrt_d;
        }
        const float mn = fmaxf(m, wave_max(s));  // finite: key j0 is valid
        const float alpha = (m == -INFINITY) ? 0.f : expf(m - mn);
        const float pj = (j < n_valid) ? expf(s - mn) : 0.f;
        l = l * alpha + wave_sum(pj);
        ps[wave][lane] = pj;
        __builtin_amdgcn_wave_barrier();
        const int cnt = min(64, n_valid - j0);
#pragma unroll
        for (int r = 0; r < kMaxD / 64; ++r) {
            const int t = lane + 64 * r;
            if (t < d) {
                float acc = o[r] * alpha;
                for (int jj = 0; jj < cnt; ++jj)
                    acc = fmaf(ps[wave][jj], vb[(size_t)(j0 + jj) * d + t], acc);
                o[r] = acc;
            }
        }
        __builtin_amdgcn_wave_barrier();
        m = mn;
    }

    if (live) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        float* orow = out + (size_t)row * d;
#pragma unroll
        for (int r = 0; r < kMaxD / 64; ++r) {
            const int t = lane + 64 * r;
            if (t < d) orow[t] = o[r] * inv;
        }
        if (lse != nullptr && lane == 0) lse[row] = l > 0.f ? m + logf(l) : -INFINITY;
    }
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s) {
    if (a.d < 1 || a.d > kMaxD) return hipErrorInvalidValue;
    const long long rows = (long long)a.B * a.H * a.Lq;
    const long long blocks = (rows + kWaves - 1) / kWaves;
    if (blocks < 1 || blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(fwd_f32_kernel, dim3((unsigned)blocks), dim3(kWaves * 64), 0, s,
                       static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                       static_cast<const float*>(a.v), static_cast<float*>(a.out), a.lse,
                       a.key_lens, rows, a.H, a.Lq, a.Lk, a.d, a.causal,
                       (float)(1.0 / sqrt((double)a.d)));
    return hipGetLastError();
}

}  // namespace sdpa
