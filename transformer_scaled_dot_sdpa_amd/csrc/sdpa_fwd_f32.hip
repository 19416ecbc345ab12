// Scaled dot-product attention forward in fp32 for any head size 1..256
// (values of their own width 1..256), any strides, scale and additive mask.
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

struct F32Params {
    const float* q;
    const float* k;
    const float* v;
    float* out;
    float* lse;
    const int32_t* key_lens;
    long long nrows;
    int H, Lq, Lk, d, dv, causal;
    float scale;
    long long q_sb, q_sh, k_sb, k_sh, v_sb, v_sh, o_sb, o_sh;
    int q_sl, k_sl, v_sl, o_sl;
    const float* mask;
    long long m_sb, m_sh;
    int m_sl;
};

__global__ void __launch_bounds__(kWaves * 64) fwd_f32_kernel(F32Params p) {
    __shared__ float qs[kWaves][kMaxD];
    __shared__ float ps[kWaves][64];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const long long row = (long long)blockIdx.x * kWaves + wave;  // flat (b, h, i)
    const bool live = row < p.nrows;
    const int i = live ? (int)(row % p.Lq) : 0;
    const long long bh = live ? row / p.Lq : 0;
    const int b = (int)(bh / p.H);
    const int hh = (int)(bh % p.H);
    const int d = p.d, dv = p.dv;

    int n_valid = 0;
    if (live) {
        n_valid = p.Lk;
        if (p.key_lens != nullptr) {
            int L = p.key_lens[b];
            L = L < 0 ? 0 : L;
            n_valid = L < n_valid ? L : n_valid;
        }
        if (p.causal && i + 1 < n_valid) n_valid = i + 1;
        const float* qrow = p.q + b * p.q_sb + hh * p.q_sh + (long long)i * p.q_sl;
        for (int t = lane; t < d; t += 64) qs[wave][t] = qrow[t];
    }
    __syncthreads();

    const float* kb = p.k + b * p.k_sb + hh * p.k_sh;
    const float* vb = p.v + b * p.v_sb + hh * p.v_sh;
    const float* mrow = p.mask ? p.mask + b * p.m_sb + hh * p.m_sh + (long long)i * p.m_sl : nullptr;
    float m = -INFINITY, l = 0.f;
    float o[kMaxD / 64];
#pragma unroll
    for (int r = 0; r < kMaxD / 64; ++r) o[r] = 0.f;

    for (int j0 = 0; j0 < n_valid; j0 += 64) {
        const int j = j0 + lane;
        float s = -INFINITY;
        if (j < n_valid) {
            const float* kr = kb + (long long)j * p.k_sl;
            float z = 0.f;
            for (int t = 0; t < d; ++t) z = fmaf(qs[wave][t], kr[t], z);
            s = z * p.scale;
            if (mrow) s += mrow[j];
        }
        const float mn = fmaxf(m, wave_max(s));
        // mn = -inf: every key so far masked; nothing to add yet
        const float alpha = (m == -INFINITY) ? 0.f : expf(m - mn);
        const float pj = (j < n_valid && mn != -INFINITY) ? expf(s - mn) : 0.f;
        l = l * alpha + wave_sum(pj);
        ps[wave][lane] = pj;
        __builtin_amdgcn_wave_barrier();
        const int cnt = min(64, n_valid - j0);
#pragma unroll
        for (int r = 0; r < kMaxD / 64; ++r) {
            const int t = lane + 64 * r;
            if (t < dv) {
                float acc = o[r] * alpha;
                for (int jj = 0; jj < cnt; ++jj)
                    acc = fmaf(ps[wave][jj], vb[(long long)(j0 + jj) * p.v_sl + t], acc);
                o[r] = acc;
            }
        }
        __builtin_amdgcn_wave_barrier();
        m = mn;
    }

    if (live) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        float* orow = p.out + b * p.o_sb + hh * p.o_sh + (long long)i * p.o_sl;
#pragma unroll
        for (int r = 0; r < kMaxD / 64; ++r) {
            const int t = lane + 64 * r;
            if (t < dv) orow[t] = o[r] * inv;
        }
        if (p.lse != nullptr && lane == 0) p.lse[row] = l > 0.f ? m + logf(l) : -INFINITY;
    }
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s) {
    if (a.d < 1 || a.d > kMaxD || a.dv < 1 || a.dv > kMaxD) return hipErrorInvalidValue;
    const long long rows = (long long)a.B * a.H * a.Lq;
    const long long blocks = (rows + kWaves - 1) / kWaves;
    if (blocks < 1 || blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    F32Params p;
    p.q = static_cast<const float*>(a.q);
    p.k = static_cast<const float*>(a.k);
    p.v = static_cast<const float*>(a.v);
    p.out = static_cast<float*>(a.out);
    p.lse = a.lse;
    p.key_lens = a.key_lens;
    p.nrows = rows;
    p.H = a.H; p.Lq = a.Lq; p.Lk = a.Lk; p.d = a.d; p.dv = a.dv; p.causal = a.causal;
    p.scale = a.scale > 0.f ? a.scale : (float)(1.0 / sqrt((double)a.d));
    p.q_sb = a.q_sb; p.q_sh = a.q_sh; p.q_sl = a.q_sl;
    p.k_sb = a.k_sb; p.k_sh = a.k_sh; p.k_sl = a.k_sl;
    p.v_sb = a.v_sb; p.v_sh = a.v_sh; p.v_sl = a.v_sl;
    p.o_sb = a.o_sb; p.o_sh = a.o_sh; p.o_sl = a.o_sl;
    p.mask = a.mask;
    p.m_sb = a.m_sb; p.m_sh = a.m_sh; p.m_sl = a.m_sl;
    hipLaunchKernelGGL(fwd_f32_kernel, dim3((unsigned)blocks), dim3(kWaves * 64), 0, s, p);
    return hipGetLastError();
}

}  // namespace sdpa
