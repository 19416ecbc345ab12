// Decode-shaped attention forward in bf16: a few query rows (1..8) against a
// long key/value sequence, the form of generating one token per step
// (cookipedia article, "全体": the decoder produces the output one position
// at a time).  Same operation and masks as the main forward
// (softmax(Q K^T / sqrt(d)) V, "Aufmerksamkeit ist alles, was Sie
// brauchen", section 3.2.1, eq. (1)).
//
// Work of this shape reads every key and value row once and does 4*d flops
// per row and query, so it is bound by HBM bandwidth; a matrix-core product
// would waste 31 of its 32 rows.  The kernel therefore uses the vector ALU:
//
// * Each (b, h) slice is split into key chunks so that the grid covers the
//   GPU even for a handful of slices.  One workgroup (4 wavefronts) takes one
//   chunk; its wavefronts stream interleaved groups of rows with 16-byte
//   loads, each row spread over d/8 lanes (a 64-lane load reads 1 KiB of
//   consecutive rows).
// * Per query row and wavefront: running maximum m (wave-uniform), and per
//   lane group a running sum l and output slice o, rescaled by 2^(m_old -
//   m_new) when m grows -- exact by the ratio identity of the formula page
//   "トランスフォーマーの注意機構", section 証明.
// * The four wavefronts' (m, l, o) are merged in LDS.  With one chunk the
//   result is written as out/lse directly; otherwise the chunk's normalised
//   o and natural-log lse go to the workspace and decode_combine merges the
//   chunks: lse = ln sum_c e^{lse_c}, o = sum_c e^{lse_c - lse} o_c, the
//   same identity with the log-sum-exp of section 広がる学問.  (Merging in
//   the workgroup that finishes a slice's last chunk, found with a counter,
//   saves the second launch but needs a device-scope release and acquire per
//   workgroup, i.e. L2 write-back and invalidation across the XCDs: on
//   MI355X that made a call of 8 slices x 32 chunks 17.9 us against 9.7 us
//   for the two launches.)
#include "sdpa_internal.h"

#include <math.h>

#include <mutex>

namespace sdpa {

// Device memory of sdpa_decode_noalloc: the per-chunk partial results live
// here instead of in a caller workspace.  One copy per GPU, held until the
// process ends; every call on a GPU shares it (calls that overlap on one GPU
// race).  The kernels write every partial they read in the same call, so
// nothing needs clearing between calls.
static __device__ __align__(256) unsigned char scratch[kDecodeNoallocScratchBytes];

namespace {

// Device address of `scratch` per device ordinal, looked up once per device
// (in host code the array's name is only a stand-in for the symbol).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

struct DParams {
    const uint16_t* __restrict__ q;
    const uint16_t* __restrict__ k;
    const uint16_t* __restrict__ v;
    uint16_t* __restrict__ out;
    float* __restrict__ lse;          // may be null
    const int32_t* __restrict__ key_lens;
    float* __restrict__ part_o;       // [splits][B*H*Lq][d] (splits > 1)
    float* __restrict__ part_lse;     // [splits][B*H*Lq]
    int H, Lq, Lk;
    int causal;
    int splits;
    int chunk;                        // keys per split (multiple of the step)
    float scale_log2;                 // log2(e) / sqrt(d)
};

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint16_t to_bf16(float x) {
    const __bf16 b = (__bf16)x;   // round to nearest even
    return __builtin_bit_cast(uint16_t, b);
}

// Sum over the lanes of one row group (CPR consecutive lanes).
template <int CPR>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int off = 1; off < CPR; off <<= 1) x += __shfl_xor(x, off);
    return x;
}
// Maximum / sum over the row groups of a wavefront (lanes l, l ^ CPR, ...).
template <int CPR>
__device__ __forceinline__ float across_groups_max(float x) {
#pragma unroll
    for (int off = CPR; off < 64; off <<= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}
template <int CPR>
__device__ __forceinline__ float across_groups_sum(float x) {
#pragma unroll
    for (int off = CPR; off < 64; off <<= 1) x += __shfl_xor(x, off);
    return x;
}

// Feature f of output row `row` from the per-chunk results: lse = ln sum_c
// e^{lse_c}, o = sum_c e^{lse_c - lse} o_c, accumulated with a running
// maximum over batches of 32 chunks whose loads are all issued before any of
// them is used (one memory latency per batch).  A row with no valid key in
// any chunk gets o = 0, lse = -inf.
template <int D>
__device__ __forceinline__ void merge_chunks(const DParams& p, size_t rows, size_t row, int f) {
    constexpr int NB = 32;
    float M = -INFINITY, Z = 0.f, O = 0.f;
    for (int c0 = 0; c0 < p.splits; c0 += NB) {
        float xs[NB], ys[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            // chunks past the last reload the last one (in bounds) and are
            // dropped below
            const int c = c0 + j < p.splits ? c0 + j : p.splits - 1;
            xs[j] = p.part_lse[(size_t)c * rows + row];
            ys[j] = p.part_o[((size_t)c * rows + row) * D + f];
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const float x = c0 + j < p.splits ? xs[j] : -INFINITY;
            const float mn = fmaxf(M, x);
            const float mref = mn == -INFINITY ? 0.f : mn;
            const float a = __expf(M - mref);                        // 0 while M = -inf
            const float w = x == -INFINITY ? 0.f : __expf(x - mref);  // 0 for an empty chunk
            Z = fmaf(Z, a, w);
            O = fmaf(O, a, w * ys[j]);
            M = mn;
        }
    }
    p.out[row * D + f] = to_bf16(Z > 0.f ? O / Z : 0.f);
    if (p.lse != nullptr && f == 0) p.lse[row] = Z > 0.f ? M + logf(Z) : -INFINITY;
}

template <int D, int NQ>
__global__ void __launch_bounds__(kThreads) decode_kernel(DParams p) {
    constexpr int CPR = D / 8;          // lanes per key row (16 bytes each)
    constexpr int G = 64 / CPR;         // key rows per wavefront step
    constexpr int STEP = G * kWaves;    // key rows per workgroup step
    constexpr int UNROLL = 4;

    __shared__ float red_m[kWaves][NQ], red_l[kWaves][NQ];
    __shared__ float red_o[kWaves][NQ][D];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int grp = lane / CPR;         // key row of this lane inside a step
    const int c = lane % CPR;           // 16-byte chunk (features 8c .. 8c + 7)

    const int split = blockIdx.x % p.splits;
    const int bh = blockIdx.x / p.splits;
    const int b = bh / p.H;
    int kv_len = p.Lk;
    if (p.key_lens != nullptr) {
        int L = p.key_lens[b];
        L = L < 0 ? 0 : L;
        kv_len = L < kv_len ? L : kv_len;
    }
    const int k_lo = split * p.chunk;
    const int k_hi = min(k_lo + p.chunk, kv_len);

    const uint16_t* kb = p.k + (size_t)bh * p.Lk * D;
    const uint16_t* vb = p.v + (size_t)bh * p.Lk * D;
    // this lane's row in step s: k_lo + s * STEP + wave * G + grp.  A lane
    // whose row is at or past k_hi loads row k_lo instead (in bounds: every
    // chunk starts below Lk) and masks it, so every batch of UNROLL steps
    // is loaded whole, without branches.
    const int row0 = k_lo + wave * G + grp;
    const int nsteps = (k_hi - k_lo + STEP - 1) / STEP;
    uint4 kw[UNROLL], vw[UNROLL];
    auto load_batch = [&](int s0) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int row = row0 + (s0 + u) * STEP;
            const int rr = row < k_hi ? row : k_lo;
            kw[u] = *reinterpret_cast<const uint4*>(kb + (size_t)rr * D + 8 * c);
            vw[u] = *reinterpret_cast<const uint4*>(vb + (size_t)rr * D + 8 * c);
        }
    };
    // the first batch goes out before the query rows are read, so that the
    // two memory latencies overlap
    if (nsteps > 0) load_batch(0);

    // query rows (pre-scaled into exp2 units) and their valid key bounds
    float qv[NQ][8];
    int n_valid[NQ];
    const size_t q_row0 = (size_t)bh * p.Lq;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        const int ii = i < p.Lq ? i : p.Lq - 1;
        const uint4 w = *reinterpret_cast<const uint4*>(p.q + (q_row0 + ii) * D + 8 * c);
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            qv[i][2 * e] = bf_lo(ww[e]) * p.scale_log2;
            qv[i][2 * e + 1] = bf_hi(ww[e]) * p.scale_log2;
        }
        int n = k_hi;
        if (p.causal) n = min(n, i + 1);
        n_valid[i] = i < p.Lq ? n : k_lo;   // rows past Lq see nothing
    }

    float m[NQ], l[NQ], o[NQ][8];
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        m[i] = -INFINITY;
        l[i] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[i][e] = 0.f;
    }

    // One key row per lane group: running maximum m (wave-uniform), sum l
    // and output slice o, rescaled when m grows.  While every row so far
    // was masked (m = -inf) the reference is 0, so the rescale factor and
    // the masked weights are exact zeros and nothing branches.
    auto consume = [&](int row, uint4 kv4, uint4 vv4) __attribute__((always_inline)) {
        const uint32_t ka[4] = {kv4.x, kv4.y, kv4.z, kv4.w};
        const uint32_t va[4] = {vv4.x, vv4.y, vv4.z, vv4.w};
        float kf[8], vf[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            kf[2 * e] = bf_lo(ka[e]);
            kf[2 * e + 1] = bf_hi(ka[e]);
            vf[2 * e] = bf_lo(va[e]);
            vf[2 * e + 1] = bf_hi(va[e]);
        }
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            float z = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) z = fmaf(qv[i][e], kf[e], z);
            z = group_sum<CPR>(z);
            const bool ok = row < n_valid[i];
            const float mn = fmaxf(m[i], across_groups_max<CPR>(ok ? z : -INFINITY));
            const float mref = mn == -INFINITY ? 0.f : mn;
            const float alpha = __builtin_amdgcn_exp2f(m[i] - mref);   // 0 when m was -inf
            const float pj = ok ? __builtin_amdgcn_exp2f(z - mref) : 0.f;
            l[i] = fmaf(l[i], alpha, pj);
#pragma unroll
            for (int e = 0; e < 8; ++e) o[i][e] = fmaf(o[i][e], alpha, pj * vf[e]);
            m[i] = mn;
        }
    };

    // batches of UNROLL steps; the next batch's loads go out before the
    // current one is consumed
    for (int s = 0; s < nsteps; s += UNROLL) {
        uint4 kc[UNROLL], vc[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            kc[u] = kw[u];
            vc[u] = vw[u];
        }
        if (s + UNROLL < nsteps) load_batch(s + UNROLL);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) consume(row0 + (s + u) * STEP, kc[u], vc[u]);
    }

    // merge the row groups of the wavefront (same m), then the wavefronts
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        l[i] = across_groups_sum<CPR>(l[i]);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[i][e] = across_groups_sum<CPR>(o[i][e]);
        if (lane < CPR) {
#pragma unroll
            for (int e = 0; e < 8; ++e) red_o[wave][i][8 * c + e] = o[i][e];
        }
        if (lane == 0) {
            red_m[wave][i] = m[i];
            red_l[wave][i] = l[i];
        }
    }
    __syncthreads();

    // thread t merges feature t % D of row t / D
    for (int t = threadIdx.x; t < NQ * D; t += kThreads) {
        const int i = t / D, f = t % D;
        if (i >= p.Lq) continue;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red_m[w][i]);
        float L = 0.f, O = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float sc = __builtin_amdgcn_exp2f(red_m[w][i] - M);   // 0 for an empty wavefront
                L = fmaf(red_l[w][i], sc, L);
                O = fmaf(red_o[w][i][f], sc, O);
            }
        }
        const size_t row = q_row0 + i;
        const float on = L > 0.f ? O / L : 0.f;
        const float ls = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
        if (p.splits == 1) {
            p.out[row * D + f] = to_bf16(on);
            if (p.lse != nullptr && f == 0) p.lse[row] = ls;
        } else {
            const size_t rows = (size_t)gridDim.x / p.splits * p.Lq;
            p.part_o[((size_t)split * rows + row) * D + f] = on;
            if (f == 0) p.part_lse[(size_t)split * rows + row] = ls;
        }
    }
}

// Thread t merges feature t % D of output row t / D (merge_chunks).
template <int D>
__global__ void __launch_bounds__(256) decode_combine(DParams p, long long rows) {
    const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
    if (t >= rows * D) return;
    merge_chunks<D>(p, (size_t)rows, (size_t)(t / D), (int)(t % D));
}

template <int D, int NQ>
hipError_t launch_nq(const DecodeArgs& a, const DecodePlan& plan, hipStream_t s) {
    DParams p;
    p.q = static_cast<const uint16_t*>(a.q);
    p.k = static_cast<const uint16_t*>(a.k);
    p.v = static_cast<const uint16_t*>(a.v);
    p.out = static_cast<uint16_t*>(a.out);
    p.lse = a.lse;
    p.key_lens = a.key_lens;
    p.H = a.H;
    p.Lq = a.Lq;
    p.Lk = a.Lk;
    p.causal = a.causal;
    p.splits = plan.splits;
    p.chunk = plan.chunk;
    p.scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    const long long rows = (long long)a.B * a.H * a.Lq;
    p.part_lse = static_cast<float*>(a.workspace);
    p.part_o = p.part_lse + (size_t)plan.splits * rows;
    const long long grid = (long long)a.B * a.H * plan.splits;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((decode_kernel<D, NQ>), dim3((unsigned)grid), dim3(kThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || plan.splits == 1) return e;
    const long long threads = rows * D;
    hipLaunchKernelGGL((decode_combine<D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, p, rows);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, const DecodePlan& plan, hipStream_t s) {
    if (a.Lq <= 1) return launch_nq<D, 1>(a, plan, s);
    if (a.Lq <= 2) return launch_nq<D, 2>(a, plan, s);
    if (a.Lq <= 4) return launch_nq<D, 4>(a, plan, s);
    return launch_nq<D, 8>(a, plan, s);
}

}  // namespace

DecodePlan plan_decode(int B, int H, int Lq, int Lk, int d, int num_cus) {
    DecodePlan plan;
    // With at least two slices per compute unit the main forward kernel,
    // one workgroup streaming a whole slice's K and V through LDS, moves the
    // bytes faster than the split kernel below (measured on MI355X, Lq = 1,
    // warmed clocks: 3-5% at d = 128 with 512-1536 slices of 2048 keys, 5-16%
    // at d = 64), except for d = 128 beyond 4096 keys, where the split
    // kernel stays about 3% ahead.
    const long long n_slices = (long long)B * H;
    const int cus = num_cus > 0 ? num_cus : 256;
    plan.use_forward = n_slices >= 2LL * cus && (d == 64 || Lk <= 4096) &&
                       (long long)Lk * d * 2 < (1LL << 32);
    if (plan.use_forward) {
        plan.splits = 1;
        plan.chunk = Lk;
        plan.workspace_bytes = 0;
        return plan;
    }
    // step of the kernel: 4 wavefronts x 64/(d/8) rows; chunks of about
    // 256 KiB of keys and values, and at least 4 workgroups per compute
    // unit, so that chunks of uneven length (key_lens) still balance; never
    // chunks under 4 steps
    const int step = kWaves * (64 / (d / 8));
    const long long slices = (long long)B * H;
    const long long target_keys = (256LL << 10) / (4LL * d);
    long long splits = (Lk + target_keys - 1) / target_keys;
    const long long want = 4LL * num_cus;
    if (slices * splits < want) splits = (want + slices - 1) / slices;
    const long long max_splits = (Lk + 4LL * step - 1) / (4LL * step);
    if (splits > max_splits) splits = max_splits;
    if (splits < 1) splits = 1;
    long long chunk = (Lk + splits - 1) / splits;
    chunk = (chunk + step - 1) / step * step;
    splits = (Lk + chunk - 1) / chunk;
    plan.splits = (int)splits;
    plan.chunk = (int)chunk;
    const long long rows = (long long)B * H * Lq;
    plan.workspace_bytes = splits > 1 ? (size_t)splits * rows * (size_t)(d + 1) * sizeof(float) : 0;
    return plan;
}

hipError_t decode_scratch_init(int device) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[device] != nullptr) return hipSuccess;
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != device) (void)hipSetDevice(cur);
    if (e != hipSuccess) return e;
    g_scratch_ptr[device] = ptr;
    return hipSuccess;
}

void* decode_scratch_ptr(int device) {
    if (device < 0 || device >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    return g_scratch_ptr[device];
}

hipError_t launch_decode_bf16(const DecodeArgs& a, const DecodePlan& plan, hipStream_t s) {
    if (a.Lq < 1 || a.Lq > kDecodeMaxLq) return hipErrorInvalidValue;
    if (plan.use_forward) {
        FwdArgs f;
        f.q = a.q; f.k = a.k; f.v = a.v; f.out = a.out; f.lse = a.lse; f.key_lens = a.key_lens;
        f.B = a.B; f.H = a.H; f.Lq = a.Lq; f.Lk = a.Lk; f.d = a.d; f.causal = a.causal;
        f.num_cus = a.num_cus;
        f.set_contiguous();
        const Bf16Tile tile{a.d, 64, 4, 1, 0, nullptr};
        return launch_fwd_bf16(f, tile, s);
    }
    if (a.d == 128) return launch_d<128>(a, plan, s);
    if (a.d == 64) return launch_d<64>(a, plan, s);
    return hipErrorInvalidValue;
}

}  // namespace sdpa
