// C ABI of the attention forward, decode forward and backward (declared in
// include/sdpa.h): handle management, argument validation and dispatch to
// the HIP kernels.
#include "sdpa.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <new>
#include <utility>

#include "sdpa_internal.h"

struct sdpa_ctx {
    sdpa_dtype_t dtype;
    int device;
    int num_cus;
    char arch[64];
};

namespace {

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

// a * b * c * d without overflowing int64 (all factors >= 1).
bool mul_fits(long long a, long long b, long long c, long long d, long long* r) {
    long long x = a;
    for (long long f : {b, c, d}) {
        if (x > INT64_MAX / f) return false;
        x *= f;
    }
    *r = x;
    return true;
}

bool is_gfx950(const char* arch) { return strncmp(arch, "gfx950", 6) == 0; }

// Resolved strides of one [B, H, L, width] view and its extent in elements
// (from the base to one past the last element).
struct View {
    long long sb, sh, sl;
    long long extent;
};

// false: invalid layout (negative stride, row stride under the width, or an
// extent that overflows int64).
bool resolve_view(const sdpa_layout_t& lay, long long B, long long H, long long L, long long width,
                  View* v) {
    if (lay.row == 0) {
        v->sl = width;
        v->sh = L * width;
        v->sb = H * L * width;
    } else {
        if (lay.batch < 0 || lay.head < 0 || lay.row < width) return false;
        v->sb = lay.batch;
        v->sh = lay.head;
        v->sl = lay.row;
    }
    // extent = (B-1) sb + (H-1) sh + (L-1) sl + width, without overflow
    long long e = width;
    for (auto [n, st] : {std::pair<long long, long long>{B - 1, v->sb}, {H - 1, v->sh}, {L - 1, v->sl}}) {
        if (st != 0 && n > (INT64_MAX - e) / st) return false;
        e += n * st;
    }
    v->extent = e;
    return true;
}

// true if no two elements of the view share an address: every dimension of
// size > 1 has a nonzero stride, and taken in increasing stride order each
// stride is at least the span of the dimensions before it (width elements
// for the contiguous last dimension).
bool one_to_one(const View& v, long long B, long long H, long long L, long long width) {
    struct Dim { long long n, st; };
    Dim dims[3] = {{B, v.sb}, {H, v.sh}, {L, v.sl}};
    for (const Dim& d : dims)
        if (d.n > 1 && d.st == 0) return false;
    // sort the three by stride (insertion sort)
    for (int i = 1; i < 3; ++i)
        for (int j = i; j > 0 && dims[j].st < dims[j - 1].st; --j) std::swap(dims[j], dims[j - 1]);
    long long span = width;
    for (const Dim& d : dims) {
        if (d.n <= 1) continue;
        if (d.st < span) return false;
        span += (d.n - 1) * d.st;   // no overflow: the extent was checked by resolve_view
    }
    return true;
}

}  // namespace

extern "C" {

sdpa_status_t sdpa_create(sdpa_handle_t* h, sdpa_dtype_t dtype, int device) {
    if (h == nullptr) return SDPA_STATUS_INVALID_VALUE;
    if (dtype != SDPA_DTYPE_FP32 && dtype != SDPA_DTYPE_BF16) return SDPA_STATUS_INVALID_VALUE;
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess) {
        (void)hipGetLastError();
        return SDPA_STATUS_HIP_ERROR;
    }
    if (device < 0 || device >= count) return SDPA_STATUS_INVALID_VALUE;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) {
        (void)hipGetLastError();
        return SDPA_STATUS_HIP_ERROR;
    }
    if (dtype == SDPA_DTYPE_BF16 && !is_gfx950(prop.gcnArchName)) return SDPA_STATUS_NOT_SUPPORTED;
    // address of the no-allocation decode scratch on this device (once per device)
    if (dtype == SDPA_DTYPE_BF16 && sdpa::decode_scratch_init(device) != hipSuccess) {
        (void)hipGetLastError();
        return SDPA_STATUS_HIP_ERROR;
    }
    sdpa_ctx* c = new (std::nothrow) sdpa_ctx;
    if (c == nullptr) return SDPA_STATUS_ALLOC_FAILED;
    c->dtype = dtype;
    c->device = device;
    c->num_cus = prop.multiProcessorCount;
    strncpy(c->arch, prop.gcnArchName, sizeof(c->arch) - 1);
    c->arch[sizeof(c->arch) - 1] = '\0';
    *h = c;
    return SDPA_STATUS_SUCCESS;
}

sdpa_status_t sdpa_destroy(sdpa_handle_t h) {
    delete h;
    return SDPA_STATUS_SUCCESS;
}

const char* sdpa_status_string(sdpa_status_t s) {
    switch (s) {
        case SDPA_STATUS_SUCCESS: return "SDPA_STATUS_SUCCESS";
        case SDPA_STATUS_INVALID_VALUE: return "SDPA_STATUS_INVALID_VALUE";
        case SDPA_STATUS_NOT_SUPPORTED: return "SDPA_STATUS_NOT_SUPPORTED";
        case SDPA_STATUS_HIP_ERROR: return "SDPA_STATUS_HIP_ERROR";
        case SDPA_STATUS_ALLOC_FAILED: return "SDPA_STATUS_ALLOC_FAILED";
    }
    return "SDPA_STATUS_UNKNOWN";
}

const char* sdpa_kernel_name(sdpa_handle_t h, int B, int H, int Lq, int Lk, int d_k,
                             int causal, int has_key_lens) {
    if (h == nullptr || B < 1 || H < 1 || Lq < 1 || Lk < 1 || d_k < 1) return nullptr;
    if (h->dtype == SDPA_DTYPE_FP32) return d_k <= 256 ? "f32_wave_per_row" : nullptr;
    sdpa::Bf16Tile t;
    if (!sdpa::select_bf16_tile(d_k, causal, has_key_lens, (long long)B * H, Lq, Lk, h->num_cus, false, &t))
        return nullptr;
    return t.name;
}

sdpa_status_t sdpa_forward(sdpa_handle_t h, const void* q, const void* k, const void* v,
                           void* out, float* lse, int B, int H, int Lq, int Lk, int d_k,
                           int causal, const int32_t* key_lens, void* stream) {
    if (h == nullptr || q == nullptr || k == nullptr || v == nullptr || out == nullptr)
        return SDPA_STATUS_INVALID_VALUE;
    if (B < 1 || H < 1 || Lq < 1 || Lk < 1 || d_k < 1) return SDPA_STATUS_INVALID_VALUE;
    if (causal != 0 && causal != 1) return SDPA_STATUS_INVALID_VALUE;
    long long nq = 0, nkv = 0;
    if (!mul_fits(B, H, Lq, d_k, &nq) || !mul_fits(B, H, Lk, d_k, &nkv))
        return SDPA_STATUS_INVALID_VALUE;
    const size_t esz = h->dtype == SDPA_DTYPE_BF16 ? 2 : 4;
    if ((unsigned long long)nq > SIZE_MAX / esz || (unsigned long long)nkv > SIZE_MAX / esz)
        return SDPA_STATUS_INVALID_VALUE;
    const size_t bq = (size_t)nq * esz, bkv = (size_t)nkv * esz;
    if (overlaps(out, bq, q, bq) || overlaps(out, bq, k, bkv) || overlaps(out, bq, v, bkv))
        return SDPA_STATUS_INVALID_VALUE;
    if (lse != nullptr) {
        const size_t bl = (size_t)B * H * Lq * sizeof(float);
        if (overlaps(lse, bl, out, bq) || overlaps(lse, bl, q, bq) || overlaps(lse, bl, k, bkv) ||
            overlaps(lse, bl, v, bkv))
            return SDPA_STATUS_INVALID_VALUE;
        if (reinterpret_cast<uintptr_t>(lse) % alignof(float) != 0) return SDPA_STATUS_INVALID_VALUE;
    }

    sdpa::FwdArgs a;
    a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse; a.key_lens = key_lens;
    a.B = B; a.H = H; a.Lq = Lq; a.Lk = Lk; a.d = d_k; a.causal = causal;
    a.num_cus = h->num_cus;
    a.set_contiguous();

    sdpa::Bf16Tile tile;
    if (h->dtype == SDPA_DTYPE_BF16) {
        if (!sdpa::select_bf16_tile(d_k, causal, key_lens != nullptr, (long long)B * H, Lq, Lk, h->num_cus,
                                    false, &tile))
            return SDPA_STATUS_NOT_SUPPORTED;
        for (const void* p : {q, k, v, (const void*)out})
            if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return SDPA_STATUS_NOT_SUPPORTED;
        // buffer loads address a (b, h) slice of k and v with 32-bit offsets
        if ((long long)Lk * d_k * 2 >= (1LL << 32)) return SDPA_STATUS_NOT_SUPPORTED;
    } else {
        if (d_k > 256) return SDPA_STATUS_NOT_SUPPORTED;
        for (const void* p : {q, k, v, (const void*)out})
            if (reinterpret_cast<uintptr_t>(p) % alignof(float) != 0) return SDPA_STATUS_INVALID_VALUE;
    }
    if (key_lens != nullptr && reinterpret_cast<uintptr_t>(key_lens) % alignof(int32_t) != 0)
        return SDPA_STATUS_INVALID_VALUE;

    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) {
        (void)hipGetLastError();
        return SDPA_STATUS_HIP_ERROR;
    }
    if (cur != h->device && hipSetDevice(h->device) != hipSuccess) {
        (void)hipGetLastError();
        return SDPA_STATUS_HIP_ERROR;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = h->dtype == SDPA_DTYPE_BF16 ? sdpa::launch_fwd_bf16(a, tile, s)
                                               : sdpa::launch_fwd_f32(a, s);
    if (cur != h->device) (void)hipSetDevice(cur);
    return e == hipSuccess ? SDPA_STATUS_SUCCESS : SDPA_STATUS_HIP_ERROR;
}

sdpa_status_t sdpa_backward(sdpa_handle_t h, const void* q, const void* k, const void* v,
                            const void* out, const void* dout, const float* lse, float* delta,
                            void* dq, void* dk, void* dv, int B, int H, int Lq, int Lk, int d_k,
                            int causal, const int32_t* key_lens, void* stream) {
    if (h == nullptr || q == nullptr || k == nullptr || v == nullptr || out == nullptr ||
        dout == nullptr || lse == nullptr || delta == nullptr || dq == nullptr || dk == nullptr ||
        dv == nullptr)
        return SDPA_STATUS_INVALID_VALUE;
    if (B < 1 || H < 1 || Lq < 1 || Lk < 1 || d_k < 1) return SDPA_STATUS_INVALID_VALUE;
    if (causal != 0 && causal != 1) return SDPA_STATUS_INVALID_VALUE;
    long long nq = 0, nkv = 0;
    if (!mul_fits(B, H, Lq, d_k, &nq) || !mul_fits(B, H, Lk, d_k, &nkv))
        return SDPA_STATUS_INVALID_VALUE;
    const size_t esz = h->dtype == SDPA_DTYPE_BF16 ? 2 : 4;
    if ((unsigned long long)nq > SIZE_MAX / esz || (unsigned long long)nkv > SIZE_MAX / esz)
        return SDPA_STATUS_INVALID_VALUE;
    const size_t bq = (size_t)nq * esz, bkv = (size_t)nkv * esz;
    const size_t bl = (size_t)B * H * Lq * sizeof(float);
    // every written buffer is disjoint from every other buffer
    struct Span { const void* p; size_t n; };
    const Span inputs[] = {{q, bq}, {k, bkv}, {v, bkv}, {out, bq}, {dout, bq}, {lse, bl}};
    const Span outputs[] = {{delta, bl}, {dq, bq}, {dk, bkv}, {dv, bkv}};
    for (size_t o = 0; o < 4; ++o) {
        for (const Span& in : inputs)
            if (overlaps(outputs[o].p, outputs[o].n, in.p, in.n)) return SDPA_STATUS_INVALID_VALUE;
        for (size_t p = o + 1; p < 4; ++p)
            if (overlaps(outputs[o].p, outputs[o].n, outputs[p].p, outputs[p].n))
                return SDPA_STATUS_INVALID_VALUE;
    }
    if (reinterpret_cast<uintptr_t>(lse) % alignof(float) != 0 ||
        reinterpret_cast<uintptr_t>(delta) % alignof(float) != 0)
        return SDPA_STATUS_INVALID_VALUE;
    if (key_lens != nullptr && reinterpret_cast<uintptr_t>(key_lens) % alignof(int32_t) != 0)
        return SDPA_STATUS_INVALID_VALUE;
    if (h->dtype == SDPA_DTYPE_BF16) {
        if (d_k != 64 && d_k != 128) return SDPA_STATUS_NOT_SUPPORTED;
        for (const void* p : {q, k, v, out, dout, (const void*)dq, (const void*)dk, (const void*)dv})
            if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return SDPA_STATUS_NOT_SUPPORTED;
        // buffer loads address a (b, h) slice of q, dO (dK/dV pass) and k, v
        // (dQ pass) with 32-bit offsets
        if ((long long)Lq * d_k * 2 >= (1LL << 32) || (long long)Lk * d_k * 2 >= (1LL << 32))
            return SDPA_STATUS_NOT_SUPPORTED;
    } else {
        if (d_k > 256) return SDPA_STATUS_NOT_SUPPORTED;
        for (const void* p : {q, k, v, out, dout, (const void*)dq, (const void*)dk, (const void*)dv})
            if (reinterpret_cast<uintptr_t>(p) % alignof(float) != 0) return SDPA_STATUS_INVALID_VALUE;
    }

    sdpa::BwdArgs a;
    a.q = q; a.k = k; a.v = v; a.out = out; a.dout = dout; a.lse = lse; a.delta = delta;
    a.dq = dq; a.dk = dk; a.dv = dv; a.key_lens = key_lens;
    a.B = B; a.H = H; a.Lq = Lq; a.Lk = Lk; a.d = d_k; a.causal = causal;
    a.num_cus = h->num_cus;

    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) {
        (void)hipGetLastError();
        return SDPA_STATUS_HIP_ERROR;
    }
    if (cur != h->device && hipSetDevice(h->device) != hipSuccess) {
        (void)hipGetLastError();
        return SDPA_STATUS_HIP_ERROR;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = h->dtype == SDPA_DTYPE_BF16 ? sdpa::launch_bwd_bf16(a, s) : sdpa::launch_bwd_f32(a, s);
    if (cur != h->device) (void)hipSetDevice(cur);
    return e == hipSuccess ? SDPA_STATUS_SUCCESS : SDPA_STATUS_HIP_ERROR;
}

sdpa_status_t sdpa_forward_ex(sdpa_handle_t h, const sdpa_forward_desc_t* desc, void* stream) {
    if (h == nullptr || desc == nullptr) return SDPA_STATUS_INVALID_VALUE;
    const sdpa_forward_desc_t& d = *desc;
    if (d.q == nullptr || d.k == nullptr || d.v == nullptr || d.out == nullptr)
        return SDPA_STATUS_INVALID_VALUE;
    if (d.B < 1 || d.H < 1 || d.Lq < 1 || d.Lk < 1 || d.d_k < 1) return SDPA_STATUS_INVALID_VALUE;
    if (d.causal != 0 && d.causal != 1) return SDPA_STATUS_INVALID_VALUE;
    const int dv = d.d_v > 0 ? d.d_v : d.d_k;
    View vq, vk, vv, vo, vm;
    if (!resolve_view(d.q_layout, d.B, d.H, d.Lq, d.d_k, &vq) ||
        !resolve_view(d.k_layout, d.B, d.H, d.Lk, d.d_k, &vk) ||
        !resolve_view(d.v_layout, d.B, d.H, d.Lk, dv, &vv) ||
        !resolve_view(d.out_layout, d.B, d.H, d.Lq, dv, &vo))
        return SDPA_STATUS_INVALID_VALUE;
    // several (b, h, row) of out at one address would be written by several
    // workgroups at once
    if (!one_to_one(vo, d.B, d.H, d.Lq, dv)) return SDPA_STATUS_INVALID_VALUE;
    if (d.mask != nullptr) {
        sdpa_layout_t ml = d.mask_layout;
        if (ml.row == 0) ml.row = d.Lk;   // all zero: one shared [Lq, Lk] matrix
        if (!resolve_view(ml, d.B, d.H, d.Lq, d.Lk, &vm)) return SDPA_STATUS_INVALID_VALUE;
    }
    const bool bf16 = h->dtype == SDPA_DTYPE_BF16;
    const size_t esz = bf16 ? 2 : 4;
    for (const View* v : {&vq, &vk, &vv, &vo})
        if ((unsigned long long)v->extent > SIZE_MAX / esz) return SDPA_STATUS_INVALID_VALUE;
    const size_t bl = (size_t)d.B * d.H * d.Lq * sizeof(float);
    const size_t bo = (size_t)vo.extent * esz;
    // out (and lse) must not overlap anything read
    struct Span { const void* p; size_t n; };
    const Span reads[] = {{d.q, (size_t)vq.extent * esz}, {d.k, (size_t)vk.extent * esz},
                          {d.v, (size_t)vv.extent * esz},
                          {d.mask, d.mask ? (size_t)vm.extent * 4 : 0}};
    for (const Span& r : reads) {
        if (r.p == nullptr || r.n == 0) continue;
        if (overlaps(d.out, bo, r.p, r.n)) return SDPA_STATUS_INVALID_VALUE;
        if (d.lse != nullptr && overlaps(d.lse, bl, r.p, r.n)) return SDPA_STATUS_INVALID_VALUE;
    }
    if (d.lse != nullptr && overlaps(d.lse, bl, d.out, bo)) return SDPA_STATUS_INVALID_VALUE;
    if (d.lse != nullptr && reinterpret_cast<uintptr_t>(d.lse) % alignof(float) != 0)
        return SDPA_STATUS_INVALID_VALUE;
    if (d.key_lens != nullptr && reinterpret_cast<uintptr_t>(d.key_lens) % alignof(int32_t) != 0)
        return SDPA_STATUS_INVALID_VALUE;
    if (d.mask != nullptr && reinterpret_cast<uintptr_t>(d.mask) % alignof(float) != 0)
        return SDPA_STATUS_INVALID_VALUE;

    sdpa::Bf16Tile tile{};
    if (bf16) {
        if ((d.d_k != 64 && d.d_k != 128) || (dv != 64 && dv != 128)) return SDPA_STATUS_NOT_SUPPORTED;
        // d_v != d_k and the additive mask are compiled into the default tile only
        const bool general = dv != d.d_k || d.mask != nullptr;
        if (d.tile != nullptr) {
            if (!sdpa::find_bf16_tile(d.d_k, d.tile, &tile)) return SDPA_STATUS_NOT_SUPPORTED;
            // the default geometry (64 keys, 4 wavefronts, no key split)
            if (general && (tile.bc != 64 || tile.waves != 4 || tile.ks != 1)) return SDPA_STATUS_NOT_SUPPORTED;
        } else {
            sdpa::select_bf16_tile(d.d_k, d.causal, d.key_lens != nullptr, (long long)d.B * d.H, d.Lq, d.Lk,
                                   h->num_cus, general, &tile);
        }
        for (const void* p : {d.q, d.k, d.v, (const void*)d.out})
            if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return SDPA_STATUS_NOT_SUPPORTED;
        for (const View* v : {&vq, &vk, &vv, &vo})
            if (v->sb % 8 != 0 || v->sh % 8 != 0 || v->sl % 8 != 0) return SDPA_STATUS_NOT_SUPPORTED;
        // buffer loads address a (b, h) slice of k and v with 32-bit offsets
        if ((long long)d.Lk * vk.sl * 2 >= (1LL << 32) || (long long)d.Lk * vv.sl * 2 >= (1LL << 32))
            return SDPA_STATUS_NOT_SUPPORTED;
        if (vq.sl > INT32_MAX || vo.sl > INT32_MAX) return SDPA_STATUS_NOT_SUPPORTED;
        if (d.mask != nullptr && ((long long)(d.Lq - 1) * vm.sl + d.Lk) * 4 >= (1LL << 31))
            return SDPA_STATUS_NOT_SUPPORTED;
    } else {
        if (d.d_k > 256 || dv > 256) return SDPA_STATUS_NOT_SUPPORTED;
        if (d.tile != nullptr && strcmp(d.tile, "f32_wave_per_row") != 0) return SDPA_STATUS_NOT_SUPPORTED;
        for (const void* p : {d.q, d.k, d.v, (const void*)d.out})
            if (reinterpret_cast<uintptr_t>(p) % alignof(float) != 0) return SDPA_STATUS_INVALID_VALUE;
        for (const View* v : {&vq, &vk, &vv, &vo})
            if (v->sl > INT32_MAX) return SDPA_STATUS_NOT_SUPPORTED;
        if (d.mask != nullptr && vm.sl > INT32_MAX) return SDPA_STATUS_NOT_SUPPORTED;
    }

    sdpa::FwdArgs a;
    a.q = d.q; a.k = d.k; a.v = d.v; a.out = d.out; a.lse = d.lse; a.key_lens = d.key_lens;
    a.B = d.B; a.H = d.H; a.Lq = d.Lq; a.Lk = d.Lk; a.d = d.d_k; a.dv = dv; a.causal = d.causal;
    a.num_cus = h->num_cus;
    a.q_sb = vq.sb; a.q_sh = vq.sh; a.q_sl = (int)vq.sl;
    a.k_sb = vk.sb; a.k_sh = vk.sh; a.k_sl = (int)vk.sl;
    a.v_sb = vv.sb; a.v_sh = vv.sh; a.v_sl = (int)vv.sl;
    a.o_sb = vo.sb; a.o_sh = vo.sh; a.o_sl = (int)vo.sl;
    a.scale = d.scale > 0.f ? d.scale : 0.f;
    a.mask = d.mask;
    a.m_sb = d.mask ? vm.sb : 0; a.m_sh = d.mask ? vm.sh : 0; a.m_sl = d.mask ? (int)vm.sl : 0;

    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) {
        (void)hipGetLastError();
        return SDPA_STATUS_HIP_ERROR;
    }
    if (cur != h->device && hipSetDevice(h->device) != hipSuccess) {
        (void)hipGetLastError();
        return SDPA_STATUS_HIP_ERROR;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (bf16) {
        e = sdpa::launch_fwd_bf16(a, tile, s);
    } else {
        e = sdpa::launch_fwd_f32(a, s);
    }
    if (cur != h->device) (void)hipSetDevice(cur);
    return e == hipSuccess ? SDPA_STATUS_SUCCESS : SDPA_STATUS_HIP_ERROR;
}

size_t sdpa_decode_workspace_size(sdpa_handle_t h, int B, int H, int Lq, int Lk, int d_k) {
    if (h == nullptr || B < 1 || H < 1 || Lq < 1 || Lk < 1 || d_k < 1) return 0;
    if (h->dtype != SDPA_DTYPE_BF16 || (d_k != 64 && d_k != 128) || Lq > sdpa::kDecodeMaxLq) return 0;
    long long n = 0;
    if (!mul_fits(B, H, Lq, d_k, &n) || !mul_fits(B, H, Lk, d_k, &n)) return 0;
    return sdpa::plan_decode(B, H, Lq, Lk, d_k, h->num_cus).workspace_bytes;
}

}  // extern "C"

namespace {

// sdpa_decode and sdpa_decode_noalloc: validation and launch.  noalloc: the
// partial results go to the library's own scratch array instead of a
// caller workspace.
sdpa_status_t decode_impl(sdpa_handle_t h, const void* q, const void* k, const void* v, void* out,
                          float* lse, int B, int H, int Lq, int Lk, int d_k, int causal,
                          const int32_t* key_lens, void* workspace, size_t workspace_bytes,
                          bool noalloc, void* stream) {
    if (h == nullptr || q == nullptr || k == nullptr || v == nullptr || out == nullptr)
        return SDPA_STATUS_INVALID_VALUE;
    if (B < 1 || H < 1 || Lq < 1 || Lk < 1 || d_k < 1) return SDPA_STATUS_INVALID_VALUE;
    if (causal != 0 && causal != 1) return SDPA_STATUS_INVALID_VALUE;
    if (h->dtype != SDPA_DTYPE_BF16 || (d_k != 64 && d_k != 128) || Lq > sdpa::kDecodeMaxLq)
        return SDPA_STATUS_NOT_SUPPORTED;
    long long nq = 0, nkv = 0;
    if (!mul_fits(B, H, Lq, d_k, &nq) || !mul_fits(B, H, Lk, d_k, &nkv))
        return SDPA_STATUS_INVALID_VALUE;
    if ((unsigned long long)nkv > SIZE_MAX / 2) return SDPA_STATUS_INVALID_VALUE;
    const size_t bq = (size_t)nq * 2, bkv = (size_t)nkv * 2;
    const size_t bl = (size_t)B * H * Lq * sizeof(float);
    const sdpa::DecodePlan plan = sdpa::plan_decode(B, H, Lq, Lk, d_k, h->num_cus);
    if (noalloc) {
        if (plan.workspace_bytes > sdpa::kDecodeNoallocScratchBytes) return SDPA_STATUS_NOT_SUPPORTED;
        workspace = plan.workspace_bytes > 0 ? sdpa::decode_scratch_ptr(h->device) : nullptr;
        if (plan.workspace_bytes > 0 && workspace == nullptr) return SDPA_STATUS_HIP_ERROR;
        workspace_bytes = plan.workspace_bytes;
    } else if (plan.workspace_bytes > 0) {
        if (workspace == nullptr || workspace_bytes < plan.workspace_bytes) return SDPA_STATUS_INVALID_VALUE;
        if (reinterpret_cast<uintptr_t>(workspace) % alignof(float) != 0) return SDPA_STATUS_INVALID_VALUE;
    }
    struct Span { const void* p; size_t n; };
    const Span inputs[] = {{q, bq}, {k, bkv}, {v, bkv}};
    // (the library's own scratch is an allocation of its own: it cannot
    // overlap caller memory)
    const Span outputs[] = {{out, bq}, {lse, lse ? bl : 0},
                            {workspace, noalloc ? 0 : plan.workspace_bytes}};
    for (size_t o = 0; o < 3; ++o) {
        if (outputs[o].p == nullptr || outputs[o].n == 0) continue;
        for (const Span& in : inputs)
            if (overlaps(outputs[o].p, outputs[o].n, in.p, in.n)) return SDPA_STATUS_INVALID_VALUE;
        for (size_t p2 = o + 1; p2 < 3; ++p2)
            if (outputs[p2].p != nullptr && outputs[p2].n != 0 &&
                overlaps(outputs[o].p, outputs[o].n, outputs[p2].p, outputs[p2].n))
                return SDPA_STATUS_INVALID_VALUE;
    }
    if (lse != nullptr && reinterpret_cast<uintptr_t>(lse) % alignof(float) != 0)
        return SDPA_STATUS_INVALID_VALUE;
    if (key_lens != nullptr && reinterpret_cast<uintptr_t>(key_lens) % alignof(int32_t) != 0)
        return SDPA_STATUS_INVALID_VALUE;
    for (const void* p : {q, k, v, (const void*)out})
        if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return SDPA_STATUS_NOT_SUPPORTED;

    sdpa::DecodeArgs a;
    a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse; a.key_lens = key_lens;
    a.workspace = workspace;
    a.B = B; a.H = H; a.Lq = Lq; a.Lk = Lk; a.d = d_k; a.causal = causal;
    a.num_cus = h->num_cus;

    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) {
        (void)hipGetLastError();
        return SDPA_STATUS_HIP_ERROR;
    }
    if (cur != h->device && hipSetDevice(h->device) != hipSuccess) {
        (void)hipGetLastError();
        return SDPA_STATUS_HIP_ERROR;
    }
    hipError_t e = sdpa::launch_decode_bf16(a, plan, static_cast<hipStream_t>(stream));
    if (cur != h->device) (void)hipSetDevice(cur);
    return e == hipSuccess ? SDPA_STATUS_SUCCESS : SDPA_STATUS_HIP_ERROR;
}

}  // namespace

extern "C" {

sdpa_status_t sdpa_decode(sdpa_handle_t h, const void* q, const void* k, const void* v, void* out,
                          float* lse, int B, int H, int Lq, int Lk, int d_k, int causal,
                          const int32_t* key_lens, void* workspace, size_t workspace_bytes,
                          void* stream) {
    return decode_impl(h, q, k, v, out, lse, B, H, Lq, Lk, d_k, causal, key_lens, workspace,
                       workspace_bytes, false, stream);
}

sdpa_status_t sdpa_decode_noalloc(sdpa_handle_t h, const void* q, const void* k, const void* v,
                                  void* out, float* lse, int B, int H, int Lq, int Lk, int d_k,
                                  int causal, const int32_t* key_lens, void* stream) {
    return decode_impl(h, q, k, v, out, lse, B, H, Lq, Lk, d_k, causal, key_lens, nullptr, 0, true,
                       stream);
}

}  // extern "C"
