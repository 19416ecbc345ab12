// Internal interface between the C ABI (sdpa_api.cpp), the tile selector and
// the HIP kernels.  Not installed; callers use include/sdpa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa {

// Arguments shared by every forward kernel.  q/k/v/out are [B, H, L, width]
// views (q/out with L = Lq, k/v with L = Lk; width d for q/k, dv for v/out)
// given by element strides of batch, head and row; the last dimension is
// contiguous.  lse is contiguous [B, H, Lq].  The bf16 kernel's default
// tile and the fp32 kernel honour strides, dv != d, scale and mask; the
// other bf16 tiles take dv = d and no mask.
struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    float* lse;               // may be null
    const int32_t* key_lens;  // device int32[B], may be null
    int B, H, Lq, Lk, d;
    int dv;
    int causal;
    int num_cus;              // compute units of the device (sizes persistent grids)
    long long q_sb, q_sh, k_sb, k_sh, v_sb, v_sh, o_sb, o_sh;
    int q_sl, k_sl, v_sl, o_sl;
    float scale;              // > 0: scores are q.k * scale; else 1/sqrt(d)
    const float* mask;        // additive fp32 mask on the scaled scores, or null
    long long m_sb, m_sh;     // mask strides (0 broadcasts)
    int m_sl;

    // contiguous [B, H, L, width] tensors, dv = d, default scale, no mask
    void set_contiguous() {
        dv = d;
        q_sl = o_sl = k_sl = v_sl = d;
        q_sh = o_sh = (long long)Lq * d;
        k_sh = v_sh = (long long)Lk * d;
        q_sb = o_sb = (long long)H * Lq * d;
        k_sb = v_sb = (long long)H * Lk * d;
        scale = 0.f;
        mask = nullptr;
        m_sb = m_sh = 0;
        m_sl = 0;
    }
};

// Arguments of the backward kernels.  Layouts as FwdArgs; dout, dq have q's
// shape, dk, dv k's shape; lse and delta are fp32 [B, H, Lq].
struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* out;
    const void* dout;
    const float* lse;
    float* delta;             // written: D_i = dout_i . out_i
    void* dq;
    void* dk;
    void* dv;
    const int32_t* key_lens;
    int B, H, Lq, Lk, d;
    int causal;
    int num_cus;              // compute units of the device (sizes the work units)
};

// Arguments of the decode-shaped forward: FwdArgs plus the caller's
// workspace (partial results of the key chunks).
struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    float* lse;               // may be null
    const int32_t* key_lens;  // may be null
    void* workspace;          // plan.workspace_bytes, 4-byte aligned (unused with one chunk)
    int B, H, Lq, Lk, d;
    int causal;
    int num_cus;              // compute units of the device
};

// Largest number of query rows the decode kernel takes.
constexpr int kDecodeMaxLq = 8;

// How a decode call is split over keys.
struct DecodePlan {
    int splits;               // key chunks per (b, h)
    int chunk;                // keys per chunk
    size_t workspace_bytes;   // 0 when splits == 1
    bool use_forward;         // enough slices to fill the GPU: the main forward
                              // kernel (one workgroup per slice, no workspace)
};
DecodePlan plan_decode(int B, int H, int Lq, int Lk, int d, int num_cus);

// One bf16 tile configuration of the forward kernel (sdpa_fwd_bf16.hip):
// waves wavefronts of 32 query rows each share K/V tiles of bc keys; with
// ks = 2 two such groups take alternate key tiles of the same rows.  pairs:
// with per-batch key lengths (and no causal mask) each workgroup runs a
// long item and a short one, batches ranked by key length.
struct Bf16Tile {
    int d;
    int bc;
    int waves;
    int ks;
    int pairs;
    const char* name;
};

// Most batches the key-length ranking takes (LDS arrays of the kernel).
constexpr int kMaxPairBatches = 512;

// Picks the bf16 tile for a problem (tile_select.cpp).  general: the call
// has d_v != d_k or an additive mask, which only the default tile takes.
// Returns false if d is not one of the compiled head sizes.
bool select_bf16_tile(int d, int causal, int has_key_lens, long long bh, int Lq, int Lk, int num_cus,
                      bool general, Bf16Tile* out);
// The compiled tile of this name and head size (tuning and tests); false if
// there is none.
bool find_bf16_tile(int d, const char* name, Bf16Tile* out);

// Kernel launchers; return hipSuccess or the launch error.
hipError_t launch_fwd_bf16(const FwdArgs& a, const Bf16Tile& t, hipStream_t s);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s);
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t s);
hipError_t launch_decode_bf16(const DecodeArgs& a, const DecodePlan& plan, hipStream_t s);

// The library's own decode scratch (sdpa_decode_noalloc): a fixed-size
// device array per GPU.  decode_scratch_init looks up its address on one
// device (once; later calls return at once) and must run before
// decode_scratch_ptr can return it; nullptr before that.
constexpr size_t kDecodeNoallocScratchBytes = (size_t)16 << 20;
hipError_t decode_scratch_init(int device);
void* decode_scratch_ptr(int device);
hipError_t launch_bwd_f32(const BwdArgs& a, hipStream_t s);

}  // namespace sdpa
