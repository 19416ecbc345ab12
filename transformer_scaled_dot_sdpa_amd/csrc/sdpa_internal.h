// Internal interface between the C ABI (sdpa_api.cpp), the tile selector and
// the HIP kernels.  Not installed; callers use include/sdpa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa {

// Arguments shared by every forward kernel.  Tensors are contiguous
// [B, H, L, d] (q/out with L = Lq, k/v with L = Lk); lse is [B, H, Lq].
struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    float* lse;               // may be null
    const int32_t* key_lens;  // device int32[B], may be null
    int B, H, Lq, Lk, d;
    int causal;
    int num_cus;              // compute units of the device (sizes persistent grids)
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
};

// Largest number of query rows the decode kernel takes.
constexpr int kDecodeMaxLq = 8;

// How a decode call is split over keys.
struct DecodePlan {
    int splits;               // key chunks per (b, h)
    int chunk;                // keys per chunk
    size_t workspace_bytes;   // 0 when splits == 1
};
DecodePlan plan_decode(int B, int H, int Lq, int Lk, int d, int num_cus);

// One bf16 tile configuration.  br = rows of Q per workgroup
// (32 per wavefront), bc = keys per K/V tile.
struct Bf16Tile {
    int d;
    int bc;
    int waves;
    int kind;   // 0: sdpa_fwd_bf16.hip, 1: sdpa_fwd_bf16_pipe.hip, 2: sdpa_fwd_bf16_pp.hip,
                // 3: sdpa_fwd_bf16_wide.hip
    const char* name;
};

// Picks the bf16 tile for a problem (tile_select.cpp).  Returns false if
// d is not one of the compiled head sizes.
bool select_bf16_tile(int d, int causal, long long bh, int Lq, int Lk, int num_cus,
                      Bf16Tile* out);

// Kernel launchers; return hipSuccess or the launch error.
hipError_t launch_fwd_bf16(const FwdArgs& a, const Bf16Tile& t, hipStream_t s);
hipError_t launch_fwd_bf16_pipe(const FwdArgs& a, const Bf16Tile& t, hipStream_t s);
hipError_t launch_fwd_bf16_pp(const FwdArgs& a, const Bf16Tile& t, hipStream_t s);
hipError_t launch_fwd_bf16_wide(const FwdArgs& a, const Bf16Tile& t, hipStream_t s);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s);
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t s);
hipError_t launch_decode_bf16(const DecodeArgs& a, const DecodePlan& plan, hipStream_t s);
hipError_t launch_bwd_f32(const BwdArgs& a, hipStream_t s);

}  // namespace sdpa
