/*
 * sdpa.h -- C ABI of the MI355X (gfx950) scaled dot-product attention forward
 * and its gradients.
 *
 * The operation is eq. (1) of "Aufmerksamkeit ist alles, was Sie brauchen"
 * (German translation of "Attention Is All You Need"), section 3.2.1:
 *
 *     Attention(Q, K, V) = softmax(Q K^T / sqrt(d_k)) V
 *
 * applied independently to every (batch b, head h) slice -- "all heads in
 * parallel" (cookipedia article "Attention Is All You Need", section
 * "Transformer の構造"; German translation, section 3.2.2).  Three forms are
 * covered, as listed in "D2L-74-Transformer", section "Attention: 3 different
 * kinds":
 *   - encoder self-attention: Lq = Lk, no mask;
 *   - decoder masked self-attention: causal = 1, the strict upper triangle of
 *     Q K^T is set to -inf before the softmax, the diagonal is kept
 *     (cookipedia article, section "原論文でのデコーダ");
 *   - encoder-decoder cross-attention: Lq != Lk, keys and values from the
 *     encoder, optionally with per-batch key lengths.
 *
 * Plain C types only; all tensor pointers are device pointers owned by the
 * caller.  The library never allocates, frees or retains caller memory.
 */
#ifndef SDPA_MI355X_H_
#define SDPA_MI355X_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Opaque handle; created by sdpa_create, owned by the library. */
typedef struct sdpa_ctx* sdpa_handle_t;

typedef enum {
    SDPA_STATUS_SUCCESS = 0,
    SDPA_STATUS_INVALID_VALUE = 1,   /* bad handle, pointer, size or flag */
    SDPA_STATUS_NOT_SUPPORTED = 2,   /* dtype / d_k / device combination not built */
    SDPA_STATUS_HIP_ERROR = 3,       /* a HIP runtime call or kernel launch failed */
    SDPA_STATUS_ALLOC_FAILED = 4     /* host allocation of the handle failed */
} sdpa_status_t;

typedef enum {
    SDPA_DTYPE_FP32 = 0,   /* q, k, v, out are float; any 1 <= d_k <= 256 */
    SDPA_DTYPE_BF16 = 1    /* q, k, v, out are bf16 (uint16 bits); d_k in {64, 128} */
} sdpa_dtype_t;

/*
 * Create a handle bound to one element type and one HIP device.
 *   h       out: the new handle (unchanged on error).
 *   dtype   element type of q, k, v and out for every call on this handle.
 *   device  HIP device ordinal; must be a gfx950 device for SDPA_DTYPE_BF16.
 * Reads the device's properties once (architecture, compute-unit count); the
 * handle is immutable afterwards, so concurrent sdpa_forward calls on
 * different streams may share it.
 * Errors: INVALID_VALUE (h == NULL, unknown dtype, bad ordinal),
 * HIP_ERROR (device query failed), NOT_SUPPORTED (bf16 on a non-gfx950
 * device), ALLOC_FAILED.
 */
sdpa_status_t sdpa_create(sdpa_handle_t* h, sdpa_dtype_t dtype, int device);

/*
 * Enqueue one attention forward on `stream`; returns without waiting.
 *
 *   q        [B, H, Lq, d_k] contiguous row-major, handle's dtype.
 *   k, v     [B, H, Lk, d_k] contiguous row-major (values have width d_k).
 *   out      [B, H, Lq, d_k] contiguous, handle's dtype; must not overlap
 *            q, k or v.  out[b,h,i,:] = sum_j a_ij v[b,h,j,:] with
 *            a_ij = softmax over the valid j of s_ij = q_i . k_j / sqrt(d_k)
 *            (German translation, section 3.2.1, eq. (1)).  Results are
 *            rounded to the output type to nearest, ties to even.
 *   lse      [B, H, Lq] float, or NULL: natural-log sum over the valid j of
 *            e^{s_ij} (the smoothed maximum of the scores named in the formula
 *            page "トランスフォーマーの注意機構", section "広がる学問").
 *   B, H, Lq, Lk, d_k   sizes, each >= 1.
 *   causal   0 or 1.  1: key j is valid for query i only if j <= i (top-left
 *            aligned for any Lq, Lk).
 *   key_lens device int32[B], or NULL: key j of batch b is valid only if
 *            j < clamp(key_lens[b], 0, Lk).  Keys and values at or past that
 *            length are never read, so they may hold any bits.
 *   stream   HIP stream (hipStream_t) as an opaque pointer; NULL = default.
 * A query row with no valid key gets out = 0 and lse = -inf.
 *
 * Accumulation is fp32 on every path.  bf16: products on bf16 matrix cores
 * with fp32 accumulation, the softmax weights rounded to bf16 before they
 * multiply V.
 *
 * Errors (returned before anything is enqueued; out and lse untouched):
 * INVALID_VALUE for a NULL handle or tensor pointer, sizes < 1, causal not
 * 0/1, overlapping out, or sizes whose element counts overflow int64;
 * NOT_SUPPORTED for d_k outside the handle dtype's range, bf16 pointers
 * not 16-byte aligned, or a bf16 (b, h) slice of k or v of 4 GiB or more
 * (Lk * d_k * 2 >= 2^32); HIP_ERROR if the launch fails.  Faults during
 * execution surface at the caller's next synchronisation, as in HIP.
 */
sdpa_status_t sdpa_forward(sdpa_handle_t h,
                           const void* q, const void* k, const void* v,
                           void* out, float* lse,
                           int B, int H, int Lq, int Lk, int d_k,
                           int causal, const int32_t* key_lens, void* stream);

/*
 * Element strides of a [B, H, L, width] view whose last dimension is
 * contiguous: element (b, h, l, t) sits at base + b*batch + h*head + l*row + t.
 * A layout with row == 0 stands for the contiguous [B, H, L, width] tensor.
 * The head-interleaved [B, L, H*width] layout that multi-head attention
 * produces and concatenates (cookipedia article, section "Transformer の構造";
 * German translation, section 3.2.2) is batch = L*H*width, head = width,
 * row = H*width.
 */
typedef struct {
    int64_t batch;
    int64_t head;
    int64_t row;
} sdpa_layout_t;

/*
 * The general forward: every argument of sdpa_forward plus
 *   d_v          width of values and outputs (German translation, section
 *                3.2.1: queries and keys of dimension d_k, values of
 *                dimension d_v); <= 0 means d_v = d_k.
 *   *_layout     strides of q, k (width d_k), v, out (width d_v).
 *   scale        scores are (q . k) * scale; <= 0 means 1/sqrt(d_k).  The
 *                temperature form of the formula page's section 証明 is
 *                scale = 1/tau.
 *   mask         NULL, or an additive fp32 term added to every scaled score
 *                before the softmax: element (b, h, i, j) of a [B, H, Lq, Lk]
 *                view with strides mask_layout (batch or head 0 broadcast;
 *                all zero: one [Lq, Lk] matrix shared by every (b, h)).
 *                Entries must be finite or -inf; -inf drops the key, as the
 *                causal mask does (formula page, section 応用; the toy model
 *                of the cookipedia article, section "トイモデル", builds its
 *                decoder mask this way).  A row whose valid keys all carry
 *                -inf gets out = 0 and lse = -inf.
 * causal and key_lens apply as in sdpa_forward, on top of the mask.
 *   tile         NULL for the configuration sdpa_forward would choose, or the
 *                name of a compiled one ("bf16_d128_bc64_w4_ks2", ...; fp32:
 *                "f32_wave_per_row").  Every configuration computes the same
 *                function; they differ in speed.  d_v != d_k and a mask run
 *                only in the default bf16 configuration of each d_k
 *                ("bf16_d64_bc64_w4", "bf16_d128_bc64_w4").
 */
typedef struct {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    float* lse;                 /* [B, H, Lq] contiguous, or NULL */
    int B, H, Lq, Lk, d_k, d_v;
    sdpa_layout_t q_layout, k_layout, v_layout, out_layout;
    int causal;
    const int32_t* key_lens;
    float scale;
    const float* mask;
    sdpa_layout_t mask_layout;
    const char* tile;           /* NULL: chosen by shape (see sdpa_kernel_name);
                                   else the name of one compiled bf16 tile
                                   configuration (sdpa_kernel_name's strings),
                                   for tuning and tests */
} sdpa_forward_desc_t;

/*
 * Enqueue the general forward described by *desc on `stream`; returns
 * without waiting.  Handle dtype as sdpa_forward.  bf16: d_k and d_v in
 * {64, 128}; every stride a multiple of 8 elements and q, k, v, out 16-byte
 * aligned; each of k and v spanning under 4 GiB per (b, h) slice (Lk * row
 * stride * 2 bytes); a mask slice under 2 GiB.  fp32: d_k, d_v <= 256, any
 * strides.  The mask is read fastest when its pointer is 16-byte aligned and
 * its strides are multiples of 4.
 * Errors (before anything is enqueued): INVALID_VALUE for desc == NULL, a
 * NULL tensor, sizes < 1, causal not 0/1, a row stride below the width, a
 * negative stride, element counts overflowing int64, an out view in which
 * two elements share an address (a zero stride on a dimension of size > 1,
 * or strides whose rows interleave), or out overlapping any input (by
 * extent); NOT_SUPPORTED for the dtype limits above, or a tile name that is
 * not compiled for this d_k (or cannot take this d_v or mask); HIP_ERROR if
 * the launch fails.
 */
sdpa_status_t sdpa_forward_ex(sdpa_handle_t h, const sdpa_forward_desc_t* desc, void* stream);

/*
 * Enqueue the gradients of one attention forward on `stream`; returns
 * without waiting.
 *
 * For a loss L with dL/d(out) = dout, the proof section (証明) of the formula
 * page "トランスフォーマーの注意機構" fixes every step: the output display
 * o = sum_j a_j v_j gives dL/dv_j and dL/da_j = dout . v_j, the Jacobian of
 * the weights da_j/ds_l = a_j (delta_jl - a_l) gives
 *     dL/ds_j = a_j (dout . v_j - D),   D = sum_l a_l (dout . v_l) = dout . out,
 * and the score display s_j = q . k_j / sqrt(d_k) gives
 *     dq_i = sum_j dL/ds_ij k_j / sqrt(d_k),
 *     dk_j = sum_i dL/ds_ij q_i / sqrt(d_k),
 *     dv_j = sum_i a_ij dout_i,
 * summed over the valid (i, j) pairs of sdpa_forward's masks.
 *
 *   q, k, v, B, H, Lq, Lk, d_k, causal, key_lens
 *            exactly as passed to the sdpa_forward call being differentiated.
 *   out      [B, H, Lq, d_k], that call's output (handle's dtype).
 *   lse      [B, H, Lq] float, that call's log-sum-exp (required here): the
 *            weights are recomputed as a_ij = e^{s_ij - lse_i}.
 *   dout     [B, H, Lq, d_k], dL/d(out), handle's dtype.
 *   delta    [B, H, Lq] float, caller-owned, written: D_i = dout_i . out_i
 *            (fp32).  It is the only intermediate the gradients need and is
 *            left holding D on return.
 *   dq       [B, H, Lq, d_k] written (handle's dtype).
 *   dk, dv   [B, H, Lk, d_k] written (handle's dtype).  Keys that no query
 *            row sees (past key_lens, or above the causal triangle) get 0;
 *            so does dq of a row with no valid key.
 *   stream   HIP stream (hipStream_t) as an opaque pointer; NULL = default.
 *
 * Accumulation is fp32 on every path.  bf16: the five products on bf16
 * matrix cores, the recomputed weights and dL/ds rounded to bf16 (RNE) as
 * operands; results rounded to bf16 (RNE).  Deterministic: no atomics.
 * dout . v_j and D are two fp32 dot products summed in different orders, so
 * where dL/ds cancels exactly in real arithmetic (a row with one valid key)
 * dq and dk hold a rounding residue of order 2^-24 d_k |dout| |v| rather
 * than an exact zero.
 *
 * Errors (returned before anything is enqueued; outputs untouched):
 * INVALID_VALUE for a NULL handle or pointer (key_lens aside), sizes < 1,
 * causal not 0/1, element counts overflowing int64, misaligned float
 * pointers, or any written buffer (delta, dq, dk, dv) overlapping another
 * argument; NOT_SUPPORTED for d_k outside the handle dtype's range (bf16:
 * 64 or 128), bf16 pointers not 16-byte aligned, or a bf16 (b, h) slice of
 * 4 GiB or more (Lq * d_k * 2 or Lk * d_k * 2 >= 2^32); HIP_ERROR if a
 * launch fails.
 */
sdpa_status_t sdpa_backward(sdpa_handle_t h,
                            const void* q, const void* k, const void* v,
                            const void* out, const void* dout, const float* lse,
                            float* delta, void* dq, void* dk, void* dv,
                            int B, int H, int Lq, int Lk, int d_k,
                            int causal, const int32_t* key_lens, void* stream);

/*
 * Decode-shaped forward: the same operation, masks and outputs as
 * sdpa_forward, for a few query rows (1 <= Lq <= 8) against a long key/value
 * sequence -- the shape of generating one position per step (cookipedia
 * article, section "全体").  bf16 handles, d_k in {64, 128}.  For the usual
 * decode step (the newest position attends to every cached key) pass
 * causal = 0 and the context length per batch in key_lens; causal = 1 keeps
 * sdpa_forward's top-left meaning.
 *
 * Each (b, h) slice is split into key chunks so that few slices still fill
 * the GPU; each chunk yields a partial output and log-sum-exp, merged as
 * lse = ln sum_c e^{lse_c}, out = sum_c e^{lse_c - lse} out_c (the ratio
 * identity of the formula page "トランスフォーマーの注意機構", section 証明,
 * with the log-sum-exp of section 広がる学問).  With at least two slices per
 * compute unit (and d_k = 64, or at most 4096 keys) the slices already fill
 * the GPU: the call then runs sdpa_forward's kernel, one workgroup per
 * slice, with no split and no workspace.  The partial results of a split
 * live in a caller-owned workspace:
 *   workspace        device memory of at least workspace_bytes, 4-byte
 *                    aligned, not overlapping any other argument; contents
 *                    on entry are ignored and on return unspecified.  May be
 *                    NULL when sdpa_decode_workspace_size returns 0.
 *   workspace_bytes  its size; must be >= sdpa_decode_workspace_size(...)
 *                    for the same arguments.
 * Other arguments as sdpa_forward.  Errors: as sdpa_forward, plus
 * INVALID_VALUE for a missing, short, misaligned or overlapping workspace and
 * NOT_SUPPORTED for fp32 handles, Lq > 8 or d_k outside {64, 128}.
 */
sdpa_status_t sdpa_decode(sdpa_handle_t h,
                          const void* q, const void* k, const void* v,
                          void* out, float* lse,
                          int B, int H, int Lq, int Lk, int d_k,
                          int causal, const int32_t* key_lens,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of workspace sdpa_decode needs for these sizes on this handle's
 * device (0: none needed, or the combination is not supported).  Depends
 * only on the arguments and the device's compute-unit count.
 */
size_t sdpa_decode_workspace_size(sdpa_handle_t h, int B, int H, int Lq, int Lk, int d_k);

/*
 * sdpa_decode for callers that cannot allocate memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * operation, arguments, kernels and results as sdpa_decode, but the partial
 * results of a split over keys go to a fixed device array that the library
 * holds per GPU (SDPA_DECODE_NOALLOC_SCRATCH_BYTES, 16 MiB, kept until the
 * process ends; its address is looked up when a bf16 handle is created on
 * that device) instead of a caller workspace.  The call itself allocates
 * nothing.  Every call on one GPU shares that array, so calls that overlap
 * on one GPU (on different streams, or from several threads) race and must
 * be serialised by the caller; the kernels write every partial result they
 * read within the call, so nothing carries over from the previous call.
 * Errors: as sdpa_decode, plus NOT_SUPPORTED when the split these sizes
 * need is larger than the array (sdpa_decode_workspace_size(...) >
 * SDPA_DECODE_NOALLOC_SCRATCH_BYTES) -- use sdpa_decode with a workspace
 * then.
 */
#define SDPA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
sdpa_status_t sdpa_decode_noalloc(sdpa_handle_t h,
                                  const void* q, const void* k, const void* v,
                                  void* out, float* lse,
                                  int B, int H, int Lq, int Lk, int d_k,
                                  int causal, const int32_t* key_lens, void* stream);

/* Release a handle (NULL is accepted).  Does not synchronise any stream. */
sdpa_status_t sdpa_destroy(sdpa_handle_t h);

/* Static, human-readable name of a status code (never NULL). */
const char* sdpa_status_string(sdpa_status_t s);

/*
 * Tile configuration that sdpa_forward would launch for these arguments,
 * written as a short static string (e.g. "bf16_d128_bc64_w4"); for logging
 * and profiling.  Returns NULL when the combination is not supported.
 */
const char* sdpa_kernel_name(sdpa_handle_t h, int B, int H, int Lq, int Lk,
                             int d_k, int causal, int has_key_lens);

#ifdef __cplusplus
}
#endif

#endif /* SDPA_MI355X_H_ */
