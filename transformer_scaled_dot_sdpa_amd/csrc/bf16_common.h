// Device-side pieces shared by the bf16 forward kernels: vector types, the
// kernel argument block, the LDS layouts of K and V tiles, and the
// workgroup -> (b, h, query block) mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa {
namespace bf16k {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLn2 = 0.69314718055994530942f;
// Lazy rescaling: the running maximum used for the exponentials is only
// raised when a new maximum exceeds it by more than 2^8 (in exp2 units), so
// weights stay <= 256 and O is rescaled rarely.  The final O / l and
// m + log2(l) are exact for whichever reference maximum was used.
constexpr float kRescaleSlack = 8.0f;
// s_waitcnt immediate that waits for all vector-memory operations (including
// direct-to-LDS loads) and nothing else: vmcnt = 0, expcnt and lgkmcnt at max.
constexpr int kWaitVmcnt0 = 0x0F70;

struct KParams {
    const uint16_t* __restrict__ q;
    const uint16_t* __restrict__ k;
    const uint16_t* __restrict__ v;
    uint16_t* __restrict__ out;
    float* __restrict__ lse;
    const int32_t* __restrict__ key_lens;
    int H, Lq, Lk;
    int num_qb;        // query blocks per (b, h)
    int num_items;     // work items = (b, h, query block) triples
    int upi;           // work items per scheduling unit (1, or 2: a long/short pair)
    int num_units;     // ceil(num_items / upi)
    int B;
    // key-length pairs (LENS kernels): batches ordered by clamped key length,
    // longest first, and unit u runs items u and num_items - 1 - u
    int lens_pairs;
    // one unit per workgroup, all resident at once, units alternating long
    // and short (causal): renumber so that the two workgroups a compute unit
    // holds take a long unit and the short one beside it (cu_pairs = compute
    // units per XCD; 0: off)
    int cu_pairs;
    float scale_log2;  // log2(e) * scale (scale = 1 / sqrt(d) unless given)
    // Element strides of the [B, H, L, width] views: batch, head, row.
    long long q_sb, q_sh, k_sb, k_sh, v_sb, v_sh, o_sb, o_sh;
    int q_sl, k_sl, v_sl, o_sl;
    // Additive fp32 mask on the scaled scores (MASK kernels): [B, H, Lq, Lk]
    // view with strides m_sb, m_sh (0 broadcasts), m_sl; inv_scale = 1 / scale
    // turns it into raw-score units.
    const float* __restrict__ mask;
    long long m_sb, m_sh;
    int m_sl;
    float inv_scale;
    int mask_vec;      // mask rows and slices 16-byte aligned: vector loads
};


// LDS row of key j inside a K tile: bits 2 and 3 swapped (an involution).
// With this order the S^T accumulator of lane (n, h) holds, at index r,
// key 16*(r/8) + 8h + r%8 of its 32-key block: eight consecutive keys per
// half, the layout the B operand of the P.V product needs.
__device__ __forceinline__ int k_lds_row(int j) {
    return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1);
}

// XOR swizzles of the 16-byte chunk index inside an LDS row, chosen so that
// the MFMA operand reads of 16 consecutive lanes hit distinct bank groups.
// The K swizzle depends only on row bits 0..3 (D = 128) or 1..3 (D = 64),
// the V swizzle only on bits 0..1 (D = 128) or 1 (D = 64), so 32-row and
// 4-row steps keep them unchanged.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
    return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int v_swz(int row) {
    return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
}

// 16-byte-per-lane buffer load straight into LDS (lane l writes dst + 16 l).
// The buffer is the nbytes bytes from base (raw, stride 0); a lane whose
// byte offset voff + soff is >= nbytes receives zeros instead, which keeps
// keys past the valid length from ever being read.  Plain arguments only:
// the buffer-resource type exists for the device compilation alone.
__device__ __forceinline__ void buffer_load_lds16(const void* base, uint32_t nbytes,
                                                  lds_void* dst, uint32_t voff, uint32_t soff) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(base), (short)0, (int)nbytes, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 0, 0);
}

typedef __attribute__((address_space(3))) uint16_t lds_u16;

// A wavefront's 32 x W block of results in the 32x32x16 accumulator layout
// (lane n + 32h, column tile t, register r: row n, column 32t + 8(r/4) +
// 4h + r%4), times the lane's `mul`, rounded to bf16 and stored as whole
// rows.  Stored straight from the accumulators, every instruction would
// write 8 bytes of each of 32 rows: partial cache lines.  Instead the block
// goes to `stage` (32*W elements of LDS, row-major, the 16-byte chunks of a
// row XOR-swizzled by the row so that the 32 rows' writes spread over the
// banks) and is read back so that consecutive lanes hold consecutive 16
// bytes of one row; 16-byte non-temporal stores then write whole lines:
// rows i < rows of the block go to dst + i * ld.  The caller makes sure no
// other wavefront still reads `stage`.
template <int W>
__device__ __forceinline__ void store_rows_bf16(const f32x16* acc, float mul, lds_u16* stage, uint16_t* dst,
                                                size_t ld, int rows, int lane) {
    constexpr int CPR = W / 8;     // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;  // rows per store instruction
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    // the empty asm keeps the compiler from computing the lane's LDS offsets
    // once at kernel start and holding them in registers through the loops
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int n = ln & 31, h = ln >> 5;
#pragma unroll
    for (int t = 0; t < W / 32; ++t)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            __bf16 w[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) w[c] = (__bf16)(acc[t][4 * g4 + c] * mul);
            const int ch = (4 * t + g4) ^ (n & (CPR - 1));
            *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(stage + n * W + ch * 8 + 4 * h) =
                __builtin_bit_cast(u32x2, w);
        }
    const int r_in = ln / CPR, c = ln % CPR;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
        const int row = i * RPI + r_in;
        const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
            stage + row * W + ((c ^ (row & (CPR - 1))) * 8));
        if (row < rows) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst + (size_t)row * ld + c * 8));
    }
}

// x combined with its value in lane l ^ 32.  v_permlane32_swap(a, b)
// returns (a[l], a[l + 32]) in lanes l < 32 and (b[l - 32], b[l]) in lanes
// l >= 32, so with a = b = x each lane gets its own value and its partner's.
// The two results pass through an empty asm: otherwise the optimizer folds
// a symmetric combination of them (max, sum) into the first result alone.
__device__ __forceinline__ void halves_pair(float x, float* p0, float* p1) {
    const unsigned a = __builtin_bit_cast(unsigned, x);
    const auto pr = __builtin_amdgcn_permlane32_swap(a, a, false, false);
    unsigned r0 = pr[0], r1 = pr[1];
    asm volatile("" : "+v"(r0), "+v"(r1));
    *p0 = __builtin_bit_cast(float, r0);
    *p1 = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ float max_across_halves(float x) {
    float p0, p1;
    halves_pair(x, &p0, &p1);
    return fmaxf(p0, p1);
}
__device__ __forceinline__ float sum_across_halves(float x) {
    float p0, p1;
    halves_pair(x, &p0, &p1);
    return p0 + p1;
}

// The unit of work of workgroup g of nwg; every launch here sizes its grid
// to one workgroup per unit.  Workgroup ids are dealt to the 8 XCDs in turn;
// each XCD gets a contiguous range of units (as many as it has workgroups)
// and its workgroups take them in order, so the workgroups running side by
// side on one XCD work on neighbouring units -- the query blocks of a few
// heads, whose K and V then stay in that XCD's L2.  (32-bit arithmetic only:
// the general form, units spread over fewer workgroups, took two 64-bit
// divisions, about 200 scalar instructions at the start of every workgroup.)
// A bijection of [0, nwg); host-callable so that it can be checked there.
__host__ __device__ __forceinline__ int unit_of_workgroup(int nwg, int g) {
    const int xcd = g & 7, j = g >> 3;
    const int per = nwg >> 3, rem = nwg & 7;
    return xcd * per + (xcd < rem ? xcd : rem) + j;
}
__device__ __forceinline__ int workgroup_unit() { return unit_of_workgroup(gridDim.x, blockIdx.x); }

// With every workgroup resident at once, the hardware hands an XCD's
// workgroups to its C compute units in turn, so the XCD's j-th and (j + C)-th
// workgroups share a compute unit.  Units that alternate long and short
// (causal query blocks) would then put two long ones on every other compute
// unit.  This renumbering gives local workgroup j < P the unit 2j and
// workgroup j + C the unit 2j + 1 (P = R - C pairs of an XCD range of R
// units), so that each compute unit holding two workgroups runs one long and
// one short unit -- of the same head, which also shares its K/V in L2.  unit
// is workgroup g's unit from unit_of_workgroup; the result is again a
// bijection of [0, nwg).
__host__ __device__ __forceinline__ int cu_pair_renumber(int nwg, int g, int cus_per_xcd, int unit) {
    const int xcd = g & 7, j = g >> 3;
    const int per = nwg >> 3, rem = nwg & 7;
    const int R = per + (xcd < rem ? 1 : 0);
    const int lo = xcd * per + (xcd < rem ? xcd : rem);
    const int C = cus_per_xcd;
    if (R <= C || R > 2 * C || (lo & 1)) return unit;
    const int P = R - C;
    const int local = j < P ? 2 * j : (j >= C ? 2 * (j - C) + 1 : 2 * P + (j - P));
    return lo + local;
}
__device__ __forceinline__ int cu_pair_unit(int cus_per_xcd, int unit) {
    return cu_pair_renumber(gridDim.x, blockIdx.x, cus_per_xcd, unit);
}

// Work items per scheduling unit for causal problems (host side).  Query
// (or key) blocks of a slice alternate long and short, so once the items
// outnumber the resident slots a unit of two consecutive items -- a long and
// a short one -- makes every unit equally long.  But pairs halve the number
// of units, and where that leaves slots idle single items under dynamic
// dispatch finish sooner: up to single_max items (pairs would fill only
// part of the slots), and, when short_steps > 0, for items of at most
// short_steps key tiles whose pairs would end in a round at most 60% full
// (short items even out by themselves).  steps: key tiles of 64 in the
// longest item.
inline int causal_items_per_unit(long long items, long long slots, long long single_max, int steps,
                                 int short_steps) {
    if (items <= slots || items <= single_max) return 1;
    const long long last = ((items + 1) / 2) % slots;   // pairs in their last round
    return (steps <= short_steps && last > 0 && 5 * last <= 3 * slots) ? 1 : 2;
}

// Work item -> (b*H + h, query block).  Causal query blocks of a head are
// ordered longest, shortest, second longest, second shortest, ...: items
// 2i and 2i + 1 of a head together take the same number of key tiles, so
// scheduling units of such pairs are all equally long.
template <bool CAUSAL>
__host__ __device__ __forceinline__ void item_block(int item, int num_qb, int* bh, int* qb) {
    *bh = item / num_qb;
    const int q = item - *bh * num_qb;
    *qb = !CAUSAL ? q : ((q & 1) ? (q >> 1) : num_qb - 1 - (q >> 1));
}

}  // namespace bf16k
}  // namespace sdpa
