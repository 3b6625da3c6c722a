// fa_common.h - types shared by the gfx950 forward kernels and their host
// dispatch, and the device helpers both kernel files use.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Everything a launch needs, passed by value as one kernel argument.
// Strides are in elements, {batch, head, seq}; the innermost axis (D, or kL
// for the mask) is contiguous.
struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* mask;
    void* o;
    float* lse;
    int64_t q_s[3];
    int64_t k_s[3];
    int64_t v_s[3];
    int64_t o_s[3];
    int64_t m_s[3];
    int B, Hq, Hkv, qL, kL;
    int group;          // Hq / Hkv: consecutive query heads per kv head
    int n_qtiles;       // ceil(qL / BM) for the chosen variant
    float scale_log2;   // |scale| * log2(e): scores live in base 2
    int neg_q;          // scale < 0: Q's sign bit is flipped on load instead
    int mask_vec;       // mask rows admit 4-element vector loads
    int pair_tiles;     // causal: the whole grid is resident at once (see causal_tile)
    // Key range split over work-groups (n_split > 1): work-group s of a
    // query tile takes key tiles [s * split_tiles, (s + 1) * split_tiles)
    // and writes its normalised O (fp32, [n_split][B][H_q][qL][D]) and its
    // natural-log L ([n_split][B][H_q][qL], -inf when no key of the range is
    // allowed) to o_part / l_part; a merge kernel combines them.
    float* o_part;
    float* l_part;
    int n_split;        // 1: no split
    int split_tiles;
    // Work-group kernel: rows [32 t, 32 t + 32) of NW query heads of one GQA
    // group per work-group, one head per wave (short query ranges).
    int head_pack;
    // Causal sliding window (the work-group kernels, bf16 and fp32):
    // window >= 1 restricts row i to keys i - window + 1 .. i; 0 is no window.
    int window;
    // Dropout (the work-group kernel's dropout variants): a P V term is kept
    // when the Philox-4x32-10 word drawn for its score position, as
    // u = (word >> 8) / 2^24, is >= drop_p, and then scaled by drop_scale.
    float drop_p;
    float drop_scale;           // 1 / (1 - p), 0 when p >= 1
    uint32_t drop_thresh;       // ceil(p 2^24) 2^8 (mod 2^32): keep iff the word is >= it
    uint32_t seed_lo, seed_hi;  // the generator's key
    uint32_t off_lo, off_hi;    // 64-bit offset added to every counter
};

enum MaskKind { MASK_NONE = 0, MASK_ADD = 1, MASK_BOOL = 2 };

// Work-groups are dispatched round-robin over the 8 XCDs (each with its own
// L2): work-group i runs on XCD i % 8.  Within the H_q consecutive
// work-groups of one (query tile, batch), slot i gets query head
// (i % 8) * (H_q / 8) + i / 8, so each XCD receives H_q / 8 consecutive
// heads -- whole GQA groups when H_kv >= 8 -- and re-reads their K/V tiles
// from its own L2.  Other head counts keep the plain order.
__device__ __forceinline__ int head_of(int slot, int Hq) {
    return (Hq % 8 == 0) ? (slot % 8) * (Hq / 8) + slot / 8 : slot;
}

// Causal query tiles differ in length (tile t sees t + 1 key blocks).
// Work-group rank r (ids in dispatch order, one rank per H_q * B ids) gets
// tile n - 1 - r, longest first, which balances a grid that runs in several
// rounds.  When the whole grid is resident at once the second half is
// reversed (shortest first), so that the work-groups placed second on each
// CU complement the first: rank r and rank r + (n + 1) / 2 get tiles n - 1 - r
// and r, n + 1 key blocks together.
__device__ __forceinline__ int causal_tile(int rank, int n, int pair) {
    if (!pair) return n - 1 - rank;
    const int half = (n + 1) / 2;
    return rank < half ? n - 1 - rank : rank - half;
}

// True when a grid of `wgs` work-groups fits on the GPU at once, given how
// many work-groups one CU holds.
inline bool grid_fits_at_once(int64_t wgs, int wgs_per_cu) {
    constexpr int kCUs = 256;
    return wgs <= (int64_t)kCUs * (wgs_per_cu > 0 ? wgs_per_cu : 1);
}

// One direct global -> LDS load (global_load_lds_dwordx4): lane l's 16
// bytes land at LDS byte address lds_base + 16 l.  It is issued from inline
// assembly so that the compiler does not track it: while a direct load it
// knows of is in flight, the compiler turns every wait for an LDS read into
// a wait for all of them, which serialises the operand reads with the
// matrix products.  Completion is ordered instead by the key loop's explicit
// vmcnt waits and barriers (a load the compiler does not know of can only
// make its own waits wait longer).
//
// M0 (the LDS base of the load) is set and left as is: a wave issues each
// instruction in ~4 cycles, and saving and restoring M0 around every load
// doubled its cost (~28 against ~13 cycles, measured on MI355X).  The
// kernels that use these loads read M0 nowhere else: they issue no
// compiler-tracked direct load and index no register array at run time (a
// test scans the built code object for any other M0 use).  The s_nop is the
// wait the hardware needs between writing M0 and the load that reads it.
__device__ __forceinline__ void lds_dma16(const void* gsrc, uint32_t lds_base) {
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, off"
        :
        : "v"(gsrc), "s"(lds_base)
        : "memory");
}

// One compiled variant: its launch function and shape facts the host needs.
typedef hipError_t (*LaunchFn)(const FwdParams&, hipStream_t);

struct Variant {
    const char* name;
    int dtype;      // 0 fp32, 1 bf16 (fa_dtype)
    int D;
    int mask;       // MaskKind
    int causal;
    int block_m;    // query rows per work-group
    LaunchFn launch;
};

// Variant tables defined by each kernel translation unit (host only).
const Variant* variants_bf16(int* n);
const Variant* variants_f32(int* n);
const Variant* variants_bf16_dropout(int* n);

}  // namespace fa
