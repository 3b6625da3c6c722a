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
    float drop_scale;           // 1 / (1 - p), 0 when p >= 1 (applied to O at the end)
    uint32_t drop_thresh;       // ceil(p 2^24) 2^8 (mod 2^32): keep iff the word is >= it
    uint32_t seed_lo, seed_hi;  // the generator's key
    uint32_t off_lo, off_hi;    // 64-bit offset added to every counter
    // Scratch for the partials of a split launch, given by the caller of the
    // launcher (fa_fwd_strided_noalloc), ws_bytes long; null: the launcher
    // takes the partials from the library's pool.
    float* ws;
    size_t ws_bytes;
};

enum MaskKind { MASK_NONE = 0, MASK_ADD = 1, MASK_BOOL = 2 };

// Everything a backward launch needs.  Tensors are contiguous head-major:
// Q, O, dO, dQ [B, H_q, qL, D]; K, V, dK, dV [B, H_kv, kL, D]; L and Delta
// [B, H_q, qL] fp32.
struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dout;
    const float* lse;   // natural-log logsumexp of the forward pass
    const void* mask;
    float* delta;       // written: rowsum(dO * O)
    void* dq;
    void* dk;
    void* dv;
    int64_t m_s[3];     // mask strides {batch, head, seq} in elements
    int B, Hq, Hkv, qL, kL;
    int group;          // Hq / Hkv
    float scale;        // natural-domain score scale (signed)
    float scale_log2;   // scale * log2(e)
    int mask_vec;       // mask rows admit 4-element vector loads
    // dK/dV grid split over the heads of each GQA group (set by the
    // launcher): kv_split work-groups per key tile, each over group /
    // kv_split query heads, writing fp32 partials [s][dK, dV][B][H_kv][kL][D]
    // that a reduction sums
    float* kv_part;
    int kv_split;
};

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
// The same from a wave-uniform base (an SGPR pair) plus this lane's 32-bit
// byte offset: half the address bytes a 64-bit per-lane address takes, which
// makes the load cheaper to issue.
__device__ __forceinline__ void lds_dma16_so(const void* gbase, uint32_t byte_off, uint32_t lds_base) {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(byte_off), "s"(gbase), "s"(lds_base)
        : "memory");
}

__device__ __forceinline__ void lds_dma16(const void* gsrc, uint32_t lds_base) {
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, off"
        :
        : "v"(gsrc), "s"(lds_base)
        : "memory");
}

// Philox-4x32 with 10 rounds (Salmon, Moraes, Dror and Shaw, "Parallel
// random numbers: as easy as 1, 2, 3", SC 2011) on the counter (c0, c1, 0, 0)
// under the key (k0, k1): each round multiplies words 0 and 2 by the round
// constants, spreads the 64-bit products as (hi(c2 M1) ^ c1 ^ k0,
// lo(c2 M1), hi(c0 M0) ^ c3 ^ k1, lo(c0 M0)) and advances the key by the
// Weyl increments.
struct Words4 {
    uint32_t w0, w1, w2, w3;
};
__device__ __forceinline__ Words4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t k0, uint32_t k1)
{
    uint32_t c2 = 0u, c3 = 0u;
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        // one 32 x 32 -> 64-bit product each (a single multiply-add
        // instruction rather than separate low and high multiplies)
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        // three-input xors, one v_bitop3_b32 each (truth table 0x96 = a ^ b ^ c)
        const uint32_t n0 = __builtin_amdgcn_bitop3_b32(hi1, c1, k0, 0x96);
        const uint32_t n2 = __builtin_amdgcn_bitop3_b32(hi0, c3, k1, 0x96);
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return Words4{c0, c1, c2, c3};
}
__device__ __forceinline__ uint32_t word_at(const Words4& w, int i)
{
    return i == 0 ? w.w0 : i == 1 ? w.w1 : i == 2 ? w.w2 : w.w3;
}

// Keep bits of the 4 consecutive score positions n0 .. n0 + 3
// (n = ((b H_q + h) qL + i) kL + j): word n mod 4 of the Philox block at
// counter offset + floor(n / 4) decides key n; 1 keeps the term, 0 drops it.
// The kernels apply the common 1 / (1 - p) to O at the end, so P times a
// keep bit stays exact in bf16.
__device__ __forceinline__ void dropout_quad(const FwdParams& p, int64_t n0, float* mult)
{
    const uint64_t off = ((uint64_t)p.off_hi << 32) | p.off_lo;
    const uint64_t ctr = off + ((uint64_t)n0 >> 2);
    const Words4 wa = philox4x32_10((uint32_t)ctr, (uint32_t)(ctr >> 32), p.seed_lo, p.seed_hi);
    // u = floor(w / 2^8) / 2^24 >= p  <=>  floor(w / 2^8) >= ceil(p 2^24)
    // <=>  w >= ceil(p 2^24) 2^8 = drop_thresh (an integer compare)
    auto keep = [&](uint32_t w) __attribute__((always_inline)) { return (w >= p.drop_thresh) ? 1.f : 0.f; };
    if ((p.kL & 3) == 0) {
        // every row starts at a multiple of 4: one block covers the quad
        mult[0] = keep(wa.w0);
        mult[1] = keep(wa.w1);
        mult[2] = keep(wa.w2);
        mult[3] = keep(wa.w3);
    } else {
        const Words4 wb = philox4x32_10((uint32_t)(ctr + 1), (uint32_t)((ctr + 1) >> 32), p.seed_lo, p.seed_hi);
        const int sh = (int)(n0 & 3);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = sh + e;
            mult[e] = keep(i < 4 ? word_at(wa, i) : word_at(wb, i - 4));
        }
    }
}

// One compiled variant: its launch function and shape facts the host needs.
// With `need` non-null a launch function only plans: it stores the scratch
// bytes its launch would take for the partials of a split key range (0 for
// none) and launches nothing.
typedef hipError_t (*LaunchFn)(const FwdParams&, hipStream_t, size_t* need);

struct Variant {
    const char* name;
    int dtype;      // 0 fp32, 1 bf16 (fa_dtype)
    int D;
    int mask;       // MaskKind
    int causal;
    int block_m;    // query rows per work-group
    LaunchFn launch;
};

// The head dims with compiled kernels; each has a translation unit per
// dtype (fa_fwd_bf16_d<D>.hip, fa_fwd_f32_d<D>.hip) defining its variant
// tables (host only).
#define FA_FOR_EACH_HEAD_DIM(X) X(16) X(32) X(48) X(64) X(80) X(96) X(128) X(256)
#define FA_DECLARE_TABLES(D)                      \
    const Variant* variants_bf16_d##D(int* n);         \
    const Variant* variants_bf16_dropout_d##D(int* n); \
    const Variant* variants_f32_d##D(int* n);          \
    const Variant* variants_f32_dropout_d##D(int* n);
FA_FOR_EACH_HEAD_DIM(FA_DECLARE_TABLES)
#undef FA_DECLARE_TABLES

// Backward variants (fa_bwd_bf16_d<D>.hip), host only.
typedef hipError_t (*BwdLaunchFn)(const BwdParams&, hipStream_t);
struct BwdVariant {
    const char* name;
    int D;
    int mask;    // MaskKind
    int causal;
    BwdLaunchFn launch;
};
#define FA_FOR_EACH_BWD_HEAD_DIM(X) X(64) X(128)
#define FA_DECLARE_BWD_TABLES(D) const BwdVariant* bwd_variants_bf16_d##D(int* n);
FA_FOR_EACH_BWD_HEAD_DIM(FA_DECLARE_BWD_TABLES)
#undef FA_DECLARE_BWD_TABLES
const BwdVariant* bwd_variants_bf16(int* n);

// Every variant of one kind, over all head dims (fa_api.cpp, host only).
const Variant* variants_bf16(int* n);
const Variant* variants_f32(int* n);
const Variant* variants_bf16_dropout(int* n);
const Variant* variants_f32_dropout(int* n);

// The stream-ordered memory pool the library creates for itself on the
// current device (fa_api.cpp): split launches take their partials from it.
hipError_t library_pool(hipMemPool_t* out);

}  // namespace fa
