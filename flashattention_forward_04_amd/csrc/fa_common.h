// fa_common.h - types shared by the gfx950 forward kernels and their host
// dispatch.  Device-side helpers live with the kernels that use them.
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

}  // namespace fa
