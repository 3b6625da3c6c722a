// fa_merge.h - the merge that ends a forward launch whose key range was split
// over work-groups (bf16 or fp32 output).
//
// Each split s leaves, per query row, its normalised partial O_s (fp32, D
// floats) and its natural-log L_s = m_s + ln l_s.  With L = ln sum_s e^{L_s},
// the row's result is O = sum_s e^{L_s - L} O_s: the rescale-and-add that the
// online softmax applies between key blocks (FlashAttention-2, Section 3.1,
// the forward pass), here applied once across the splits.
#pragma once

#include "fa_common.h"

#include <math.h>

namespace fa {
namespace {

// A work-group of four waves takes 4 / WPR query rows, WPR waves each.  A
// partial row is D/4 lanes of four floats, so one wave load covers 64 / (D/4)
// partial rows; the WPR waves of a row take its splits in turn, keep several
// loads in flight each, and meet in LDS.  Ranges with no allowed key
// (L_s = -inf) weigh 0; a row with none at all gets O = 0, L = 0.  Every
// partial is finite (an empty range writes zeros).
template <int D, bool BF16, int WPR>
__global__ void __launch_bounds__(256) merge_splits_kernel(const FwdParams p)
{
    typedef float v4 __attribute__((ext_vector_type(4)));
    typedef uint32_t w2 __attribute__((ext_vector_type(2)));
    typedef float v2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    constexpr int C4 = D / 4;     // lanes per partial row
    constexpr int SPW = 64 / C4;  // partial rows per wave load
    static_assert(D % 4 == 0 && C4 <= 64, "head dim");
    static_assert(WPR == 1 || WPR == 2 || WPR == 4, "waves per row");
    constexpr float kLog2e_ = 1.4426950408889634f;
    constexpr float kLn2_ = 0.6931471805599453f;
    __shared__ v4 red[256];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int part = wave % WPR;  // this wave's share of its row's splits
    const int64_t rows = (int64_t)p.B * p.Hq * p.qL;
    const int64_t row = (int64_t)blockIdx.x * (4 / WPR) + wave / WPR;
    const bool live = row < rows;
    // the largest L_s, and sum_s e^{L_s - max}: every wave for itself (the
    // n_split values of one row are a few hundred bytes)
    float lmax = -INFINITY;
    if (live)
        for (int s = lane; s < p.n_split; s += 64) lmax = fmaxf(lmax, p.l_part[s * rows + row]);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) lmax = fmaxf(lmax, __shfl_xor(lmax, m));
    float sum = 0.f;
    v4 acc = {0.f, 0.f, 0.f, 0.f};
    if (lmax != -INFINITY) {
        for (int s = lane; s < p.n_split; s += 64)
            sum += __builtin_amdgcn_exp2f((p.l_part[s * rows + row] - lmax) * kLog2e_);
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) sum += __shfl_xor(sum, m);
        const int sub = lane / C4, c = lane - sub * C4;
        if (sub < SPW) {
#pragma unroll 4
            for (int s = part * SPW + sub; s < p.n_split; s += WPR * SPW) {
                const float w = __builtin_amdgcn_exp2f((p.l_part[s * rows + row] - lmax) * kLog2e_);
                const v4 o = *(const v4*)(p.o_part + (s * rows + row) * D + 4 * c);
                acc[0] = __builtin_fmaf(w, o[0], acc[0]);
                acc[1] = __builtin_fmaf(w, o[1], acc[1]);
                acc[2] = __builtin_fmaf(w, o[2], acc[2]);
                acc[3] = __builtin_fmaf(w, o[3], acc[3]);
            }
        }
    }
    if (WPR * SPW > 1) {
        red[threadIdx.x] = acc;
        __syncthreads();
    }
    // the first wave of each row sums its row's WPR x SPW partial sums
    if (!live || part != 0 || lane >= C4) return;
    v4 t = acc;
    if (WPR * SPW > 1) {
        t = v4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < WPR * SPW; ++k) {
            const v4 r = red[(wave + k / SPW) * 64 + (k % SPW) * C4 + lane];
            t[0] += r[0];
            t[1] += r[1];
            t[2] += r[2];
            t[3] += r[3];
        }
    }
    const float inv = (sum > 0.f) ? 1.f / sum : 0.f;
    const int i = (int)(row % p.qL);
    const int64_t bh = row / p.qL;
    const int h = (int)(bh % p.Hq), b = (int)(bh / p.Hq);
    const int64_t at = b * p.o_s[0] + h * p.o_s[1] + (int64_t)i * p.o_s[2] + 4 * lane;
    if constexpr (BF16) {
        // round to nearest even, two elements per conversion
        w2 out;
        out[0] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v2{t[0] * inv, t[1] * inv}, b2));
        out[1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v2{t[2] * inv, t[3] * inv}, b2));
        *(w2*)((uint16_t*)p.o + at) = out;
    } else {
        *(v4*)((float*)p.o + at) = v4{t[0] * inv, t[1] * inv, t[2] * inv, t[3] * inv};
    }
    if (lane == 0) p.lse[row] = (sum > 0.f) ? lmax + __builtin_amdgcn_logf(sum) * kLn2_ : 0.f;
}

// Launch of the merge: waves per row by the loads a row takes (about four
// or more in flight per wave).
template <int D, bool BF16>
hipError_t launch_merge(const FwdParams& q, int64_t rows, hipStream_t st)
{
    constexpr int SPW = 64 / (D / 4);
    const int loads = (q.n_split + SPW - 1) / SPW;  // wave loads per row
    if (loads >= 16) {
        hipLaunchKernelGGL((merge_splits_kernel<D, BF16, 4>), dim3((unsigned)rows), dim3(256), 0, st, q);
    } else if (loads >= 8) {
        hipLaunchKernelGGL((merge_splits_kernel<D, BF16, 2>), dim3((unsigned)((rows + 1) / 2)), dim3(256), 0, st, q);
    } else {
        hipLaunchKernelGGL((merge_splits_kernel<D, BF16, 1>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, q);
    }
    return hipGetLastError();
}

}  // namespace
}  // namespace fa
