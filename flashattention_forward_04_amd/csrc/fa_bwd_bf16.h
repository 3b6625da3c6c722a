// fa_bwd_bf16.h - FlashAttention-2 backward (dQ, dK, dV), bf16 in/out, for
// gfx950: the kernel templates and their launcher.  Each fa_bwd_bf16_d<D>.hip
// instantiates the variants of one head dim.
//
// What is computed (forge flash_attention_mma.metal, the backward section's
// header; mlx-native flash_attn_train.rs, "Phase 2 -- FA-2 backward kernel";
// ruDNN dense_attention.rs, `backward_kv_owned`): with P_ij = exp(s_ij - L_i)
// the forward pass's softmax weights (L its natural-log logsumexp; 0 for keys
// that are not allowed),
//     Delta_i = rowsum(dO_i * O_i)
//     dP_ij   = dO_i . V_j,      dS_ij = P_ij (dP_ij - Delta_i)
//     dQ_i    = scale sum_j dS_ij K_j
//     dK_j    = scale sum_{i, heads of j's group} dS_ij Q_i
//     dV_j    = sum_{i, heads of j's group} P_ij dO_i
// No online rescale is needed: L fixes the normalisation.
//
// Three launches, no atomics, deterministic (the split the forge header
// describes; the KV-owned grid covers whole GQA groups as ruDNN's
// `backward_kv_owned` does):
//   * delta: Delta = rowsum(dO * O) in fp32, one row per 16 lanes (D = 128)
//   * dQ: one work-group per (query tile of 32 NW rows, head); Q and dO stay
//     in VGPRs; K and V tiles stream through LDS.  Per key tile:
//       S^T = K Q^T and dP^T = V dO^T on the matrix cores (lane l holds 16
//       keys of query row l%32, as in the forward kernel), P and dS in the
//       accumulator layout, then dQ^T += K^T dS^T with K^T read by
//       transposing LDS reads and dS^T fed straight from the accumulators.
//   * dK, dV: one work-group per (key tile of 32 NW keys, kv head); K and V
//     stay in VGPRs; the Q and dO tiles of every query head of the group
//     stream through LDS.  Per query tile:
//       S = Q K^T and dP = dO V^T (lane l holds 16 queries of key l%32),
//       P and dS, then dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T
//       read by transposing LDS reads.
//   S and dP are formed in both grids (seven matrix products where an atomic
//   dQ would take five); that is the price of owning every output row.
// bf16 P and dS feed the matrix products (fp32 accumulation); Delta, P and dS
// are fp32 before that rounding.
#pragma once

#include "fa_common.h"

#include <math.h>

#include <algorithm>

namespace fa {
namespace {

typedef __bf16 bwd_bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bwd_bf16x2 __attribute__((ext_vector_type(2)));
typedef float bwd_f32x16 __attribute__((ext_vector_type(16)));
typedef float bwd_f32x2 __attribute__((ext_vector_type(2)));
typedef float bwd_f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t bwd_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t bwd_u32x2 __attribute__((ext_vector_type(2)));
typedef short bwd_i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bwd_i16x4 bwd_lds_i16x4;

constexpr float kBwdLog2e = 1.4426950408889634f;

__device__ __forceinline__ uint32_t bwd_pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(bwd_f32x2{a, b}, bwd_bf16x2));
}

__device__ __forceinline__ float bwd_bf16_to_float(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// ds_read_b64_tr_b16: within each 16-lane group, source lane 4e + a reads 4
// consecutive bf16 of row e (of four rows) at column 4a; destination lane t
// receives column t of all four rows.
__device__ __forceinline__ bwd_i16x4 bwd_lds_read_tr(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((bwd_lds_i16x4*)p);
}

// Rows [r0, r0 + ROWS) of a bf16 matrix with D columns and a row stride of
// `stride` elements, staged into LDS with row pitch PITCH elements by direct
// global -> LDS loads (global_load_lds_dwordx4, tracked by the compiler).
// The LDS tile is padded to whole 1 KiB blocks: block i is filled by one load
// of wave i % NW, whose lane l writes 16-byte slot 64 i + l (slots in a row's
// pad are skipped).  Rows past `nrows` repeat row nrows - 1 (finite values,
// masked by the caller).
// UNTRACKED: issued from inline assembly (lds_dma16), which the compiler
// does not count, so that its waits for LDS operand reads stay narrow; the
// kernel's own vmcnt(0) before each barrier retires them.
template <int D, int PITCH, int ROWS, int NW, bool UNTRACKED = false>
__device__ __forceinline__ void bwd_stage_rows(const uint16_t* gbase, int64_t stride, int r0, int nrows,
                                               uint16_t* lds, int wave, int lane)
{
    constexpr int SPR = PITCH / 8;
    constexpr int NINS = (ROWS * SPR + 63) / 64;
#pragma unroll
    for (int k = 0; k < (NINS + NW - 1) / NW; ++k) {
        const int i = wave + k * NW;
        if (NINS % NW != 0 && i >= NINS) break;
        const int slot = 64 * i + lane;
        const int row = slot / SPR, ch = slot % SPR;
        if (ch < D / 8 && row < ROWS) {
            const int rr = min(r0 + row, nrows - 1);
            if constexpr (UNTRACKED)
                lds_dma16(gbase + (int64_t)rr * stride + ch * 8,
                          __builtin_amdgcn_readfirstlane(
                              (uint32_t)(size_t)(__attribute__((address_space(3))) void*)(lds + 512 * i)));
            else
                __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(gbase + (int64_t)rr * stride + ch * 8),
                                                 (__attribute__((address_space(3))) void*)(lds + 512 * i), 16, 0, 0);
        }
    }
}

template <int ROWS, int PITCH>
constexpr int bwd_tile_elems() { return ((ROWS * PITCH / 8 + 63) / 64) * 512; }

// Row pitch padding (elements) of the tiles read both as rows and by
// transposing reads (K in the dQ grid, Q and dO in the dK/dV grid).
#ifndef FA_BWD_TILE_PAD
#define FA_BWD_TILE_PAD 24
#endif

__device__ __forceinline__ void bwd_wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// The dQ grid stages its K and V tiles with untracked direct loads (3 %
// faster at the 8k D = 128 shape); the dK/dV grid keeps the builtin, with
// which it does not spill (it spilled 24 bytes and ran 23 % slower with the
// untracked form).
#ifndef FA_BWD_DQ_UNTRACKED
#define FA_BWD_DQ_UNTRACKED 1
#endif

// ---------------------------------------------------------------- Delta
// Delta[row] = sum_d dO[row, d] O[row, d] in fp32; D/8 lanes per row, each
// with 8 elements (16 bytes).
template <int D>
__global__ void __launch_bounds__(256) bwd_delta_kernel(const BwdParams p)
{
    constexpr int LPR = D / 8;  // lanes per row
    const int64_t rows = (int64_t)p.B * p.Hq * p.qL;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = t / LPR;
    const int part = (int)(t % LPR);
    float acc = 0.f;
    if (row < rows) {
        const bwd_u32x4 a = *(const bwd_u32x4*)((const uint16_t*)p.o + row * D + 8 * part);
        const bwd_u32x4 b = *(const bwd_u32x4*)((const uint16_t*)p.dout + row * D + 8 * part);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc = __builtin_fmaf(bwd_bf16_to_float(a[e] & 0xffffu), bwd_bf16_to_float(b[e] & 0xffffu), acc);
            acc = __builtin_fmaf(bwd_bf16_to_float(a[e] >> 16), bwd_bf16_to_float(b[e] >> 16), acc);
        }
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, LPR);
    if (row < rows && part == 0) p.delta[row] = acc;
}

// ---------------------------------------------------------------- dQ
template <int D, int MASK, bool CAUSAL, int NW, int BN, int WPE>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
bwd_dq_kernel(const BwdParams p)
{
    constexpr int BM = NW * 32;
    constexpr int KP = D + FA_BWD_TILE_PAD;  // K tile pitch: row reads and transposing reads
    constexpr int VP = D + 8;   // V tile pitch: row reads only
    constexpr int KT = bwd_tile_elems<BN, KP>();
    constexpr int VT = bwd_tile_elems<BN, VP>();
    constexpr int DK = D / 16;  // k-steps over the head dim
    constexpr int NC = BN / 32;  // 32-key blocks per tile
    constexpr int ND = D / 32;   // 32-wide blocks of dQ^T
    static_assert(D % 32 == 0 && BN % 32 == 0, "tile shape");
    __shared__ __attribute__((aligned(1024))) uint16_t Ks[2][KT];
    __shared__ __attribute__((aligned(1024))) uint16_t Vs[2][VT];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r32 = lane & 31, g = lane >> 5, lt = lane & 15;

    int id = blockIdx.x;
    const int h = head_of(id % p.Hq, p.Hq);
    id /= p.Hq;
    const int b = id % p.B;
    id /= p.B;
    const int n_qt = (p.qL + BM - 1) / BM;
    const int qt = CAUSAL ? n_qt - 1 - id : id;  // causal: longest tiles first
    const int q0 = qt * BM;
    const int wq0 = q0 + wave * 32;
    const int qrow = wq0 + r32;
    const int hk = h / p.group;
    const bool row_in = qrow < p.qL;

    const int64_t qoff = (((int64_t)b * p.Hq + h) * p.qL) * D;
    const uint16_t* Kb = (const uint16_t*)p.k + ((int64_t)b * p.Hkv + hk) * p.kL * D;
    const uint16_t* Vb = (const uint16_t*)p.v + ((int64_t)b * p.Hkv + hk) * p.kL * D;

    // Q and dO of this lane's row as B operands (elements 16 ks + 8 g .. + 7)
    bwd_bf16x8 qf[DK], of[DK];
    {
        const int rr = row_in ? qrow : 0;
        const bwd_u32x4* qs = (const bwd_u32x4*)((const uint16_t*)p.q + qoff + (int64_t)rr * D);
        const bwd_u32x4* os = (const bwd_u32x4*)((const uint16_t*)p.dout + qoff + (int64_t)rr * D);
#pragma unroll
        for (int ks = 0; ks < DK; ++ks) {
            qf[ks] = __builtin_bit_cast(bwd_bf16x8, row_in ? qs[2 * ks + g] : bwd_u32x4{0, 0, 0, 0});
            of[ks] = __builtin_bit_cast(bwd_bf16x8, row_in ? os[2 * ks + g] : bwd_u32x4{0, 0, 0, 0});
        }
    }
    const int64_t srow = ((int64_t)b * p.Hq + h) * p.qL + (row_in ? qrow : 0);
    const float l2 = row_in ? p.lse[srow] * kBwdLog2e : 0.f;  // base-2 logsumexp
    const float delta = row_in ? p.delta[srow] : 0.f;
    const float c2 = p.scale_log2;
    const uint8_t* mrow = nullptr;
    if (MASK != MASK_NONE) {
        const int esz = MASK == MASK_BOOL ? 1 : 2;
        mrow = (const uint8_t*)p.mask + (b * p.m_s[0] + h * p.m_s[1] + (int64_t)min(qrow, p.qL - 1) * p.m_s[2]) * esz;
    }

    bwd_f32x16 dq[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) dq[d] = bwd_f32x16{};

    const int kv_end = CAUSAL ? min(p.kL, min(p.qL, q0 + BM)) : p.kL;
    const int n_tiles = (kv_end + BN - 1) / BN;
    // this wave needs tiles 0 .. t_last (causal rows never see later keys)
    int t_last = n_tiles - 1;
    if (CAUSAL) t_last = min(t_last, (wq0 + 31) / BN);
    if (wq0 >= p.qL) t_last = -1;

    auto stage = [&](int t, int buf) __attribute__((always_inline)) {
        bwd_stage_rows<D, KP, BN, NW, FA_BWD_DQ_UNTRACKED>(Kb, D, t * BN, p.kL, Ks[buf], wave, lane);
        bwd_stage_rows<D, VP, BN, NW, FA_BWD_DQ_UNTRACKED>(Vb, D, t * BN, p.kL, Vs[buf], wave, lane);
    };
    if (n_tiles > 0) stage(0, 0);
    for (int t = 0; t < n_tiles; ++t) {
        const int buf = t & 1;
        bwd_wait_loads();
        __syncthreads();  // tile t is in LDS; every wave is done with buffer buf ^ 1
        if (t + 1 < n_tiles) stage(t + 1, buf ^ 1);
        if (t > t_last) continue;
        const uint16_t* kt = Ks[buf];
        const uint16_t* vt = Vs[buf];
        const int j0 = t * BN;
        // S^T = K Q^T and dP^T = V dO^T
        bwd_f32x16 s[NC], dp[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            s[c] = bwd_f32x16{};
            dp[c] = bwd_f32x16{};
        }
#pragma unroll
        for (int ks = 0; ks < DK; ++ks)
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const bwd_bf16x8 ka = *(const bwd_bf16x8*)(kt + (32 * c + r32) * KP + (2 * ks + g) * 8);
                const bwd_bf16x8 va = *(const bwd_bf16x8*)(vt + (32 * c + r32) * VP + (2 * ks + g) * 8);
                s[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s[c], 0, 0, 0);
                dp[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, of[ks], dp[c], 0, 0, 0);
            }
        // P = exp2(s c2 (+ mask log2 e) - l2) over the allowed keys; dS = P (dP - Delta)
        const bool edge = (j0 + BN > p.kL) || (CAUSAL && j0 + BN - 1 > wq0) || MASK != MASK_NONE;
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int jb = j0 + 32 * c + 8 * rq + 4 * g;  // 4 consecutive keys
                bwd_u32x2 mw = {0u, 0u};
                if (MASK != MASK_NONE) {
                    if (p.mask_vec && jb + 3 < p.kL) {
                        if (MASK == MASK_ADD) mw = *(const bwd_u32x2*)(mrow + 2 * (int64_t)jb);
                        else mw[0] = *(const uint32_t*)(mrow + jb);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            if (jb + e >= p.kL) continue;
                            if (MASK == MASK_ADD) mw[e >> 1] |= (uint32_t)((const uint16_t*)mrow)[jb + e] << (16 * (e & 1));
                            else if (mrow[jb + e] != 0) mw[0] |= 1u << (8 * e);
                        }
                    }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * rq + e;
                    const int j = jb + e;
                    float x = __builtin_fmaf(s[c][r], c2, -l2);
                    bool ok = true;
                    if (edge) {
                        ok = j < p.kL && row_in;
                        if (CAUSAL) ok = ok && j <= qrow;
                        if (MASK == MASK_BOOL) ok = ok && ((mw[0] >> (8 * e)) & 0xffu) != 0;
                        if (MASK == MASK_ADD) x = __builtin_fmaf(bwd_bf16_to_float((mw[e >> 1] >> (16 * (e & 1))) & 0xffffu), kBwdLog2e, x);
                    }
                    const float pr = ok ? __builtin_amdgcn_exp2f(x) : 0.f;
                    s[c][r] = pr * (dp[c][r] - delta);  // dS
                }
            }
        // dQ^T += K^T dS^T: 16-key chunks, K^T by transposing reads in the
        // key order the dS registers hold
#pragma unroll
        for (int kidx = 0; kidx < 2 * NC; ++kidx) {
            const int c = kidx >> 1, hh = kidx & 1;
            bwd_u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = bwd_pack_bf16x2(s[c][8 * hh + 2 * e], s[c][8 * hh + 2 * e + 1]);
            const bwd_bf16x8 dsf = __builtin_bit_cast(bwd_bf16x8, w);
            const int row0 = 16 * kidx + 4 * g + (lt >> 2);
#pragma unroll
            for (int d = 0; d < ND; ++d) {
                const int col = 32 * d + 16 * ((lane >> 4) & 1) + 4 * (lt & 3);
                const bwd_i16x4 a0 = bwd_lds_read_tr(kt + row0 * KP + col);
                const bwd_i16x4 a1 = bwd_lds_read_tr(kt + (row0 + 8) * KP + col);
                const bwd_bf16x8 kta = __builtin_bit_cast(bwd_bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
                dq[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kta, dsf, dq[d], 0, 0, 0);
            }
        }
    }
    // dQ = scale dQ^T, row qrow, head-dim 32 d + 8 rq + 4 g + {0..3}
    if (row_in) {
        uint16_t* orow = (uint16_t*)p.dq + qoff + (int64_t)qrow * D;
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                bwd_u32x2 w;
                w[0] = bwd_pack_bf16x2(dq[d][4 * rq] * p.scale, dq[d][4 * rq + 1] * p.scale);
                w[1] = bwd_pack_bf16x2(dq[d][4 * rq + 2] * p.scale, dq[d][4 * rq + 3] * p.scale);
                *(bwd_u32x2*)(orow + 32 * d + 8 * rq + 4 * g) = w;
            }
    }
}

// ---------------------------------------------------------------- dK, dV
// KVS: the grid is split kv_split ways per key tile (fp32 partials): the
// work-group of split s takes steps s, s + kv_split, ... of the key tile's
// (query head, query tile) steps.  The unsplit kernel is a separate
// instantiation so that its code is unchanged.
template <int D, int MASK, bool CAUSAL, int NW, int BQ, int WPE, bool KVS>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
bwd_dkdv_kernel(const BwdParams p)
{
    constexpr int BK = NW * 32;  // keys per work-group
    constexpr int TP = D + FA_BWD_TILE_PAD;  // Q and dO tile pitch: row reads and transposing reads
    constexpr int TT = bwd_tile_elems<BQ, TP>();
    constexpr int DK = D / 16;
    constexpr int NQ = BQ / 32;  // 32-query blocks per tile
    constexpr int ND = D / 32;
    static_assert(D % 32 == 0 && BQ % 32 == 0 && BQ <= 64, "tile shape");
    __shared__ __attribute__((aligned(1024))) uint16_t Qs[2][TT];
    __shared__ __attribute__((aligned(1024))) uint16_t Os[2][TT];
    __shared__ __attribute__((aligned(16))) float Ls[2][64];  // L2 of the tile's rows (raw L, natural log)
    __shared__ __attribute__((aligned(16))) float Ds[2][64];  // Delta of the tile's rows

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r32 = lane & 31, g = lane >> 5, lt = lane & 15;

    // kv head innermost: with H_kv a multiple of 8 every work-group of a kv
    // head runs on one XCD and re-reads that group's Q and dO from its L2.
    int id = blockIdx.x;
    const int hk = id % p.Hkv;
    id /= p.Hkv;
    const int kvs = KVS ? p.kv_split : 1;
    const int split = KVS ? id % kvs : 0;
    id /= kvs;
    const int h_first = hk * p.group;
    const int b = id % p.B;
    id /= p.B;
    const int k0 = id * BK;  // causal: the first key tiles see the most queries (issued first)
    const int wk0 = k0 + wave * 32;
    const int key = wk0 + r32;
    const bool key_in = key < p.kL;

    const int64_t kvoff = (((int64_t)b * p.Hkv + hk) * p.kL) * D;
    bwd_bf16x8 kf[DK], vf[DK];
    {
        const int kk = key_in ? key : 0;
        const bwd_u32x4* ks_ = (const bwd_u32x4*)((const uint16_t*)p.k + kvoff + (int64_t)kk * D);
        const bwd_u32x4* vs_ = (const bwd_u32x4*)((const uint16_t*)p.v + kvoff + (int64_t)kk * D);
#pragma unroll
        for (int ks = 0; ks < DK; ++ks) {
            kf[ks] = __builtin_bit_cast(bwd_bf16x8, key_in ? ks_[2 * ks + g] : bwd_u32x4{0, 0, 0, 0});
            vf[ks] = __builtin_bit_cast(bwd_bf16x8, key_in ? vs_[2 * ks + g] : bwd_u32x4{0, 0, 0, 0});
        }
    }
    const float c2 = p.scale_log2;

    bwd_f32x16 dk[ND], dv[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) {
        dk[d] = bwd_f32x16{};
        dv[d] = bwd_f32x16{};
    }

    // query tiles of one head: causal keys [k0, k0 + BK) are seen by rows >= k0 only
    const int qt0 = CAUSAL ? min(k0, p.qL) / BQ : 0;
    const int n_qt = (p.qL + BQ - 1) / BQ;
    const int per_head = max(0, n_qt - qt0);
    // the key tile's steps (query head, query tile); a split work-group takes
    // every kvs-th of them, from its own
    const int n_all = (k0 < p.kL) ? per_head * p.group : 0;
    const int n_steps = KVS ? (n_all > split ? (n_all - split + kvs - 1) / kvs : 0) : n_all;
    auto at = [&](int step) __attribute__((always_inline)) { return KVS ? split + step * kvs : step; };

    auto stage = [&](int step, int buf) __attribute__((always_inline)) {
        const int h = h_first + at(step) / per_head;
        const int q0 = (qt0 + at(step) % per_head) * BQ;
        const int64_t qoff = (((int64_t)b * p.Hq + h) * p.qL) * D;
        bwd_stage_rows<D, TP, BQ, NW>((const uint16_t*)p.q + qoff, D, q0, p.qL, Qs[buf], wave, lane);
        bwd_stage_rows<D, TP, BQ, NW>((const uint16_t*)p.dout + qoff, D, q0, p.qL, Os[buf], wave, lane);
        if (wave == NW - 1 && lane < BQ) {
            // L and Delta of the tile's rows (rows past qL repeat row qL - 1)
            const int64_t r = ((int64_t)b * p.Hq + h) * p.qL + min(q0 + lane, p.qL - 1);
            __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(p.lse + r),
                                             (__attribute__((address_space(3))) void*)(&Ls[buf][0]), 4, 0, 0);
            __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(p.delta + r),
                                             (__attribute__((address_space(3))) void*)(&Ds[buf][0]), 4, 0, 0);
        }
    };
    if (n_steps > 0) stage(0, 0);
    for (int step = 0; step < n_steps; ++step) {
        const int buf = step & 1;
        bwd_wait_loads();
        __syncthreads();  // this step's tiles are in LDS; buffer buf ^ 1 is free
        if (step + 1 < n_steps) stage(step + 1, buf ^ 1);
        const int h = h_first + at(step) / per_head;
        const int q0 = (qt0 + at(step) % per_head) * BQ;
        // a wave whose keys all follow the tile's last row skips it
        if (wk0 >= p.kL) continue;
        if (CAUSAL && wk0 > q0 + BQ - 1) continue;
        const uint16_t* qt = Qs[buf];
        const uint16_t* ot = Os[buf];
        // S = Q K^T and dP = dO V^T: lane l holds key l%32 and queries
        // 32 qb + 8 (r/4) + 4 g + r%4
        bwd_f32x16 s[NQ], dp[NQ];
#pragma unroll
        for (int qb = 0; qb < NQ; ++qb) {
            s[qb] = bwd_f32x16{};
            dp[qb] = bwd_f32x16{};
        }
#pragma unroll
        for (int ks = 0; ks < DK; ++ks)
#pragma unroll
            for (int qb = 0; qb < NQ; ++qb) {
                const bwd_bf16x8 qa = *(const bwd_bf16x8*)(qt + (32 * qb + r32) * TP + (2 * ks + g) * 8);
                const bwd_bf16x8 oa = *(const bwd_bf16x8*)(ot + (32 * qb + r32) * TP + (2 * ks + g) * 8);
                s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[ks], s[qb], 0, 0, 0);
                dp[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, vf[ks], dp[qb], 0, 0, 0);
            }
        // P and dS; this lane's 16 rows per block are 4 runs of 4 consecutive rows
        const bool edge = (q0 + BQ > p.qL) || (CAUSAL && q0 < wk0 + 31) || !key_in || MASK != MASK_NONE;
        const uint8_t* mcol = nullptr;
        if (MASK != MASK_NONE) {
            const int esz = MASK == MASK_BOOL ? 1 : 2;
            mcol = (const uint8_t*)p.mask + (b * p.m_s[0] + h * p.m_s[1]) * esz + (int64_t)min(key, p.kL - 1) * esz;
        }
#pragma unroll
        for (int qb = 0; qb < NQ; ++qb)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int ib = 32 * qb + 8 * rq + 4 * g;  // first of 4 rows within the tile
                const bwd_f32x4 lv = *(const bwd_f32x4*)(&Ls[buf][ib]);
                const bwd_f32x4 dv4 = *(const bwd_f32x4*)(&Ds[buf][ib]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * rq + e;
                    const int i = q0 + ib + e;
                    float x = __builtin_fmaf(s[qb][r], c2, -lv[e] * kBwdLog2e);
                    bool ok = true;
                    if (edge) {
                        ok = i < p.qL && key_in;
                        if (CAUSAL) ok = ok && key <= i;
                        if (MASK != MASK_NONE && ok) {
                            const uint8_t* mp = mcol + (int64_t)i * p.m_s[2] * (MASK == MASK_BOOL ? 1 : 2);
                            if (MASK == MASK_BOOL) ok = *mp != 0;
                            else x = __builtin_fmaf(bwd_bf16_to_float(*(const uint16_t*)mp), kBwdLog2e, x);
                        }
                    }
                    const float pr = ok ? __builtin_amdgcn_exp2f(x) : 0.f;
                    dp[qb][r] = pr * (dp[qb][r] - dv4[e]);  // dS
                    s[qb][r] = pr;                           // P
                }
            }
        // dV^T += dO^T P and dK^T += Q^T dS over 16-query chunks
#pragma unroll
        for (int kidx = 0; kidx < 2 * NQ; ++kidx) {
            const int qb = kidx >> 1, hh = kidx & 1;
            bwd_u32x4 wp, wd;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                wp[e] = bwd_pack_bf16x2(s[qb][8 * hh + 2 * e], s[qb][8 * hh + 2 * e + 1]);
                wd[e] = bwd_pack_bf16x2(dp[qb][8 * hh + 2 * e], dp[qb][8 * hh + 2 * e + 1]);
            }
            const bwd_bf16x8 pf = __builtin_bit_cast(bwd_bf16x8, wp);
            const bwd_bf16x8 dsf = __builtin_bit_cast(bwd_bf16x8, wd);
            const int row0 = 16 * kidx + 4 * g + (lt >> 2);
#pragma unroll
            for (int d = 0; d < ND; ++d) {
                const int col = 32 * d + 16 * ((lane >> 4) & 1) + 4 * (lt & 3);
                const bwd_i16x4 o0 = bwd_lds_read_tr(ot + row0 * TP + col);
                const bwd_i16x4 o1 = bwd_lds_read_tr(ot + (row0 + 8) * TP + col);
                const bwd_i16x4 q0v = bwd_lds_read_tr(qt + row0 * TP + col);
                const bwd_i16x4 q1v = bwd_lds_read_tr(qt + (row0 + 8) * TP + col);
                const bwd_bf16x8 ota = __builtin_bit_cast(bwd_bf16x8, __builtin_shufflevector(o0, o1, 0, 1, 2, 3, 4, 5, 6, 7));
                const bwd_bf16x8 qta = __builtin_bit_cast(bwd_bf16x8, __builtin_shufflevector(q0v, q1v, 0, 1, 2, 3, 4, 5, 6, 7));
                dv[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ota, pf, dv[d], 0, 0, 0);
                dk[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qta, dsf, dk[d], 0, 0, 0);
            }
        }
    }
    if constexpr (KVS) {
        // fp32 partials of this work-group's heads.  A lane holds 4
        // consecutive head-dim elements of its key per register quad; each
        // wave passes its 32 keys through a 32 x 36 float region of the idle
        // Q/dO buffers, one 32-column block at a time, so that every store
        // writes whole 128-byte lines of four key rows.
        constexpr int XP = 36, XE = 32 * XP * 2;  // region pitch (floats), size (16-bit elements)
        constexpr int R = TT / XE;                // regions per buffer
        static_assert(4 * R >= NW, "a partial region per wave");
        __syncthreads();  // every wave is past its last read of the Q/dO buffers
        const int w = wave;
        float* xs = (float*)(w < R       ? &Qs[0][w * XE]
                             : w < 2 * R ? &Qs[1][(w - R) * XE]
                             : w < 3 * R ? &Os[0][(w - 2 * R) * XE]
                                         : &Os[1][(w - 3 * R) * XE]);
        const int64_t plane = (int64_t)p.B * p.Hkv * p.kL * D;  // one partial dK or dV
        float* base = p.kv_part + 2 * (int64_t)split * plane + kvoff + (int64_t)wk0 * D;
#pragma unroll
        for (int which = 0; which < 2; ++which)
#pragma unroll
            for (int d = 0; d < ND; ++d) {
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    const bwd_f32x16& a = which == 0 ? dk[d] : dv[d];
                    *(bwd_f32x4*)(xs + r32 * XP + 8 * rq + 4 * g) =
                        bwd_f32x4{a[4 * rq], a[4 * rq + 1], a[4 * rq + 2], a[4 * rq + 3]};
                }
                // lane l reads columns 4 (l % 8) .. +3 of key rows 8 i + l / 8
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rr = 8 * i + (lane >> 3), c4 = 4 * (lane & 7);
                    const bwd_f32x4 v = *(const bwd_f32x4*)(xs + rr * XP + c4);
                    if (wk0 + rr < p.kL)
                        *(bwd_f32x4*)(base + which * plane + (int64_t)rr * D + 32 * d + c4) = v;
                }
            }
        return;
    }
    // dK = scale dK^T, dV = dV^T: key row `key`, head-dim 32 d + 8 rq + 4 g + {0..3}
    if (key_in) {
        uint16_t* krow = (uint16_t*)p.dk + kvoff + (int64_t)key * D;
        uint16_t* vrow = (uint16_t*)p.dv + kvoff + (int64_t)key * D;
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                bwd_u32x2 wk, wv;
                wk[0] = bwd_pack_bf16x2(dk[d][4 * rq] * p.scale, dk[d][4 * rq + 1] * p.scale);
                wk[1] = bwd_pack_bf16x2(dk[d][4 * rq + 2] * p.scale, dk[d][4 * rq + 3] * p.scale);
                wv[0] = bwd_pack_bf16x2(dv[d][4 * rq], dv[d][4 * rq + 1]);
                wv[1] = bwd_pack_bf16x2(dv[d][4 * rq + 2], dv[d][4 * rq + 3]);
                *(bwd_u32x2*)(krow + 32 * d + 8 * rq + 4 * g) = wk;
                *(bwd_u32x2*)(vrow + 32 * d + 8 * rq + 4 * g) = wv;
            }
    }
}

// Sum of the kv_split partials of a split dK/dV grid: dK = scale sum_s dK_s,
// dV = sum_s dV_s in bf16; each thread takes 4 consecutive elements of one
// key row of both.
template <int D>
__global__ void __launch_bounds__(256) bwd_dkdv_reduce_kernel(const BwdParams p)
{
    const int64_t plane = (int64_t)p.B * p.Hkv * p.kL * D;
    const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (e >= plane) return;
    bwd_f32x4 sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < p.kv_split; ++s) {
        sk += *(const bwd_f32x4*)(p.kv_part + 2 * (int64_t)s * plane + e);
        sv += *(const bwd_f32x4*)(p.kv_part + (2 * (int64_t)s + 1) * plane + e);
    }
    bwd_u32x2 wk, wv;
    wk[0] = bwd_pack_bf16x2(sk[0] * p.scale, sk[1] * p.scale);
    wk[1] = bwd_pack_bf16x2(sk[2] * p.scale, sk[3] * p.scale);
    wv[0] = bwd_pack_bf16x2(sv[0], sv[1]);
    wv[1] = bwd_pack_bf16x2(sv[2], sv[3]);
    *(bwd_u32x2*)((uint16_t*)p.dk + e) = wk;
    *(bwd_u32x2*)((uint16_t*)p.dv + e) = wv;
}

// Work-groups each key tile's steps are split over (1: none).  A non-causal
// grid with fewer work-groups than CUs splits them over up to 512 /
// work-groups.  A causal grid (small, or of up to ~two resident rounds)
// splits them over up to FA_BWD_CAUSAL_MAX_WGS / work-groups: its first key
// tiles see every query tile and its last almost none, and with every
// work-group resident at once the launch lasts as long as the longest one
// (at 32 heads x 8192 keys, 1024 steps against 520 on average); split, the
// longest takes half as many steps and the rest fill in behind it.  Up to
// 1024 work-groups then, and at most kMaxSplit ways.
#ifndef FA_BWD_CAUSAL_MAX_WGS
#define FA_BWD_CAUSAL_MAX_WGS 1024
#endif
inline int bwd_kv_split(int64_t kv_wgs, bool causal)
{
    constexpr int kCUs = 256, kMaxWgs = 512, kMaxSplit = 16;
    if (kv_wgs <= 0 || (kv_wgs >= kCUs && !causal)) return 1;
    // (a small causal grid takes the causal cap too: at 2 x 4 kv heads x 2048
    // keys, D = 64, 8 ways against 4 took the dK/dV kernel from 72 to 62 us
    // and the reduction from 6.3 to 10.9, 5.5 us less per call)
    const int64_t cap = causal ? FA_BWD_CAUSAL_MAX_WGS : kMaxWgs;
    return (int)std::max<int64_t>(1, std::min<int64_t>(kMaxSplit, cap / kv_wgs));
}

// Launch shapes: work-group waves and tile rows of the dQ and dK/dV grids.
template <int D, int MASK, bool CAUSAL, int QNW, int BN, int QWPE, int KNW, int BQ, int KWPE>
hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t st)
{
    const int64_t rows = (int64_t)p.B * p.Hq * p.qL;
    const int64_t delta_threads = rows * (D / 8);
    hipLaunchKernelGGL((bwd_delta_kernel<D>), dim3((unsigned)((delta_threads + 255) / 256)), dim3(256), 0, st, p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t dq_wgs = (int64_t)((p.qL + QNW * 32 - 1) / (QNW * 32)) * p.Hq * p.B;
    hipLaunchKernelGGL((bwd_dq_kernel<D, MASK, CAUSAL, QNW, BN, QWPE>), dim3((unsigned)dq_wgs), dim3(QNW * 64), 0, st, p);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t kv_wgs = (int64_t)((p.kL + KNW * 32 - 1) / (KNW * 32)) * p.Hkv * p.B;
    BwdParams q = p;
    q.kv_split = bwd_kv_split(kv_wgs, CAUSAL);
    q.kv_part = nullptr;
    if (q.kv_split == 1) {
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, MASK, CAUSAL, KNW, BQ, KWPE, false>), dim3((unsigned)kv_wgs),
                           dim3(KNW * 64), 0, st, q);
        return hipGetLastError();
    }
    // the partials come from the library's stream-ordered pool and go back
    // to it once the reduction has read them; every partial element the
    // reduction reads is written by the split grid first
    const int64_t plane = (int64_t)p.B * p.Hkv * p.kL * D;
    hipMemPool_t pool;
    err = library_pool(&pool);
    if (err != hipSuccess) return err;
    void* ws = nullptr;
    err = hipMallocFromPoolAsync(&ws, (size_t)(2 * q.kv_split * plane) * sizeof(float), pool, st);
    if (err != hipSuccess) return err;
    q.kv_part = (float*)ws;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, MASK, CAUSAL, KNW, BQ, KWPE, true>), dim3((unsigned)(kv_wgs * q.kv_split)),
                       dim3(KNW * 64), 0, st, q);
    err = hipGetLastError();
    if (err == hipSuccess) {
        hipLaunchKernelGGL((bwd_dkdv_reduce_kernel<D>), dim3((unsigned)((plane / 4 + 255) / 256)), dim3(256), 0, st, q);
        err = hipGetLastError();
    }
    const hipError_t ferr = hipFreeAsync(ws, st);
    return err != hipSuccess ? err : ferr;
}

}  // namespace

// Launch shapes per head dim: dQ grid (waves, keys per tile, waves per SIMD),
// dK/dV grid (waves, queries per tile, waves per SIMD).
#ifndef FA_BWD_D64_CFG
#define FA_BWD_D64_CFG 4, 64, 2, 4, 64, 2
#endif
#ifndef FA_BWD_D128_CFG
#define FA_BWD_D128_CFG 4, 32, 2, 4, 32, 2
#endif

#define FA_BWD_VARIANT(D, MASK, CAUSAL, NAME, QNW, BN, QWPE, KNW, BQ, KWPE) \
    {NAME, D, MASK, CAUSAL, &launch_bwd_bf16<D, MASK, CAUSAL, QNW, BN, QWPE, KNW, BQ, KWPE>}
#define FA_BWD_VARIANT_CFG(...) FA_BWD_VARIANT(__VA_ARGS__)
#define FA_BWD_FOR_D(D, CFG)                                                      \
    FA_BWD_VARIANT_CFG(D, MASK_NONE, false, "bwd_bf16_d" #D "_nomask", CFG),         \
    FA_BWD_VARIANT_CFG(D, MASK_NONE, true, "bwd_bf16_d" #D "_nomask_causal", CFG),   \
    FA_BWD_VARIANT_CFG(D, MASK_ADD, false, "bwd_bf16_d" #D "_additive", CFG),        \
    FA_BWD_VARIANT_CFG(D, MASK_ADD, true, "bwd_bf16_d" #D "_additive_causal", CFG),  \
    FA_BWD_VARIANT_CFG(D, MASK_BOOL, false, "bwd_bf16_d" #D "_bool", CFG),           \
    FA_BWD_VARIANT_CFG(D, MASK_BOOL, true, "bwd_bf16_d" #D "_bool_causal", CFG)

}  // namespace fa
