// fa_fwd_bf16.hip - FlashAttention-2 forward, bf16 in/out, for gfx950.
//
// What is computed (mlx-native flash_attn_train.rs, module doc "Algorithm";
// oxibonsai dit_attention_flash.rs, module doc "Flash-attention v2
// structure"): per query tile, stream the keys in tiles of BN, compute the
// score tile S = scale * Q K^T on the matrix cores, keep a running row max m
// and row sum l, rescale the output accumulator by exp(m_old - m_new), add
// P V, and finish with O /= l and L = m + ln l.  Scores are kept in base 2
// (the log2(e) factor is folded into the scale, as the mlx-native module doc
// "Scale convention" describes) so every exponential is one v_exp_f32.
//
// How it maps onto CDNA4:
//   * One work-group = NW wavefronts of 64 lanes; wave w owns 32 query rows.
//   * Both products run on v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
//     The score tile is formed transposed, S^T = K Q^T (K is the A operand
//     from LDS, Q the B operand held in VGPRs for the whole kernel).  In the
//     32x32 accumulator layout lane l then holds 16 keys of ONE query row
//     (row l%32; keys 8(r/4) + 4(l/32) + r%4 for register r), so the row max
//     and row sum are 16 in-register operations plus one exchange with lane
//     l^32.
//   * The output is accumulated transposed too, O^T = V^T P^T, so lane l
//     again owns query row l%32 and the per-row rescale is a plain multiply
//     of the lane's own accumulator registers by its own factor: no
//     diagonal-matrix product (the forge flash_attention_mma.metal header
//     explains why Metal needed one; CDNA4's accumulator layout is
//     documented, so it is not needed here).
//   * P goes from the S^T accumulator straight into the B operand of the
//     O^T product: the 8 keys a lane contributes per k-step are a
//     permutation of a 16-key chunk, and V^T is staged in LDS in that same
//     permuted key order so the A operand is one 16-byte LDS read per lane.
//   * K is staged in LDS row-major with a 16-byte pad per row; V is staged
//     transposed ([D][BN] with the key permutation) from coalesced 16-byte
//     global loads, packing 4 keys per 8-byte LDS write.
//   * Causal work-groups are issued longest-first, and key tiles past the
//     last query row of a work-group are never loaded (forge
//     flash_attention_mma.metal, the causal j_end bound); a wave whose rows
//     all precede a key tile skips that tile's arithmetic.
//   * Ragged tails: query rows past qL load zeros and are not stored; key
//     rows past kL are staged as zeros and their scores masked to -inf.
#include "fa_common.h"

#include <math.h>

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even fp32 -> bf16 pair, packed low = a, high = b.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    __bf16 x = (__bf16)a;
    __bf16 y = (__bf16)b;
    return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

template <int D, int MASK, bool CAUSAL, int NW, int BN>
__global__ void __launch_bounds__(NW * 64)
fwd_bf16_kernel(const FwdParams p)
{
    constexpr int NT = NW * 64;
    constexpr int BM = NW * 32;
    constexpr int KP = D + 8;   // K row pitch in LDS (elements), 16-byte pad
    constexpr int VP = BN + 8;  // V^T row pitch in LDS (elements), 16-byte pad
    constexpr int DK = D / 16;  // k-steps of S^T over the head dimension
    constexpr int NC = BN / 32; // 32-key blocks per key tile
    constexpr int ND = D / 32;  // 32-wide blocks of O^T along the head dimension
    static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");

    __shared__ __attribute__((aligned(16))) uint16_t Ks[BN * KP];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VP];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r32 = lane & 31;
    const int g = lane >> 5;

    // ---- which (query tile, head, batch) this work-group owns ----
    int id = blockIdx.x;
    const int h = id % p.Hq;
    id /= p.Hq;
    const int b = id % p.B;
    id /= p.B;
    const int qt = CAUSAL ? (p.n_qtiles - 1 - id) : id;  // longest causal tiles first
    const int q0 = qt * BM;
    const int hk = h / p.group;
    const int wq0 = q0 + wave * 32;
    const int qrow = wq0 + r32;

    const uint16_t* Qb = (const uint16_t*)p.q + b * p.q_s[0] + h * p.q_s[1];
    const uint16_t* Kb = (const uint16_t*)p.k + b * p.k_s[0] + hk * p.k_s[1];
    const uint16_t* Vb = (const uint16_t*)p.v + b * p.v_s[0] + hk * p.v_s[1];

    // ---- Q fragments: row qrow, elements 16ks + 8g .. +7 ----
    bf16x8 qf[DK];
    {
        const bool in = qrow < p.qL;
        const u32x4* src = (const u32x4*)(Qb + (int64_t)(in ? qrow : 0) * p.q_s[2]);
        const uint32_t flip = p.neg_q ? 0x80008000u : 0u;
#pragma unroll
        for (int ks = 0; ks < DK; ++ks) {
            u32x4 w = in ? src[2 * ks + g] : u32x4{0, 0, 0, 0};
            w ^= flip;
            qf[ks] = __builtin_bit_cast(bf16x8, w);
        }
    }

    const float c2 = p.scale_log2;
    const int kv_end = CAUSAL ? min(p.kL, min(p.qL, q0 + BM)) : p.kL;

    // mask row of this lane (clamped so ragged rows read in bounds)
    const uint8_t* mrow = nullptr;
    if (MASK != MASK_NONE) {
        const int qc = min(qrow, p.qL - 1);
        const int esz = (MASK == MASK_BOOL) ? 1 : 2;
        mrow = (const uint8_t*)p.mask + (b * p.m_s[0] + h * p.m_s[1] + (int64_t)qc * p.m_s[2]) * esz;
    }

    f32x16 o[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) o[d] = f32x16{};
    float m_run = -INFINITY;  // running max, base 2
    float l_run = 0.f;        // running sum

    for (int j0 = 0; j0 < kv_end; j0 += BN) {
        __syncthreads();  // the previous tile's LDS reads are done
        // ---- stage K (row-major) ----
        constexpr int KCH = BN * D / 8;
#pragma unroll
        for (int it = 0; it < (KCH + NT - 1) / NT; ++it) {
            const int c = tid + it * NT;
            if (KCH % NT != 0 && c >= KCH) break;
            const int row = c / (D / 8);
            const int col = c % (D / 8);
            const int j = j0 + row;
            u32x4 w = u32x4{0, 0, 0, 0};
            if (j < p.kL) w = *(const u32x4*)(Kb + (int64_t)j * p.k_s[2] + col * 8);
            *(u32x4*)(Ks + row * KP + col * 8) = w;
        }
        // ---- stage V transposed, keys permuted within each 16-key chunk ----
        // key quad qd (keys 4qd..4qd+3) lands at position 16(qd/4) + 4*perm[qd%4]
        // with perm = {0, 2, 1, 3}: a lane in half g then finds keys
        // {4g..4g+3, 8+4g..8+4g+3} of the chunk as 8 contiguous elements.
        constexpr int VU = (BN / 4) * (D / 8);
#pragma unroll
        for (int it = 0; it < (VU + NT - 1) / NT; ++it) {
            const int u = tid + it * NT;
            if (VU % NT != 0 && u >= VU) break;
            const int w8 = u % (D / 8);
            const int qd = u / (D / 8);
            u32x4 r[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = j0 + 4 * qd + e;
                r[e] = u32x4{0, 0, 0, 0};
                if (j < p.kL) r[e] = *(const u32x4*)(Vb + (int64_t)j * p.v_s[2] + w8 * 8);
            }
            const int pq = qd & 3;
            const int pos = 16 * (qd >> 2) + 4 * ((pq == 1) ? 2 : (pq == 2) ? 1 : pq);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int wd = i >> 1;
                uint32_t lo, hi;
                if (i & 1) {
                    lo = (r[0][wd] >> 16) | (r[1][wd] & 0xffff0000u);
                    hi = (r[2][wd] >> 16) | (r[3][wd] & 0xffff0000u);
                } else {
                    lo = (r[0][wd] & 0xffffu) | (r[1][wd] << 16);
                    hi = (r[2][wd] & 0xffffu) | (r[3][wd] << 16);
                }
                *(u32x2*)(Vt + (8 * w8 + i) * VP + pos) = u32x2{lo, hi};
            }
        }
        __syncthreads();

        // a wave whose rows all precede this key tile has nothing to do here
        if (CAUSAL && j0 > wq0 + 31) continue;

        // ---- S^T = K Q^T ----
        f32x16 s[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) s[c] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < DK; ++ks) {
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const bf16x8 kop = *(const bf16x8*)(Ks + (32 * c + r32) * KP + 16 * ks + 8 * g);
                s[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qf[ks], s[c], 0, 0, 0);
            }
        }

        // ---- masking: tail keys, causal diagonal, user mask ----
        const bool fast = (MASK == MASK_NONE) && (j0 + BN <= p.kL) && (!CAUSAL || j0 + BN - 1 <= wq0);
        float cs = c2;
        if (!fast) {
            cs = 1.f;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    const int jb = j0 + 32 * c + 8 * rq + 4 * g;  // first of 4 consecutive keys
                    float mv[4] = {0.f, 0.f, 0.f, 0.f};
                    bool mb[4] = {true, true, true, true};
                    if (MASK == MASK_ADD) {
                        if (p.mask_vec && jb + 3 < p.kL) {
                            const u32x2 w = *(const u32x2*)(mrow + 2 * (int64_t)jb);
                            mv[0] = bf16_bits_to_float(w[0] & 0xffffu);
                            mv[1] = bf16_bits_to_float(w[0] >> 16);
                            mv[2] = bf16_bits_to_float(w[1] & 0xffffu);
                            mv[3] = bf16_bits_to_float(w[1] >> 16);
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (jb + e < p.kL)
                                    mv[e] = bf16_bits_to_float(((const uint16_t*)mrow)[jb + e]);
                        }
                    } else if (MASK == MASK_BOOL) {
                        if (p.mask_vec && jb + 3 < p.kL) {
                            const uint32_t w = *(const uint32_t*)(mrow + jb);
#pragma unroll
                            for (int e = 0; e < 4; ++e) mb[e] = ((w >> (8 * e)) & 0xffu) != 0;
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e) mb[e] = (jb + e < p.kL) ? (mrow[jb + e] != 0) : false;
                        }
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int j = jb + e;
                        bool ok = (j < p.kL) && mb[e];
                        if (CAUSAL) ok = ok && (j <= qrow);
                        float t = s[c][4 * rq + e] * c2;
                        if (MASK == MASK_ADD) t = __builtin_fmaf(mv[e], kLog2e, t);
                        s[c][4 * rq + e] = ok ? t : -INFINITY;
                    }
                }
            }
        }

        // ---- online softmax for this lane's row ----
        float mx = s[0][0];
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[c][r]);
        mx = fmaxf(mx, xor32(mx));
        const float m_new = fmaxf(m_run, mx * cs);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float corr = __builtin_amdgcn_exp2f(m_run - m_use);
        float rs = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[c][r], cs, -m_use));
                s[c][r] = e;
                rs += e;
            }
        rs += xor32(rs);
        l_run = l_run * corr + rs;
        m_run = m_new;
#pragma unroll
        for (int d = 0; d < ND; ++d) o[d] *= corr;

        // ---- O^T += V^T P^T ----
#pragma unroll
        for (int c = 0; c < NC; ++c) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                u32x4 pw;
#pragma unroll
                for (int e = 0; e < 4; ++e) pw[e] = pack_bf16x2(s[c][8 * hh + 2 * e], s[c][8 * hh + 2 * e + 1]);
                const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
                const int kidx = 2 * c + hh;
#pragma unroll
                for (int d = 0; d < ND; ++d) {
                    const bf16x8 vop = *(const bf16x8*)(Vt + (32 * d + r32) * VP + 16 * kidx + 8 * g);
                    o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pf, o[d], 0, 0, 0);
                }
            }
        }
    }

    // ---- epilogue: O = O / l, L = m ln2 + ln l (O = 0, L = 0 if no key) ----
    if (qrow < p.qL) {
        const float inv = (l_run > 0.f) ? 1.f / l_run : 0.f;
        uint16_t* orow = (uint16_t*)p.o + b * p.o_s[0] + h * p.o_s[1] + (int64_t)qrow * p.o_s[2];
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                u32x2 w;
                w[0] = pack_bf16x2(o[d][4 * rq + 0] * inv, o[d][4 * rq + 1] * inv);
                w[1] = pack_bf16x2(o[d][4 * rq + 2] * inv, o[d][4 * rq + 3] * inv);
                *(u32x2*)(orow + 32 * d + 8 * rq + 4 * g) = w;
            }
        if (g == 0) {
            const float lse = (l_run > 0.f) ? (m_run + __builtin_amdgcn_logf(l_run)) * kLn2 : 0.f;
            p.lse[((int64_t)b * p.Hq + h) * p.qL + qrow] = lse;
        }
    }
}

template <int D, int MASK, bool CAUSAL, int NW, int BN>
hipError_t launch_bf16(const FwdParams& p, hipStream_t st)
{
    const dim3 grid((unsigned)p.n_qtiles * p.Hq * p.B);
    hipLaunchKernelGGL((fwd_bf16_kernel<D, MASK, CAUSAL, NW, BN>), grid, dim3(NW * 64), 0, st, p);
    return hipGetLastError();
}

}  // namespace

#define FA_BF16_VARIANT(D, MASK, CAUSAL, NW, BN, NAME) \
    {NAME, 1, D, MASK, CAUSAL, NW * 32, &launch_bf16<D, MASK, CAUSAL, NW, BN>}

#define FA_BF16_FOR_D(D, NW, BN)                                                          \
    FA_BF16_VARIANT(D, MASK_NONE, false, NW, BN, "fwd_bf16_d" #D "_nomask"),              \
    FA_BF16_VARIANT(D, MASK_NONE, true, NW, BN, "fwd_bf16_d" #D "_nomask_causal"),        \
    FA_BF16_VARIANT(D, MASK_ADD, false, NW, BN, "fwd_bf16_d" #D "_additive"),             \
    FA_BF16_VARIANT(D, MASK_ADD, true, NW, BN, "fwd_bf16_d" #D "_additive_causal"),       \
    FA_BF16_VARIANT(D, MASK_BOOL, false, NW, BN, "fwd_bf16_d" #D "_bool"),                \
    FA_BF16_VARIANT(D, MASK_BOOL, true, NW, BN, "fwd_bf16_d" #D "_bool_causal")

// Host-only accessor: a namespace-scope const table would also be emitted
// for the device, where the launch functions do not exist.
const Variant* variants_bf16(int* n)
{
    static const Variant table[] = {
    FA_BF16_FOR_D(64, 4, 64),
    FA_BF16_FOR_D(128, 4, 64),
    FA_BF16_FOR_D(256, 4, 32),
};
    *n = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace fa
