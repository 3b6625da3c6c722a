// fa_fwd_f32.h - FlashAttention-2 forward, fp32 in/out, for gfx950: the
// kernel template and its launcher.  Each fa_fwd_f32_d<D>.hip instantiates
// the variants of one head dim.
//
// Same algorithm as the bf16 kernel (mlx-native flash_attn_train.rs, module
// doc "Algorithm"), with every operand kept in fp32: Q, K, V, the scores, P
// and the accumulators.  The oxibonsai dit_attention_flash.rs module doc
// reports that staging full-range values in half precision broke its 1e-3
// parity bound, so this path never rounds P or the operands down.
//
// CDNA4 mapping:
//   * Both products run on v_mfma_f32_32x32x2_f32.  As in the bf16 kernel the
//     score tile is formed transposed, S^T = K Q^T, so lane l holds 16 keys
//     of query row l%32 and row reductions stay in-lane plus one exchange
//     with lane l^32; the output is accumulated as O^T = V^T P^T so the
//     per-row rescale multiplies the lane's own registers.
//   * The head dimension is contracted in an order that lets one 16-byte LDS
//     read of K feed four MFMAs: step 4t+e uses element 8t + 4(l/32) + e.  Q
//     is held in VGPRs in the matching order.
//   * Score register r of S^T is the P operand of one O^T step directly
//     (fp32 MFMAs take one k element per lane), and V^T is staged in LDS so
//     one 16-byte read yields the V operand of four consecutive steps.
//   * Output rows are written through the caller's strides, which is how the
//     token-major [seq, heads*D] layout of the DiT joint attention
//     (oxibonsai dit_attention_flash.rs, module doc) is produced in place.
#pragma once

#include "fa_common.h"
#include "fa_merge.h"

#include <math.h>

namespace fa {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// The running max is moved, and O and l rescaled, only when a row's new max
// exceeds it by more than this (base-2 units): the same softmax, with the
// rescale of the accumulators skipped on almost every tile.  Measured: the
// DiT shape (24 heads x 4096 x 4096, D = 128) 1708 -> 1670 us, the fp32
// decode shape's main kernel 110.6 -> 105.3 us.
constexpr float kRescaleSlackF32 = 8.f;

// PACK (query ranges of at most 16 rows, GQA groups of a multiple of 4
// heads): a wave's 32 rows are 16 rows each of two query heads of one group
// (lane rows 0-15 the first, 16-31 the second), and a work-group takes 2 NW
// heads of the group, so every matrix row is a real row and the work-group's
// K/V tiles serve all of its heads.
template <int D, int MASK, bool CAUSAL, int NW, int BN, bool DROP = false, bool PACK = false>
__global__ void __launch_bounds__(NW * 64)
fwd_f32_kernel(const FwdParams p)
{
    constexpr int NT = NW * 64;
    constexpr int BM = NW * 32;
    constexpr int KP = D + 4;   // K row pitch in LDS (floats)
    constexpr int VP = BN + 4;  // V^T row pitch in LDS (floats)
    constexpr int DT = D / 8;   // groups of four k-steps over the head dimension
    constexpr int NC = BN / 32;
    // 32-wide blocks of O^T; a head dim that is not a multiple of 32 is
    // rounded up, and the extra rows of the last block (which only ever
    // meet V^T rows past D) are never stored
    constexpr int ND = (D + 31) / 32;
    constexpr int DP = 32 * ND;  // V^T rows in LDS (the rows past D are read, never written)
    static_assert(BN % 32 == 0 && D % 16 == 0, "tile shape");

    // two buffers each: K row-major (filled by direct global -> LDS loads,
    // padded to whole 1 KiB blocks) and V transposed (filled from registers)
    constexpr int KSPR = KP / 4;                 // 16-byte slots per K row
    constexpr int KINS = (BN * KSPR + 63) / 64;  // 1 KiB blocks per K tile
    __shared__ __attribute__((aligned(1024))) float Ks0[KINS * 256];
    __shared__ __attribute__((aligned(1024))) float Ks1[KINS * 256];
    __shared__ __attribute__((aligned(16))) float Vt0[DP * VP];
    __shared__ __attribute__((aligned(16))) float Vt1[DP * VP];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r32 = lane & 31;
    const int g = lane >> 5;

    int id = blockIdx.x;
    int h, hk, split, b, q0, wq0, qrow;
    if constexpr (PACK) {
        // kv head innermost (a group's work-groups on one XCD when H_kv is a
        // multiple of 8), then the group's chunk of 2 NW heads, then the split
        const int nch = p.group / (2 * NW);
        hk = id % p.Hkv;
        id /= p.Hkv;
        const int c = id % nch;
        id /= nch;
        split = id % p.n_split;
        id /= p.n_split;
        b = id % p.B;
        h = hk * p.group + c * 2 * NW + 2 * wave + (r32 >> 4);  // this lane's head
        q0 = 0;
        wq0 = 0;
        qrow = r32 & 15;
    } else {
        h = head_of(id % p.Hq, p.Hq);
        id /= p.Hq;
        // key range split over work-groups (n_split > 1): this work-group takes
        // key tiles [split * split_tiles, (split + 1) * split_tiles)
        split = id % p.n_split;
        id /= p.n_split;
        b = id % p.B;
        id /= p.B;
        const int qt = CAUSAL ? causal_tile(id, p.n_qtiles, p.pair_tiles) : id;
        q0 = qt * BM;
        hk = h / p.group;
        wq0 = q0 + wave * 32;
        qrow = wq0 + r32;
    }
    // the last row any lane of this wave holds
    const int wq_last = PACK ? 15 : wq0 + 31;

    const float* Qb = (const float*)p.q + b * p.q_s[0] + h * p.q_s[1];
    const float* Kb = (const float*)p.k + b * p.k_s[0] + hk * p.k_s[1];
    const float* Vb = (const float*)p.v + b * p.v_s[0] + hk * p.v_s[1];

    // Q: qf[t] = Q[qrow][8t + 4g .. +3]
    f32x4 qf[DT];
    {
        const bool in = qrow < p.qL;
        const f32x4* src = (const f32x4*)(Qb + (int64_t)(in ? qrow : 0) * p.q_s[2]);
        const float sgn = p.neg_q ? -1.f : 1.f;
#pragma unroll
        for (int t = 0; t < DT; ++t) qf[t] = in ? src[2 * t + g] * sgn : f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // dropout: the score position of this lane's row at key 0
    const int64_t drow = DROP ? (((int64_t)b * p.Hq + h) * p.qL + qrow) * p.kL : 0;

    const float c2 = p.scale_log2;
    const int kv_end = CAUSAL ? min(p.kL, min(p.qL, PACK ? 16 : q0 + BM)) : p.kL;
    // causal sliding window: rows see keys from i - window + 1 on, so the
    // work-group starts at the tile of its first row's first key
    const bool win = CAUSAL && p.window > 0;
    const int t_first = (win ? max(0, q0 - p.window + 1) / BN : 0) + split * p.split_tiles;

    const uint8_t* mrow = nullptr;
    if (MASK != MASK_NONE) {
        const int qc = min(qrow, p.qL - 1);
        const int esz = (MASK == MASK_BOOL) ? 1 : 4;
        mrow = (const uint8_t*)p.mask + (b * p.m_s[0] + h * p.m_s[1] + (int64_t)qc * p.m_s[2]) * esz;
    }

    f32x16 o[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) o[d] = f32x16{};
    float m_run = -INFINITY;
    float l_run = 0.f;

    // ---- one key tile: j0, its K (row-major) and V^T staged at Ks, Vt ----
    auto tile = [&](int j0, const float* Ks, const float* Vt) __attribute__((always_inline)) {
        // ---- S^T = K Q^T ----
        f32x16 s[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) s[c] = f32x16{};
#pragma unroll
        for (int t = 0; t < DT; ++t) {
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const f32x4 kv = *(const f32x4*)(Ks + (32 * c + r32) * KP + 8 * t + 4 * g);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    s[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[e], qf[t][e], s[c], 0, 0, 0);
            }
        }

        // (a tile reaching below the window of the wave's last row is masked too)
        const bool w_edge = win && j0 < wq_last + 1 - p.window;
        const bool fast = (MASK == MASK_NONE) && (j0 + BN <= p.kL) && (!CAUSAL || j0 + BN - 1 <= wq0) && !w_edge;
        float cs = c2;
        if (!fast) {
            cs = 1.f;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    const int jb = j0 + 32 * c + 8 * rq + 4 * g;
                    float mv[4] = {0.f, 0.f, 0.f, 0.f};
                    bool mb[4] = {true, true, true, true};
                    if (MASK == MASK_ADD) {
                        if (p.mask_vec && jb + 3 < p.kL) {
                            const f32x4 w = *(const f32x4*)(mrow + 4 * (int64_t)jb);
#pragma unroll
                            for (int e = 0; e < 4; ++e) mv[e] = w[e];
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (jb + e < p.kL) mv[e] = ((const float*)mrow)[jb + e];
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
                        if (CAUSAL) ok = ok && (!w_edge || j > qrow - p.window);
                        float t = s[c][4 * rq + e] * c2;
                        if (MASK == MASK_ADD) t = __builtin_fmaf(mv[e], kLog2e, t);
                        s[c][4 * rq + e] = ok ? t : -INFINITY;
                    }
                }
            }
        }

        float mx = s[0][0];
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[c][r]);
        mx = fmaxf(mx, xor32(mx));
        // the running max moves (and O, l are rescaled) only when a row's
        // tile max exceeds it by more than kRescaleSlackF32; P is taken
        // against m_run, so it stays <= 2^kRescaleSlackF32
        const float m_tile = mx * cs;
        if (__builtin_amdgcn_ballot_w64(m_tile > m_run + kRescaleSlackF32) != 0) {
            const float m_new = fmaxf(m_run, m_tile);
            if (m_run != -INFINITY && m_new != m_run) {
                const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
                l_run *= corr;
#pragma unroll
                for (int d = 0; d < ND; ++d) o[d] *= corr;
            }
            m_run = m_new;
        }
        const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
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
        l_run += rs;
        if constexpr (DROP) {
            // the row sum above takes P before dropout (l and L are those
            // without it); only the P V product sees the multipliers
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    float mlt[4];
                    dropout_quad(p, drow + j0 + 32 * c + 8 * rq + 4 * g, mlt);
#pragma unroll
                    for (int e = 0; e < 4; ++e) s[c][4 * rq + e] *= mlt[e];
                }
        }

        // ---- O^T += V^T P^T: step r of key block c is key 32c + 8(r/4) + 4g + r%4 ----
#pragma unroll
        for (int c = 0; c < NC; ++c) {
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
#pragma unroll
                for (int d = 0; d < ND; ++d) {
                    const f32x4 vv = *(const f32x4*)(Vt + (32 * d + r32) * VP + 32 * c + 8 * rq + 4 * g);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        o[d] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv[e], s[c][4 * rq + e], o[d], 0, 0, 0);
                }
            }
        }
    };

    const int n_all = (kv_end + BN - 1) / BN;
    // (tiles are numbered from 0 at key 0; a split work-group ends its range early)
    const int n_tiles = p.n_split > 1 ? min(n_all, t_first + p.split_tiles) : n_all;
    // this wave needs tiles 0..t_last (causal rows never see later keys)
    int t_last = n_tiles - 1;
    if (CAUSAL) t_last = min(t_last, wq_last / BN);
    if (wq0 >= p.qL) t_last = -1;  // every row of this wave is past qL: it only helps stage tiles

    // A full tile (all BN rows below kL) loads from a tile base that is the
    // same for every lane (SGPRs) plus per-lane 32-bit byte offsets computed
    // once; the tail tile takes the clamped per-slot path.
    const bool off32 = (int64_t)BN * max(p.k_s[2], p.v_s[2]) * 4 < ((int64_t)1 << 31);
    auto uniform_base = [](const float* ptr) __attribute__((always_inline)) {
        const uint64_t a = (uint64_t)(size_t)ptr;
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
        return (const char*)(size_t)(((uint64_t)hi << 32) | (uint64_t)lo);
    };
    constexpr int KIT = (KINS + NW - 1) / NW;
    uint32_t koff[KIT];
#pragma unroll
    for (int k = 0; k < KIT; ++k) {
        const int slot = 64 * (wave + k * NW) + lane;
        koff[k] = (uint32_t)(((int64_t)(slot / KSPR) * p.k_s[2] + (slot % KSPR) * 4) * 4);
    }

    // K tile t -> LDS directly: 1 KiB block i by wave i % NW, lane l writing
    // slot 64i + l; pad slots are skipped, rows past kL repeat row kL - 1
    auto issue_k = [&](int t, float* kt) __attribute__((always_inline)) {
        if (MASK == MASK_NONE && (t + 1) * BN <= p.kL && off32) {
            const char* tbase = uniform_base(Kb + (int64_t)t * BN * p.k_s[2]);
#pragma unroll
            for (int k = 0; k < KIT; ++k) {
                const int i = wave + k * NW;
                if (KINS % NW != 0 && i >= KINS) break;
                const int slot = 64 * i + lane;
                if (slot % KSPR < D / 4 && slot / KSPR < BN)
                    lds_dma16_so(tbase, koff[k], (uint32_t)(size_t)(__attribute__((address_space(3))) void*)(kt + 256 * i));
            }
            return;
        }
#pragma unroll
        for (int k = 0; k < (KINS + NW - 1) / NW; ++k) {
            const int i = wave + k * NW;
            if (KINS % NW != 0 && i >= KINS) break;
            const int slot = 64 * i + lane;
            const int row = slot / KSPR;
            const int ch = slot % KSPR;
            if (ch < D / 4 && row < BN) {
                const int j = min(t * BN + row, p.kL - 1);
                const float* src = Kb + (int64_t)j * p.k_s[2] + ch * 4;
                if (MASK == MASK_NONE) {
                    lds_dma16(src, (uint32_t)(size_t)(__attribute__((address_space(3))) void*)(kt + 256 * i));
                } else {
                    // tracked by the compiler: the mask loads' waits count exactly
                    __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)src,
                                                     (__attribute__((address_space(3))) void*)(kt + 256 * i), 16, 0,
                                                     0);
                }
            }
        }
    };
    // V tile t -> registers (4 keys x 4 dims per unit), stored transposed
    // into LDS once the current tile is done with the other buffer
    constexpr int VU = (BN / 4) * (D / 4);
    constexpr int VIT = (VU + NT - 1) / NT;
    f32x4 vr[VIT][4];
    uint32_t voff[VIT][4];
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
        const int u = min(tid + it * NT, VU - 1);
        const int w4 = u % (D / 4);
        const int qd = u / (D / 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) voff[it][e] = (uint32_t)(((int64_t)(4 * qd + e) * p.v_s[2] + w4 * 4) * 4);
    }
    auto load_v = [&](int t) __attribute__((always_inline)) {
        if ((t + 1) * BN <= p.kL && off32) {
            // (formed from Vb itself, not through readfirstlane: the loads
            // stay global ones; a pointer rebuilt from integers would make
            // them flat loads, which an LDS-read wait also waits for)
            const char* tbase = (const char*)(Vb + (int64_t)t * BN * p.v_s[2]);
#pragma unroll
            for (int it = 0; it < VIT; ++it) {
                const int u = tid + it * NT;
                if (VU % NT != 0 && u >= VU) break;
#pragma unroll
                for (int e = 0; e < 4; ++e) vr[it][e] = *(const f32x4*)(tbase + voff[it][e]);
            }
            return;
        }
#pragma unroll
        for (int it = 0; it < VIT; ++it) {
            const int u = tid + it * NT;
            if (VU % NT != 0 && u >= VU) break;
            const int w4 = u % (D / 4);
            const int qd = u / (D / 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = min(t * BN + 4 * qd + e, p.kL - 1);
                vr[it][e] = *(const f32x4*)(Vb + (int64_t)j * p.v_s[2] + w4 * 4);
            }
        }
    };
    auto store_v = [&](float* vt) __attribute__((always_inline)) {
#pragma unroll
        for (int it = 0; it < VIT; ++it) {
            const int u = tid + it * NT;
            if (VU % NT != 0 && u >= VU) break;
            const int w4 = u % (D / 4);
            const int qd = u / (D / 4);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *(f32x4*)(vt + (4 * w4 + i) * VP + 4 * qd) =
                    f32x4{vr[it][0][i], vr[it][1][i], vr[it][2][i], vr[it][3][i]};
        }
    };

    // the first tile, then the loop: tile t+1 is loaded (K straight into
    // LDS, V into registers) while tile t is computed; V goes to LDS after
    // tile t.  (Rows past kL are clamped to kL - 1, so a first tile past the
    // key range loads in bounds and the loop does not run.)
    issue_k(t_first, Ks0);
    load_v(t_first);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    store_v(Vt0);
    __syncthreads();
    auto step = [&](int t, const float* Ks, const float* Vt, float* kn, float* vn) __attribute__((always_inline)) {
        const int j0 = t * BN;
        const bool more = t + 1 < n_tiles;
        if (more) {
            issue_k(t + 1, kn);
            load_v(t + 1);
        }
        if (t <= t_last) {
            tile(j0, Ks, Vt);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): K of tile t+1 in LDS, V in registers
        if (more) store_v(vn);
        __syncthreads();
    };
    for (int t = t_first; t < n_tiles; t += 2) {
        step(t, Ks0, Vt0, Ks1, Vt1);
        if (t + 1 < n_tiles) step(t + 1, Ks1, Vt1, Ks0, Vt0);
    }

    if (qrow < p.qL && p.n_split > 1) {
        // one key range of a split launch: its normalised O and natural-log L
        // (-inf when the range holds no allowed key), merged afterwards
        const float inv = (l_run > 0.f) ? (DROP ? p.drop_scale : 1.f) / l_run : 0.f;
        const int64_t rows = (int64_t)p.B * p.Hq * p.qL;
        const int64_t row = ((int64_t)b * p.Hq + h) * p.qL + qrow;
        float* orow = p.o_part + ((int64_t)split * rows + row) * D;
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                if (32 * d + 8 * rq >= D) continue;
                *(f32x4*)(orow + 32 * d + 8 * rq + 4 * g) =
                    f32x4{o[d][4 * rq + 0], o[d][4 * rq + 1], o[d][4 * rq + 2], o[d][4 * rq + 3]} * inv;
            }
        if (g == 0)
            p.l_part[(int64_t)split * rows + row] =
                (l_run > 0.f) ? (m_run + __builtin_amdgcn_logf(l_run)) * kLn2 : -INFINITY;
    } else if (qrow < p.qL) {
        // dropout's 1 / (1 - p) scales every kept term alike: it is applied here
        const float inv = (l_run > 0.f) ? (DROP ? p.drop_scale : 1.f) / l_run : 0.f;
        float* orow = (float*)p.o + b * p.o_s[0] + h * p.o_s[1] + (int64_t)qrow * p.o_s[2];
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                if (32 * d + 8 * rq >= D) continue;  // rows of the rounded-up last block
                const f32x4 w = f32x4{o[d][4 * rq + 0], o[d][4 * rq + 1], o[d][4 * rq + 2], o[d][4 * rq + 3]} * inv;
                *(f32x4*)(orow + 32 * d + 8 * rq + 4 * g) = w;
            }
        if (g == 0) {
            const float lse = (l_run > 0.f) ? (m_run + __builtin_amdgcn_logf(l_run)) * kLn2 : 0.f;
            p.lse[((int64_t)b * p.Hq + h) * p.qL + qrow] = lse;
        }
    }
}

// How many work-groups a query tile's key range is split over (1: none): a
// grid that leaves more than half of the CUs idle while each work-group walks
// a long key range (at least 2 kMinSplitTiles tiles) splits that range, up to
// one full GPU of work-groups, at least kMinSplitTiles tiles each (a multiple
// of 2).  A tiny grid (at most 8 work-groups) splits down to one tile per
// work-group: its time is one CU's latency and matrix work, which the split
// spreads over CUs.  Measured on 1 head x 128 x 128 keys at D = 64: 15.2 ->
// 12.4 us (8.3 in the main kernel, 4.1 in the merge).  Each work-group
// starts its own ring at buffer 0, so any number of tiles per range works.
template <bool CAUSAL, int BN>
int split_plan_f32(const FwdParams& p, int64_t wgs, int* split_tiles, int wgs_per_cu = 1)
{
    constexpr int kCUs = 256;
    const int kMinSplitTiles = wgs <= 8 ? 1 : 8;
    const int kv_max = CAUSAL ? min(p.kL, p.qL) : p.kL;
    const int n_kt = (kv_max + BN - 1) / BN;
    *split_tiles = 0;
    if (p.window > 0 || wgs * 2 > kCUs || n_kt < 2 * kMinSplitTiles) return 1;
    const int64_t want = (int64_t)kCUs * wgs_per_cu / wgs;  // wgs_per_cu work-groups per CU
    const int by_len = n_kt / kMinSplitTiles;
    const int s0 = (int)(want < by_len ? want : (int64_t)by_len);
    if (s0 < 2) return 1;
    int st = (n_kt + s0 - 1) / s0;
    if (kMinSplitTiles > 1) st = (st + 1) / 2 * 2;
    *split_tiles = st;
    return (n_kt + st - 1) / st;
}

template <int D, int MASK, bool CAUSAL, int NW, int BN, bool DROP = false, bool PACK = false>
hipError_t launch_f32(const FwdParams& p, hipStream_t st, size_t* need = nullptr)
{
    // the kernel divides its grid index by n_split
    if (p.n_split < 1) return hipErrorInvalidValue;
    FwdParams q = p;
    // (packed: one work-group per 2 NW heads of a group, all query rows)
    const int64_t wgs = PACK ? (int64_t)p.B * p.Hkv * (p.group / (2 * NW)) : (int64_t)p.n_qtiles * p.Hq * p.B;
    int split_tiles = 0;
    // (the packed shape fits two work-groups per CU)
    const int n_split = split_plan_f32<CAUSAL, BN>(p, wgs, &split_tiles, PACK ? 2 : 1);
    const int64_t rows = (int64_t)p.B * p.Hq * p.qL;
    const size_t ws_bytes = n_split < 2 ? 0 : (size_t)n_split * rows * (D + 1) * sizeof(float);
    if (need) {
        *need = ws_bytes;
        return hipSuccess;
    }
    if (n_split < 2) {
        q.pair_tiles = CAUSAL && grid_fits_at_once(wgs, 1);
        hipLaunchKernelGGL((fwd_f32_kernel<D, MASK, CAUSAL, NW, BN, DROP, PACK>), dim3((unsigned)wgs), dim3(NW * 64), 0,
                           st, q);
        return hipGetLastError();
    }
    // partials in the caller's scratch or from the library's stream-ordered
    // pool (freed for reuse once the merge has read them); every partial the
    // merge reads is written by this launch first
    void* ws = p.ws;
    hipError_t err = hipSuccess;
    if (ws != nullptr) {
        if (p.ws_bytes < ws_bytes) return hipErrorInvalidValue;
    } else {
        hipMemPool_t pool;
        err = library_pool(&pool);
        if (err != hipSuccess) return err;
        err = hipMallocFromPoolAsync(&ws, ws_bytes, pool, st);
        if (err != hipSuccess) return err;
    }
    q.o_part = (float*)ws;
    q.l_part = q.o_part + (int64_t)n_split * rows * D;
    q.n_split = n_split;
    q.split_tiles = split_tiles;
    q.pair_tiles = CAUSAL && grid_fits_at_once(wgs * n_split, 1);
    hipLaunchKernelGGL((fwd_f32_kernel<D, MASK, CAUSAL, NW, BN, DROP, PACK>), dim3((unsigned)(wgs * n_split)),
                       dim3(NW * 64), 0, st, q);
    err = hipGetLastError();
    if (err == hipSuccess) {
        err = launch_merge<D, false>(q, rows, st);
    }
    if (p.ws != nullptr) return err;
    const hipError_t ferr = hipFreeAsync(ws, st);
    return err != hipSuccess ? err : ferr;
}

// Query ranges of at most 16 rows in GQA groups of a multiple of 4 heads (a
// decode step) take the packed shape: 2-wave work-groups of 4 heads x 16
// rows with 32-key tiles (two work-groups per CU).  Everything else takes the
// head dim's own shape.
template <int D, int MASK, bool CAUSAL, int NW, int BN, bool DROP = false>
hipError_t launch_f32_any(const FwdParams& p, hipStream_t st, size_t* need = nullptr)
{
    if (p.qL <= 16 && p.group % 4 == 0 && p.window == 0) {
        FwdParams q = p;
        q.n_qtiles = 1;
        return launch_f32<D, MASK, CAUSAL, 2, 32, DROP, true>(q, st, need);
    }
    return launch_f32<D, MASK, CAUSAL, NW, BN, DROP>(p, st, need);
}

}  // namespace

#define FA_F32_VARIANT(D, MASK, CAUSAL, NW, BN, NAME) \
    {NAME, 0, D, MASK, CAUSAL, NW * 32, &launch_f32_any<D, MASK, CAUSAL, NW, BN>}

#define FA_F32_FOR_D(D, NW, BN)                                                         \
    FA_F32_VARIANT(D, MASK_NONE, false, NW, BN, "fwd_f32_d" #D "_nomask"),              \
    FA_F32_VARIANT(D, MASK_NONE, true, NW, BN, "fwd_f32_d" #D "_nomask_causal"),        \
    FA_F32_VARIANT(D, MASK_ADD, false, NW, BN, "fwd_f32_d" #D "_additive"),             \
    FA_F32_VARIANT(D, MASK_ADD, true, NW, BN, "fwd_f32_d" #D "_additive_causal"),       \
    FA_F32_VARIANT(D, MASK_BOOL, false, NW, BN, "fwd_f32_d" #D "_bool"),                \
    FA_F32_VARIANT(D, MASK_BOOL, true, NW, BN, "fwd_f32_d" #D "_bool_causal")

// Launch shapes per head dimension (waves per work-group, keys per tile);
// overridable at build time for tuning sweeps.
#ifndef FA_F32_D16_CFG
#define FA_F32_D16_CFG 4, 32
#endif
#ifndef FA_F32_D48_CFG
#define FA_F32_D48_CFG 4, 32
#endif
#ifndef FA_F32_D80_CFG
#define FA_F32_D80_CFG 4, 64
#endif
#ifndef FA_F32_D32_CFG
#define FA_F32_D32_CFG 4, 32
#endif
#ifndef FA_F32_D64_CFG
#define FA_F32_D64_CFG 4, 32
#endif
#ifndef FA_F32_D128_CFG
#define FA_F32_D128_CFG 4, 64
#endif
#ifndef FA_F32_D96_CFG
#define FA_F32_D96_CFG 4, 64
#endif
#ifndef FA_F32_D256_CFG
#define FA_F32_D256_CFG 4, 32
#endif
// expands a CFG macro into separate arguments before FA_F32_FOR_D sees them
#define FA_F32_FOR_D_CFG(D, ...) FA_F32_FOR_D(D, __VA_ARGS__)

// Dropout variants: the same kernel at the same launch shapes, with the
// multipliers applied to the fp32 P before P V.
#define FA_F32_DROP_VARIANT(D, MASK, CAUSAL, NW, BN, NAME) \
    {NAME, 0, D, MASK, CAUSAL, NW * 32, &launch_f32_any<D, MASK, CAUSAL, NW, BN, true>}
#define FA_F32_DROP_FOR_D(D, NW, BN)                                                           \
    FA_F32_DROP_VARIANT(D, MASK_NONE, false, NW, BN, "fwd_f32_d" #D "_nomask_dropout"),        \
    FA_F32_DROP_VARIANT(D, MASK_NONE, true, NW, BN, "fwd_f32_d" #D "_nomask_causal_dropout"),  \
    FA_F32_DROP_VARIANT(D, MASK_ADD, false, NW, BN, "fwd_f32_d" #D "_additive_dropout"),       \
    FA_F32_DROP_VARIANT(D, MASK_ADD, true, NW, BN, "fwd_f32_d" #D "_additive_causal_dropout"), \
    FA_F32_DROP_VARIANT(D, MASK_BOOL, false, NW, BN, "fwd_f32_d" #D "_bool_dropout"),          \
    FA_F32_DROP_VARIANT(D, MASK_BOOL, true, NW, BN, "fwd_f32_d" #D "_bool_causal_dropout")
#define FA_F32_DROP_FOR_D_CFG(D, ...) FA_F32_DROP_FOR_D(D, __VA_ARGS__)

}  // namespace fa
