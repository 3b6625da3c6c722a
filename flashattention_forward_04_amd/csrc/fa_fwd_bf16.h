// fa_fwd_bf16.h - FlashAttention-2 forward, bf16 in/out, for gfx950: the
// kernel templates and their launchers.  Each fa_fwd_bf16_d<D>.hip
// instantiates the variants of one head dim (so the library compiles in
// parallel).
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
//     permutation of a 16-key chunk, and the V^T operand is read in that same
//     key order with two gfx950 transposing LDS reads (ds_read_b64_tr_b16),
//     so V is staged exactly like K: no VALU transposition.
//   * K and V are staged in LDS row-major with padded row pitches that
//     measure conflict-free on gfx950 for every access the kernel makes
//     (TileLayout).  Tiles go straight from global memory into LDS
//     (global_load_lds_dwordx4, no registers) round a ring of LDS buffers,
//     loaded one or more tiles ahead, with one barrier per tile.
//   * Two instruction schedules: plain (score products of tile t, then its
//     softmax with the P V products interleaved block by block) and
//     pipelined (the score products of tile t+1 are spread through the
//     softmax of tile t, so a wave always has matrix work beside its vector
//     work).  Which one each head dimension uses was chosen by timing.
//   * Causal work-groups are issued longest-first, and key tiles past the
//     last query row of a work-group are never loaded (forge
//     flash_attention_mma.metal, the causal j_end bound); a wave whose rows
//     all precede a key tile skips that tile's arithmetic.
//   * Ragged tails: query rows past qL load zeros and are not stored; key
//     rows past kL repeat row kL - 1 (finite values) and their scores are
//     masked to -inf.
#pragma once

#include "fa_common.h"
#include "fa_merge.h"

#include <math.h>

#include <cstring>
#include <mutex>
#include <type_traits>

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Round-to-nearest-even fp32 -> bf16 pair, packed low = a, high = b (one
// v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Cross-half reductions: lanes l and l^32 hold the two halves of one query
// row's keys.  v_permlane32_swap(x, x) returns x[l%32] and x[l%32 + 32] in
// every lane, so one VALU op replaces an LDS-routed shuffle.
__device__ __forceinline__ float row_max_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float row_sum_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The running max is only moved (and O, l rescaled) when a row's new max
// exceeds it by more than kRescaleSlack (base-2 units).  Until then P is
// computed against the stale max, so every P stays <= 2^kRescaleSlack: the
// result is the same softmax, and the rescale of the accumulator is skipped
// on almost every tile.
constexpr float kRescaleSlack = 8.f;

// Vector instructions placed after each matrix product in the softmax
// stages (chosen by timing on MI355X).
#ifndef FA_SCHED_PV
#define FA_SCHED_PV 4
#endif
// K operand reads kept in flight ahead of the score products of a whole
// tile (0 = leave it to the compiler).
#ifndef FA_SCHED_S
#define FA_SCHED_S 4
#endif

// Walk the key range of causal grids that fit at once in two halves per
// work-group (see launch_bf16_any).
#ifndef FA_KEY_HALVES
#define FA_KEY_HALVES 1
#endif

// Split long key ranges of small grids over work-groups (see launch_bf16).
#ifndef FA_SPLIT_KV
#define FA_SPLIT_KV 1
#endif

// K and V tiles live in LDS row-major ([BN][D], one key per row) with a
// padded row pitch: D + 8 elements for K; for V, D + 32, or 96 at D = 48
// and 80.  Measured on gfx950, the K pitch has no bank conflicts for the
// 16-byte staging writes and the 16-byte K operand reads, and the
// transposing V reads are conflict-free when the V pitch is 32 elements
// past a multiple of 64 (D + 32 is that at D = 64, 128 and 256).  At
// D = 16, 32 and 96 such a pitch removed the conflicts (up to 33 % of CU
// cycles at D = 96) without making the kernel faster, so those keep D + 32.
// The pitches keep every operand address a per-lane base plus a
// compile-time offset.
template <int D>
constexpr int k_pitch()
{
#ifdef FA_BF16_KPAD
    return D + FA_BF16_KPAD;
#else
    return D + 8;
#endif
}
template <int D>
constexpr int v_pitch()
{
#ifdef FA_BF16_VPAD
    return D + FA_BF16_VPAD;
#else
    return (D == 48 || D == 80) ? 96 : D + 32;
#endif
}
template <int P>
struct TileLayout {
    static constexpr int PITCH = P;
    __device__ static __forceinline__ int off(int row, int chunk) { return row * P + chunk * 8; }
};

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// ds_read_b64_tr_b16: within each 16-lane group, source lane 4e + a reads 4
// consecutive bf16 of row e (of four rows) at column 4a; destination lane t
// receives column t of all four rows.  Two of these give a lane the 8 keys
// of one V^T operand row (head-dim index) without any VALU transposition.
__device__ __forceinline__ i16x4 lds_read_tr(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
}

// One work-group: NW waves of 32 query rows each, BN keys per tile, WPE
// waves per SIMD the register allocation must leave room for.
//
// PIPE (software pipelining across key tiles): the score products of tile
// t+1 are issued in between the softmax instructions of tile t.  A wave's
// vector instructions run while its own matrix products execute, but hardly
// while another wave's do, so a wave that interleaves both kinds of work
// keeps the matrix cores busy through the softmax.  K is then staged one
// tile ahead of V.
//
// K/V tiles are loaded straight from global memory into LDS (no registers),
// round a ring of NB buffers, with one barrier per tile.
//
// KSPLIT (key halves): the NW waves form two halves of NW / 2 waves on the
// same NW / 2 row blocks.  Half 0 walks the first half of the work-group's
// key tiles and half 1 the second, each round its own ring of LDS buffers,
// so a long causal row block takes half as many steps.  At the end the two
// softmax states (m, l, O) of each row are merged through LDS -- the same
// combination the online softmax applies between key blocks.
//
// RPACK (query ranges of at most 16 rows, GQA groups of a multiple of 2 NW
// heads): a wave's 32 rows are 16 rows each of two query heads of one group
// (lanes with row bit 4 clear the first, set the second), and the work-group
// takes 2 NW heads of the group; every matrix row is then a real row.
template <int D, int MASK, bool CAUSAL, int NW, int BN, int WPE, int SCHED, int NB, bool DROP = false,
          bool KSPLIT = false, bool RPACK = false>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
fwd_bf16_kernel(const FwdParams p)
{
    static_assert(SCHED == 0 || SCHED == 1, "schedule: 0 plain, 1 pipelined");
    constexpr bool PIPE = SCHED != 0;  // next tile's scores formed during this tile's softmax
    constexpr int NH = KSPLIT ? 2 : 1;  // key halves
    constexpr int WH = NW / NH;         // waves per half; the halves share the query rows
    constexpr int BM = WH * 32;         // query rows per work-group
    using KL = TileLayout<k_pitch<D>()>;  // K tile layout in LDS
    using VL = TileLayout<v_pitch<D>()>;  // V tile layout in LDS
    // tiles are padded to whole 1 KiB blocks: one direct load of a wave
    // fills exactly one block
    constexpr int KSPR = KL::PITCH / 8;          // 16-byte slots per K row
    constexpr int VSPR = VL::PITCH / 8;          // 16-byte slots per V row
    constexpr int KINS = (BN * KSPR + 63) / 64;  // 1 KiB blocks per K tile
    constexpr int VINS = (BN * VSPR + 63) / 64;  // 1 KiB blocks per V tile
    constexpr int KTILE = KINS * 512;            // elements per K buffer
    constexpr int VTILE = VINS * 512;            // elements per V buffer
    constexpr int DK = D / 16;                   // k-steps of S^T over the head dimension
    constexpr int NC = BN / 32;                  // 32-key blocks per key tile
    // 32-wide blocks of O^T along the head dimension, rounded up: the rows
    // past D of the last block read V^T columns past D (inside the padded
    // LDS rows, never written) and are never stored
    constexpr int ND = (D + 31) / 32;
    constexpr int NP = DK * NC;                  // score products per tile
    static_assert(BN % 32 == 0 && D % 16 == 0, "tile shape");
    static_assert(32 * ND <= v_pitch<D>(), "the V^T reads of the last block stay inside a padded V row");
    static_assert(k_pitch<D>() % 8 == 0 && v_pitch<D>() % 8 == 0, "16-byte rows");

    // NB buffers each for K and V, as separate arrays so that the compiler
    // can tell the buffer being loaded from the ones being read
    static_assert(NB == 2 || NB == 4, "ring depth");
    // key halves: buffers 0-1 are half 0's ring, 2-3 half 1's; the merge
    // passes each row block's state through one V buffer
    static_assert(!KSPLIT || (NB == 2 && !DROP && NW % 2 == 0 && WH <= 4 &&
                              (1024 * ((D + 31) / 32) + 128) * 4 <= VTILE * 2), "key halves");
    constexpr int KT2 = (NB > 2 || KSPLIT) ? KTILE : 1, VT2 = (NB > 2 || KSPLIT) ? VTILE : 1;
    __shared__ __attribute__((aligned(1024))) uint16_t Ks0[KTILE];
    __shared__ __attribute__((aligned(1024))) uint16_t Ks1[KTILE];
    __shared__ __attribute__((aligned(1024))) uint16_t Ks2[KT2];
    __shared__ __attribute__((aligned(1024))) uint16_t Ks3[KT2];
    __shared__ __attribute__((aligned(1024))) uint16_t Vs0[VTILE];
    __shared__ __attribute__((aligned(1024))) uint16_t Vs1[VTILE];
    __shared__ __attribute__((aligned(1024))) uint16_t Vs2[VT2];
    __shared__ __attribute__((aligned(1024))) uint16_t Vs3[VT2];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // the wave index is uniform across the wave; saying so keeps the per-wave
    // branches below (causal skip, masked tiles) scalar
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r32 = lane & 31;
    const int g = lane >> 5;
    const int half = KSPLIT ? wave / WH : 0;  // key half of this wave (0 without KSPLIT)
    const int wrow = KSPLIT ? wave % WH : wave;  // row block of this wave

    // buffer i of this wave's ring
    auto kbuf = [&](auto i_c) __attribute__((always_inline)) -> uint16_t* {
        constexpr int I = decltype(i_c)::value;
        if constexpr (KSPLIT) return half ? (I == 0 ? Ks2 : Ks3) : (I == 0 ? Ks0 : Ks1);
        return I == 0 ? Ks0 : I == 1 ? Ks1 : I == 2 ? Ks2 : Ks3;
    };
    auto vbuf = [&](auto i_c) __attribute__((always_inline)) -> uint16_t* {
        constexpr int I = decltype(i_c)::value;
        if constexpr (KSPLIT) return half ? (I == 0 ? Vs2 : Vs3) : (I == 0 ? Vs0 : Vs1);
        return I == 0 ? Vs0 : I == 1 ? Vs1 : I == 2 ? Vs2 : Vs3;
    };
    // the same by a (fully unrolled, hence constant) index
    auto kbuf_dyn = [&](int i) __attribute__((always_inline)) -> uint16_t* {
        if (KSPLIT) i += 2 * half;
        return i == 0 ? Ks0 : i == 1 ? Ks1 : i == 2 ? Ks2 : Ks3;
    };
    auto vbuf_dyn = [&](int i) __attribute__((always_inline)) -> uint16_t* {
        if (KSPLIT) i += 2 * half;
        return i == 0 ? Vs0 : i == 1 ? Vs1 : i == 2 ? Vs2 : Vs3;
    };

    // ---- which (query tile, head, batch) this work-group owns ----
    // Normally one query head and NW * 32 consecutive rows.  With head_pack
    // (a query range of at most 32 rows in a GQA group) rows [q0, q0 + 32) of
    // NW query heads of one kv head's group: wave w takes the w-th of them,
    // so the heads share every K/V tile the work-group stages.
    int id = blockIdx.x;
    int h, hk, split, b, q0, wq0;
    bool head_ok = true;  // false: a packed wave past the end of its group
    if constexpr (RPACK) {
        // kv head innermost, then the group's chunk of 2 NW heads, then the split
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
    } else if (p.head_pack) {
        // kv head innermost: the work-groups of one kv head's group sit H_kv
        // ids apart, on one XCD (one L2) when H_kv is a multiple of 8
        const int nch = (p.group + NW - 1) / NW;
        hk = id % p.Hkv;
        id /= p.Hkv;
        const int c = id % nch;
        id /= nch;
        split = id % p.n_split;
        id /= p.n_split;
        b = id % p.B;
        id /= p.B;
        q0 = id * 32;
        const int hg = c * NW + wave;
        head_ok = hg < p.group;
        h = hk * p.group + min(hg, p.group - 1);
        wq0 = q0;
    } else {
        h = head_of(id % p.Hq, p.Hq);
        id /= p.Hq;
        split = id % p.n_split;
        id /= p.n_split;
        b = id % p.B;
        id /= p.B;
        const int qt = CAUSAL ? causal_tile(id, p.n_qtiles, p.pair_tiles) : id;
        q0 = qt * BM;
        hk = h / p.group;
        wq0 = q0 + wrow * 32;  // first query row of this wave
    }
    const int qrow = RPACK ? (r32 & 15) : wq0 + r32;  // this lane's query row
    const int wq_last = RPACK ? 15 : wq0 + 31;         // the last row any lane of this wave holds

    const uint16_t* Qb = (const uint16_t*)p.q + b * p.q_s[0] + h * p.q_s[1];
    const uint16_t* Kb = (const uint16_t*)p.k + b * p.k_s[0] + hk * p.k_s[1];
    const uint16_t* Vb = (const uint16_t*)p.v + b * p.v_s[0] + hk * p.v_s[1];

    // ---- Q fragments: row qrow, elements 16ks + 8g .. +7 (zeros past qL) ----
    bf16x8 qf[DK];
    {
        const bool in = head_ok && qrow < p.qL;
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
    const int kv_end = CAUSAL ? min(p.kL, min(p.qL, q0 + (RPACK ? 16 : p.head_pack ? 32 : BM))) : p.kL;
    // key tiles of this query tile; a split work-group takes tiles
    // [tb, tb + split_tiles) of them, numbered from 0 below.  A sliding
    // window starts the range at the tile of the first row's first key.
    const bool win = CAUSAL && p.window > 0;
    const int n_all = (kv_end + BN - 1) / BN;
    const int tb_wg = (win ? max(0, q0 - p.window + 1) / BN : 0) + split * p.split_tiles;
    const int n_wg = max(0, (p.n_split > 1 ? min(n_all, tb_wg + p.split_tiles) : n_all) - tb_wg);
    // key halves: half 0 takes tiles [0, nh) of the range, half 1 the rest;
    // both run nh steps (the barriers are shared)
    const int nh = KSPLIT ? (n_wg + 1) / 2 : n_wg;
    const int tb = tb_wg + (half ? nh : 0);                            // this wave's first tile
    const int n_tiles = KSPLIT ? (half ? n_wg - nh : nh) : n_wg;      // and how many it takes
    const int n_steps = nh;                                            // loop steps of the work-group
    // this wave needs tiles 0..t_last (a prefix: causal rows never see later keys)
    int t_last = n_tiles - 1;
    if (CAUSAL) t_last = min(t_last, wq_last / BN - tb);
    if (wq0 >= p.qL || !head_ok) t_last = -1;

    // dropout: the score position of this lane's row at key 0, and the
    // dropout multipliers of the 4 consecutive keys from position n0
    const int64_t drow = DROP ? (((int64_t)b * p.Hq + h) * p.qL + qrow) * p.kL : 0;
    auto drop_quad = [&](int64_t n0, float* mult) __attribute__((always_inline)) { dropout_quad(p, n0, mult); };

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
    float m_run = -INFINITY;  // running max (base 2) that P is taken against
    float l_run = 0.f;        // running sum of P

    // Direct global -> LDS staging: 1 KiB block i of a tile is filled by one
    // global_load_lds_dwordx4 of wave i % NW, whose lane l writes slot 64i + l
    // (the hardware places lane l's 16 bytes at the block base + 16 l).  A
    // slot in a row's pad is skipped; rows past kL load row kL - 1 (finite
    // values; their scores are masked, so they only meet P = 0).
    // A lane's slots are the same in every tile: their element offsets
    // within a tile (row * stride + chunk * 8) are computed once, so a full
    // tile's load address is one add; only the tail tile (rows past kL,
    // clamped) recomputes them.
    constexpr int KIT = (KINS + WH - 1) / WH;  // direct loads per wave per K tile (at most)
    constexpr int VIT = (VINS + WH - 1) / WH;
    // (32-bit byte offsets within a tile: a full tile takes them when BN rows
    // of the larger stride fit in 31 bits, else the per-slot path)
    const bool off32 = (int64_t)BN * max(p.k_s[2], p.v_s[2]) * 2 < ((int64_t)1 << 31);
    uint32_t koff[KIT], voff[VIT];
    auto slot_offsets = [&](uint32_t* off, int64_t stride, auto spr_c, auto nins_c) __attribute__((always_inline)) {
        constexpr int SPR = decltype(spr_c)::value;
        constexpr int NINS = decltype(nins_c)::value;
#pragma unroll
        for (int k = 0; k < (NINS + WH - 1) / WH; ++k) {
            const int slot = 64 * (wrow + k * WH) + lane;
            off[k] = (uint32_t)(((int64_t)(slot / SPR) * stride + (slot % SPR) * 8) * 2);
        }
    };
    slot_offsets(koff, p.k_s[2], std::integral_constant<int, KSPR>{}, std::integral_constant<int, KINS>{});
    slot_offsets(voff, p.v_s[2], std::integral_constant<int, VSPR>{}, std::integral_constant<int, VINS>{});
    auto issue_tile = [&](const uint16_t* gbase, int64_t stride, int j0, uint16_t* lds, const uint32_t* off,
                          auto spr_c, auto nins_c) __attribute__((always_inline)) {
        constexpr int SPR = decltype(spr_c)::value;
        constexpr int NINS = decltype(nins_c)::value;
        auto all_slots = [&](auto full_c) __attribute__((always_inline)) {
            constexpr bool FULL = decltype(full_c)::value;
            // the tile's base is the same for every lane: keep it in SGPRs
            const uint64_t tb64 = (uint64_t)(size_t)(gbase + (int64_t)j0 * stride);
            // (readfirstlane returns int: each half goes through uint32_t so
            // that the low half is zero-extended, not sign-extended)
            const uint32_t tb_hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(tb64 >> 32));
            const uint32_t tb_lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)tb64);
            const uint16_t* tbase = (const uint16_t*)(size_t)(((uint64_t)tb_hi << 32) | (uint64_t)tb_lo);
#pragma unroll
            for (int k = 0; k < (NINS + WH - 1) / WH; ++k) {
                const int i = wrow + k * WH;
                if (NINS % WH != 0 && i >= NINS) break;
                const int slot = 64 * i + lane;
                const int row = slot / SPR;
                const int ch = slot % SPR;
                if (ch < D / 8 && row < BN) {
                    const uint16_t* src =
                        FULL ? (const uint16_t*)((const char*)tbase + off[k])
                             : gbase + (int64_t)min(j0 + row, p.kL - 1) * stride + ch * 8;
                    // (the compiler does not count these loads: a wait it
                    // places for a later ordinary load, e.g. of mask words,
                    // counts fewer loads in flight than there are, so it
                    // waits longer, never shorter; the tiles themselves are
                    // waited for explicitly at the end of each step)
                    if (FULL)
                        lds_dma16_so(tbase, off[k], (uint32_t)(size_t)(__attribute__((address_space(3))) void*)(lds + 512 * i));
                    else
                        lds_dma16(src, (uint32_t)(size_t)(__attribute__((address_space(3))) void*)(lds + 512 * i));
                }
            }
        };
        if (j0 + BN <= p.kL && off32)
            all_slots(std::true_type{});
        else
            all_slots(std::false_type{});
    };
    auto issue_k = [&](int t, uint16_t* kt) __attribute__((always_inline)) {
        issue_tile(Kb, p.k_s[2], (tb + t) * BN, kt, koff, std::integral_constant<int, KSPR>{},
                   std::integral_constant<int, KINS>{});
    };
    auto issue_v = [&](int t, uint16_t* vt) __attribute__((always_inline)) {
        issue_tile(Vb, p.v_s[2], (tb + t) * BN, vt, voff, std::integral_constant<int, VSPR>{},
                   std::integral_constant<int, VINS>{});
    };
    // all of this wave's direct loads have landed in LDS
    auto wait_loads = []() __attribute__((always_inline)) { __builtin_amdgcn_s_waitcnt(0x0F70); };

    // ---- S^T = K Q^T for the key tile staged at kt: products [i0, i1) of
    // the NP, in k-step-major order (consecutive products feed different
    // accumulators) ----
    auto score_products = [&](f32x16 (&s)[NC], const uint16_t* kt, int i0, int i1) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            if (i < i0 || i >= i1) continue;
            const int ks = i / NC, c = i % NC;
            const bf16x8 kop = *(const bf16x8*)(kt + KL::off(32 * c + r32, 2 * ks + g));
            s[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qf[ks], ks == 0 ? f32x16{} : s[c], 0, 0, 0);
        }
#if FA_SCHED_S
        // keep FA_SCHED_S operand reads in flight ahead of the products
        if (i0 == 0 && i1 == NP) {
            __builtin_amdgcn_sched_group_barrier(0x100, FA_SCHED_S, 3);
#pragma unroll
            for (int i = 0; i < NP - FA_SCHED_S; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 3);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 3);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, FA_SCHED_S, 3);
        }
#endif
    };

    // ---- scores of key tile j0 -> base 2, excluded keys at -inf: keys past
    // kL, keys after the row (causal), and the user mask ----
    // Raw mask words of one key tile for this lane: for 32-key block c and
    // quad rq, the 4 keys j0 + 32c + 8rq + 4g + {0..3} (bf16 bit pairs in x
    // and y for an additive mask; one byte each in x for a bool mask, nonzero
    // = attend).  Loaded one tile ahead so the global load latency is
    // covered by a tile of work.
    typedef u32x2 MaskWords[NC][4];
    auto load_mask = [&](int j0, MaskWords& mw) __attribute__((always_inline)) {
        // one decision per tile (a per-quad one would split the loads into
        // branches the compiler's wait counting merges pessimistically)
        const bool vec = p.mask_vec && j0 + BN <= p.kL;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int jb = j0 + 32 * c + 8 * rq + 4 * g;  // first of 4 consecutive keys
                u32x2 w = {0u, 0u};
                if (vec) {
                    // whole tile inside the row, rows aligned: one load per quad
                    if (MASK == MASK_ADD) w = *(const u32x2*)(mrow + 2 * (int64_t)jb);
                    if (MASK == MASK_BOOL) w[0] = *(const uint32_t*)(mrow + jb);
                } else if (MASK == MASK_ADD) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (jb + e < p.kL) w[e >> 1] |= (uint32_t)((const uint16_t*)mrow)[jb + e] << (16 * (e & 1));
                } else if (MASK == MASK_BOOL) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (jb + e < p.kL && mrow[jb + e] != 0) w[0] |= 1u << (8 * e);
                }
                mw[c][rq] = w;
            }
        }
    };

    // ---- scores of key tile j0 -> base 2, excluded keys at -inf: keys past
    // kL, keys after the row (causal), and the user mask (its words in mw) ----
    auto apply_mask = [&](f32x16 (&s)[NC], int j0, const MaskWords& mw) __attribute__((always_inline)) {
        // the tile reaches below the window of the wave's last row
        const bool w_edge = win && j0 < wq0 + 32 - p.window;
        if (MASK == MASK_NONE) {
            // key j0 + 32c + 8rq + 4g + e is allowed iff 32c + 8rq + e <= lim
            // (and, on a window's edge, >= lo)
            int lim = p.kL - 1;
            if (CAUSAL) lim = min(lim, qrow);
            lim -= j0 + 4 * g;
            if (w_edge) {
                const int lo = qrow - p.window + 1 - (j0 + 4 * g);
#pragma unroll
                for (int c = 0; c < NC; ++c)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int x = 32 * c + 8 * (r >> 2) + (r & 3);
                        s[c][r] = (x <= lim && x >= lo) ? s[c][r] * c2 : -INFINITY;
                    }
                return;
            }
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    s[c][r] = (32 * c + 8 * (r >> 2) + (r & 3) <= lim) ? s[c][r] * c2 : -INFINITY;
            return;
        }
        // the bias of element e of a quad: bf16 bits in the low or high half
        // (a bias of -inf excludes the key by itself)
        auto bias = [&](const u32x2& w, int e) __attribute__((always_inline)) {
            return __uint_as_float((e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16));
        };
        // Tiles inside the key range, below the causal diagonal and the
        // window's edge: only the user mask decides (wave-uniform branch)
        if (j0 + BN <= p.kL && !(CAUSAL && j0 + BN - 1 > wq0) && !w_edge) {
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    const u32x2 w = mw[c][rq];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float x = s[c][4 * rq + e];
                        if (MASK == MASK_ADD) s[c][4 * rq + e] = __builtin_fmaf(bias(w, e), kLog2e, x * c2);
                        if (MASK == MASK_BOOL) s[c][4 * rq + e] = ((w[0] >> (8 * e)) & 0xffu) != 0 ? x * c2 : -INFINITY;
                    }
                }
            return;
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) {
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int jb = j0 + 32 * c + 8 * rq + 4 * g;
                const u32x2 w = mw[c][rq];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = jb + e;
                    bool ok = j < p.kL;
                    if (MASK == MASK_BOOL) ok = ok && ((w[0] >> (8 * e)) & 0xffu) != 0;
                    if (CAUSAL) ok = ok && (j <= qrow);
                    if (CAUSAL) ok = ok && (!w_edge || j > qrow - p.window);
                    float x = s[c][4 * rq + e] * c2;
                    if (MASK == MASK_ADD) x = __builtin_fmaf(bias(w, e), kLog2e, x);
                    s[c][4 * rq + e] = ok ? x : -INFINITY;
                }
            }
        }
    };

    // ---- online softmax of s (raw when cs == c2, base 2 when cs == 1), then
    // O^T += V^T P^T from the value tile staged at vt; in pipelined mode the
    // next tile's score products (into sn, from the K tile staged at kn) are
    // interleaved.
    //
    // The work is laid out as a static software pipeline so that every
    // matrix product has vector work beside it and every LDS operand is read
    // one stage before it is used:
    //   stage -1: row max and rescale decision; score products of group 0
    //   stage r (0 .. NCH): P V of 16-key block r-1, score products of
    //             group r+1, P of block r; reads V^T operands of block r and
    //             K operands of group r+2.
    // Stages are fenced (sched_barrier), and inside a stage the products and
    // vector instructions are issued alternately (sched_group_barrier).
    auto softmax_pv = [&](f32x16 (&s)[NC], float cs, const uint16_t* vt, f32x16 (&sn)[NC], const uint16_t* kn,
                          int j0) __attribute__((always_inline)) {
        constexpr int NCH = 2 * NC;                            // 16-key blocks per tile
        constexpr int NS = PIPE ? NP : 0;                      // next-tile score products
        constexpr int SS = PIPE ? (NP + NCH) / (NCH + 1) : 0;  // products per group
        constexpr int SSB = SS > 0 ? SS : 1;
        bf16x8 kb[2][SSB];  // K operands, by group parity
        bf16x8 vb[2][ND];   // V^T operands, by block parity
        bf16x8 pf[2];       // P operands, by block parity
        const int lt = lane & 15;

        auto k_read = [&](int grp) __attribute__((always_inline)) {
#pragma unroll
            for (int jj = 0; jj < SS; ++jj) {
                const int i = grp * SS + jj;
                if (i < NS) kb[grp & 1][jj] = *(const bf16x8*)(kn + KL::off(32 * (i % NC) + r32, 2 * (i / NC) + g));
            }
        };
        auto s_mma = [&](int grp) __attribute__((always_inline)) {
#pragma unroll
            for (int jj = 0; jj < SS; ++jj) {
                const int i = grp * SS + jj;
                if (i < NS) {
                    const int ks = i / NC, c = i % NC;
                    sn[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[grp & 1][jj], qf[ks], ks == 0 ? f32x16{} : sn[c],
                                                                     0, 0, 0);
                }
            }
        };
        auto v_read = [&](int kidx) __attribute__((always_inline)) {
#pragma unroll
            for (int d = 0; d < ND; ++d) {
                // lane l: head-dim column 32d + l%32, keys 16kidx + 4g + {0..3}
                // and 16kidx + 8 + 4g + {0..3}, the order P is packed in
                const int col = 32 * d + 16 * ((lane >> 4) & 1) + 4 * (lt & 3);
                const int row0 = 16 * kidx + 4 * g + (lt >> 2);
                const i16x4 v0 = lds_read_tr(vt + VL::off(row0, 0) + col);
                const i16x4 v1 = lds_read_tr(vt + VL::off(row0 + 8, 0) + col);
                vb[kidx & 1][d] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
            }
        };
        auto pv_mma = [&](int kidx) __attribute__((always_inline)) {
#pragma unroll
            for (int d = 0; d < ND; ++d)
                o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb[kidx & 1][d], pf[kidx & 1], o[d], 0, 0, 0);
        };

        // stage -1: group 0's operands are needed at once (their latency is
        // covered by the row max); group 1's are read behind the first product
        k_read(0);
        float mx = s[0][0];
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[c][r]);
        const float m_tile = row_max_halves(mx) * cs;
        s_mma(0);
        k_read(1);
        if (PIPE) {
            __builtin_amdgcn_sched_group_barrier(0x100, SS, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, SS, 0);
#pragma unroll
            for (int i = 1; i < SS; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (__builtin_amdgcn_ballot_w64(m_tile > m_run + kRescaleSlack) != 0) {
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
        // the row sum is taken in fp32 before P is rounded to bf16: L must
        // stay within 1e-3 even for rows that see only a few keys
        float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
        for (int r = 0; r <= NCH; ++r) {
            if (r < NCH) v_read(r);
            if (r + 2 <= NCH) k_read(r + 2);
            if (r >= 1) pv_mma(r - 1);
            if (r + 1 <= NCH) s_mma(r + 1);
            if (r < NCH) {
                const int c = r >> 1, hh = r & 1;
                // dropout multipliers of this 16-key chunk: keys
                // j0 + 32c + 8(2hh + qq) + 4g + {0..3}, qq = 0, 1
                float mlt[8];
                if constexpr (DROP) {
                    drop_quad(drow + j0 + 32 * c + 16 * hh + 4 * g, mlt);
                    drop_quad(drow + j0 + 32 * c + 16 * hh + 8 + 4 * g, mlt + 4);
                }
                u32x4 pw;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float a = __builtin_amdgcn_exp2f(__builtin_fmaf(s[c][8 * hh + 2 * e], cs, -m_use));
                    const float z = __builtin_amdgcn_exp2f(__builtin_fmaf(s[c][8 * hh + 2 * e + 1], cs, -m_use));
                    // the row sum takes P before dropout (l and L are those
                    // without it); only the P V product sees the multipliers
                    if constexpr (DROP)
                        pw[e] = pack_bf16x2(a * mlt[4 * (e >> 1) + 2 * (e & 1)], z * mlt[4 * (e >> 1) + 2 * (e & 1) + 1]);
                    else
                        pw[e] = pack_bf16x2(a, z);
                    rs0 += a;
                    rs1 += z;
                }
                pf[r & 1] = __builtin_bit_cast(bf16x8, pw);
            }
            // one product first (its wait retires the previous stage's
            // reads, so no more than one stage of reads is ever in flight),
            // then this stage's reads, then products and vector work
            // alternately
            constexpr int kMfma = ND + SS;
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * ND + SS, 1);
#pragma unroll
            for (int i = 1; i < kMfma; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x002, FA_SCHED_PV, 1);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        l_run += row_sum_halves(rs0 + rs1);
    };

    // softmax and P V of tile t with its scores in s
    auto finish_tile = [&](int t, f32x16 (&s)[NC], const uint16_t* vt, f32x16 (&sn)[NC], const uint16_t* kn,
                           const MaskWords& mw) __attribute__((always_inline)) {
        const int j0 = (tb + t) * BN;
        // (a window's left edge: the wave's last row starts at key wq0 + 32 - window)
        const bool masked = (MASK != MASK_NONE) || (j0 + BN > p.kL) || (CAUSAL && j0 + BN - 1 > wq0) ||
                            (win && j0 < wq0 + 32 - p.window);
        // one softmax for both kinds of tile, so that the accumulators and
        // the next tile's scores are written in one place (two copies of the
        // softmax would make the register allocator move them at the join)
        if (masked) apply_mask(s, j0, mw);
        const float cs = masked ? 1.f : c2;
        softmax_pv(s, cs, vt, sn, kn, j0);
    };

    f32x16 sa[NC], sb[NC];  // score tiles (two, for the pipelined schedule)

    // ---- the key loop.  K and V tiles go round rings of NB LDS buffers
    // (tile t in buffer t % NB); step t loads K of tile t + PK and V of tile
    // t + PV, each into the buffer that was last read in step t - 1, so one
    // barrier per step covers every reuse.  The loop is unrolled by NB so
    // every buffer choice is static.
    constexpr int PK = PIPE ? NB : NB - 1;  // load-ahead distance of K
    constexpr int PV = NB - 1;              // load-ahead distance of V
    // loads this wave issues per tile (the fewest any wave issues)
    constexpr int kLoadsPerStep = KINS / WH + VINS / WH;
    // At the end of step t, what step t+1 reads was issued at step t+2-NB or
    // earlier, so the loads of the last NB-2 steps may stay in flight (when
    // all of them were issued; near the end everything is waited for).
    constexpr int kPending = (NB - 2) * kLoadsPerStep;
    static_assert(kPending < 64, "vmcnt range");
    auto end_step = [&](int t) __attribute__((always_inline)) {
        if (kPending > 0 && t + PK < n_tiles)
            __builtin_amdgcn_s_waitcnt(0x0F70 | (kPending & 15) | ((kPending >> 4) << 14));
        else
            wait_loads();
        __syncthreads();
    };
    MaskWords ma, mb;  // mask words of the current and the next tile
    auto step = [&](int t, auto u_c) __attribute__((always_inline)) {
        constexpr int U = decltype(u_c)::value;  // t % NB
        f32x16(&sc)[NC] = (U & 1) ? sb : sa;
        f32x16(&sn)[NC] = (U & 1) ? sa : sb;
        MaskWords& mc = (U & 1) ? mb : ma;
        MaskWords& mn = (U & 1) ? ma : mb;
        if (t + PK < n_tiles) issue_k(t + PK, kbuf(std::integral_constant<int, (U + PK) % NB>{}));
        if (t + PV < n_tiles) issue_v(t + PV, vbuf(std::integral_constant<int, (U + PV) % NB>{}));
        if (MASK != MASK_NONE && t + 1 <= t_last) load_mask((tb + t + 1) * BN, mn);
        if (t <= t_last) {
            const uint16_t* vr = vbuf(std::integral_constant<int, U>{});
            if (PIPE) {
                // the next tile's scores are formed even past t_last (from
                // whatever its K buffer holds): keeping them unconditional
                // keeps them in the same instruction stream as this softmax,
                // and a result that is not needed is never read
                finish_tile(t, sc, vr, sn, kbuf(std::integral_constant<int, (U + 1) % NB>{}), mc);
            } else {
                const uint16_t* kr = kbuf(std::integral_constant<int, U>{});
                score_products(sa, kr, 0, NP);
                finish_tile(t, sa, vr, sb, kr, mc);
            }
        }
        end_step(t);
    };

    // prologue: the first PK K tiles and PV V tiles
#pragma unroll
    for (int u = 0; u < NB; ++u) {
        if (u < PK && u < n_tiles) issue_k(u, kbuf_dyn(u));
        if (u < PV && u < n_tiles) issue_v(u, vbuf_dyn(u));
    }
    if (MASK != MASK_NONE && t_last >= 0) load_mask(tb * BN, ma);
    wait_loads();
    __syncthreads();
    if (PIPE) {
        if (t_last >= 0) score_products(sa, kbuf_dyn(0), 0, NP);
        __syncthreads();  // K of tile 0 is read before tile NB replaces it
    }
    for (int t0 = 0; t0 < n_steps; t0 += NB) {
        step(t0, std::integral_constant<int, 0>{});
        if (t0 + 1 < n_steps) step(t0 + 1, std::integral_constant<int, 1>{});
        if (NB > 2) {
            if (t0 + 2 < n_steps) step(t0 + 2, std::integral_constant<int, 2 % NB>{});
            if (t0 + 3 < n_steps) step(t0 + 3, std::integral_constant<int, 3 % NB>{});
        }
    }

    if constexpr (KSPLIT) {
        // The halves' softmax states meet in LDS: wave wrow of half 1 leaves
        // its (O^T, m, l) in V buffer wrow (lane-major, so each lane reads
        // back its own values), and wave wrow of half 0 -- the same rows and
        // the same accumulator layout -- folds it in: m = max(m0, m1),
        // l = l0 2^(m0 - m) + l1 2^(m1 - m), O likewise (a half with no
        // allowed key, m = -inf, weighs 0).
        __syncthreads();  // every wave is past its last read of the K/V buffers; no load is in flight
        float* xb = (float*)(wrow == 0 ? Vs0 : wrow == 1 ? Vs1 : wrow == 2 ? Vs2 : Vs3);
        if (half == 1) {
#pragma unroll
            for (int d = 0; d < ND; ++d)
#pragma unroll
                for (int r = 0; r < 16; ++r) xb[(d * 16 + r) * 64 + lane] = o[d][r];
            xb[ND * 1024 + lane] = m_run;
            xb[ND * 1024 + 64 + lane] = l_run;
        }
        __syncthreads();
        if (half == 0) {
            const float m1 = xb[ND * 1024 + lane], l1 = xb[ND * 1024 + 64 + lane];
            const float m = fmaxf(m_run, m1);
            const float c0 = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m);
            const float c1 = (m1 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m1 - m);
#pragma unroll
            for (int d = 0; d < ND; ++d)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[d][r] = __builtin_fmaf(o[d][r], c0, xb[(d * 16 + r) * 64 + lane] * c1);
            l_run = __builtin_fmaf(l_run, c0, l1 * c1);
            m_run = m;
        }
    }

    // ---- epilogue: O = O / l, L = (m + log2 l) ln2 (O = 0, L = 0 if no key) ----
    // Per-wave regions of the (by now idle) K/V buffers for whole-line
    // stores: 32 rows of XP floats, or of 2 XP bf16 elements.
    constexpr int XP = 36;                        // region row pitch, floats
    constexpr int XE = 32 * XP * 2;               // region size in 16-bit elements
    constexpr int RK = KTILE / XE, RV = VTILE / XE;
    constexpr bool XPOSE = 2 * RK + 2 * RV >= NW;  // (every wave gets a region)
    auto region = [&](int w) __attribute__((always_inline)) -> uint16_t* {
        return w < RK ? Ks0 + w * XE : w < 2 * RK ? Ks1 + (w - RK) * XE
                    : w < 2 * RK + RV ? Vs0 + (w - 2 * RK) * XE : Vs1 + (w - 2 * RK - RV) * XE;
    };
    if constexpr (XPOSE && D % 64 == 0 && !RPACK) {
        if (p.n_split == 1 && p.head_pack == 0) {
            // O of an unsplit launch: stored straight from the accumulators,
            // an instruction writes 16 bytes of each of 32 rows; instead each
            // wave passes 64 columns at a time through its region and stores
            // whole 128-byte lines of 8 rows, nontemporally (O is not read
            // again here)
            __syncthreads();  // every wave (both key halves) is past its last read of the K/V buffers
            if (KSPLIT && half != 0) return;  // half 0 writes the merged rows
            const float inv = (l_run > 0.f) ? (DROP ? p.drop_scale : 1.f) / l_run : 0.f;
            constexpr int OP = 2 * XP;  // region row pitch, bf16 elements
            uint16_t* xs = region(wave);
            uint16_t* obase = (uint16_t*)p.o + b * p.o_s[0] + h * p.o_s[1];
#pragma unroll
            for (int hc = 0; hc < D / 64; ++hc) {
#pragma unroll
                for (int dd = 0; dd < 2; ++dd)
#pragma unroll
                    for (int rq = 0; rq < 4; ++rq) {
                        const int d = 2 * hc + dd;
                        u32x2 w;
                        w[0] = pack_bf16x2(o[d][4 * rq + 0] * inv, o[d][4 * rq + 1] * inv);
                        w[1] = pack_bf16x2(o[d][4 * rq + 2] * inv, o[d][4 * rq + 3] * inv);
                        *(u32x2*)(xs + r32 * OP + 32 * dd + 8 * rq + 4 * g) = w;
                    }
                // (the region is this wave's own, and a wave's LDS accesses
                // take effect in order)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rr = 8 * i + (lane >> 3), c8 = 8 * (lane & 7);
                    const u32x4 v = *(const u32x4*)(xs + rr * OP + c8);
                    if (wq0 + rr < p.qL)
                        __builtin_nontemporal_store(v, (u32x4*)(obase + (int64_t)(wq0 + rr) * p.o_s[2] + 64 * hc + c8));
                }
            }
            if (qrow < p.qL && g == 0) {
                const float lse = (l_run > 0.f) ? (m_run + __builtin_amdgcn_logf(l_run)) * kLn2 : 0.f;
                p.lse[((int64_t)b * p.Hq + h) * p.qL + qrow] = lse;
            }
            return;
        }
    }
    if (KSPLIT && half != 0) return;  // half 0 writes the merged rows
    if (p.n_split > 1) {
        // one key range of a split launch: normalised fp32 O and natural-log
        // L of this range (-inf when it holds no allowed key)
        // dropout's 1 / (1 - p) scales every kept term alike: it is applied here
        const float inv = (l_run > 0.f) ? (DROP ? p.drop_scale : 1.f) / l_run : 0.f;
        const int64_t rows = (int64_t)p.B * p.Hq * p.qL;
        const bool row_ok = qrow < p.qL && head_ok;
        // A lane's O^T registers hold 4 consecutive head-dim elements of one
        // row per quad, so a store straight from them writes 32 bytes of
        // each of 32 rows, and the partial cache lines cost HBM writes well
        // beyond their bytes.  Each wave instead passes its rows through a
        // 32 x XP float region of the (by now idle) K/V buffers, one 32-column
        // block at a time, and each store then covers whole 128-byte lines
        // of four rows.
        if constexpr (XPOSE) {
            __syncthreads();  // every wave is past its last read of the K/V buffers
            float* xs = (float*)region(wave);
            // this wave's first row (RPACK: of the wave's first head; its
            // second head's rows start 16 region rows later)
            const int64_t row0 = ((int64_t)b * p.Hq + (RPACK ? hk * p.group + (h - hk * p.group) / 2 * 2 : h)) * p.qL + wq0;
#pragma unroll
            for (int d = 0; d < ND; ++d) {
#pragma unroll
                for (int rq = 0; rq < 4; ++rq)
                    *(f32x4*)(xs + r32 * XP + 8 * rq + 4 * g) =
                        f32x4{o[d][4 * rq + 0], o[d][4 * rq + 1], o[d][4 * rq + 2], o[d][4 * rq + 3]} * inv;
                // lane l reads columns 4 (l % 8) .. +3 of rows 8 i + l / 8
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rr = 8 * i + (lane >> 3), c4 = 4 * (lane & 7);
                    const f32x4 v = *(const f32x4*)(xs + rr * XP + c4);
                    // (RPACK: region row rr is row rr % 16 of the wave's head rr / 16)
                    const int rq_ = RPACK ? (rr & 15) : wq0 + rr;
                    const int64_t ri = RPACK ? row0 + (int64_t)(rr >> 4) * p.qL + (rr & 15) : row0 + rr;
                    if (32 * d + c4 < D && rq_ < p.qL && head_ok)
                        *(f32x4*)(p.o_part + ((int64_t)split * rows + ri) * D + 32 * d + c4) = v;
                }
            }
        } else if (row_ok) {
            float* orow = p.o_part + ((int64_t)split * rows + ((int64_t)b * p.Hq + h) * p.qL + qrow) * D;
#pragma unroll
            for (int d = 0; d < ND; ++d)
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    if (32 * d + 8 * rq >= D) continue;
                    *(f32x4*)(orow + 32 * d + 8 * rq + 4 * g) =
                        f32x4{o[d][4 * rq + 0], o[d][4 * rq + 1], o[d][4 * rq + 2], o[d][4 * rq + 3]} * inv;
                }
        }
        if (row_ok && g == 0)
            p.l_part[(int64_t)split * rows + ((int64_t)b * p.Hq + h) * p.qL + qrow] =
                (l_run > 0.f) ? (m_run + __builtin_amdgcn_logf(l_run)) * kLn2 : -INFINITY;
    } else if (qrow < p.qL && head_ok) {
        // dropout's 1 / (1 - p) scales every kept term alike: it is applied here
        const float inv = (l_run > 0.f) ? (DROP ? p.drop_scale : 1.f) / l_run : 0.f;
        uint16_t* orow = (uint16_t*)p.o + b * p.o_s[0] + h * p.o_s[1] + (int64_t)qrow * p.o_s[2];
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                if (32 * d + 8 * rq >= D) continue;  // rows of the rounded-up last block
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

// Work-groups of the work-group kernel one CU holds: by waves per SIMD, and
// by LDS (tiles padded to 1 KiB blocks, NB buffers each for K and V).
template <int D, int NW, int BN, int WPE, int NB>
constexpr int wgs_per_cu()
{
    constexpr int kLdsPerWg = NB * ((BN * k_pitch<D>() / 8 + 63) / 64 + (BN * v_pitch<D>() / 8 + 63) / 64) * 1024;
    return (4 * WPE / NW < 160 * 1024 / kLdsPerWg) ? 4 * WPE / NW : 160 * 1024 / kLdsPerWg;
}

// How many work-groups a query tile's key range is split over (1: none).
// A grid that leaves more than half of the CUs idle while each work-group
// walks a long key range splits that range (at least kMinSplitTiles key
// tiles each, a multiple of the ring depth), up to one full GPU of
// work-groups; the partials are merged afterwards.
template <bool CAUSAL, int BN, int NB>
int split_plan(const FwdParams& p, int64_t wgs, int wgs_per_cu_, int* split_tiles)
{
    constexpr int kCUs = 256;
    constexpr int kMinSplitTiles = 8;
    const int kv_max = CAUSAL ? min(p.kL, p.qL) : p.kL;
    const int n_kt = (kv_max + BN - 1) / BN;
    *split_tiles = 0;
    if (!FA_SPLIT_KV || p.window > 0 || wgs * 2 > kCUs || n_kt < 2 * kMinSplitTiles) return 1;
    const int64_t want = (int64_t)kCUs * wgs_per_cu_ / wgs;
    const int by_len = n_kt / kMinSplitTiles;
    const int s0 = (int)(want < by_len ? want : (int64_t)by_len);
    if (s0 < 2) return 1;
    int st = (n_kt + s0 - 1) / s0;
    st = (st + NB - 1) / NB * NB;
    *split_tiles = st;
    return (n_kt + st - 1) / st;
}

template <int D, int MASK, bool CAUSAL, int NW, int BN, int WPE, int SCHED, int NB, bool DROP = false,
          bool KSPLIT = false, bool RPACK = false>
hipError_t launch_bf16(const FwdParams& p, hipStream_t st, size_t* need = nullptr)
{
    // the work-group kernel divides its grid index by n_split
    if (p.n_split < 1) return hipErrorInvalidValue;
    // (key halves: twice the LDS ring, and never a split over work-groups)
    constexpr int kWgsPerCu = wgs_per_cu<D, NW, BN, WPE, KSPLIT ? 2 * NB : NB>();
    FwdParams q = p;
    const int64_t wgs = RPACK       ? (int64_t)p.B * p.Hkv * (p.group / (2 * NW))
                        : p.head_pack ? (int64_t)p.n_qtiles * ((p.group + NW - 1) / NW) * p.Hkv * p.B
                                      : (int64_t)p.n_qtiles * p.Hq * p.B;
    int split_tiles = 0;
    const int n_split = KSPLIT ? 1 : split_plan<CAUSAL, BN, NB>(p, wgs, kWgsPerCu, &split_tiles);
    const int64_t rows = (int64_t)p.B * p.Hq * p.qL;
    const size_t ws_bytes = n_split < 2 ? 0 : (size_t)n_split * rows * (D + 1) * sizeof(float);
    if (need) {
        *need = ws_bytes;
        return hipSuccess;
    }
    if (n_split < 2) {
        q.pair_tiles = CAUSAL && grid_fits_at_once(wgs, kWgsPerCu);
        hipLaunchKernelGGL((fwd_bf16_kernel<D, MASK, CAUSAL, NW, BN, WPE, SCHED, NB, DROP, KSPLIT, RPACK>),
                           dim3((unsigned)wgs), dim3(NW * 64), 0, st, q);
        return hipGetLastError();
    }
    // partials in the caller's scratch, or from the library's stream-ordered
    // pool, freed (for reuse by later calls on this stream) once the merge has
    // read them.  Every partial the merge reads is written by this launch
    // first, so the scratch needs no clearing.
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
    q.pair_tiles = CAUSAL && grid_fits_at_once(wgs * n_split, kWgsPerCu);
    hipLaunchKernelGGL((fwd_bf16_kernel<D, MASK, CAUSAL, NW, BN, WPE, SCHED, NB, DROP, KSPLIT, RPACK>),
                       dim3((unsigned)(wgs * n_split)), dim3(NW * 64), 0, st, q);
    err = hipGetLastError();
    if (err == hipSuccess) {
        err = launch_merge<D, true>(q, rows, st);
    }
    if (p.ws != nullptr) return err;
    const hipError_t ferr = hipFreeAsync(ws, st);
    return err != hipSuccess ? err : ferr;
}

// ---------------------------------------------------------------------------
// Key-split forward for few, wide rows.  At D = 256 a wave needs a whole SIMD
// of registers, so a launch with fewer than one work-group per CU leaves most
// SIMDs idle (an 8-head 1024-row problem has 256 waves of 32 rows for 1024
// SIMDs).  Here a work-group owns only 32 query rows and its NS waves split
// the key range instead (wave w takes key tiles w, w + NS, ...), each with
// its own LDS buffers and no barrier in the loop.  The waves' partial
// softmax states are merged through LDS at the end -- the same merge of
// (O, m, l) partials that combines key blocks in the online softmax -- so no
// scratch memory is needed.
//
// Per tile a wave loads K (and the mask words) ahead of V: the K buffer is
// refilled as soon as the score operands are in registers, the V buffer as
// soon as the P V operands are, so each load has a softmax or a score phase
// to land in.
template <int D, int MASK, bool CAUSAL, int NS, int BN>
__global__ void __launch_bounds__(NS * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
fwd_bf16_split_kernel(const FwdParams p)
{
    using KL = TileLayout<k_pitch<D>()>;
    using VL = TileLayout<v_pitch<D>()>;
    constexpr int KSPR = KL::PITCH / 8;
    constexpr int VSPR = VL::PITCH / 8;
    constexpr int KINS = (BN * KSPR + 63) / 64;  // 1 KiB blocks (and loads) per K tile
    constexpr int VINS = (BN * VSPR + 63) / 64;  // 1 KiB blocks (and loads) per V tile
    constexpr int KTILE = KINS * 512;
    constexpr int VTILE = VINS * 512;
    constexpr int DK = D / 16;
    constexpr int NC = BN / 32;
    constexpr int ND = D / 32;
    constexpr int OPITCH = D + 4;                // floats per row of a partial O in LDS
    constexpr int NMASK = (MASK == MASK_NONE) ? 0 : NC * 4;  // mask loads per tile (vector path)
    static_assert(NS == 4 && ND % NS == 0, "the merge gives each wave ND / NS blocks of O");
    static_assert(2 * 32 * OPITCH * 4 <= NS * KTILE * 2 && 2 * 32 * OPITCH * 4 <= NS * VTILE * 2,
                  "two partial O tiles fit in each of the K and V areas");
    static_assert(KINS < 48 && VINS + NMASK < 48, "vmcnt range");

    __shared__ __attribute__((aligned(1024))) uint16_t Kall[NS * KTILE];
    __shared__ __attribute__((aligned(1024))) uint16_t Vall[NS * VTILE];
    __shared__ float Mpart[NS][32];
    __shared__ float Lpart[NS][32];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r32 = lane & 31;
    const int g = lane >> 5;

    int id = blockIdx.x;
    const int h = head_of(id % p.Hq, p.Hq);
    id /= p.Hq;
    const int b = id % p.B;
    id /= p.B;
    const int qt = CAUSAL ? causal_tile(id, p.n_qtiles, p.pair_tiles) : id;
    const int q0 = qt * 32;
    const int qrow = q0 + r32;
    const int hk = h / p.group;

    const uint16_t* Qb = (const uint16_t*)p.q + b * p.q_s[0] + h * p.q_s[1];
    const uint16_t* Kb = (const uint16_t*)p.k + b * p.k_s[0] + hk * p.k_s[1];
    const uint16_t* Vb = (const uint16_t*)p.v + b * p.v_s[0] + hk * p.v_s[1];

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
    const int kv_end = CAUSAL ? min(p.kL, min(p.qL, q0 + 32)) : p.kL;
    const int n_tiles = (q0 < p.qL) ? (kv_end + BN - 1) / BN : 0;

    const uint8_t* mrow = nullptr;
    if (MASK != MASK_NONE) {
        const int qc = min(qrow, p.qL - 1);
        const int esz = (MASK == MASK_BOOL) ? 1 : 2;
        mrow = (const uint8_t*)p.mask + (b * p.m_s[0] + h * p.m_s[1] + (int64_t)qc * p.m_s[2]) * esz;
    }

    f32x16 o[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) o[d] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    uint16_t* Kw = Kall + wave * KTILE;
    uint16_t* Vw = Vall + wave * VTILE;
    // the whole tile by this wave: block i is one direct load (see the
    // work-group kernel); rows past kL load row kL - 1.  Here the compiler
    // tracks the loads: the mask words are ordinary loads, and a wait for
    // them would otherwise also wait for every untracked load issued after
    // them, i.e. for the next K tile.
    auto issue_tile = [&](const uint16_t* gbase, int64_t stride, int j0, uint16_t* lds, auto spr_c, auto nins_c)
        __attribute__((always_inline)) {
        constexpr int SPR = decltype(spr_c)::value;
        constexpr int NINS = decltype(nins_c)::value;
#pragma unroll
        for (int i = 0; i < NINS; ++i) {
            const int slot = 64 * i + lane;
            const int row = slot / SPR;
            const int ch = slot % SPR;
            if (ch < D / 8 && row < BN) {
                const int j = min(j0 + row, p.kL - 1);
                __builtin_amdgcn_global_load_lds(
                    (__attribute__((address_space(1))) void*)(gbase + (int64_t)j * stride + ch * 8),
                    (__attribute__((address_space(3))) void*)(lds + 512 * i), 16, 0, 0);
            }
        }
    };

    typedef u32x2 MaskWords[NC][4];
    auto load_mask = [&](int j0, MaskWords& mw) __attribute__((always_inline)) {
        // one decision per tile (a per-quad one would split the loads into
        // branches the compiler's wait counting merges pessimistically)
        const bool vec = p.mask_vec && j0 + BN <= p.kL;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int jb = j0 + 32 * c + 8 * rq + 4 * g;
                u32x2 w = {0u, 0u};
                if (vec) {
                    // whole tile inside the row, rows aligned: one load per quad
                    if (MASK == MASK_ADD) w = *(const u32x2*)(mrow + 2 * (int64_t)jb);
                    if (MASK == MASK_BOOL) w[0] = *(const uint32_t*)(mrow + jb);
                } else if (MASK == MASK_ADD) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (jb + e < p.kL) w[e >> 1] |= (uint32_t)((const uint16_t*)mrow)[jb + e] << (16 * (e & 1));
                } else if (MASK == MASK_BOOL) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (jb + e < p.kL && mrow[jb + e] != 0) w[0] |= 1u << (8 * e);
                }
                mw[c][rq] = w;
            }
        }
    };
    // K (and the mask words) of tile t, then V of tile t
    auto issue_k = [&](int t, MaskWords& mw) __attribute__((always_inline)) {
        issue_tile(Kb, p.k_s[2], t * BN, Kw, std::integral_constant<int, KSPR>{}, std::integral_constant<int, KINS>{});
        if (MASK != MASK_NONE) load_mask(t * BN, mw);
    };
    auto issue_v = [&](int t) __attribute__((always_inline)) {
        issue_tile(Vb, p.v_s[2], t * BN, Vw, std::integral_constant<int, VSPR>{}, std::integral_constant<int, VINS>{});
    };

    MaskWords mw, mwn;
    int t = wave;
    if (t < n_tiles) {
        issue_k(t, mw);
        issue_v(t);
    }
    const int lt = lane & 15;
    for (; t < n_tiles; t += NS) {
        const int tn = t + NS;
        const int j0 = t * BN;
        // K and the mask words of tile t have landed (V, issued after them,
        // may still be in flight)
        __builtin_amdgcn_s_waitcnt(0x0F70 | (VINS & 15) | ((VINS >> 4) << 14));
        f32x16 s[NC];
#pragma unroll
        for (int ks = 0; ks < DK; ++ks)
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const bf16x8 kop = *(const bf16x8*)(Kw + KL::off(32 * c + r32, 2 * ks + g));
                s[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qf[ks], ks == 0 ? f32x16{} : s[c], 0, 0, 0);
            }
        const bool masked = (MASK != MASK_NONE) || (j0 + BN > p.kL) || (CAUSAL && j0 + BN - 1 > q0);
        if (masked) {
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    const int jb = j0 + 32 * c + 8 * rq + 4 * g;
                    const u32x2 w = mw[c][rq];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int j = jb + e;
                        bool ok = j < p.kL;
                        if (MASK == MASK_BOOL) ok = ok && ((w[0] >> (8 * e)) & 0xffu) != 0;
                        if (CAUSAL) ok = ok && (j <= qrow);
                        float x = s[c][4 * rq + e] * c2;
                        if (MASK == MASK_ADD) {
                            const uint32_t bits = (w[e >> 1] >> (16 * (e & 1))) & 0xffffu;
                            x = __builtin_fmaf(bf16_bits_to_float(bits), kLog2e, x);
                        }
                        s[c][4 * rq + e] = ok ? x : -INFINITY;
                    }
                }
        }
        // the score operands are in registers and this tile's mask words are
        // used: refill the K buffer (and fetch the next mask words).  Issued
        // only now, so that the compiler's wait for this tile's mask words
        // does not also wait for these loads.
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        if (tn < n_tiles) issue_k(tn, mwn);
        const float cs = masked ? 1.f : c2;
        float mx = s[0][0];
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[c][r]);
        const float m_tile = row_max_halves(mx) * cs;
        if (__builtin_amdgcn_ballot_w64(m_tile > m_run + kRescaleSlack) != 0) {
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
        // V of tile t has landed (only K and mask words of tile tn are newer)
        if (tn < n_tiles)
            __builtin_amdgcn_s_waitcnt(0x0F70 | ((KINS + NMASK) & 15) | (((KINS + NMASK) >> 4) << 14));
        else
            __builtin_amdgcn_s_waitcnt(0x0F70);
        float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int kidx = 2 * c + hh;
                u32x4 pw;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float a = __builtin_amdgcn_exp2f(__builtin_fmaf(s[c][8 * hh + 2 * e], cs, -m_use));
                    const float z = __builtin_amdgcn_exp2f(__builtin_fmaf(s[c][8 * hh + 2 * e + 1], cs, -m_use));
                    pw[e] = pack_bf16x2(a, z);
                    rs0 += a;
                    rs1 += z;
                }
                const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
                for (int d = 0; d < ND; ++d) {
                    const int col = 32 * d + 16 * ((lane >> 4) & 1) + 4 * (lt & 3);
                    const int row0 = 16 * kidx + 4 * g + (lt >> 2);
                    const i16x4 v0 = lds_read_tr(Vw + VL::off(row0, 0) + col);
                    const i16x4 v1 = lds_read_tr(Vw + VL::off(row0 + 8, 0) + col);
                    const bf16x8 vop =
                        __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
                    o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pf, o[d], 0, 0, 0);
                }
            }
        }
        l_run += row_sum_halves(rs0 + rs1);
        // the P V operands are in registers: refill the V buffer
        __builtin_amdgcn_s_waitcnt(0xC07F);
        if (tn < n_tiles) issue_v(tn);
        if (MASK != MASK_NONE) {
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) mw[c][rq] = mwn[c][rq];
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // no load of this wave is still writing LDS

    // ---- merge the NS partial softmax states of each row ----
    __syncthreads();  // every wave is done with its K and V buffers
    if (g == 0) Mpart[wave][r32] = m_run;
    __syncthreads();
    float m_fin = -INFINITY;
#pragma unroll
    for (int w = 0; w < NS; ++w) m_fin = fmaxf(m_fin, Mpart[w][r32]);
    const float corr = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_fin);
    float* opart = (wave < 2) ? (float*)Kall + wave * (32 * OPITCH) : (float*)Vall + (wave - 2) * (32 * OPITCH);
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
            f32x4 v = {o[d][4 * rq] * corr, o[d][4 * rq + 1] * corr, o[d][4 * rq + 2] * corr, o[d][4 * rq + 3] * corr};
            *(f32x4*)(opart + r32 * OPITCH + 32 * d + 8 * rq + 4 * g) = v;
        }
    if (g == 0) Lpart[wave][r32] = l_run * corr;
    __syncthreads();
    float l_fin = 0.f;
#pragma unroll
    for (int w = 0; w < NS; ++w) l_fin += Lpart[w][r32];
    if (qrow < p.qL) {
        const float inv = (l_fin > 0.f) ? 1.f / l_fin : 0.f;
        uint16_t* orow = (uint16_t*)p.o + b * p.o_s[0] + h * p.o_s[1] + (int64_t)qrow * p.o_s[2];
        // wave w finishes head-dimension blocks [w ND/NS, (w+1) ND/NS)
#pragma unroll
        for (int dd = 0; dd < ND / NS; ++dd) {
            const int d = wave * (ND / NS) + dd;
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int off = r32 * OPITCH + 32 * d + 8 * rq + 4 * g;
                f32x4 acc = *(const f32x4*)((float*)Kall + off);
                acc += *(const f32x4*)((float*)Kall + 32 * OPITCH + off);
                acc += *(const f32x4*)((float*)Vall + off);
                acc += *(const f32x4*)((float*)Vall + 32 * OPITCH + off);
                u32x2 w;
                w[0] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
                w[1] = pack_bf16x2(acc[2] * inv, acc[3] * inv);
                *(u32x2*)(orow + 32 * d + 8 * rq + 4 * g) = w;
            }
        }
        if (wave == 0 && g == 0) {
            const float lse = (l_fin > 0.f) ? (m_fin + __builtin_amdgcn_logf(l_fin)) * kLn2 : 0.f;
            p.lse[((int64_t)b * p.Hq + h) * p.qL + qrow] = lse;
        }
    }
}

// ---------------------------------------------------------------------------
// Streaming forward for short key ranges (kL <= 32 NT).  The cost of such a
// launch is reading Q and writing O once (flop per byte about kL, below the
// matrix ridge), so the kernel is built to keep HBM busy:
//   * a work-group stays on one kv head, loads all of its K and V into LDS
//     once (at most NT tiles of 32 keys), and then needs no barrier;
//   * each wave walks a strided list of 32-row query blocks of that head's
//     query-head group; the next block's Q is loaded into registers while
//     the current block is computed and its O stored (the raw words are
//     converted only where they are used, so nothing waits for them early);
//   * the grid is sized to the number of work-groups the GPU holds at once;
//   * O leaves through a small per-wave LDS region, so that each store
//     covers whole 128-byte lines of 8 rows (stored straight from the
//     accumulators, an instruction writes 16 bytes of each of 32 rows, and
//     those scattered writes cost more than the rest of the kernel: 40
//     against 30 us at 32 heads x 8192 rows x 32 keys, 26.5 with the whole
//     lines stored nontemporally; a nontemporal hint on the scattered pieces
//     made it 4x slower).  With NT = 4 and 4 waves there is no LDS room for
//     the region beside two work-groups per CU, so NT = 4 takes 8-wave
//     work-groups, one per CU.
template <int D, bool CAUSAL, int NW, int NT>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
fwd_bf16_stream_kernel(const FwdParams p, int wgs_per_head)
{
    constexpr int BN = 32;
    using KL = TileLayout<k_pitch<D>()>;
    using VL = TileLayout<v_pitch<D>()>;
    constexpr int KSPR = KL::PITCH / 8, VSPR = VL::PITCH / 8;
    constexpr int KINS = (BN * KSPR + 63) / 64, VINS = (BN * VSPR + 63) / 64;
    constexpr int KTILE = KINS * 512, VTILE = VINS * 512;
    constexpr int DK = D / 16, ND = D / 32;
    __shared__ __attribute__((aligned(1024))) uint16_t Ks[NT * KTILE];
    __shared__ __attribute__((aligned(1024))) uint16_t Vs[NT * VTILE];
    // O staging: per wave 32 rows x 64 columns (128 bytes of a row), pitch
    // 72 elements
    constexpr bool STAGE = (NT <= 2 || NW == 8) && D % 64 == 0;
    constexpr int OP = 72;
    __shared__ __attribute__((aligned(16))) uint16_t Ost[STAGE ? NW * 32 * OP : 8];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r32 = lane & 31, g = lane >> 5, lt = lane & 15;

    // work-group -> (batch, kv head, slot among the head's work-groups)
    const int slot = blockIdx.x % wgs_per_head;
    const int bh = blockIdx.x / wgs_per_head;
    const int hk = bh % p.Hkv;
    const int b = bh / p.Hkv;
    const uint16_t* Kb = (const uint16_t*)p.k + b * p.k_s[0] + hk * p.k_s[1];
    const uint16_t* Vb = (const uint16_t*)p.v + b * p.v_s[0] + hk * p.v_s[1];
    const int n_tiles = (p.kL + BN - 1) / BN;  // <= NT

    // ---- all K and V tiles of this head into LDS (rows past kL repeat row kL - 1) ----
    auto load_tile = [&](const uint16_t* gbase, int64_t stride, uint16_t* lds, auto spr_c, auto nins_c, int t)
        __attribute__((always_inline)) {
        constexpr int SPR = decltype(spr_c)::value;
        constexpr int NINS = decltype(nins_c)::value;
        for (int i = wave; i < NINS; i += NW) {
            const int sl = 64 * i + lane;
            const int row = sl / SPR, ch = sl % SPR;
            if (ch < D / 8 && row < BN) {
                const int j = min(t * BN + row, p.kL - 1);
                lds_dma16(gbase + (int64_t)j * stride + ch * 8,
                          (uint32_t)(size_t)(__attribute__((address_space(3))) void*)(lds + 512 * i));
            }
        }
    };
    for (int t = 0; t < n_tiles; ++t) {
        load_tile(Kb, p.k_s[2], Ks + t * KTILE, std::integral_constant<int, KSPR>{},
                  std::integral_constant<int, KINS>{}, t);
        load_tile(Vb, p.v_s[2], Vs + t * VTILE, std::integral_constant<int, VSPR>{},
                  std::integral_constant<int, VINS>{}, t);
    }

    // ---- this wave's query blocks: block q of the group's group * nqb ----
    const int nqb = (p.qL + 31) / 32;
    const int nblk = p.group * nqb;
    const int stride_blk = wgs_per_head * NW;
    const float c2 = p.scale_log2;
    const uint32_t flip = p.neg_q ? 0x80008000u : 0u;

    // raw Q words of a block; the sign flip and the zeroing of rows past qL
    // are applied where the block is computed, so nothing waits for these
    // loads before then.  Always DK loads (from an in-range row), so the
    // number of loads in flight is known when waiting below.
    auto q_load = [&](int blk, u32x4 (&qw)[DK]) __attribute__((always_inline)) {
        const int bc = min(blk, nblk - 1);
        const int h = hk * p.group + bc / nqb;
        const int qrow = min((bc % nqb) * 32 + r32, p.qL - 1);
        const u32x4* src =
            (const u32x4*)((const uint16_t*)p.q + b * p.q_s[0] + h * p.q_s[1] + (int64_t)qrow * p.q_s[2]);
#pragma unroll
        for (int ks = 0; ks < DK; ++ks) qw[ks] = src[2 * ks + g];
    };

    auto block = [&](int blk, const u32x4 (&qw)[DK]) __attribute__((always_inline)) {
        const int h = hk * p.group + blk / nqb;
        const int q0 = (blk % nqb) * 32;
        const int qrow = q0 + r32;
        bf16x8 qf[DK];
#pragma unroll
        for (int ks = 0; ks < DK; ++ks)
            qf[ks] = __builtin_bit_cast(bf16x8, qrow < p.qL ? (qw[ks] ^ flip) : u32x4{0, 0, 0, 0});
        f32x16 o[ND];
#pragma unroll
        for (int d = 0; d < ND; ++d) o[d] = f32x16{};
        float m_run = -INFINITY, l_run = 0.f;
        const int t_end = CAUSAL ? min(n_tiles, (q0 + 31) / BN + 1) : n_tiles;
        for (int t = 0; t < t_end; ++t) {
            const uint16_t* kt = Ks + t * KTILE;
            const uint16_t* vt = Vs + t * VTILE;
            const int j0 = t * BN;
            f32x16 s = f32x16{};
#pragma unroll
            for (int ks = 0; ks < DK; ++ks) {
                const bf16x8 kop = *(const bf16x8*)(kt + KL::off(r32, 2 * ks + g));
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qf[ks], s, 0, 0, 0);
            }
            const bool masked = (j0 + BN > p.kL) || (CAUSAL && j0 + BN - 1 > q0);
            if (masked) {
                int lim = p.kL - 1;
                if (CAUSAL) lim = min(lim, qrow);
                lim -= j0 + 4 * g;
#pragma unroll
                for (int r = 0; r < 16; ++r) s[r] = (8 * (r >> 2) + (r & 3) <= lim) ? s[r] * c2 : -INFINITY;
            }
            const float cs = masked ? 1.f : c2;
            float mx = s[0];
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
            const float m_tile = row_max_halves(mx) * cs;
            if (__builtin_amdgcn_ballot_w64(m_tile > m_run + kRescaleSlack) != 0) {
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
            float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                u32x4 pw;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float a = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * hh + 2 * e], cs, -m_use));
                    const float z = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * hh + 2 * e + 1], cs, -m_use));
                    pw[e] = pack_bf16x2(a, z);
                    rs0 += a;
                    rs1 += z;
                }
                const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
                for (int d = 0; d < ND; ++d) {
                    const int col = 32 * d + 16 * ((lane >> 4) & 1) + 4 * (lt & 3);
                    const int row0 = 16 * hh + 4 * g + (lt >> 2);
                    const i16x4 v0 = lds_read_tr(vt + VL::off(row0, 0) + col);
                    const i16x4 v1 = lds_read_tr(vt + VL::off(row0 + 8, 0) + col);
                    const bf16x8 vop =
                        __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
                    o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pf, o[d], 0, 0, 0);
                }
            }
            l_run += row_sum_halves(rs0 + rs1);
        }
        const float inv = (l_run > 0.f) ? 1.f / l_run : 0.f;
        if constexpr (STAGE) {
            // 64 columns at a time: the lanes' 4-element runs into the
            // wave's region, then rows back out as 16-byte pieces, 8 lanes
            // per row (the region is the wave's own, and a wave's LDS
            // accesses take effect in order, so no barrier is needed)
            uint16_t* xs = Ost + wave * (32 * OP);
            uint16_t* obase = (uint16_t*)p.o + b * p.o_s[0] + h * p.o_s[1];
#pragma unroll
            for (int hc = 0; hc < D / 64; ++hc) {
#pragma unroll
                for (int dd = 0; dd < 2; ++dd)
#pragma unroll
                    for (int rq = 0; rq < 4; ++rq) {
                        const int d = 2 * hc + dd;
                        u32x2 w;
                        w[0] = pack_bf16x2(o[d][4 * rq + 0] * inv, o[d][4 * rq + 1] * inv);
                        w[1] = pack_bf16x2(o[d][4 * rq + 2] * inv, o[d][4 * rq + 3] * inv);
                        *(u32x2*)(xs + r32 * OP + 32 * dd + 8 * rq + 4 * g) = w;
                    }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rr = 8 * i + (lane >> 3), c8 = 8 * (lane & 7);
                    const u32x4 v = *(const u32x4*)(xs + rr * OP + c8);
                    // (nontemporal: O is not read again here; whole lines
                    // so marked go out without a read-modify-write)
                    if (q0 + rr < p.qL)
                        __builtin_nontemporal_store(v, (u32x4*)(obase + (int64_t)(q0 + rr) * p.o_s[2] + 64 * hc + c8));
                }
            }
        }
        if (qrow < p.qL) {
            if constexpr (!STAGE) {
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
            }
            if (g == 0) {
                const float lse = (l_run > 0.f) ? (m_run + __builtin_amdgcn_logf(l_run)) * kLn2 : 0.f;
                p.lse[((int64_t)b * p.Hq + h) * p.qL + qrow] = lse;
            }
        }
    };

    // two Q buffers, unrolled by two: the next block's Q is in flight while
    // a block computes and stores (the first is issued before waiting for
    // the K/V staging)
    u32x4 qa[DK], qb[DK];
    int blk = slot * NW + wave;
    q_load(blk, qa);
    // K and V in LDS; the DK loads of the first Q block, issued after them,
    // may still be in flight
    static_assert(DK < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (DK & 15) | ((DK >> 4) << 14));
    __syncthreads();
    for (; blk < nblk; blk += 2 * stride_blk) {
        q_load(blk + stride_blk, qb);
        block(blk, qa);
        if (blk + stride_blk >= nblk) break;
        q_load(blk + 2 * stride_blk, qa);
        block(blk + stride_blk, qb);
    }
}

// Launch: the work-group kernel, or for wide rows whose grid would not give
// every CU a work-group, the key-split kernel
// (D = 256 only: narrower rows leave room for more waves per SIMD instead.)
// At D = 128, key ranges up to kShortKeys take a work-group shape suited to
// HBM-bound launches.
constexpr int kShortKeys = 256;
// Query ranges up to this many rows take 2-wave work-groups.
constexpr int kShortQueries = 64;
// Waves per work-group, keys per tile, waves per SIMD, schedule and ring
// depth of the packed short-query shape (by default 2-wave work-groups with
// the head dim's main tile shape).
#ifndef FA_BF16_RPACK_SHAPE
#define FA_BF16_RPACK_SHAPE 2, BN, WPE, SCHED, NB
#endif
template <int D, int MASK, bool CAUSAL, int NW, int BN, int WPE, int SCHED, int NB>
hipError_t launch_bf16_any(const FwdParams& p, hipStream_t st, size_t* need = nullptr)
{
    // (the work-group launcher rejects n_split < 1; the other kernels ignore it)
    if (p.n_split < 1) return hipErrorInvalidValue;
    if constexpr (D == 128) {
        // Short key ranges are HBM-bound (Q in, O out).
        if (MASK == MASK_NONE && p.kL <= 4 * 32 && p.window == 0) {
            // streaming kernel: enough work-groups per kv head to fill the
            // GPU twice over, each with at least a few query blocks per wave
            constexpr int kResident = 2 * 256;
            const int heads = p.B * p.Hkv;
            const int blocks = p.group * ((p.qL + 31) / 32);
            int per_head = (kResident + heads - 1) / heads;
            per_head = max(1, min(per_head, blocks / 4));
            const dim3 grid((unsigned)(per_head * heads));
            if (need) {
                *need = 0;
                return hipSuccess;
            }
            // K/V LDS sized to the key range (one, two or four 32-key tiles)
            if (p.kL <= 32)
                hipLaunchKernelGGL((fwd_bf16_stream_kernel<D, CAUSAL, 4, 1>), grid, dim3(4 * 64), 0, st, p, per_head);
            else if (p.kL <= 64)
                hipLaunchKernelGGL((fwd_bf16_stream_kernel<D, CAUSAL, 4, 2>), grid, dim3(4 * 64), 0, st, p, per_head);
            else {
                // 8-wave work-groups, one per CU
                int per_head8 = (kResident / 2 + heads - 1) / heads;
                per_head8 = max(1, min(per_head8, blocks / 8));
                hipLaunchKernelGGL((fwd_bf16_stream_kernel<D, CAUSAL, 8, 4>), dim3((unsigned)(per_head8 * heads)),
                                   dim3(8 * 64), 0, st, p, per_head8);
            }
            return hipGetLastError();
        }
    }
    if constexpr (NW > 2) {
        // Short query ranges (a decode step): 2-wave work-groups of 64 rows,
        // so that waves are not spent on rows past qL and more work-groups
        // fit per CU (the split plan then cuts a long key range finer).
        if (p.qL <= kShortQueries) {
            FwdParams q = p;
            if (p.qL <= 16 && p.group % 4 == 0 && p.window == 0) {
                // at most 16 rows: each wave holds two query heads' rows
                q.n_qtiles = 1;
                return launch_bf16<D, MASK, CAUSAL, FA_BF16_RPACK_SHAPE, false, false, true>(q, st, need);
            }
            if (p.qL <= 32 && p.group >= 2) {
                // one 32-row tile: pack two query heads of a GQA group
                q.head_pack = 1;
                q.n_qtiles = 1;
            } else {
                q.n_qtiles = (p.qL + 63) / 64;
            }
            return launch_bf16<D, MASK, CAUSAL, 2, BN, WPE, SCHED, NB>(q, st, need);
        }
    }
    if constexpr (D == 256) {
        // Fewer query tiles than CUs: split the key range over work-groups
        // when it is long enough (measured 73 against 80 us on 8 heads x
        // 1024 rows x 3072 keys), else over the waves of one work-group.
        constexpr int kCUs = 256;
        int split_tiles = 0;
        if (p.window == 0 && (int64_t)p.n_qtiles * p.Hq * p.B < kCUs &&
            split_plan<CAUSAL, BN, NB>(p, (int64_t)p.n_qtiles * p.Hq * p.B, wgs_per_cu<D, NW, BN, WPE, NB>(),
                                       &split_tiles) < 2) {
            FwdParams q = p;
            q.n_qtiles = (p.qL + 31) / 32;
            q.pair_tiles = CAUSAL && grid_fits_at_once((int64_t)q.n_qtiles * q.Hq * q.B, 1);
            const dim3 grid((unsigned)q.n_qtiles * q.Hq * q.B);
            if (need) {
                *need = 0;
                return hipSuccess;
            }
            hipLaunchKernelGGL((fwd_bf16_split_kernel<D, MASK, CAUSAL, 4, 32>), grid, dim3(4 * 64), 0, st, q);
            return hipGetLastError();
        }
    }
    if constexpr (D == 128) {
        // Key ranges up to kShortKeys: 4-wave work-groups with 32-key tiles
        // keep two work-groups per CU resident, so one's loads overlap the
        // other's stores (kL = 32: 49 -> 38 us for 32 heads x 8192 rows);
        // long ones keep the 8-wave shape.
        if (p.kL <= kShortKeys) {
            FwdParams q = p;
            q.n_qtiles = (p.qL + 127) / 128;
            return launch_bf16<D, MASK, CAUSAL, 4, 32, 2, 0, 2>(q, st, need);
        }
    }
    if constexpr (FA_KEY_HALVES && CAUSAL && NW <= 4 && BN >= 64 && NB == 2) {
        // Causal grids that fit on the GPU at once but are too large to split
        // over work-groups (e.g. 2 x 16 heads x 2048 rows at D = 64): a long
        // row block would run its key tiles alone at the end, so each
        // work-group walks its key range in two halves side by side (twice
        // the waves, the same rows) and merges them.
        const int64_t wgs = (int64_t)p.n_qtiles * p.Hq * p.B;
        const int n_kt = (min(p.kL, p.qL) + BN - 1) / BN;
        if (p.window == 0 && p.head_pack == 0 && wgs * 2 > 256 && n_kt >= 8 &&
            grid_fits_at_once(wgs, wgs_per_cu<D, NW, BN, WPE, NB>()))
            return launch_bf16<D, MASK, CAUSAL, 2 * NW, BN, WPE, SCHED, NB, false, true>(p, st, need);
    }
    return launch_bf16<D, MASK, CAUSAL, NW, BN, WPE, SCHED, NB>(p, st, need);
}

}  // namespace

// Launch shapes per head dimension and mask use: waves per work-group, keys
// per tile, waves per SIMD, pipelined (1) or not (0), LDS ring depth (2 or
// 4).  Overridable at build time for tuning sweeps.
#ifndef FA_BF16_D16_CFG
#define FA_BF16_D16_CFG 4, 64, 2, 1, 2
#endif
#ifndef FA_BF16_D16_MASKED_CFG
#define FA_BF16_D16_MASKED_CFG 4, 64, 2, 0, 2
#endif
#ifndef FA_BF16_D48_CFG
#define FA_BF16_D48_CFG 4, 64, 2, 1, 2
#endif
#ifndef FA_BF16_D48_MASKED_CFG
#define FA_BF16_D48_MASKED_CFG 4, 64, 2, 0, 2
#endif
#ifndef FA_BF16_D80_CFG
#define FA_BF16_D80_CFG 8, 64, 2, 0, 2
#endif
#ifndef FA_BF16_D80_MASKED_CFG
#define FA_BF16_D80_MASKED_CFG 8, 64, 2, 0, 2
#endif
#ifndef FA_BF16_D32_CFG
#define FA_BF16_D32_CFG 4, 64, 2, 1, 2
#endif
#ifndef FA_BF16_D32_MASKED_CFG
#define FA_BF16_D32_MASKED_CFG 4, 64, 2, 0, 2
#endif
#ifndef FA_BF16_D64_CFG
#define FA_BF16_D64_CFG 4, 64, 2, 1, 2
#endif
#ifndef FA_BF16_D64_MASKED_CFG
#define FA_BF16_D64_MASKED_CFG 4, 64, 2, 0, 2
#endif
#ifndef FA_BF16_D128_CFG
#define FA_BF16_D128_CFG 8, 64, 2, 0, 2
#endif
#ifndef FA_BF16_D128_MASKED_CFG
#define FA_BF16_D128_MASKED_CFG 8, 64, 2, 0, 2
#endif
#ifndef FA_BF16_D96_CFG
#define FA_BF16_D96_CFG 8, 64, 2, 0, 2
#endif
#ifndef FA_BF16_D96_MASKED_CFG
#define FA_BF16_D96_MASKED_CFG 8, 64, 2, 0, 2
#endif
#ifndef FA_BF16_D256_CFG
#define FA_BF16_D256_CFG 4, 32, 1, 1, 2
#endif
#ifndef FA_BF16_D256_MASKED_CFG
#define FA_BF16_D256_MASKED_CFG 4, 32, 1, 1, 2
#endif

#define FA_BF16_VARIANT(D, MASK, CAUSAL, NAME, NW, BN, WPE, SCHED, NB) \
    {NAME, 1, D, MASK, CAUSAL, NW * 32, &launch_bf16_any<D, MASK, CAUSAL, NW, BN, WPE, SCHED, NB>}
// expands a CFG macro into separate arguments before FA_BF16_VARIANT sees them
#define FA_BF16_VARIANT_CFG(...) FA_BF16_VARIANT(__VA_ARGS__)

#define FA_BF16_FOR_D(D, CFG, MCFG)                                                       \
    FA_BF16_VARIANT_CFG(D, MASK_NONE, false, "fwd_bf16_d" #D "_nomask", CFG),             \
    FA_BF16_VARIANT_CFG(D, MASK_NONE, true, "fwd_bf16_d" #D "_nomask_causal", CFG),       \
    FA_BF16_VARIANT_CFG(D, MASK_ADD, false, "fwd_bf16_d" #D "_additive", MCFG),           \
    FA_BF16_VARIANT_CFG(D, MASK_ADD, true, "fwd_bf16_d" #D "_additive_causal", MCFG),     \
    FA_BF16_VARIANT_CFG(D, MASK_BOOL, false, "fwd_bf16_d" #D "_bool", MCFG),              \
    FA_BF16_VARIANT_CFG(D, MASK_BOOL, true, "fwd_bf16_d" #D "_bool_causal", MCFG)

// Dropout variants: the work-group kernel at the head dims' own launch
// shapes (no short-key or short-query special cases).
#define FA_BF16_DROP_VARIANT(D, MASK, CAUSAL, NAME, NW, BN, WPE, SCHED, NB) \
    {NAME, 1, D, MASK, CAUSAL, NW * 32, &launch_bf16<D, MASK, CAUSAL, NW, BN, WPE, SCHED, NB, true>}
#define FA_BF16_DROP_VARIANT_CFG(...) FA_BF16_DROP_VARIANT(__VA_ARGS__)
#define FA_BF16_DROP_FOR_D(D, CFG, MCFG)                                                           \
    FA_BF16_DROP_VARIANT_CFG(D, MASK_NONE, false, "fwd_bf16_d" #D "_nomask_dropout", CFG),         \
    FA_BF16_DROP_VARIANT_CFG(D, MASK_NONE, true, "fwd_bf16_d" #D "_nomask_causal_dropout", CFG),   \
    FA_BF16_DROP_VARIANT_CFG(D, MASK_ADD, false, "fwd_bf16_d" #D "_additive_dropout", MCFG),       \
    FA_BF16_DROP_VARIANT_CFG(D, MASK_ADD, true, "fwd_bf16_d" #D "_additive_causal_dropout", MCFG), \
    FA_BF16_DROP_VARIANT_CFG(D, MASK_BOOL, false, "fwd_bf16_d" #D "_bool_dropout", MCFG),          \
    FA_BF16_DROP_VARIANT_CFG(D, MASK_BOOL, true, "fwd_bf16_d" #D "_bool_causal_dropout", MCFG)

}  // namespace fa
