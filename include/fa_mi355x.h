/*
 * fa_mi355x.h - C ABI of libfa_mi355x, a FlashAttention-2 forward pass (and
 * its backward pass) for AMD Instinct MI355X (gfx950).
 *
 * The operation (mlx-native flash_attn_train.rs, module doc "Algorithm" and
 * "Buffer layout"; oxibonsai dit_attention_flash.rs, module doc "Flash-attention
 * v2 structure"; ruDNN dense_attention.rs, `forward`):
 *
 *   for batch b, query head h, query row i, kv head g = h / (H_q / H_kv):
 *     s_ij   = scale * sum_d Q[b,h,i,d] K[b,g,j,d]   (+ mask[b,h,i,j], additive)
 *     key j is allowed iff j <= i when causal (top-left: row i sees keys
 *     0..i, whatever qL and kL are), the bool mask entry is nonzero, and
 *     s_ij != -inf
 *     O[b,h,i,:] = sum_j softmax_j(s_ij) V[b,g,j,:]   over the allowed keys
 *     L[b,h,i]   = ln sum_j exp(s_ij)                 (natural log)
 *   A row with no allowed key gets O = 0 and L = 0 (forge
 *   flash_attention_mma.metal, epilogue of flash_attn_fwd_mma).
 *
 * `scale` is the natural-domain factor, typically 1/sqrt(D); the library
 * folds log2(e) in itself (mlx-native flash_attn_train.rs, module doc "Scale
 * convention").  The additive mask is added after scaling (ruDNN `forward`).
 *
 * Conventions shared by every entry point:
 *   - Every pointer is a DEVICE pointer on the current HIP device; the caller
 *     owns all of them.  Q, K, V and the mask are read-only; O and L are
 *     overwritten in full (rows beyond qL and padding are never touched).
 *   - The call enqueues work on `hip_stream` (a hipStream_t; NULL = the null
 *     stream) and returns without synchronising.
 *   - Allocation: the forward path allocates no device memory, with one
 *     stated exception.  A call (bf16 or fp32) whose grid of query tiles
 *     leaves most CUs idle while its key range is long (for fp32 grids of
 *     at most 8 work-groups, two or more 32-key tiles) splits that range
 *     over work-groups, and needs fp32 partials (n_split * B * H_q * qL *
 *     (D + 1) * 4 bytes, at most ~34 MB).  They go to a workspace the
 *     library keeps for each (device, stream) pair it has been called with,
 *     taken from a stream-ordered memory pool that the library creates for
 *     itself on each device (hipMemPoolCreate; it keeps up to 256 MiB of
 *     freed memory for reuse) and grown, on `hip_stream`, when a call needs
 *     more than it holds.  Each use waits for the previous one through an
 *     event.  A workspace is held until the process ends; a device keeps at
 *     most 8, and calls on further streams take their partials from the pool
 *     per call and return them after the merge.  The device's default pool
 *     and every other process-wide allocator setting are left untouched.
 *     Callers that cannot allocate use fa_fwd_strided_noalloc.  fa_bwd takes
 *     the partials of a split dK/dV grid from the same pool, per call (see
 *     fa_bwd).
 *   - All argument checks run before any launch: a failed check writes
 *     nothing, launches nothing and returns FA_ERR_INVALID_ARGUMENT (or
 *     FA_ERR_UNSUPPORTED for a valid combination that is not built), with a
 *     message in fa_last_error().  A failed launch returns FA_ERR_HIP.
 *   - Buffer sizes cannot be checked through raw pointers; the Python binding
 *     checks them (cf. mlx-native flash_attn_train.rs, validate_buffer_size).
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 1

typedef enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARGUMENT = 1, /* a check below failed; nothing was launched */
    FA_ERR_UNSUPPORTED = 2,      /* valid but not built (e.g. an unbuilt head_dim) */
    FA_ERR_HIP = 3               /* the HIP runtime reported an error at launch */
} fa_status;

typedef enum {
    FA_DTYPE_F32 = 0, /* Q, K, V, O fp32; fp32 matrix products, P kept in fp32 */
    FA_DTYPE_BF16 = 1 /* Q, K, V, O bf16; fp32 accumulation, P rounded to bf16 */
} fa_dtype;

typedef enum {
    FA_MASK_NONE = 0,
    FA_MASK_ADDITIVE = 1, /* same dtype as Q; added to the scaled score; -inf excludes */
    FA_MASK_BOOL = 2      /* uint8; nonzero = attend (ruDNN `forward`, mask_kind 1) */
} fa_mask_kind;

/*
 * fa_fwd - the forward pass on contiguous head-major tensors.
 *
 *   Q    [B, H_q,  qL, D]   dtype            (read)
 *   K    [B, H_kv, kL, D]   dtype            (read)
 *   V    [B, H_kv, kL, D]   dtype            (read)
 *   mask [B, H_q,  qL, kL]  see fa_mask_kind (read; NULL iff FA_MASK_NONE)
 *   O    [B, H_q,  qL, D]   dtype            (written)
 *   L    [B, H_q,  qL]      fp32             (written)
 *
 * Checks (mlx-native flash_attn_train.rs, validate_params, plus this
 * library's own): B, H_q, H_kv, qL, kL > 0; H_q % H_kv == 0; D in
 * {16, 32, 48, 64, 80, 96, 128, 256}; known dtype and mask kind; mask non-NULL iff a mask kind
 * is given; Q, K, V, O, L non-NULL and 16-byte aligned; scale finite;
 * element counts fit in int64.
 */
fa_status fa_fwd(const void* Q, const void* K, const void* V, const void* mask,
                 void* O, float* L,
                 int B, int H_q, int H_kv, int qL, int kL, int D,
                 float scale, int causal,
                 fa_dtype dtype, fa_mask_kind mask_kind, void* hip_stream);

/*
 * Element strides {batch, head, seq} of each tensor; the D axis (the kL axis
 * for the mask) is always contiguous.  An all-zero triple selects the
 * contiguous head-major default shown for fa_fwd.  A mask stride of 0 on a
 * non-default triple broadcasts that axis (ruDNN dense_attention.rs,
 * mask_offset).  Token-major O ([qL, H_q*D] per batch, the oxibonsai
 * dit_attention_flash.rs output layout) is o = {qL*H_q*D, D, H_q*D}.
 * Q, K, V and O strides must be non-negative multiples of 16 bytes' worth of
 * elements (8 for bf16, 4 for fp32) so rows stay 16-byte aligned; mask
 * strides may be any non-negative value.
 */
typedef struct {
    int64_t q[3];
    int64_t k[3];
    int64_t v[3];
    int64_t o[3];
    int64_t mask[3];
} fa_strides;

/* fa_fwd with explicit strides (NULL = all defaults).  Same checks, plus the
 * stride rules above; L is always contiguous [B, H_q, qL]. */
fa_status fa_fwd_strided(const void* Q, const void* K, const void* V, const void* mask,
                         void* O, float* L,
                         int B, int H_q, int H_kv, int qL, int kL, int D,
                         float scale, int causal,
                         fa_dtype dtype, fa_mask_kind mask_kind,
                         const fa_strides* strides, void* hip_stream);

/*
 * fa_fwd_strided_noalloc - fa_fwd_strided for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc.  Same arguments, checks and results: the
 * same kernels and split plan run, so O and L are bitwise those of
 * fa_fwd_strided.  The fp32 partials of a split key range go to a static
 * scratch array of FA_NOALLOC_SCRATCH_BYTES in the library's device image,
 * one per GPU, held until the process ends.  The split plan never needs more
 * than 65536 * (D + 1) * 4 bytes (33.8 MB at D = 128), so every shape fits;
 * a call that would need more returns FA_ERR_INVALID_ARGUMENT before
 * launching anything.  The first call on a device looks the array up there
 * (hipGetSymbolAddress); no call allocates or calls an allocating routine.
 * Every call on a GPU shares that GPU's scratch and leaves its partials
 * there: calls that overlap on one GPU (on different streams or from
 * different host threads) race, and the caller must serialise them.  Nothing
 * in the scratch needs to start at zero: a launch writes every partial it
 * reads.
 */
#define FA_NOALLOC_SCRATCH_BYTES (36u << 20)
fa_status fa_fwd_strided_noalloc(const void* Q, const void* K, const void* V, const void* mask,
                                 void* O, float* L,
                                 int B, int H_q, int H_kv, int qL, int kL, int D,
                                 float scale, int causal,
                                 fa_dtype dtype, fa_mask_kind mask_kind,
                                 const fa_strides* strides, void* hip_stream);

/*
 * fa_fwd_strided with dropout on the attention weights (ruDNN
 * dense_attention.rs: `keep`, `keep_global` and the dropout branch of
 * `forward_flash`).  Each allowed term of the P V sum is multiplied by
 * k_ij / (1 - p_drop); the softmax denominator, and so L, are those
 * without dropout.  k_ij = 1 when u_ij >= p_drop (never when p_drop = 1),
 * where u_ij = floor(w / 2^8) / 2^24 and w is word (n mod 4) of
 * Philox-4x32-10 (Salmon et al., SC 2011) applied to the 128-bit counter
 * (offset + floor(n / 4) as a 64-bit value, low word first, then two zero
 * words) under the key (seed low word, seed high word), for the score
 * position n = ((b * H_q + h) * qL + i) * kL + j.  The same (seed, offset)
 * reproduces the same mask; a caller drawing several masks advances offset
 * by ceil(B * H_q * qL * kL / 4) between calls.
 * p_drop must lie in [0, 1] (else FA_ERR_INVALID_ARGUMENT).  Built for bf16
 * and fp32 at every D, every mask kind, causal or not (the work-group
 * kernels at each head dim's launch shape; D = 256 never takes the key-split
 * kernel here).  Everything else as fa_fwd_strided.
 */
fa_status fa_fwd_dropout(const void* Q, const void* K, const void* V, const void* mask,
                         void* O, float* L,
                         int B, int H_q, int H_kv, int qL, int kL, int D,
                         float scale, int causal,
                         fa_dtype dtype, fa_mask_kind mask_kind,
                         float p_drop, uint64_t seed, uint64_t offset,
                         const fa_strides* strides, void* hip_stream);

/*
 * fa_fwd_strided restricted to a causal sliding window: query row i attends
 * to keys i - window + 1 .. i (and within them to what the mask allows).
 * The forge flash_attention_mma.metal header carries a `window` field in
 * FlashParams that it routes to kernels it does not show and never defines;
 * this causal-window meaning is the reading taken here.  window >= kL (more
 * generally, >= qL) is plain causal attention.  A row left with no key gets
 * O = 0 and L = 0, as in fa_fwd.
 * window must be >= 1 and causal must be 1 (else FA_ERR_INVALID_ARGUMENT).
 * Built for bf16 and fp32 at every D and mask kind.
 * A windowed launch never splits its key range over work-groups, so it
 * allocates nothing.  Everything else as fa_fwd_strided.
 */
fa_status fa_fwd_window(const void* Q, const void* K, const void* V, const void* mask,
                        void* O, float* L,
                        int B, int H_q, int H_kv, int qL, int kL, int D,
                        float scale, int causal,
                        fa_dtype dtype, fa_mask_kind mask_kind,
                        int window, const fa_strides* strides, void* hip_stream);

/*
 * fa_bwd - the backward pass: gradients dQ, dK, dV of the forward output O
 * for an upstream gradient dO (forge flash_attention_mma.metal, the backward
 * section's header and its dq / dv / dk kernels; mlx-native
 * flash_attn_train.rs, "Phase 2 -- FA-2 backward kernel": compute D, then
 * the backward kernel; ruDNN dense_attention.rs, `backward_kv_owned`).  With
 * P_ij = exp(s_ij - L_i) the forward pass's softmax weights (0 for keys that
 * are not allowed; same rules as fa_fwd):
 *
 *     Delta_i = sum_d dO[i,d] O[i,d]          (written to Delta)
 *     dS_ij   = P_ij (dO_i . V_j - Delta_i)
 *     dQ_i    = scale sum_j dS_ij K_j
 *     dK_j    = scale sum over the query heads of j's kv head and rows i of dS_ij Q_i
 *     dV_j    = sum over the query heads of j's kv head and rows i of P_ij dO_i
 *
 *   Q, O, dO [B, H_q,  qL, D]  dtype   (read; O and L are fa_fwd's outputs
 *   K, V     [B, H_kv, kL, D]  dtype    for the same Q, K, V, mask, scale
 *   L        [B, H_q,  qL]     fp32     and causal)
 *   mask     [B, H_q,  qL, kL] as fa_fwd (read; NULL iff FA_MASK_NONE); no
 *            gradient is formed for it
 *   Delta    [B, H_q,  qL]     fp32    (written: a caller-owned workspace that
 *                                       holds rowsum(dO * O) on return)
 *   dQ       [B, H_q,  qL, D]  dtype   (written)
 *   dK, dV   [B, H_kv, kL, D]  dtype   (written)
 * All tensors are contiguous head-major.  Built for bf16 at D = 64 and 128,
 * every mask kind, causal or not; other valid combinations return
 * FA_ERR_UNSUPPORTED.  Three launches on `hip_stream` (Delta, then dQ, then
 * dK and dV); no atomics, so the result is deterministic.  When the dK/dV
 * grid would leave CUs idle (fewer than 256 work-groups of 128 keys, e.g.
 * B = 2, H_kv = 4, kL = 2048), or is causal with at most 1023 work-groups
 * (its first key tiles see every query tile, e.g. B = 1, H_kv = 8,
 * kL = 8192), each key tile's (query head, query tile) steps are split over
 * up to 16 work-groups (at most 512 in all, 1024 if causal); their fp32
 * partial dK and dV (2 * split * B * H_kv * kL * D * 4 bytes, at most
 * ~134 MB) come from the library's stream-ordered pool (as fa_fwd's split
 * partials) and are summed, in a fixed order, by a fourth launch.
 * Otherwise nothing is allocated.  Checks as fa_fwd, plus dO, Delta, dQ, dK, dV non-NULL and
 * aligned (16 bytes; 4 for L and Delta).
 */
fa_status fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* L,
                 const void* mask, float* Delta, void* dQ, void* dK, void* dV,
                 int B, int H_q, int H_kv, int qL, int kL, int D,
                 float scale, int causal,
                 fa_dtype dtype, fa_mask_kind mask_kind, void* hip_stream);

/* 1 if (dtype, D, mask_kind, causal) has a compiled kernel, else 0. */
int fa_supported(fa_dtype dtype, int D, fa_mask_kind mask_kind, int causal);

/* 1 if fa_bwd has a compiled kernel for (dtype, D, mask_kind, causal), else 0. */
int fa_bwd_supported(fa_dtype dtype, int D, fa_mask_kind mask_kind, int causal);

/* Number of compiled kernel variants -- every (dtype, D, mask kind, causal)
 * of fa_fwd, then of fa_fwd_dropout, then of fa_bwd -- and the name of
 * variant i (NULL past the end); the names are static strings (cf. the
 * kernel-name lists that mlx-native flash_attn_train.rs exposes to its
 * tests). */
int fa_variant_count(void);
const char* fa_variant_name(int i);

/* Static text for a status code. */
const char* fa_status_string(fa_status s);

/* Message of the last non-OK status on the calling thread ("" if none);
 * valid until the next call on that thread. */
const char* fa_last_error(void);

/* FA_ABI_VERSION of the loaded library. */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
