/*
 * fa_oracle.c - reference attention forward pass, fp64, on the CPU.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker that the GPU kernels
 * are compared against.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load it; the product library never does,
 * and the two share no source, header, table or helper.
 *
 * What it computes is the plain definition of scaled dot-product attention
 * with a softmax over the allowed keys, written out without any tiling,
 * online rescaling or reordering:
 *
 *   for every batch b, query head h and query row i, with kv head
 *   g = floor(h / (Hq / Hkv))   (consecutive query heads share a kv head:
 *   ruDNN dense_attention.rs, `forward`, the `kh` index; forge
 *   flash_attention_mma.metal, the `hkv` index of flash_attn_fwd_mma)
 *
 *     s_ij = scale * sum_d Q[b,h,i,d] * K[b,g,j,d]      (+ mask[b,h,i,j] when
 *            the mask is additive: the score is scaled first, the mask added
 *            after, as in ruDNN `forward`)
 *
 *     j is allowed iff  j <= i when causal (top-left alignment, ruDNN
 *     `forward`: token <= row), the bool mask entry is nonzero (ruDNN
 *     `forward`: mask_kind 1), and s_ij != -inf (ruDNN `forward`: an additive
 *     -inf excludes the score).
 *
 *     m_i = max over allowed j of s_ij
 *     p_ij = exp(s_ij - m_i) for allowed j, 0 otherwise;   l_i = sum_j p_ij
 *     O[b,h,i,:] = sum_j p_ij V[b,g,j,:] / l_i
 *     L[b,h,i]   = m_i + ln(l_i)                (natural-log logsumexp:
 *                  mlx-native flash_attn_train.rs, module doc "Algorithm")
 *
 *   Sliding window (fa_oracle_fwd_window; the forge header's FlashParams
 *   carries a `window` field that it routes elsewhere and never defines, so
 *   this is a reading): with window W >= 1 and causal, key j is allowed only
 *   when additionally i - j < W, i.e. row i sees keys i - W + 1 .. i.
 *
 *   A row with no allowed key gets O = 0 and L = 0 (forge
 *   flash_attention_mma.metal, epilogue of flash_attn_fwd_mma: l = 0 writes
 *   zeros for both).
 *
 * The score row S[i, 0..kL) is materialised in full before the softmax, one
 * query row at a time.  Rows are independent and run in parallel (OpenMP).
 *
 * Layouts (all contiguous, row-major, fp64):
 *   Q [B, Hq, qL, D], K and V [B, Hkv, kL, D], mask [B, Hq, qL, kL] (or NULL),
 *   O [nrows, D], L [nrows] where row r of the output is query row rows[r],
 *   a flat index (b*Hq + h)*qL + i.  rows == NULL means every row in order.
 *
 * mask_kind: 0 none, 1 additive (added to the scaled score), 2 bool (nonzero
 * attends).
 *
 * Returns 0, or -1 when an argument is out of range.
 *
 * Dropout (fa_oracle_fwd_dropout; ruDNN dense_attention.rs, `keep`,
 * `keep_global` and the `dropout` branch of `forward_flash`): each allowed
 * term of the P V sum is multiplied by k_ij / (1 - p), where k_ij = 1 when a
 * uniform u_ij >= p and 0 otherwise (all 0 when p >= 1).  The denominator
 * l_i and hence L are those without dropout.  u_ij comes from the position
 * n = ((b*Hq + h)*qL + i)*kL + j: the Philox-4x32 block cipher with 10
 * rounds (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy
 * as 1, 2, 3", SC 2011) is applied to the 128-bit counter
 * (offset + floor(n / 4), 64-bit, low word first; then two zero words)
 * under the 64-bit key `seed` (low word first); word n mod 4 of the result,
 * w, gives u = floor(w / 2^8) / 2^24.
 * The generator and the position-to-word map are pinned exactly against
 * rocRAND's independent host implementation of Philox-4x32-10 (whole blocks
 * at arbitrary counters and keys, and the word at stream position n with the
 * carry from the low counter word into the high one).
 *
 * Backward pass (fa_oracle_bwd; forge flash_attention_mma.metal, the
 * backward section's header and kernels flash_attn_bwd_dq_mma,
 * flash_attn_bwd_dv_mma and flash_attn_bwd_dk_mma; mlx-native
 * flash_attn_train.rs, "Phase 2 -- FA-2 backward kernel"; ruDNN
 * dense_attention.rs, `backward_kv_owned`): for an upstream gradient dO of
 * the output O, with P_ij the softmax weights of the forward pass (0 for
 * keys that are not allowed), the gradients are the chain rule through
 * O = P V and the row softmax, written out plainly:
 *
 *     dP_ij    = dO_i . V_j
 *     dS_ij    = P_ij (dP_ij - sum_k P_ik dP_ik)     (the softmax Jacobian)
 *     dQ_i     = scale sum_j dS_ij K_j
 *     dK_j     = scale sum_{h in j's group, i} dS_ij Q_i
 *     dV_j     = sum_{h in j's group, i} P_ij dO_i
 *
 * The row sum sum_k P_ik dP_ik is taken from the weights themselves (the
 * definition), not through the identity rowsum(dO_i * O_i) the kernels use.
 * A row with no allowed key contributes nothing.  The mask is an input
 * constant: no gradient is formed for it.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int fa_oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* One Philox-4x32 round function, then the key schedule, 10 times: the
 * two 32x32 -> 64-bit products of words 0 and 2 with the round multipliers
 * are spread over the four words as (hi(c2 M1) ^ c1 ^ k0, lo(c2 M1),
 * hi(c0 M0) ^ c3 ^ k1, lo(c0 M0)); the key words advance by the Weyl
 * increments (the golden ratio and sqrt(3) - 1, as 32-bit fractions). */
void fa_oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    const uint64_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        const uint64_t p0 = M0 * (uint64_t)c0;
        const uint64_t p1 = M1 * (uint64_t)c2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n1 = (uint32_t)p1;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        const uint32_t n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += W0;
        k1 += W1;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* k_n / (1 - p) for score position n (see the header): 0 or 1 / (1 - p). */
double fa_oracle_dropout_multiplier(int64_t n, float p, uint64_t seed, uint64_t offset)
{
    if (!(p < 1.0f)) return 0.0;
    const uint64_t ctr64 = offset + (uint64_t)(n / 4);
    const uint32_t ctr[4] = {(uint32_t)ctr64, (uint32_t)(ctr64 >> 32), 0u, 0u};
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t w[4];
    fa_oracle_philox4x32_10(ctr, key, w);
    const double u = (double)(w[n % 4] >> 8) / 16777216.0;
    return (u >= (double)p) ? 1.0 / (1.0 - (double)p) : 0.0;
}

typedef struct {
    int on;
    float p;
    uint64_t seed, offset;
} dropout_t;

static void one_row(const double* Q, const double* K, const double* V,
                    const double* mask, int mask_kind,
                    int Hq, int Hkv, int qL, int kL, int D, double scale,
                    int causal, int window, int64_t flat, double* s, unsigned char* ok,
                    double* o, double* lse, const dropout_t* drop)
{
    const int64_t i = flat % qL;
    const int64_t bh = flat / qL;
    const int64_t h = bh % Hq;
    const int64_t b = bh / Hq;
    const int64_t group = Hq / Hkv;
    const int64_t g = h / group;
    const double* q = Q + flat * D;
    const double* kbase = K + (b * Hkv + g) * (int64_t)kL * D;
    const double* vbase = V + (b * Hkv + g) * (int64_t)kL * D;
    const double* mrow = mask ? mask + flat * (int64_t)kL : NULL;

    /* 1. the score row, in full */
    for (int64_t j = 0; j < kL; ++j) {
        const double* k = kbase + j * D;
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += q[d] * k[d];
        double sc = scale * dot;
        int allowed = 1;
        if (causal && j > i) allowed = 0;
        if (window > 0 && i - j >= window) allowed = 0;
        if (mask_kind == 1) sc = sc + mrow[j];
        if (mask_kind == 2 && mrow[j] == 0.0) allowed = 0;
        if (sc == -INFINITY) allowed = 0;
        s[j] = sc;
        ok[j] = (unsigned char)allowed;
    }

    /* 2. the row max over the allowed keys */
    double m = -INFINITY;
    int64_t n_allowed = 0;
    for (int64_t j = 0; j < kL; ++j)
        if (ok[j]) {
            if (s[j] > m) m = s[j];
            ++n_allowed;
        }

    for (int d = 0; d < D; ++d) o[d] = 0.0;
    if (n_allowed == 0) {
        *lse = 0.0;
        return;
    }

    /* 3. p = exp(s - m), l = sum p, O = sum p V / l */
    double l = 0.0;
    for (int64_t j = 0; j < kL; ++j) {
        if (!ok[j]) continue;
        const double p = exp(s[j] - m);
        l += p;
        const double pv = drop->on ? p * fa_oracle_dropout_multiplier(flat * kL + j, drop->p, drop->seed,
                                                                      drop->offset)
                                   : p;
        const double* v = vbase + j * D;
        for (int d = 0; d < D; ++d) o[d] += pv * v[d];
    }
    for (int d = 0; d < D; ++d) o[d] = o[d] / l;
    *lse = m + log(l);
}

static int run_rows(const double* Q, const double* K, const double* V,
                    const double* mask, int mask_kind,
                    int B, int Hq, int Hkv, int qL, int kL, int D,
                    double scale, int causal, int window,
                    const int64_t* rows, int64_t nrows,
                    double* O, double* L, const dropout_t* drop)
{
    if (window < 0 || (window > 0 && !causal)) return -1;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || qL <= 0 || kL <= 0 || D <= 0) return -1;
    if (Hq % Hkv != 0) return -1;
    if (mask_kind < 0 || mask_kind > 2) return -1;
    if ((mask_kind != 0) != (mask != NULL)) return -1;
    const int64_t total = (int64_t)B * Hq * qL;
    if (rows == NULL) nrows = total;
    for (int64_t r = 0; r < nrows && rows; ++r)
        if (rows[r] < 0 || rows[r] >= total) return -1;

    int bad = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)kL);
        unsigned char* ok = (unsigned char*)malloc((size_t)kL);
        if (!s || !ok) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t r = 0; r < nrows; ++r) {
                const int64_t flat = rows ? rows[r] : r;
                one_row(Q, K, V, mask, mask_kind, Hq, Hkv, qL, kL, D, scale,
                        causal, window, flat, s, ok, O + r * D, L + r, drop);
            }
        }
        free(s);
        free(ok);
    }
    return bad ? -1 : 0;
}

int fa_oracle_fwd(const double* Q, const double* K, const double* V,
                  const double* mask, int mask_kind,
                  int B, int Hq, int Hkv, int qL, int kL, int D,
                  double scale, int causal,
                  const int64_t* rows, int64_t nrows,
                  double* O, double* L)
{
    const dropout_t none = {0, 0.0f, 0, 0};
    return run_rows(Q, K, V, mask, mask_kind, B, Hq, Hkv, qL, kL, D, scale, causal, 0, rows, nrows, O, L, &none);
}

/* fa_oracle_fwd restricted to a causal sliding window of `window` >= 1 keys
 * (see the header); returns -1 unless causal. */
int fa_oracle_fwd_window(const double* Q, const double* K, const double* V,
                         const double* mask, int mask_kind,
                         int B, int Hq, int Hkv, int qL, int kL, int D,
                         double scale, int causal,
                         const int64_t* rows, int64_t nrows,
                         double* O, double* L, int window)
{
    if (window < 1) return -1;
    const dropout_t none = {0, 0.0f, 0, 0};
    return run_rows(Q, K, V, mask, mask_kind, B, Hq, Hkv, qL, kL, D, scale, causal, window, rows, nrows, O, L,
                    &none);
}

/* fa_oracle_fwd with dropout of rate p (0 <= p <= 1) under `seed` and
 * counter `offset` (see the header). */
int fa_oracle_fwd_dropout(const double* Q, const double* K, const double* V,
                          const double* mask, int mask_kind,
                          int B, int Hq, int Hkv, int qL, int kL, int D,
                          double scale, int causal,
                          const int64_t* rows, int64_t nrows,
                          double* O, double* L,
                          float p, uint64_t seed, uint64_t offset)
{
    if (!(p >= 0.0f && p <= 1.0f)) return -1;
    const dropout_t drop = {1, p, seed, offset};
    return run_rows(Q, K, V, mask, mask_kind, B, Hq, Hkv, qL, kL, D, scale, causal, 0, rows, nrows, O, L, &drop);
}

/* ------------------------------------------------------------------ backward */

/* The score s_ij and whether key j is allowed for query row `flat` (the same
 * rules as one_row: causal top-left, bool mask, additive mask, -inf). */
static double score_of(const double* Q, const double* K, const double* mask, int mask_kind,
                       int Hq, int Hkv, int qL, int kL, int D, double scale, int causal,
                       int64_t flat, int64_t j, int* allowed)
{
    const int64_t i = flat % qL;
    const int64_t bh = flat / qL;
    const int64_t head = bh % Hq;
    const int64_t b = bh / Hq;
    const int64_t g = head / (Hq / Hkv);
    /* keys excluded by position or by the bool mask need no score */
    if ((causal && j > i) || (mask_kind == 2 && mask[flat * (int64_t)kL + j] == 0.0)) {
        *allowed = 0;
        return -INFINITY;
    }
    const double* qrow = Q + flat * D;
    const double* krow = K + ((b * Hkv + g) * (int64_t)kL + j) * D;
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += qrow[d] * krow[d];
    double score = scale * dot;
    if (mask_kind == 1) score = score + mask[flat * (int64_t)kL + j];
    *allowed = score != -INFINITY;
    return score;
}

/* dP_ij = dO_i . V_j */
static double dp_of(const double* dO, const double* V, int Hq, int Hkv, int qL, int kL, int D,
                    int64_t flat, int64_t j)
{
    const int64_t bh = flat / qL;
    const int64_t head = bh % Hq;
    const int64_t b = bh / Hq;
    const int64_t g = head / (Hq / Hkv);
    const double* go = dO + flat * D;
    const double* v = V + ((b * Hkv + g) * (int64_t)kL + j) * D;
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += go[d] * v[d];
    return dot;
}

/*
 * fa_oracle_bwd - dQ, dK, dV of attention (see the header), fp64.
 *
 * Q, dO [B, Hq, qL, D]; K, V [B, Hkv, kL, D]; mask [B, Hq, qL, kL] or NULL.
 * qrows: flat query rows (b*Hq + h)*qL + i whose dQ is wanted (NULL = all,
 * in order), nq of them; dQ is [nq, D].
 * krows: flat key rows (b*Hkv + g)*kL + j whose dK and dV are wanted (NULL =
 * all), nk of them; dK and dV are [nk, D].
 * Returns 0, or -1 when an argument is out of range.
 */
int fa_oracle_bwd(const double* Q, const double* K, const double* V, const double* dO,
                  const double* mask, int mask_kind,
                  int B, int Hq, int Hkv, int qL, int kL, int D,
                  double scale, int causal,
                  const int64_t* qrows, int64_t nq, const int64_t* krows, int64_t nk,
                  double* dQ, double* dK, double* dV)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || qL <= 0 || kL <= 0 || D <= 0) return -1;
    if (Hq % Hkv != 0) return -1;
    if (mask_kind < 0 || mask_kind > 2) return -1;
    if ((mask_kind != 0) != (mask != NULL)) return -1;
    const int64_t total_q = (int64_t)B * Hq * qL;
    const int64_t total_k = (int64_t)B * Hkv * kL;
    if (qrows == NULL) nq = total_q;
    if (krows == NULL) nk = total_k;
    for (int64_t r = 0; r < nq && qrows; ++r)
        if (qrows[r] < 0 || qrows[r] >= total_q) return -1;
    for (int64_t r = 0; r < nk && krows; ++r)
        if (krows[r] < 0 || krows[r] >= total_k) return -1;

    /* 1. per query row: the softmax normaliser (as m and l) and the row sum
     *    sum_k P_ik dP_ik, over the allowed keys */
    double* row_m = (double*)malloc(sizeof(double) * (size_t)total_q);
    double* row_l = (double*)malloc(sizeof(double) * (size_t)total_q);
    double* row_pdp = (double*)malloc(sizeof(double) * (size_t)total_q);
    if (!row_m || !row_l || !row_pdp) {
        free(row_m);
        free(row_l);
        free(row_pdp);
        return -1;
    }
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t r = 0; r < total_q; ++r) {
        double m = -INFINITY;
        for (int64_t j = 0; j < kL; ++j) {
            int ok;
            const double sc = score_of(Q, K, mask, mask_kind, Hq, Hkv, qL, kL, D, scale, causal, r, j, &ok);
            if (ok && sc > m) m = sc;
        }
        double l = 0.0, pdp = 0.0;
        if (m != -INFINITY) {
            for (int64_t j = 0; j < kL; ++j) {
                int ok;
                const double sc = score_of(Q, K, mask, mask_kind, Hq, Hkv, qL, kL, D, scale, causal, r, j, &ok);
                if (!ok) continue;
                const double e = exp(sc - m);
                l += e;
                pdp += e * dp_of(dO, V, Hq, Hkv, qL, kL, D, r, j);
            }
            pdp /= l;
        }
        row_m[r] = m;
        row_l[r] = l;
        row_pdp[r] = pdp;
    }

    /* 2. dQ_i = scale sum_j dS_ij K_j */
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t r = 0; r < nq; ++r) {
        const int64_t flat = qrows ? qrows[r] : r;
        const int64_t bh = flat / qL;
        const int64_t b = bh / Hq;
        const int64_t g = (bh % Hq) / (Hq / Hkv);
        double* out = dQ + r * D;
        for (int d = 0; d < D; ++d) out[d] = 0.0;
        if (row_m[flat] == -INFINITY) continue;
        for (int64_t j = 0; j < kL; ++j) {
            int ok;
            const double sc = score_of(Q, K, mask, mask_kind, Hq, Hkv, qL, kL, D, scale, causal, flat, j, &ok);
            if (!ok) continue;
            const double p = exp(sc - row_m[flat]) / row_l[flat];
            const double ds = p * (dp_of(dO, V, Hq, Hkv, qL, kL, D, flat, j) - row_pdp[flat]);
            const double* k = K + ((b * Hkv + g) * (int64_t)kL + j) * D;
            for (int d = 0; d < D; ++d) out[d] += scale * ds * k[d];
        }
    }

    /* 3. dK_j and dV_j: every query row of every head of key j's group */
    const int64_t group = Hq / Hkv;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t r = 0; r < nk; ++r) {
        const int64_t flat = krows ? krows[r] : r;
        const int64_t j = flat % kL;
        const int64_t bg = flat / kL;
        const int64_t g = bg % Hkv;
        const int64_t b = bg / Hkv;
        double* gk = dK + r * D;
        double* gv = dV + r * D;
        for (int d = 0; d < D; ++d) gk[d] = gv[d] = 0.0;
        for (int64_t h = g * group; h < (g + 1) * group; ++h)
            for (int64_t i = 0; i < qL; ++i) {
                const int64_t qf = (b * Hq + h) * qL + i;
                if (row_m[qf] == -INFINITY) continue;
                int ok;
                const double sc = score_of(Q, K, mask, mask_kind, Hq, Hkv, qL, kL, D, scale, causal, qf, j, &ok);
                if (!ok) continue;
                const double p = exp(sc - row_m[qf]) / row_l[qf];
                const double ds = p * (dp_of(dO, V, Hq, Hkv, qL, kL, D, qf, j) - row_pdp[qf]);
                const double* q = Q + qf * D;
                const double* go = dO + qf * D;
                for (int d = 0; d < D; ++d) {
                    gk[d] += scale * ds * q[d];
                    gv[d] += p * go[d];
                }
            }
    }
    free(row_m);
    free(row_l);
    free(row_pdp);
    return 0;
}
