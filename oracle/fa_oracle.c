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

static void one_row(const double* Q, const double* K, const double* V,
                    const double* mask, int mask_kind,
                    int Hq, int Hkv, int qL, int kL, int D, double scale,
                    int causal, int64_t flat, double* s, unsigned char* ok,
                    double* o, double* lse)
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
        const double* v = vbase + j * D;
        for (int d = 0; d < D; ++d) o[d] += p * v[d];
    }
    for (int d = 0; d < D; ++d) o[d] = o[d] / l;
    *lse = m + log(l);
}

int fa_oracle_fwd(const double* Q, const double* K, const double* V,
                  const double* mask, int mask_kind,
                  int B, int Hq, int Hkv, int qL, int kL, int D,
                  double scale, int causal,
                  const int64_t* rows, int64_t nrows,
                  double* O, double* L)
{
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
                        causal, flat, s, ok, O + r * D, L + r);
            }
        }
        free(s);
        free(ok);
    }
    return bad ? -1 : 0;
}
