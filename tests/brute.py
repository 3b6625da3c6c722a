"""Pure-Python brute-force attention for tiny shapes (an oracle pin).

Written independently of the C oracle and with a different formula: the
softmax is taken without subtracting the row max, p_ij = exp(s_ij) / sum_j
exp(s_ij) and L_i = ln(sum_j exp(s_ij)), summed with math.fsum.  That is
only safe for small scores, which the tiny pin inputs guarantee (|s| < 50).
Nested lists in, nested lists out; no numpy arithmetic.
"""
import math


def brute_attention(q, k, v, scale, causal=False, mask=None, mask_kind="none"):
    """q[b][h][i][d], k/v[b][g][j][d], mask[b][h][i][j] -> (O[b][h][i][d], L[b][h][i])."""
    B, Hq, qL, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv, kL = len(k[0]), len(k[0][0])
    per_kv = Hq // Hkv
    O = [[[[0.0] * D for _ in range(qL)] for _ in range(Hq)] for _ in range(B)]
    L = [[[0.0] * qL for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h // per_kv
            for i in range(qL):
                weights = []
                for j in range(kL):
                    if causal and j > i:
                        continue
                    s = scale * math.fsum(q[b][h][i][d] * k[b][g][j][d] for d in range(D))
                    if mask_kind == "additive":
                        s = s + mask[b][h][i][j]
                    if mask_kind == "bool" and not mask[b][h][i][j]:
                        continue
                    if s == -math.inf:
                        continue
                    weights.append((j, math.exp(s)))
                if not weights:
                    continue  # O stays 0, L stays 0
                total = math.fsum(w for _, w in weights)
                for d in range(D):
                    O[b][h][i][d] = math.fsum(w * v[b][g][j][d] for j, w in weights) / total
                L[b][h][i] = math.log(total)
    return O, L
