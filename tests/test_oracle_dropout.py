"""Pins of the oracle's dropout (ruDNN dense_attention.rs: `keep`,
`keep_global`, the `dropout` branch of `forward_flash`) and of its generator,
Philox-4x32-10 (Salmon, Moraes, Dror and Shaw, SC 2011).

The generator's exact output stream is pinned against rocRAND in
test_oracle_philox.py; the properties checked here (a bijection per key,
uniform and independent-looking words, full avalanche, the keep rate) are a
second line of defence.  The dropout
semantics are pinned exactly: p = 0 and p = 1, L unchanged, a pure-Python
evaluation of sum_j softmax_ij k_ij / (1 - p) V_j at the oracle's positions
n = ((b*Hq + h)*qL + i)*kL + j, and unbiasedness over seeds.
"""
import math

import numpy as np
import pytest

from oracle import attention_fwd, dropout_multiplier, philox4x32_10

pytestmark = pytest.mark.filterwarnings("ignore")


def _small(seed, B=1, Hq=2, Hkv=1, qL=5, kL=37, D=8):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, Hq, qL, D)), rng.standard_normal((B, Hkv, kL, D)),
            rng.standard_normal((B, Hkv, kL, D)))


def test_p0_is_no_dropout_and_p1_drops_everything():
    q, k, v = _small(1)
    O, L = attention_fwd(q, k, v, scale=0.3)
    O0, L0 = attention_fwd(q, k, v, scale=0.3, dropout_p=0.0, seed=7)
    assert np.array_equal(O0, O) and np.array_equal(L0, L)
    O1, L1 = attention_fwd(q, k, v, scale=0.3, dropout_p=1.0, seed=7)
    assert np.all(O1 == 0) and np.array_equal(L1, L)


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_L_is_unchanged_and_O_matches_a_direct_sum(p):
    q, k, v = _small(2)
    B, Hq, qL, D = q.shape
    kL = k.shape[2]
    seed, offset = 0x1234_5678_9ABC_DEF0, 3
    Od, Ld = attention_fwd(q, k, v, scale=0.3, causal=True, dropout_p=p, seed=seed, offset=offset)
    _, L = attention_fwd(q, k, v, scale=0.3, causal=True)
    assert np.array_equal(Ld, L)
    group = Hq // k.shape[1]
    for b in range(B):
        for h in range(Hq):
            for i in range(qL):
                keys = range(i + 1)  # causal, top-left
                s = [0.3 * float(np.dot(q[b, h, i], k[b, h // group, j])) for j in keys]
                m = max(s)
                w = [math.exp(x - m) for x in s]
                l = math.fsum(w)
                flat = (b * Hq + h) * qL + i
                ref = [math.fsum(w[j] / l * dropout_multiplier(flat * kL + j, p, seed, offset) * v[b, h // group, j, d]
                                 for j in keys) for d in range(D)]
                assert np.max(np.abs(np.array(ref) - Od[b, h, i])) < 1e-12


def test_dropout_is_unbiased_over_seeds():
    q, k, v = _small(3, qL=3, kL=16, D=4)
    O, _ = attention_fwd(q, k, v, scale=0.5)
    draws = np.stack([attention_fwd(q, k, v, scale=0.5, dropout_p=0.3, seed=s)[0] for s in range(3000)])
    mean, sd = draws.mean(0), draws.std(0)
    assert np.all(np.abs(mean - O) <= 5 * sd / math.sqrt(len(draws)) + 1e-12)


@pytest.mark.parametrize("p", [0.05, 0.3, 0.75])
def test_keep_rate_and_values(p):
    n = 200_000
    m = np.array([dropout_multiplier(i, p, seed=99, offset=12345) for i in range(n)])
    assert set(np.unique(m)) <= {0.0, 1.0 / (1.0 - np.float32(p).item())}
    kept = np.mean(m > 0)
    assert abs(kept - (1 - p)) < 5 * math.sqrt(p * (1 - p) / n)


def test_philox_is_a_bijection_with_uniform_words():
    key = (0xDEADBEEF, 0x01234567)
    outs = np.array([philox4x32_10((i, 0, 0, 0), key) for i in range(1 << 15)], dtype=np.uint64)
    assert len({tuple(r) for r in outs.tolist()}) == len(outs)
    u = outs / 2.0 ** 32
    for w in range(4):
        assert abs(u[:, w].mean() - 0.5) < 5 * math.sqrt(1 / 12 / len(u))
        # consecutive counters give uncorrelated words
        assert abs(np.corrcoef(u[:-1, w], u[1:, w])[0, 1]) < 5 / math.sqrt(len(u))
    assert philox4x32_10((1, 0, 0, 0), key) != philox4x32_10((1, 0, 0, 0), (key[0] ^ 1, key[1]))


def test_philox_avalanche():
    rng = np.random.default_rng(5)
    flips = []
    for _ in range(64):
        ctr = [int(x) for x in rng.integers(0, 2 ** 32, 4)]
        key = [int(x) for x in rng.integers(0, 2 ** 32, 2)]
        base = philox4x32_10(ctr, key)
        for bit in range(128):
            c = list(ctr)
            c[bit // 32] ^= 1 << (bit % 32)
            out = philox4x32_10(c, key)
            flips.append(sum(bin(a ^ b).count("1") for a, b in zip(base, out)))
    assert 62 < np.mean(flips) < 66 and min(flips) > 30
