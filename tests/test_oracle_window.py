"""Pins of the oracle's causal sliding window (row i sees keys i - W + 1 .. i).

The pages carry a `window` field without defining it (the forge header routes
window > 0 to kernels it does not show); the reading taken is the causal
sliding window.  These tests pin that reading against closed forms, plain
causal attention, and a brute-force softmax written here over the band.
"""
import math

import numpy as np
import pytest

from oracle import attention_fwd


def draw(seed, B=1, Hq=4, Hkv=2, qL=23, kL=29, D=16):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, qL, D))
    k = rng.standard_normal((B, Hkv, kL, D))
    v = rng.standard_normal((B, Hkv, kL, D))
    return q, k, v


def brute(q, k, v, scale, window, allow=None):
    """Softmax over the band max(0, i - W + 1) .. min(i, kL - 1), one row at a time, with fsum."""
    B, Hq, qL, D = q.shape
    Hkv, kL = k.shape[1], k.shape[2]
    O = np.zeros((B, Hq, qL, D))
    L = np.zeros((B, Hq, qL))
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            for i in range(qL):
                js = [j for j in range(max(0, i - window + 1), min(i, kL - 1) + 1)
                      if allow is None or allow[b, h, i, j]]
                if not js:
                    continue
                s = [scale * math.fsum(q[b, h, i] * k[b, g, j]) for j in js]
                m = max(s)
                p = [math.exp(x - m) for x in s]
                l = math.fsum(p)
                for d in range(D):
                    O[b, h, i, d] = math.fsum(pj * v[b, g, j, d] for pj, j in zip(p, js)) / l
                L[b, h, i] = m + math.log(l)
    return O, L


@pytest.mark.parametrize("qL,kL", [(23, 29), (29, 23), (16, 16)])
def test_a_window_wider_than_every_row_is_plain_causal(qL, kL):
    q, k, v = draw(1, qL=qL, kL=kL)
    O0, L0 = attention_fwd(q, k, v, scale=0.25, causal=True)
    for w in (qL, qL + 5, 1 << 20):
        O, L = attention_fwd(q, k, v, scale=0.25, causal=True, window=w)
        assert np.array_equal(O, O0) and np.array_equal(L, L0)


def test_rows_inside_the_window_match_plain_causal():
    q, k, v = draw(2)
    W = 7
    O0, L0 = attention_fwd(q, k, v, scale=0.25, causal=True)
    O, L = attention_fwd(q, k, v, scale=0.25, causal=True, window=W)
    assert np.array_equal(O[:, :, :W], O0[:, :, :W]) and np.array_equal(L[:, :, :W], L0[:, :, :W])
    assert not np.allclose(O[:, :, W:], O0[:, :, W:])


def test_window_of_one_is_the_diagonal():
    q, k, v = draw(3, Hq=2, Hkv=1, qL=12, kL=12)
    scale = 0.4
    O, L = attention_fwd(q, k, v, scale=scale, causal=True, window=1)
    assert np.array_equal(O[0, :], np.broadcast_to(v[0, 0], O[0].shape))
    closed = scale * np.einsum("hid,id->hi", q[0], k[0, 0])
    np.testing.assert_allclose(L[0], closed, rtol=0, atol=1e-13)


def test_window_of_one_past_the_keys_is_empty():
    # rows i >= kL see no key in a window of one: O = 0 and L = 0
    q, k, v = draw(4, Hq=2, Hkv=2, qL=10, kL=6)
    O, L = attention_fwd(q, k, v, scale=0.3, causal=True, window=1)
    assert np.all(O[:, :, 6:] == 0) and np.all(L[:, :, 6:] == 0)
    assert np.all(L[:, :, :6] != 0)


@pytest.mark.parametrize("W", [2, 3, 5, 11])
def test_matches_brute_force_over_the_band(W):
    q, k, v = draw(10 + W)
    O, L = attention_fwd(q, k, v, scale=0.3, causal=True, window=W)
    Ob, Lb = brute(q, k, v, 0.3, W)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, Lb, rtol=0, atol=1e-12)


def test_window_combines_with_a_bool_mask():
    q, k, v = draw(5)
    rng = np.random.default_rng(6)
    allow = rng.random((1, 4, 23, 29)) < 0.6
    O, L = attention_fwd(q, k, v, scale=0.3, causal=True, window=4, mask=allow.astype(np.uint8),
                         mask_kind="bool")
    Ob, Lb = brute(q, k, v, 0.3, 4, allow=allow)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, Lb, rtol=0, atol=1e-12)


@pytest.mark.parametrize("kw", [dict(causal=False, window=4), dict(causal=True, window=0),
                                dict(causal=True, window=-3)])
def test_rejects_windows_outside_the_reading(kw):
    q, k, v = draw(7)
    with pytest.raises(ValueError):
        attention_fwd(q, k, v, scale=0.3, **kw)


@pytest.mark.parametrize("qL,kL,W", [(10, 6, 3), (17, 17, 5), (8, 20, 100), (33, 12, 1)])
def test_workload_flop_count_is_the_allowed_pair_count(qL, kL, W):
    """The benchmark's FLOP figure for a windowed workload: 4 D per allowed
    (row, key) pair, counted here one pair at a time."""
    import workloads as Wl
    w = Wl.WINDOW[0].with_(B=1, Hq=1, Hkv=1, qL=qL, kL=kL, D=1, window=W)
    pairs = sum(1 for i in range(qL) for j in range(kL) if j <= i and i - j < W)
    assert w.flops() == 4.0 * pairs
