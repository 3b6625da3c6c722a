"""Pins of the oracle's backward pass (fa_oracle_bwd): dQ, dK, dV of attention.

What pins it, independently of how it is written:
  * central finite differences of the forward oracle (itself pinned) on the
    scalar loss sum(O * dO), for every element of Q, K and V of tiny shapes,
    under every mask kind, causal and GQA;
  * torch's float64 autograd through softmax(scale Q K^T + mask) V, a library
    routine sharing nothing with the oracle;
  * closed forms and invariants: a row that allows one key passes its dO to
    that key's dV and no gradient to Q or K; dK summed over a head's keys is 0
    (each row's dS sums to 0); GQA gradients are MHA gradients with K, V
    repeated and dK, dV summed over each group; an additive row shift changes
    nothing; a row with no allowed key contributes nothing;
  * requested row subsets equal the full computation.
Planted mistakes in copies of the oracle (test at the end) must fail a pin.
"""
import numpy as np
import pytest
import torch

from oracle import OracleLib, attention_bwd, attention_fwd

RNG_SHAPES = [
    # B, Hq, Hkv, qL, kL, D, causal, mask_kind
    (1, 2, 1, 6, 9, 5, False, "none"),
    (1, 2, 1, 7, 7, 4, True, "none"),
    (2, 2, 2, 5, 8, 3, True, "additive"),
    (1, 4, 2, 6, 5, 4, False, "bool"),
]


def _inputs(B, Hq, Hkv, qL, kL, D, mask_kind, seed, p_masked=0.3):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, qL, D))
    k = rng.standard_normal((B, Hkv, kL, D))
    v = rng.standard_normal((B, Hkv, kL, D))
    do = rng.standard_normal((B, Hq, qL, D))
    mask = None
    if mask_kind != "none":
        masked = rng.random((B, Hq, qL, kL)) < p_masked
        masked[..., 0] = False  # every row keeps key 0
        if mask_kind == "bool":
            mask = (~masked).astype(np.uint8)
        else:
            mask = np.where(masked, -np.inf, rng.standard_normal(masked.shape))
    return q, k, v, do, mask


def _fd_check(bwd, fwd, shape, seed, eps=1e-6):
    B, Hq, Hkv, qL, kL, D, causal, kind = shape
    q, k, v, do, mask = _inputs(B, Hq, Hkv, qL, kL, D, kind, seed)
    scale = 0.7
    dq, dk, dv = bwd(q, k, v, do, scale=scale, causal=causal, mask=mask, mask_kind=kind)

    def loss(qq, kk, vv):
        O, _ = fwd(qq, kk, vv, scale=scale, causal=causal, mask=mask, mask_kind=kind)
        return float(np.sum(O * do))

    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + eps
            up = loss(q, k, v)
            x[idx] = old - eps
            dn = loss(q, k, v)
            x[idx] = old
            num[idx] = (up - dn) / (2 * eps)
        assert np.max(np.abs(num - g)) <= 1e-6 * max(1.0, np.max(np.abs(num))), (shape, np.max(np.abs(num - g)))


def _torch_ref(q, k, v, do, scale, causal, mask, kind):
    Q, K, V = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    grp = q.shape[1] // k.shape[1]
    Kr, Vr = K.repeat_interleave(grp, dim=1), V.repeat_interleave(grp, dim=1)
    s = scale * torch.matmul(Q, Kr.transpose(-1, -2).contiguous())
    qL, kL = q.shape[2], k.shape[2]
    allowed = torch.ones((qL, kL), dtype=torch.bool)
    if causal:
        allowed = allowed.tril()
    allowed = allowed.expand(s.shape)
    if kind == "additive":
        s = s + torch.tensor(mask)
    elif kind == "bool":
        allowed = allowed & torch.tensor(mask != 0)
    s = s.masked_fill(~allowed, float("-inf"))
    O = torch.matmul(torch.softmax(s, dim=-1), Vr)
    (O * torch.tensor(do)).sum().backward()
    return Q.grad.numpy(), K.grad.numpy(), V.grad.numpy()


def _autograd_check(bwd, shape, seed):
    B, Hq, Hkv, qL, kL, D, causal, kind = shape
    q, k, v, do, mask = _inputs(B, Hq, Hkv, qL, kL, D, kind, seed)
    got = bwd(q, k, v, do, scale=0.3, causal=causal, mask=mask, mask_kind=kind)
    ref = _torch_ref(q, k, v, do, 0.3, causal, mask, kind)
    for g, r in zip(got, ref):
        assert np.max(np.abs(g - r)) <= 1e-11 * max(1.0, np.max(np.abs(r)))


# ---- the pins, each taking the oracle's bwd (and fwd) callables ----

def pin_finite_differences(bwd, fwd):
    for n, shape in enumerate(RNG_SHAPES):
        _fd_check(bwd, fwd, shape, seed=100 + n)


def pin_torch_autograd(bwd, fwd):
    for n, shape in enumerate([(1, 4, 2, 33, 47, 16, False, "none"), (2, 4, 1, 40, 40, 8, True, "none"),
                               (1, 2, 2, 31, 50, 16, True, "additive"), (1, 6, 3, 29, 17, 8, False, "bool")]):
        _autograd_check(bwd, shape, seed=200 + n)


def pin_single_allowed_key(bwd, fwd):
    """A row whose mask allows only key j* has P = 1 there: dS = 0, so it adds
    nothing to dQ or dK, and its dO goes to dV_{j*} whole."""
    B, Hq, Hkv, qL, kL, D = 1, 2, 1, 5, 6, 4
    q, k, v, do, _ = _inputs(B, Hq, Hkv, qL, kL, D, "none", 300)
    jstar = np.array([[3, 1, 3, 0, 5], [2, 2, 4, 0, 1]])
    mask = np.zeros((B, Hq, qL, kL), dtype=np.uint8)
    for h in range(Hq):
        for i in range(qL):
            mask[0, h, i, jstar[h, i]] = 1
    dq, dk, dv = bwd(q, k, v, do, scale=0.9, mask=mask, mask_kind="bool")
    assert np.max(np.abs(dq)) < 1e-13 and np.max(np.abs(dk)) < 1e-13
    ref = np.zeros_like(dv)
    for h in range(Hq):
        for i in range(qL):
            ref[0, 0, jstar[h, i]] += do[0, h, i]
    assert np.max(np.abs(dv - ref)) < 1e-13


def pin_dk_sums_to_zero(bwd, fwd):
    """Each row's dS sums to 0 over its keys, so sum_j dK_j = 0 per kv head."""
    q, k, v, do, mask = _inputs(2, 4, 2, 23, 31, 8, "additive", 301)
    for causal in (False, True):
        _, dk, _ = bwd(q, k, v, do, scale=0.5, causal=causal, mask=mask, mask_kind="additive")
        assert np.max(np.abs(dk.sum(axis=2))) < 1e-12 * max(1.0, np.max(np.abs(dk)))


def pin_gqa_is_summed_mha(bwd, fwd):
    q, k, v, do, _ = _inputs(1, 6, 2, 17, 19, 8, "none", 302)
    dq, dk, dv = bwd(q, k, v, do, scale=0.4, causal=True)
    dq2, dk2, dv2 = bwd(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), do, scale=0.4, causal=True)
    assert np.max(np.abs(dq - dq2)) < 1e-12
    assert np.max(np.abs(dk - dk2.reshape(1, 2, 3, 19, 8).sum(2))) < 1e-12
    assert np.max(np.abs(dv - dv2.reshape(1, 2, 3, 19, 8).sum(2))) < 1e-12


def pin_row_shift_changes_nothing(bwd, fwd):
    q, k, v, do, mask = _inputs(1, 2, 1, 9, 12, 4, "additive", 303)
    shift = np.random.default_rng(1).standard_normal((1, 2, 9, 1)) * 5
    a = bwd(q, k, v, do, scale=0.6, mask=mask, mask_kind="additive")
    b = bwd(q, k, v, do, scale=0.6, mask=mask + shift, mask_kind="additive")
    for x, y in zip(a, b):
        assert np.max(np.abs(x - y)) < 1e-11


def pin_empty_rows_contribute_nothing(bwd, fwd):
    q, k, v, do, _ = _inputs(1, 2, 1, 6, 7, 4, "none", 304)
    mask = np.ones((1, 2, 6, 7), dtype=np.uint8)
    mask[0, 1, 3] = 0  # row 3 of head 1 allows no key
    dq, dk, dv = bwd(q, k, v, do, scale=0.8, mask=mask, mask_kind="bool")
    assert np.all(dq[0, 1, 3] == 0)
    do2 = do.copy()
    do2[0, 1, 3] = 123.0
    _, dk2, dv2 = bwd(q, k, v, do2, scale=0.8, mask=mask, mask_kind="bool")
    assert np.array_equal(dk, dk2) and np.array_equal(dv, dv2)


def pin_row_subsets(bwd, fwd):
    q, k, v, do, mask = _inputs(2, 4, 2, 13, 15, 8, "bool", 305)
    dq, dk, dv = bwd(q, k, v, do, scale=0.5, causal=True, mask=mask, mask_kind="bool")
    qrows = np.array([0, 5, 12, 13, 50, 103])
    krows = np.array([0, 1, 14, 15, 33, 59])
    sq, sk, sv = bwd(q, k, v, do, scale=0.5, causal=True, mask=mask, mask_kind="bool", qrows=qrows, krows=krows)
    assert np.array_equal(sq, dq.reshape(-1, 8)[qrows])
    assert np.array_equal(sk, dk.reshape(-1, 8)[krows]) and np.array_equal(sv, dv.reshape(-1, 8)[krows])


ALL_BWD_PINS = [pin_finite_differences, pin_torch_autograd, pin_single_allowed_key, pin_dk_sums_to_zero,
                pin_gqa_is_summed_mha, pin_row_shift_changes_nothing, pin_empty_rows_contribute_nothing,
                pin_row_subsets]


@pytest.mark.parametrize("pin", ALL_BWD_PINS, ids=lambda f: f.__name__)
def test_bwd_pin(pin):
    pin(attention_bwd, attention_fwd)


BWD_MUTANTS = {
    "softmax_row_sum_not_subtracted": (
        "const double ds = p * (dp_of(dO, V, Hq, Hkv, qL, kL, D, flat, j) - row_pdp[flat]);",
        "const double ds = p * dp_of(dO, V, Hq, Hkv, qL, kL, D, flat, j);"),
    "row_sum_not_normalised": ("            pdp /= l;\n", "\n"),
    "dk_unscaled": ("gk[d] += scale * ds * q[d];", "gk[d] += ds * q[d];"),
    "dv_takes_ds": ("gv[d] += p * go[d];", "gv[d] += ds * go[d];"),
    "dq_sums_v": ("            const double* k = K + ((b * Hkv + g) * (int64_t)kL + j) * D;\n"
                  "            for (int d = 0; d < D; ++d) out[d] += scale * ds * k[d];",
                  "            const double* k = V + ((b * Hkv + g) * (int64_t)kL + j) * D;\n"
                  "            for (int d = 0; d < D; ++d) out[d] += scale * ds * k[d];"),
    "causal_off_by_one": ("if ((causal && j > i) || (mask_kind == 2", "if ((causal && j >= i) || (mask_kind == 2"),
    "group_one_head": ("for (int64_t h = g * group; h < (g + 1) * group; ++h)", "for (int64_t h = g; h < g + 1; ++h)"),
    "mask_subtracted": ("if (mask_kind == 1) score = score + mask[flat * (int64_t)kL + j];",
                        "if (mask_kind == 1) score = score - mask[flat * (int64_t)kL + j];"),
    "dq_sign": ("for (int d = 0; d < D; ++d) out[d] += scale * ds * k[d];",
                "for (int d = 0; d < D; ++d) out[d] -= scale * ds * k[d];"),
}


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_bwd_mutant_is_caught(tmp_path, name):
    from test_oracle_mutants import _build_mutant

    old, new = BWD_MUTANTS[name]
    lib = OracleLib(_build_mutant(str(tmp_path), name, old, new))
    caught = []
    for pin in ALL_BWD_PINS:
        try:
            pin(lib.bwd, attention_fwd)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
