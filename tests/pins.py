"""Pins for the fp64 oracle: checks against what the mathematics fixes.

Each pin takes an attention callable with the oracle's signature
fwd(q, k, v, *, scale, causal, mask, mask_kind, rows) -> (O, L) and raises
AssertionError if the callable disagrees with a closed form, an invariant, a
brute-force loop or a library routine.  The same pins run against the real
oracle (all must pass) and against copies of it with planted mistakes (at
least one must fail), so a pin that cannot tell right from wrong shows up.

Definition being pinned (see oracle/fa_oracle.c): s = scale*Q.K^T (+ additive
mask), softmax over the allowed keys (causal j <= i, bool mask nonzero,
s != -inf), O = P.V, L = natural-log logsumexp of the allowed scores, and
O = 0, L = 0 for a row with no allowed key.
"""
import math

import numpy as np
import torch

from brute import brute_attention

TOL = 1e-12


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert np.all(np.isfinite(a)) == np.all(np.isfinite(b)), f"{what}: finiteness differs"
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


def _rng(seed):
    return np.random.default_rng(seed)


def pin_zero_query(fwd):
    """Q = 0 makes every score 0: L_i = ln|A_i|, O_i = mean of V over A_i."""
    r = _rng(1)
    B, H, qL, kL, D = 1, 2, 5, 7, 4
    q = np.zeros((B, H, qL, D))
    k = r.standard_normal((B, H, kL, D))
    v = r.standard_normal((B, H, kL, D))
    O, L = fwd(q, k, v, scale=0.7)
    _close(L, np.full((B, H, qL), math.log(kL)), what="zero-Q L (non-causal)")
    _close(O, np.broadcast_to(v.mean(axis=2, keepdims=True), O.shape), what="zero-Q O")
    # causal: row i sees keys 0..i
    O, L = fwd(q, k, v, scale=0.7, causal=True)
    for i in range(qL):
        _close(L[:, :, i], np.full((B, H), math.log(i + 1)), what=f"zero-Q causal L row {i}")
        _close(O[:, :, i], v[:, :, : i + 1].mean(axis=2), what=f"zero-Q causal O row {i}")
    # with an additive mask m: L_i = ln sum_j exp(m_ij), O_i = softmax(m_i) . V
    m = r.standard_normal((B, H, qL, kL))
    O, L = fwd(q, k, v, scale=0.7, mask=m, mask_kind="additive")
    for b in range(B):
        for h in range(H):
            for i in range(qL):
                w = [math.exp(x) for x in m[b, h, i]]
                tot = math.fsum(w)
                _close(L[b, h, i], math.log(tot), what="zero-Q masked L")
                exp_o = [math.fsum(w[j] * v[b, h, j, d] for j in range(kL)) / tot for d in range(D)]
                _close(O[b, h, i], exp_o, what="zero-Q masked O")


def pin_dominant_key(fwd):
    """One key aligned with the query: L = ln(e^sig + n - 1), O = (e^sig V* + sum_other V)/(e^sig + n - 1)."""
    r = _rng(2)
    kL, D, jstar = 9, 8, 5
    for alpha, beta, scale in ((2.0, 1.5, 0.5), (10.0, 3.0, 1.0), (40.0, 2.0, 0.25)):
        q = np.zeros((1, 1, 3, D))
        q[..., 0] = alpha
        k = r.standard_normal((1, 1, kL, D))
        k[..., 0] = 0.0
        k[0, 0, jstar] = 0.0
        k[0, 0, jstar, 0] = beta
        v = r.standard_normal((1, 1, kL, D))
        sig = scale * alpha * beta
        O, L = fwd(q, k, v, scale=scale)
        den = math.exp(sig) + kL - 1
        expL = math.log(den)
        others = v[0, 0].sum(axis=0) - v[0, 0, jstar]
        expO = (math.exp(sig) * v[0, 0, jstar] + others) / den
        _close(L, np.full((1, 1, 3), expL), tol=1e-12 * max(1.0, abs(expL)), what="dominant L")
        _close(O, np.broadcast_to(expO, O.shape), what="dominant O")
        if sig > 15:  # the limit O -> V*
            _close(O[0, 0, 0], v[0, 0, jstar], tol=kL * math.exp(-sig) * 10 + 1e-12, what="dominant limit")
    # A score far beyond exp's range: a max-subtracted softmax stays finite and
    # exact, L = sig + ln(1 + (n-1)e^-sig) = sig in fp64, O = V*.
    q = np.zeros((1, 1, 2, D))
    q[..., 0] = 2000.0
    k = r.standard_normal((1, 1, kL, D))
    k[..., 0] = 0.0
    k[0, 0, jstar, 0] = 1.0
    v = r.standard_normal((1, 1, kL, D))
    O, L = fwd(q, k, v, scale=1.0)
    _close(L, np.full((1, 1, 2), 2000.0), tol=1e-12 * 2000, what="huge-score L")
    _close(O, np.broadcast_to(v[0, 0, jstar], O.shape), what="huge-score O")


def pin_rows_are_distributions(fwd):
    """With V = I (kL = D) the output row is the softmax row: nonnegative, sums to 1; V = 1 gives O = 1."""
    r = _rng(3)
    D = 6
    q = r.standard_normal((1, 2, 4, D))
    k = r.standard_normal((1, 2, D, D))
    v = np.broadcast_to(np.eye(D), (1, 2, D, D)).copy()
    for causal in (False, True):
        O, _ = fwd(q, k, v, scale=0.9, causal=causal)
        assert np.all(O >= 0), "softmax row has a negative entry"
        _close(O.sum(axis=-1), np.ones((1, 2, 4)), what="softmax rows sum to 1")
        if causal:
            for i in range(4):
                assert np.all(O[0, :, i, i + 1:] == 0), "causal row has weight on a future key"
    O, _ = fwd(q, k, np.ones((1, 2, D, D)), scale=0.9)
    _close(O, np.ones_like(O), what="V = 1 gives O = 1")


def pin_causal_first_row(fwd):
    """Causal row 0 sees only key 0: O_0 = V_0, L_0 = s_00 (+ mask_00)."""
    r = _rng(4)
    q = r.standard_normal((2, 3, 6, 5))
    k = r.standard_normal((2, 3, 6, 5))
    v = r.standard_normal((2, 3, 6, 5))
    m = r.standard_normal((2, 3, 6, 6))
    for mask, kind in ((None, "none"), (m, "additive")):
        O, L = fwd(q, k, v, scale=0.3, causal=True, mask=mask, mask_kind=kind)
        s00 = 0.3 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0])
        if mask is not None:
            s00 = s00 + m[:, :, 0, 0]
        _close(O[:, :, 0], v[:, :, 0], what="causal row 0 O")
        _close(L[:, :, 0], s00, what="causal row 0 L")


def pin_causal_last_row(fwd):
    """With qL = kL the last causal row sees every key: equal to the non-causal row."""
    r = _rng(5)
    q, k, v = (r.standard_normal((1, 2, 7, 4)) for _ in range(3))
    Oc, Lc = fwd(q, k, v, scale=0.6, causal=True)
    On, Ln = fwd(q, k, v, scale=0.6)
    _close(Oc[:, :, -1], On[:, :, -1], what="causal last row O")
    _close(Lc[:, :, -1], Ln[:, :, -1], what="causal last row L")
    assert np.max(np.abs(Lc[:, :, 0] - Ln[:, :, 0])) > 1e-3, "causal had no effect on row 0"


def pin_one_key(fwd):
    """An additive mask that is -inf everywhere but key j_i gives O_i = V_j, L_i = s_ij."""
    r = _rng(6)
    B, H, qL, kL, D = 1, 2, 5, 8, 3
    q, k, v = r.standard_normal((B, H, qL, D)), r.standard_normal((B, H, kL, D)), r.standard_normal((B, H, kL, D))
    keep = r.integers(0, kL, (B, H, qL))
    m = np.full((B, H, qL, kL), -np.inf)
    np.put_along_axis(m, keep[..., None], 0.25, axis=-1)
    O, L = fwd(q, k, v, scale=0.8, mask=m, mask_kind="additive")
    for h in range(H):
        for i in range(qL):
            j = keep[0, h, i]
            _close(O[0, h, i], v[0, h, j], what="one-key O")
            _close(L[0, h, i], 0.8 * float(q[0, h, i] @ k[0, h, j]) + 0.25, what="one-key L")


def pin_mask_shift(fwd):
    """Adding c_i to a row of the additive mask leaves O alone and shifts L by c_i."""
    r = _rng(7)
    q, k, v = r.standard_normal((1, 2, 4, 5)), r.standard_normal((1, 2, 6, 5)), r.standard_normal((1, 2, 6, 5))
    m = r.standard_normal((1, 2, 4, 6))
    c = r.standard_normal((1, 2, 4, 1)) * 3
    O1, L1 = fwd(q, k, v, scale=0.5, mask=m, mask_kind="additive")
    O2, L2 = fwd(q, k, v, scale=0.5, mask=m + c, mask_kind="additive")
    _close(O2, O1, tol=1e-12, what="shift O")
    _close(L2, L1 + c[..., 0], tol=1e-12, what="shift L")


def pin_permutation(fwd):
    """Non-causal, unmasked attention does not depend on the order of the (K, V) rows."""
    r = _rng(8)
    q, k, v = r.standard_normal((1, 2, 3, 4)), r.standard_normal((1, 2, 9, 4)), r.standard_normal((1, 2, 9, 4))
    perm = r.permutation(9)
    O1, L1 = fwd(q, k, v, scale=0.7)
    O2, L2 = fwd(q, k[:, :, perm], v[:, :, perm], scale=0.7)
    _close(O2, O1, what="perm O")
    _close(L2, L1, what="perm L")


def pin_gqa(fwd):
    """GQA equals MHA with each kv head repeated for its consecutive group of query heads."""
    r = _rng(9)
    B, Hq, Hkv, qL, kL, D = 2, 6, 2, 4, 5, 3
    q = r.standard_normal((B, Hq, qL, D))
    k, v = r.standard_normal((B, Hkv, kL, D)), r.standard_normal((B, Hkv, kL, D))
    m = r.standard_normal((B, Hq, qL, kL))
    rep = Hq // Hkv
    O1, L1 = fwd(q, k, v, scale=0.4, mask=m, mask_kind="additive")
    O2, L2 = fwd(q, np.repeat(k, rep, axis=1), np.repeat(v, rep, axis=1), scale=0.4, mask=m, mask_kind="additive")
    _close(O1, O2, what="gqa O")
    _close(L1, L2, what="gqa L")


def pin_scale_homogeneity(fwd):
    """attention(Q, scale s) == attention(s*Q, scale 1)."""
    r = _rng(10)
    q, k, v = r.standard_normal((1, 1, 4, 6)), r.standard_normal((1, 1, 7, 6)), r.standard_normal((1, 1, 7, 6))
    O1, L1 = fwd(q, k, v, scale=0.37)
    O2, L2 = fwd(0.37 * q, k, v, scale=1.0)
    _close(O1, O2, tol=1e-13 * 10, what="homog O")
    _close(L1, L2, tol=1e-13 * 10, what="homog L")


def pin_bool_equals_additive(fwd):
    """A bool mask equals the additive mask that is 0 where it attends and -inf elsewhere."""
    r = _rng(11)
    q, k, v = r.standard_normal((1, 2, 6, 4)), r.standard_normal((1, 2, 7, 4)), r.standard_normal((1, 2, 7, 4))
    attend = r.random((1, 2, 6, 7)) < 0.6
    attend[..., 0] = True
    add = np.where(attend, 0.0, -np.inf)
    for causal in (False, True):
        O1, L1 = fwd(q, k, v, scale=0.5, causal=causal, mask=attend.astype(np.uint8), mask_kind="bool")
        O2, L2 = fwd(q, k, v, scale=0.5, causal=causal, mask=add, mask_kind="additive")
        _close(O1, O2, what="bool vs additive O")
        _close(L1, L2, what="bool vs additive L")


def pin_empty_rows(fwd):
    """A row with no allowed key gives O = 0 and L = 0 (bool all-zero row, or additive all -inf row)."""
    r = _rng(12)
    q, k, v = r.standard_normal((1, 1, 4, 3)), r.standard_normal((1, 1, 5, 3)), r.standard_normal((1, 1, 5, 3))
    attend = np.ones((1, 1, 4, 5), dtype=np.uint8)
    attend[0, 0, 2] = 0
    O, L = fwd(q, k, v, scale=1.0, mask=attend, mask_kind="bool")
    assert np.all(O[0, 0, 2] == 0) and L[0, 0, 2] == 0, "empty bool row is not O=0, L=0"
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    add = np.zeros((1, 1, 4, 5))
    add[0, 0, 1] = -np.inf
    O, L = fwd(q, k, v, scale=1.0, mask=add, mask_kind="additive")
    assert np.all(O[0, 0, 1] == 0) and L[0, 0, 1] == 0, "empty additive row is not O=0, L=0"
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))


def pin_brute_force(fwd):
    """Agreement to 1e-12 with the pure-Python loop on tiny shapes, every mask kind, causal and GQA."""
    r = _rng(13)
    cases = [
        dict(B=1, Hq=1, Hkv=1, qL=3, kL=4, D=2, causal=False, kind="none"),
        dict(B=2, Hq=4, Hkv=2, qL=5, kL=5, D=3, causal=True, kind="none"),
        dict(B=1, Hq=3, Hkv=1, qL=4, kL=6, D=4, causal=False, kind="additive"),
        dict(B=2, Hq=2, Hkv=2, qL=6, kL=4, D=2, causal=True, kind="additive"),
        dict(B=1, Hq=2, Hkv=1, qL=5, kL=7, D=3, causal=False, kind="bool"),
        dict(B=1, Hq=4, Hkv=4, qL=8, kL=8, D=8, causal=True, kind="bool"),
        dict(B=1, Hq=2, Hkv=2, qL=7, kL=3, D=5, causal=True, kind="none"),
    ]
    for c in cases:
        q = r.standard_normal((c["B"], c["Hq"], c["qL"], c["D"]))
        k = r.standard_normal((c["B"], c["Hkv"], c["kL"], c["D"]))
        v = r.standard_normal((c["B"], c["Hkv"], c["kL"], c["D"]))
        mask = None
        if c["kind"] == "additive":
            mask = r.standard_normal((c["B"], c["Hq"], c["qL"], c["kL"]))
            mask[r.random(mask.shape) < 0.25] = -np.inf
        elif c["kind"] == "bool":
            mask = (r.random((c["B"], c["Hq"], c["qL"], c["kL"])) < 0.7).astype(np.uint8)
        O, L = fwd(q, k, v, scale=0.6, causal=c["causal"], mask=mask, mask_kind=c["kind"])
        Ob, Lb = brute_attention(q.tolist(), k.tolist(), v.tolist(), 0.6, c["causal"],
                                 None if mask is None else mask.tolist(), c["kind"])
        _close(O, Ob, tol=1e-12, what=f"brute O {c}")
        _close(L, Lb, tol=1e-12, what=f"brute L {c}")


def pin_torch_sdpa(fwd):
    """Agreement with torch's CPU float64 scaled_dot_product_attention and logsumexp (library routines)."""
    r = _rng(14)
    B, Hq, Hkv, qL, kL, D = 2, 4, 2, 33, 47, 16
    q = torch.from_numpy(r.standard_normal((B, Hq, qL, D)))
    k = torch.from_numpy(r.standard_normal((B, Hkv, kL, D)))
    v = torch.from_numpy(r.standard_normal((B, Hkv, kL, D)))
    kr, vr = k.repeat_interleave(Hq // Hkv, dim=1), v.repeat_interleave(Hq // Hkv, dim=1)
    add = torch.from_numpy(r.standard_normal((B, Hq, qL, kL)))
    scale = 0.21
    for causal, mask in ((False, None), (True, None), (False, add)):
        if causal:
            # top-left causal: key j is visible to row i iff j <= i
            tmask = torch.ones(qL, kL, dtype=torch.bool).tril()
            ref = torch.nn.functional.scaled_dot_product_attention(q, kr, vr, attn_mask=tmask, scale=scale)
            s = (q @ kr.transpose(-1, -2)) * scale
            s = s.masked_fill(~tmask, -math.inf)
        else:
            ref = torch.nn.functional.scaled_dot_product_attention(q, kr, vr, attn_mask=mask, scale=scale)
            s = (q @ kr.transpose(-1, -2)) * scale + (mask if mask is not None else 0)
        refL = torch.logsumexp(s, dim=-1)
        O, L = fwd(q.numpy(), k.numpy(), v.numpy(), scale=scale, causal=causal,
                   mask=None if mask is None else mask.numpy(), mask_kind="none" if mask is None else "additive")
        _close(O, ref.numpy(), tol=1e-12, what=f"torch sdpa O causal={causal}")
        _close(L, refL.numpy(), tol=1e-12, what=f"torch logsumexp causal={causal}")


def pin_row_subset(fwd):
    """Asking for a subset of rows returns exactly those rows of the full result."""
    r = _rng(15)
    q, k, v = r.standard_normal((2, 3, 9, 4)), r.standard_normal((2, 1, 11, 4)), r.standard_normal((2, 1, 11, 4))
    O, L = fwd(q, k, v, scale=0.5, causal=True)
    rows = np.array([0, 5, 9, 26, 27, 53], dtype=np.int64)
    Os, Ls = fwd(q, k, v, scale=0.5, causal=True, rows=rows)
    _close(Os, O.reshape(-1, 4)[rows], tol=0, what="row subset O")
    _close(Ls, L.reshape(-1)[rows], tol=0, what="row subset L")


ALL_PINS = [
    pin_zero_query, pin_dominant_key, pin_rows_are_distributions, pin_causal_first_row,
    pin_causal_last_row, pin_one_key, pin_mask_shift, pin_permutation, pin_gqa,
    pin_scale_homogeneity, pin_bool_equals_additive, pin_empty_rows, pin_brute_force,
    pin_torch_sdpa, pin_row_subset,
]
