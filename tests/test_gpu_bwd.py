"""GPU parity of the backward pass (fa_bwd) against the fp64 oracle.

Every test runs the forward pass on the GPU (its bf16 O and fp32 L feed the
backward pass, as in training), then fa_bwd through the C ABI, and compares
dQ, dK and dV with the oracle's gradients on the same seeded inputs.

Tolerance (bf16 inputs and outputs): for each of dQ, dK, dV,
    max |gpu - oracle| <= TOL_GRAD * max |oracle| + ABS_FLOOR,
    TOL_GRAD = 2^-6, ABS_FLOOR = 1e-5.
TOL_GRAD is four bf16 rounding units at the tensor's largest entry: the
output is rounded to bf16 (at most 2^-8 of an entry), and the kernels round P
and dS to bf16 before the matrix products and take Delta from the bf16
forward output O; each of those adds error of the order of 2^-8 of the
magnitudes it multiplies, which for these inputs stay within the tensor's
largest entry.  ABS_FLOOR covers tensors whose exact value is 0 (a row with
one allowed key has dS = 0, so dQ = dK = 0 exactly): there the fp32 rounding
of dP - Delta leaves ~1e-7.
"""
import math

import numpy as np
import pytest
import torch

import flashattention_forward_04_amd as fa
import workloads as W
from oracle import attention_bwd

pytestmark = pytest.mark.gpu

TOL_GRAD = 2.0 ** -6
ABS_FLOOR = 1e-5


def _inputs(B, Hq, Hkv, qL, kL, D, seed, mask_kind="none", p_masked=0.3, empty_row=False):
    g = np.random.default_rng(seed)
    q, k, v, do = (torch.from_numpy(g.standard_normal(s, dtype=np.float32)).to(torch.bfloat16)
                   for s in ((B, Hq, qL, D), (B, Hkv, kL, D), (B, Hkv, kL, D), (B, Hq, qL, D)))
    mask = None
    if mask_kind != "none":
        masked = W.draw_masked(g, (B, Hq, qL, kL), p_masked)
        if empty_row:
            masked[0, 0, min(3, qL - 1)] = True  # one row allows no key at all
        if mask_kind == "bool":
            mask = torch.from_numpy((~masked).astype(np.uint8))
        else:
            m = g.standard_normal(masked.shape).astype(np.float32)
            m[masked] = -np.inf
            mask = torch.from_numpy(m).to(torch.bfloat16)
    return q, k, v, do, mask


def _gpu(q, k, v, do, mask, causal, scale):
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    md = None if mask is None else mask.to(dev)
    O, L = fa.fwd(qd, kd, vd, mask=md, causal=causal, scale=scale)
    dq, dk, dv, delta = fa.bwd(qd, kd, vd, O, dod, L, mask=md, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return (dq.double().cpu().numpy(), dk.double().cpu().numpy(), dv.double().cpu().numpy(),
            delta.double().cpu().numpy(), O.double().cpu().numpy())


def _oracle(q, k, v, do, mask, causal, scale, qrows=None, krows=None):
    kind, m = "none", None
    if mask is not None:
        kind = "bool" if mask.dtype == torch.uint8 else "additive"
        m = mask.numpy() if kind == "bool" else mask.double().numpy()
    return attention_bwd(q.double().numpy(), k.double().numpy(), v.double().numpy(), do.double().numpy(),
                         scale=scale, causal=causal, mask=m, mask_kind=kind, qrows=qrows, krows=krows)


def _assert_grads(got, ref, what):
    for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
        assert np.all(np.isfinite(a)), f"{what}: {name} not finite"
        scale = float(np.max(np.abs(b))) if b.size else 0.0
        err = float(np.max(np.abs(a - b))) if b.size else 0.0
        rel = err / scale if scale > 0 else err
        print(f"[bwd parity] {what} {name}: max|d| = {err:.3e}, max|ref| = {scale:.3e}, ratio {rel:.2e} "
              f"(tol {TOL_GRAD:.2e})", flush=True)
        assert err <= TOL_GRAD * scale + ABS_FLOOR, f"{what}: {name} error {err:.3e} > {TOL_GRAD} x {scale:.3e}"


def _case(B, Hq, Hkv, qL, kL, D, causal, seed, mask_kind="none", empty_row=False, scale=None):
    scale = 1 / math.sqrt(D) if scale is None else scale
    what = f"B={B} Hq={Hq} Hkv={Hkv} qL={qL} kL={kL} D={D} causal={causal} mask={mask_kind} seed={seed}"
    print(f"[case] {what}", flush=True)
    q, k, v, do, mask = _inputs(B, Hq, Hkv, qL, kL, D, seed, mask_kind, empty_row=empty_row)
    dq, dk, dv, delta, O = _gpu(q, k, v, do, mask, causal, scale)
    ref = _oracle(q, k, v, do, mask, causal, scale)
    _assert_grads((dq, dk, dv), ref, what)
    # Delta is rowsum(dO * O) of the forward output the backward pass was given
    exp_delta = (do.double().numpy() * O).sum(-1)
    assert np.max(np.abs(delta - exp_delta)) <= 1e-4 * max(1.0, float(np.max(np.abs(exp_delta))))
    return dq, dk, dv


def test_causal_gqa_training_shape():
    """The causal GQA bf16 training shape (B = 2, 16 / 4 heads, 2048 x 2048, D = 64), every element."""
    _case(2, 16, 4, 2048, 2048, 64, True, 500)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("qL,kL", [(256, 256), (127, 129), (300, 500), (500, 64), (1, 1), (1, 300), (300, 1),
                                   (1000, 1000)])
def test_shapes(D, causal, qL, kL):
    """Ragged and unequal lengths (tails of every tile kind), GQA, both head dims."""
    _case(1, 4, 2, qL, kL, D, causal, 501 + qL + 7 * kL + D)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv,kind,causal", [(16, 2, "none", False), (16, 2, "bool", True), (24, 4, "additive", False),
                                               (8, 8, "none", True)], ids=lambda x: str(x))
def test_group_splits(D, Hq, Hkv, kind, causal):
    """Small dK/dV grids whose key tiles' (head, query tile) steps are split
    over up to 16 work-groups (GQA groups of 8 and 6, and MHA); the partials
    are summed in a fixed order."""
    _case(1, Hq, Hkv, 200, 333, D, causal, 650 + D + Hq, mask_kind=kind, empty_row=kind != "none")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kind", ["additive", "bool"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_masks(D, kind, causal):
    """Both mask kinds, with a row that allows no key (it contributes nothing)."""
    dq, _, _ = _case(1, 4, 2, 193, 257, D, causal, 600 + D, mask_kind=kind, empty_row=True)
    assert np.all(dq[0, 0, 3] == 0)


@pytest.mark.parametrize("D", [64, 128])
def test_long_context_d128_shape_sampled(D):
    """The long-context causal shape (B = 1, 32 / 8 heads, 8192 x 8192) at D = 64 and 128: dQ of 384 query
    rows and dK, dV of 384 key rows against the oracle; every gradient finite."""
    B, Hq, Hkv, L = 1, 32, 8, 8192
    scale = 1 / math.sqrt(D)
    print(f"[case] long context B={B} Hq={Hq} Hkv={Hkv} L={L} D={D} causal", flush=True)
    q, k, v, do, _ = _inputs(B, Hq, Hkv, L, L, D, 700 + D)
    dq, dk, dv, _, _ = _gpu(q, k, v, do, None, True, scale)
    g = np.random.default_rng(7)
    qrows = np.unique(np.concatenate([g.integers(0, B * Hq * L, 368), [0, L - 1, L, 2 * L - 1, 5 * L + 4095,
                                                                       B * Hq * L - 1]]))
    krows = np.unique(np.concatenate([g.integers(0, B * Hkv * L, 368), [0, 1, L - 1, L, 3 * L + 4096,
                                                                        B * Hkv * L - 1]]))
    rq, rk, rv = _oracle(q, k, v, do, None, True, scale, qrows=qrows, krows=krows)
    _assert_grads((dq.reshape(-1, D)[qrows], dk.reshape(-1, D)[krows], dv.reshape(-1, D)[krows]), (rq, rk, rv),
                  f"long context D={D} sampled")


def test_gqa_equals_repeated_mha_summed():
    """dK, dV of a GQA call equal the repeated-MHA gradients summed over each group (same kernels, different
    summation order: within the tolerance)."""
    q, k, v, do, _ = _inputs(1, 8, 2, 400, 400, 128, 800)
    dq, dk, dv, _, _ = _gpu(q, k, v, do, None, True, 1 / math.sqrt(128))
    kr, vr = k.repeat_interleave(4, dim=1).contiguous(), v.repeat_interleave(4, dim=1).contiguous()
    dq2, dk2, dv2, _, _ = _gpu(q, kr, vr, do, None, True, 1 / math.sqrt(128))
    assert np.max(np.abs(dq - dq2)) == 0.0  # dQ's work-groups see the same data in the same order
    for a, b in ((dk, dk2.reshape(1, 2, 4, 400, 128).sum(2)), (dv, dv2.reshape(1, 2, 4, 400, 128).sum(2))):
        assert np.max(np.abs(a - b)) <= TOL_GRAD * np.max(np.abs(a))


def test_deterministic():
    """No atomics: two calls give the same bits."""
    q, k, v, do, _ = _inputs(2, 4, 2, 333, 333, 64, 801)
    a = _gpu(q, k, v, do, None, True, 0.125)
    b = _gpu(q, k, v, do, None, True, 0.125)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_rejections():
    z = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.zeros((1, 1, 8), dtype=torch.float32, device="cuda:0")
    with pytest.raises(fa.FaError) as e:
        fa.bwd(z.float(), z.float(), z.float(), z.float(), z.float(), lse)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED
    z96 = torch.zeros((1, 1, 8, 96), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(fa.FaError) as e:
        fa.bwd(z96, z96, z96, z96, z96, lse)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED
