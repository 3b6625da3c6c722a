"""Helpers shared by the GPU parity tests: run the HIP path, run the oracle,
compare at the tolerances the method fixes (max abs error on O: 1e-4 for fp32
outputs, 2e-2 for bf16 outputs; on L: 1e-3)."""
import numpy as np
import torch

import flashattention_forward_04_amd as fa
from oracle import attention_fwd

TOL_O = {"f32": 1e-4, "bf16": 2e-2}
TOL_L = 1e-3


def dtype_name(t):
    return "bf16" if t.dtype == torch.bfloat16 else "f32"


def run_gpu(q, k, v, mask=None, *, causal=False, scale=None, token_major=False, out=None):
    """Upload, run fa.fwd, download.  Returns (O [B,Hq,qL,D] float64, L float64, raw out tensor)."""
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    md = None if mask is None else mask.to(dev)
    B, Hq, qL, D = q.shape
    if out is None and token_major:
        out = torch.empty((B, qL, Hq, D), dtype=q.dtype, device=dev).transpose(1, 2)
    O, L = fa.fwd(qd, kd, vd, mask=md, causal=causal, scale=scale, out=out)
    torch.cuda.synchronize()
    return O.double().cpu().numpy(), L.double().cpu().numpy(), O


def run_oracle(q, k, v, mask=None, *, causal=False, scale, rows=None):
    kind = "none"
    m = None
    if mask is not None:
        kind = "bool" if mask.dtype in (torch.uint8, torch.bool) else "additive"
        m = mask.double().numpy() if kind == "additive" else mask.numpy()
    return attention_fwd(q.double().numpy(), k.double().numpy(), v.double().numpy(), scale=scale, causal=causal,
                         mask=m, mask_kind=kind, rows=rows)


def max_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    if a.size == 0:
        return 0.0
    if not np.all(np.isfinite(a)):
        return float("inf")
    return float(np.max(np.abs(a - b)))


def assert_parity(O, L, Oref, Lref, dt, what=""):
    eo, el = max_err(O, Oref), max_err(L, Lref)
    print(f"[parity] {what}: max|dO| = {eo:.3e} (tol {TOL_O[dt]:.0e}), max|dL| = {el:.3e} (tol {TOL_L:.0e})",
          flush=True)
    assert eo <= TOL_O[dt], f"{what}: O error {eo:.3e} > {TOL_O[dt]}"
    assert el <= TOL_L, f"{what}: L error {el:.3e} > {TOL_L}"
