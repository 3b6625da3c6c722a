"""Seeded synthetic workloads for the attention forward pass.

Shared by the tests and the benchmark.  This module only draws random
tensors and describes shapes: it holds none of the attention arithmetic, and
both the GPU path and the oracle receive exactly the tensors drawn here.

Recipe (the pages publish no dataset; every input is synthetic):
  * generator: numpy.random.default_rng(seed) (PCG64);
  * Q, K, V are drawn in that order with standard_normal(dtype=float32) in
    [B, H, L, D] order, then cast to bf16 with round-to-nearest-even for the
    bf16 workloads;
  * the additive mask (when present) is drawn after V: each entry is masked
    with probability p_masked, then one uniformly chosen key per row is forced
    unmasked; masked entries are -inf, the rest 0, stored in the input dtype;
  * a bool mask is the same draw stored as uint8 (1 = attend).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "bf16" or "f32": Q, K, V, O (L is always f32)
    B: int
    Hq: int
    Hkv: int
    qL: int
    kL: int
    D: int
    scale: float
    causal: bool = False
    mask_kind: str = "none"   # "none" | "additive" | "bool"
    p_masked: float = 0.0
    token_major_out: bool = False
    seed: int = 0
    dropout_p: float | None = None  # dropout rate on the attention weights (seed = the workload seed)
    window: int | None = None       # causal sliding window: row i sees keys i - window + 1 .. i
    backward: bool = False          # time fa_bwd (dQ, dK, dV) instead of the forward pass
    note: str = ""

    def flops(self) -> float:
        """Algorithmic FLOP: 4*B*Hq*qL*kL*D, halved when causal; with a window,
        4*B*Hq*D times the exact count of allowed (row, key) pairs.  The
        backward pass counts its five matrix products (S, dP, dV, dK, dQ):
        2.5 times the forward figure."""
        if self.backward:
            return 2.5 * self.with_(backward=False).flops()
        if self.window is not None:
            i = np.arange(self.qL, dtype=np.int64)
            pairs = np.minimum(np.minimum(i + 1, self.window), np.maximum(0, self.kL - np.maximum(0, i - self.window + 1)))
            return 4.0 * self.B * self.Hq * self.D * float(pairs.sum())
        f = 4.0 * self.B * self.Hq * self.qL * self.kL * self.D
        return f / 2 if self.causal else f

    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads of the method's hot path.
C1 = Workload("tiny_f32_d64", "f32", 1, 1, 1, 128, 128, 64, 1 / math.sqrt(64), seed=1,
              note="tiny non-causal fp32 SDPA")
C2 = Workload("causal_gqa_bf16_d64", "bf16", 2, 16, 4, 2048, 2048, 64, 1 / 8, causal=True, seed=2,
              note="causal GQA bf16 training forward")
C3 = Workload("causal_bf16_d128_8k", "bf16", 1, 32, 8, 8192, 8192, 128, 1 / math.sqrt(128),
              causal=True, seed=3, note="long-context causal bf16, the headline shape")
C4 = Workload("dit_f32_d128_tokmajor", "f32", 1, 24, 24, 4096, 4096, 128, 1 / math.sqrt(128),
              token_major_out=True, seed=4, note="DiT joint attention, fp32, token-major output")
C5 = Workload("masked_bf16_d256", "bf16", 1, 8, 8, 1024, 3072, 256, 1 / math.sqrt(256),
              mask_kind="additive", p_masked=0.2, seed=5, note="additive 0/-inf mask, D=256")

CONFIGS = {w.name: w for w in (C1, C2, C3, C4, C5)}
HEADLINE = C3

# Short-key shapes whose cost is the HBM traffic of Q and O (flop per byte
# about kL, below the bf16 matrix ridge of ~315): the achieved HBM GB/s is
# their figure of merit.
SHORT_KL = [
    Workload(f"short_kl{kl}_bf16_d128", "bf16", 1, 32, 8, 8192, kl, 128, 1 / math.sqrt(128), seed=20 + kl,
             note=f"short-key bf16, kL={kl}: HBM-bound (Q and O dominate the bytes)")
    for kl in (32, 64, 128)
]

# The headline shape at the further head dims the kernels support: parity
# cases and benchmark workloads of their own.
HEAD_DIMS = [
    Workload(f"causal_bf16_d{d}_8k", "bf16", 1, 32, 8, 8192, 8192, d, 1 / math.sqrt(d), causal=True,
             seed=40 + d, note=f"long-context causal bf16 at head dim {d}")
    for d in (16, 32, 48, 80, 96)
]

# Short query ranges over long key ranges (a decode step): too few query
# tiles to fill the GPU, so the key range is split over work-groups and the
# partials merged.  HBM-bound: K and V dominate the bytes.
SPLIT_KV = [
    Workload("decode_bf16_d128_32k", "bf16", 1, 32, 8, 16, 32768, 128, 1 / math.sqrt(128), seed=60,
             note="16 query rows over 32768 keys, bf16 D=128 (K/V-read bound)"),
    Workload("decode_f32_d128_32k", "f32", 1, 32, 8, 16, 32768, 128, 1 / math.sqrt(128), seed=61,
             note="16 query rows over 32768 keys, fp32 D=128 (K/V-read bound)"),
]

# The headline shape with dropout on the attention weights (rate 0.1).
DROPOUT = [
    Workload("causal_bf16_d128_8k_dropout", "bf16", 1, 32, 8, 8192, 8192, 128, 1 / math.sqrt(128), causal=True,
             seed=70, dropout_p=0.1, note="long-context causal bf16 with dropout 0.1 on the attention weights"),
]

# The headline shape under a causal sliding window of 4096 keys (the reading
# taken of the pages' `window` field).
WINDOW = [
    Workload("causal_bf16_d128_8k_window4k", "bf16", 1, 32, 8, 8192, 8192, 128, 1 / math.sqrt(128), causal=True,
             seed=80, window=4096, note="long-context causal bf16 under a 4096-key sliding window"),
]

# The backward pass (dQ, dK, dV) at the causal GQA training shape and the
# long-context shape; dO ~ N(0, 1) drawn by draw_grad.
BACKWARD = [
    C2.with_(name="bwd_causal_gqa_bf16_d64", backward=True, note="backward pass, causal GQA bf16 training shape"),
    C3.with_(name="bwd_causal_bf16_d128_8k", backward=True, note="backward pass, long-context causal bf16 D=128"),
]

# Ragged shapes that are not tile multiples (the configs above all are).
RAGGED = [
    Workload("ragged_masked_d256", "bf16", 1, 2, 2, 1000, 3000, 256, 1 / 16, mask_kind="additive",
             p_masked=0.2, seed=11),
    Workload("ragged_f32_seq8", "f32", 1, 3, 3, 8, 8, 128, 1 / math.sqrt(128), seed=12),
    Workload("ragged_f32_seq40", "f32", 1, 3, 3, 40, 40, 128, 1 / math.sqrt(128), seed=13),
    Workload("ragged_f32_seq50", "f32", 1, 3, 3, 50, 50, 128, 1 / math.sqrt(128), seed=14),
    Workload("ragged_bf16_127x129", "bf16", 2, 4, 2, 127, 129, 64, 0.125, causal=True, seed=15),
]


def draw(w: Workload):
    """Draw (q, k, v, mask) as CPU torch tensors for workload `w`.

    q [B,Hq,qL,D], k/v [B,Hkv,kL,D] in the workload dtype; mask is None,
    an additive [B,Hq,qL,kL] tensor in the workload dtype, or a uint8 bool
    tensor of that shape (1 = attend).
    """
    rng = np.random.default_rng(w.seed)
    q = rng.standard_normal((w.B, w.Hq, w.qL, w.D), dtype=np.float32)
    k = rng.standard_normal((w.B, w.Hkv, w.kL, w.D), dtype=np.float32)
    v = rng.standard_normal((w.B, w.Hkv, w.kL, w.D), dtype=np.float32)
    td = w.torch_dtype()
    q, k, v = (torch.from_numpy(x).to(td) for x in (q, k, v))
    mask = None
    if w.mask_kind != "none":
        masked = draw_masked(rng, (w.B, w.Hq, w.qL, w.kL), w.p_masked)
        if w.mask_kind == "bool":
            mask = torch.from_numpy((~masked).astype(np.uint8))
        else:
            m = np.zeros(masked.shape, dtype=np.float32)
            m[masked] = -np.inf
            mask = torch.from_numpy(m).to(td)
    return q, k, v, mask


def draw_masked(rng, shape, p_masked):
    """Bernoulli(p_masked) 'masked' flags with one unmasked key forced per row."""
    masked = rng.random(shape) < p_masked
    keep = rng.integers(0, shape[-1], shape[:-1])
    np.put_along_axis(masked, keep[..., None], False, axis=-1)
    return masked


def sample_rows(w: Workload, n: int, seed: int = 1234) -> np.ndarray:
    """Flat row indices (b*Hq + h)*qL + i for sampled parity checks.

    Always includes the first and last row of every head and the rows on both
    sides of 64- and 128-row tile edges near the start and the end; the rest
    are drawn uniformly.
    """
    rng = np.random.default_rng(seed)
    rows = set()
    for bh in range(w.B * w.Hq):
        for i in (0, 1, 31, 32, 63, 64, 127, 128, w.qL - 129, w.qL - 128, w.qL - 65, w.qL - 64, w.qL - 1):
            if 0 <= i < w.qL:
                rows.add(bh * w.qL + i)
    extra = rng.integers(0, w.B * w.Hq * w.qL, size=max(0, n - len(rows)))
    rows.update(int(x) for x in extra)
    return np.array(sorted(rows), dtype=np.int64)


def draw_grad(w: Workload):
    """The upstream gradient dO ~ N(0, 1) [B, Hq, qL, D] in the workload dtype
    (its own generator, seeded from the workload seed)."""
    rng = np.random.default_rng(w.seed + 1000)
    return torch.from_numpy(rng.standard_normal((w.B, w.Hq, w.qL, w.D), dtype=np.float32)).to(w.torch_dtype())
