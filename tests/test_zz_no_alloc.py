"""The allocation-free entry point, fa_fwd_strided_noalloc, against
fa_fwd_strided through the C ABI.

Both run the same kernels with the same split plan, so O and L must agree
bit for bit.  Each case makes two calls in a row, the second with a smaller
input, so the second reads a scratch that still holds the first call's
partials.  The cases cover a decode-shaped launch whose key range is split
over 32 work-groups (8.4 MB of partials), the masked D = 256 shape whose
range is split in 4 (33.7 MB), and a launch that does not split at all.
"""
import numpy as np
import pytest
import torch

import flashattention_forward_04_amd as fa
import workloads as W

pytestmark = pytest.mark.gpu

CASES = [
    ("decode_split32", W.SPLIT_KV[0], W.Workload("decode_small", "bf16", 1, 8, 2, 16, 8192, 128, 0.088, seed=61)),
    ("masked_d256_split4", W.C5, W.Workload("masked_d256_small", "bf16", 1, 4, 4, 512, 3072, 256, 0.0625,
                                            mask_kind="additive", p_masked=0.2, seed=62)),
    ("f32_decode_split", W.Workload("f32_decode", "f32", 1, 8, 2, 16, 16384, 128, 0.088, seed=65),
     W.Workload("f32_decode_small", "f32", 1, 4, 2, 8, 4096, 64, 0.125, causal=False, seed=66)),
    ("unsplit_causal_gqa", W.Workload("gqa_300", "bf16", 2, 4, 2, 300, 300, 64, 0.125, causal=True, seed=63),
     W.Workload("gqa_100", "bf16", 1, 4, 2, 100, 120, 64, 0.125, causal=True, seed=64)),
]


def _run(w, no_alloc):
    q, k, v, mask = W.draw(w)
    dev = torch.device("cuda:0")
    O, L = fa.fwd(q.to(dev), k.to(dev), v.to(dev), mask=None if mask is None else mask.to(dev), causal=w.causal,
                  scale=w.scale, no_alloc=no_alloc)
    torch.cuda.synchronize()
    return O.cpu(), L.cpu()


@pytest.mark.parametrize("name,first,second", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_the_allocating_entry_point(name, first, second):
    for w in (first, second):
        print(f"[case] {name}: {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} qL={w.qL} kL={w.kL} D={w.D}", flush=True)
        O_ref, L_ref = _run(w, no_alloc=False)
        O, L = _run(w, no_alloc=True)
        assert torch.equal(O, O_ref), f"{w.name}: O differs from fa_fwd_strided"
        assert torch.equal(L, L_ref), f"{w.name}: L differs from fa_fwd_strided"
        assert np.all(np.isfinite(O.float().numpy())) and np.all(np.isfinite(L.numpy()))


def test_noalloc_refuses_window_and_dropout_in_the_wrapper():
    q = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(ValueError):
        fa.fwd(q, q, q, causal=True, window=4, no_alloc=True)
    with pytest.raises(ValueError):
        fa.fwd(q, q, q, dropout_p=0.5, no_alloc=True)
