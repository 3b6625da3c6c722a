"""GPU parity: the HIP path against the fp64 oracle, element by element.

Every test calls the library through its C ABI (via the ctypes binding) on
cuda:0 and compares with the oracle on the same seeded inputs.  Tolerances:
max abs error on O <= 1e-4 (fp32 outputs) or 2e-2 (bf16 outputs), on L
<= 1e-3.  The full-size workloads (causal bf16 8k at every head dim, with
dropout and under a window, and the fp32 DiT shape) are compared on every
row: the multithreaded oracle finishes each in seconds.
"""
import math

import numpy as np
import pytest
import torch

import flashattention_forward_04_amd as fa
import workloads as W
from gpu_util import TOL_L, TOL_O, assert_parity, dtype_name, max_err, run_gpu, run_oracle
from oracle import attention_fwd

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32


def _draw(w):
    print(f"[case] {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} qL={w.qL} kL={w.kL} D={w.D} {w.dtype} "
          f"causal={w.causal} mask={w.mask_kind} seed={w.seed}", flush=True)
    return W.draw(w)


def _full_parity(w):
    q, k, v, mask = _draw(w)
    O, L, _ = run_gpu(q, k, v, mask, causal=w.causal, scale=w.scale, token_major=w.token_major_out)
    Oref, Lref = run_oracle(q, k, v, mask, causal=w.causal, scale=w.scale)
    assert_parity(O, L, Oref, Lref, w.dtype, w.name)


@pytest.mark.parametrize("w", [W.C1, W.C2, W.C5], ids=lambda w: w.name)
def test_config_full(w):
    _full_parity(w)


@pytest.mark.parametrize("w", W.RAGGED, ids=lambda w: w.name)
def test_ragged(w):
    _full_parity(w)


@pytest.mark.parametrize("w", [W.C3, W.C4, *W.HEAD_DIMS, *W.DROPOUT, *W.WINDOW],
                         ids=lambda x: getattr(x, "name", str(x)))
def test_config_full_size(w):
    """Full-size launch (the configuration the benchmark times), compared with
    the oracle on every row."""
    q, k, v, mask = _draw(w)
    if w.dropout_p is None and w.window is None:
        O, L, raw = run_gpu(q, k, v, mask, causal=w.causal, scale=w.scale, token_major=w.token_major_out)
        Oref, Lref = run_oracle(q, k, v, mask, causal=w.causal, scale=w.scale)
    else:
        dev = torch.device("cuda:0")
        raw, Lt = fa.fwd(q.to(dev), k.to(dev), v.to(dev), causal=w.causal, scale=w.scale, dropout_p=w.dropout_p,
                         seed=w.seed, window=w.window)
        torch.cuda.synchronize()
        O, L = raw.double().cpu().numpy(), Lt.double().cpu().numpy()
        Oref, Lref = attention_fwd(q.double().numpy(), k.double().numpy(), v.double().numpy(), scale=w.scale,
                                   causal=w.causal, dropout_p=w.dropout_p, seed=w.seed, window=w.window)
    assert_parity(O, L, Oref, Lref, w.dtype, w.name + " (every row)")
    if w.token_major_out:
        # the output buffer itself is [B, qL, H*D]: out[b, i, h*D + d] = O[b, h, i, d]
        buf = raw.transpose(1, 2).reshape(w.B, w.qL, w.Hq * w.D).double().cpu().numpy()
        assert np.array_equal(buf, np.transpose(O, (0, 2, 1, 3)).reshape(w.B, w.qL, w.Hq * w.D))


@pytest.mark.parametrize("w", W.SHORT_KL + W.SPLIT_KV, ids=lambda w: w.name)
def test_short_key_shapes(w):
    """The HBM-bound short-key and decode shapes at full size (the launch the
    benchmark times for them), compared on every row."""
    _full_parity(w)


# ---------------------------------------------------------------- edge cases


def _rand(shape, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32).to(dtype)


@pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "f32"])
@pytest.mark.parametrize("D", [16, 32, 48, 64, 80, 96, 128, 256])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_head_dims_and_dtypes(dtype, D, causal):
    q = _rand((1, 4, 200, D), dtype, 1)
    k = _rand((1, 2, 200, D), dtype, 2)
    v = _rand((1, 2, 200, D), dtype, 3)
    scale = 1 / math.sqrt(D)
    O, L, _ = run_gpu(q, k, v, causal=causal, scale=scale)
    Oref, Lref = run_oracle(q, k, v, causal=causal, scale=scale)
    assert_parity(O, L, Oref, Lref, dtype_name(q), f"D={D} {dtype} causal={causal}")


@pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "f32"])
@pytest.mark.parametrize("kind", ["additive", "bool"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("D", [16, 32, 48, 64, 80, 96])
def test_masks(dtype, kind, causal, D):
    q, k, v = _rand((2, 2, 70, D), dtype, 4), _rand((2, 2, 90, D), dtype, 5), _rand((2, 2, 90, D), dtype, 6)
    rng = np.random.default_rng(7)
    masked = W.draw_masked(rng, (2, 2, 70, 90), 0.3)
    masked[0, 1, 5, :] = True  # a row with no allowed key
    if kind == "bool":
        mask = torch.from_numpy((~masked).astype(np.uint8))
    else:
        m = rng.standard_normal(masked.shape).astype(np.float32)
        m[masked] = -np.inf
        mask = torch.from_numpy(m).to(dtype)
    O, L, _ = run_gpu(q, k, v, mask, causal=causal, scale=0.125)
    Oref, Lref = run_oracle(q, k, v, mask, causal=causal, scale=0.125)
    assert_parity(O, L, Oref, Lref, dtype_name(q), f"{kind} mask causal={causal} D={D}")
    assert np.all(O[0, 1, 5] == 0) and L[0, 1, 5] == 0, "row with no allowed key is not O = 0, L = 0"


@pytest.mark.parametrize("kind", ["none", "additive", "bool"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_wide_rows_key_split(kind, causal):
    """D = 256 bf16 with too few query tiles to give every CU a work-group:
    the key range is split across a work-group's waves and merged in LDS.
    Ragged lengths, a key count that is not a multiple of any tile, and a
    masked row with no allowed key."""
    qL, kL = 100, 333
    q, k, v = _rand((1, 3, qL, 256), BF16, 21), _rand((1, 3, kL, 256), BF16, 22), _rand((1, 3, kL, 256), BF16, 23)
    mask = None
    if kind != "none":
        rng = np.random.default_rng(24)
        masked = W.draw_masked(rng, (1, 3, qL, kL), 0.25)
        masked[0, 2, 7, :] = True
        if kind == "bool":
            mask = torch.from_numpy((~masked).astype(np.uint8))
        else:
            m = rng.standard_normal(masked.shape).astype(np.float32)
            m[masked] = -np.inf
            mask = torch.from_numpy(m).to(BF16)
    O, L, _ = run_gpu(q, k, v, mask, causal=causal, scale=1 / 16)
    Oref, Lref = run_oracle(q, k, v, mask, causal=causal, scale=1 / 16)
    assert_parity(O, L, Oref, Lref, "bf16", f"D=256 key split {kind} causal={causal}")
    if kind != "none":
        assert np.all(O[0, 2, 7] == 0) and L[0, 2, 7] == 0, "row with no allowed key is not O = 0, L = 0"


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_wide_rows_work_group_path(causal):
    """D = 256 bf16 with a grid that fills the GPU (16 heads x 16 tiles of 128
    rows): the work-group kernel, not the key split; every row."""
    w = W.Workload("d256_wg_path", "bf16", 1, 16, 4, 2048, 2048, 256, 1 / 16, causal=causal, seed=25)
    _full_parity(w)


@pytest.mark.parametrize("kind", ["none", "additive", "bool"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_long_keys_d128(kind, causal):
    """D = 128 bf16 with more keys than the short-key shape takes (kL > 256):
    the 8-wave work-group path, ragged in both lengths, every mask kind."""
    qL, kL = 300, 700
    q, k, v = _rand((2, 4, qL, 128), BF16, 31), _rand((2, 2, kL, 128), BF16, 32), _rand((2, 2, kL, 128), BF16, 33)
    mask = None
    if kind != "none":
        rng = np.random.default_rng(34)
        masked = W.draw_masked(rng, (2, 4, qL, kL), 0.3)
        if kind == "bool":
            mask = torch.from_numpy((~masked).astype(np.uint8))
        else:
            m = rng.standard_normal(masked.shape).astype(np.float32)
            m[masked] = -np.inf
            mask = torch.from_numpy(m).to(BF16)
    O, L, _ = run_gpu(q, k, v, mask, causal=causal, scale=1 / math.sqrt(128))
    Oref, Lref = run_oracle(q, k, v, mask, causal=causal, scale=1 / math.sqrt(128))
    assert_parity(O, L, Oref, Lref, "bf16", f"D=128 kL=700 {kind} causal={causal}")


@pytest.mark.parametrize("qL,kL,causal", [(300, 100, True), (300, 100, False), (97, 33, True), (64, 128, False),
                                          (1, 7, False), (200, 1, True)])
def test_short_keys_streaming(qL, kL, causal):
    """D = 128 bf16 unmasked with kL <= 128: the streaming kernel (K/V held
    in LDS, query blocks walked per wave), GQA group of 4, ragged lengths."""
    q, k, v = _rand((2, 8, qL, 128), BF16, 41), _rand((2, 2, kL, 128), BF16, 42), _rand((2, 2, kL, 128), BF16, 43)
    O, L, _ = run_gpu(q, k, v, None, causal=causal, scale=1 / math.sqrt(128))
    Oref, Lref = run_oracle(q, k, v, None, causal=causal, scale=1 / math.sqrt(128))
    assert_parity(O, L, Oref, Lref, "bf16", f"streaming qL={qL} kL={kL} causal={causal}")


@pytest.mark.parametrize("qL,causal", [(665, False), (1184, True)])
def test_short_keys_streaming_many_blocks(qL, causal):
    """The streaming kernel at 65-128 keys walks its query blocks round two
    Q buffers.  With 256 kv heads each head gets one 8-wave work-group, so
    wave w takes blocks w, w + 8, ...: qL = 665 (21 blocks) gives waves 3
    and 2 blocks, qL = 1184 (37 blocks) 5 and 4, which leaves the loop at
    each of its exits."""
    H = 256
    q, k, v = _rand((1, H, qL, 128), BF16, 51), _rand((1, H, 100, 128), BF16, 52), _rand((1, H, 100, 128), BF16, 53)
    O, L, _ = run_gpu(q, k, v, None, causal=causal, scale=1 / math.sqrt(128))
    Oref, Lref = run_oracle(q, k, v, None, causal=causal, scale=1 / math.sqrt(128))
    assert_parity(O, L, Oref, Lref, "bf16", f"streaming many blocks qL={qL} causal={causal}")


def test_bool_mask_equals_additive():
    q, k, v = _rand((1, 2, 64, 128), BF16, 8), _rand((1, 2, 96, 128), BF16, 9), _rand((1, 2, 96, 128), BF16, 10)
    attend = torch.from_numpy(np.random.default_rng(11).random((1, 2, 64, 96)) < 0.5)
    attend[..., 3] = True
    add = torch.zeros(attend.shape, dtype=BF16).masked_fill(~attend, float("-inf"))
    O1, L1, _ = run_gpu(q, k, v, attend.to(torch.uint8), scale=0.1)
    O2, L2, _ = run_gpu(q, k, v, add, scale=0.1)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_mask_broadcast_strides():
    """A [1, 1, qL, kL] mask expanded over batch and heads (stride 0) equals the materialised one."""
    q, k, v = _rand((2, 3, 40, 64), BF16, 12), _rand((2, 3, 56, 64), BF16, 13), _rand((2, 3, 56, 64), BF16, 14)
    m = torch.from_numpy(np.where(np.random.default_rng(15).random((1, 1, 40, 56)) < 0.3, -np.inf, 0.0)
                         .astype(np.float32)).to(BF16)
    m[..., 0] = 0
    O1, L1, _ = run_gpu(q, k, v, m.expand(2, 3, 40, 56), scale=0.125)
    O2, L2, _ = run_gpu(q, k, v, m.expand(2, 3, 40, 56).contiguous(), scale=0.125)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
    Oref, Lref = run_oracle(q, k, v, m.expand(2, 3, 40, 56).contiguous(), scale=0.125)
    assert_parity(O1, L1, Oref, Lref, "bf16", "broadcast mask")


@pytest.mark.parametrize("qL,kL", [(1, 1), (1, 300), (300, 1), (64, 500), (500, 64), (129, 33)])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_degenerate_lengths(qL, kL, causal):
    """Single rows/keys and qL != kL; causal is top-left aligned (row i sees keys 0..i)."""
    q, k, v = _rand((1, 2, qL, 64), BF16, 16), _rand((1, 1, kL, 64), BF16, 17), _rand((1, 1, kL, 64), BF16, 18)
    O, L, _ = run_gpu(q, k, v, causal=causal, scale=0.125)
    Oref, Lref = run_oracle(q, k, v, causal=causal, scale=0.125)
    assert_parity(O, L, Oref, Lref, "bf16", f"qL={qL} kL={kL} causal={causal}")


def test_zero_query_closed_form():
    """Q = 0: L_i = ln kL (ln(i+1) causal) and O_i = mean of the visible V rows."""
    kL = 333
    q = torch.zeros((1, 2, 300, 128), dtype=F32)
    k, v = _rand((1, 2, kL, 128), F32, 19), _rand((1, 2, kL, 128), F32, 20)
    O, L, _ = run_gpu(q, k, v, scale=0.3)
    assert max_err(L, np.full(L.shape, math.log(kL))) <= TOL_L
    assert max_err(O, np.broadcast_to(v.double().mean(dim=2, keepdim=True).numpy(), O.shape)) <= TOL_O["f32"]
    O, L, _ = run_gpu(q, k, v, causal=True, scale=0.3)
    i = np.arange(300)
    assert max_err(L, np.broadcast_to(np.log(i + 1.0), L.shape)) <= TOL_L
    csum = np.cumsum(v.double().numpy()[:, :, :300], axis=2) / (i + 1.0)[None, None, :, None]
    assert max_err(O, csum) <= TOL_O["f32"]


def test_dominant_key_closed_form():
    """One key aligned with the query: O -> that key's V row, L = ln(e^sig + n - 1)."""
    n, D, jstar, sig = 257, 64, 100, 30.0
    q = torch.zeros((1, 1, 96, D), dtype=F32)
    q[..., 0] = 1.0
    k = _rand((1, 1, n, D), F32, 21)
    k[..., 0] = 0.0
    k[0, 0, jstar, 0] = sig / 0.5
    v = _rand((1, 1, n, D), F32, 22)
    O, L, _ = run_gpu(q, k, v, scale=0.5)
    den = math.exp(sig) + n - 1
    expO = (math.exp(sig) * v[0, 0, jstar].double() + (v[0, 0].double().sum(0) - v[0, 0, jstar].double())) / den
    assert max_err(L, np.full(L.shape, math.log(den))) <= TOL_L
    assert max_err(O, np.broadcast_to(expO.numpy(), O.shape)) <= TOL_O["f32"]


@pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_row_max_growing_across_tiles(dtype, D, causal):
    """Scores stepping up by 7 (natural units, ~10 in base 2) every 128 keys,
    three times, so the running max is exceeded by more than the slack the
    kernels allow before rescaling O and l, on several tiles of a row (128
    keys span one or more tiles of every launch shape).  16 heads keep the
    grids large enough that the key range is not split into single tiles.
    The scores stay near 20, where fp32 still resolves them to ~1e-6."""
    g = torch.Generator().manual_seed(31)
    qL, kL = 160, 600
    q = torch.randn((1, 16, qL, D), generator=g) * 0.3
    k = torch.randn((1, 4, kL, D), generator=g) * 0.3
    v = torch.randn((1, 4, kL, D), generator=g)
    q[..., 0] = 1.0
    k[..., 0] = torch.clamp(torch.arange(kL) // 128, max=3).to(torch.float32) * (7.0 / 0.125)
    q, k, v = q.to(dtype), k.to(dtype), v.to(dtype)
    O, L, _ = run_gpu(q, k, v, causal=causal, scale=0.125)
    Oref, Lref = run_oracle(q, k, v, causal=causal, scale=0.125)
    assert_parity(O, L, Oref, Lref, dtype_name(q), f"growing max D={D} causal={causal}")


@pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "f32"])
def test_causal_first_row(dtype):
    """Causal row 0 sees only key 0: O_0 = V_0 and L_0 = scale q_0.k_0."""
    q, k, v = _rand((2, 4, 130, 128), dtype, 23), _rand((2, 2, 130, 128), dtype, 24), _rand((2, 2, 130, 128), dtype, 25)
    O, L, _ = run_gpu(q, k, v, causal=True, scale=0.09)
    vr = v.double().repeat_interleave(2, dim=1).numpy()
    kr = k.double().repeat_interleave(2, dim=1)
    s00 = 0.09 * (q.double()[:, :, 0] * kr[:, :, 0]).sum(-1).numpy()
    assert max_err(O[:, :, 0], vr[:, :, 0]) <= (TOL_O[dtype_name(q)] if dtype == BF16 else 1e-6)
    assert max_err(L[:, :, 0], s00) <= TOL_L


def test_gqa_equals_repeated_mha():
    q, k, v = _rand((1, 8, 100, 64), BF16, 26), _rand((1, 2, 120, 64), BF16, 27), _rand((1, 2, 120, 64), BF16, 28)
    O1, L1, _ = run_gpu(q, k, v, causal=True, scale=0.125)
    O2, L2, _ = run_gpu(q, k.repeat_interleave(4, dim=1), v.repeat_interleave(4, dim=1), causal=True, scale=0.125)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_token_major_equals_head_major():
    q, k, v = _rand((2, 3, 77, 128), F32, 29), _rand((2, 3, 91, 128), F32, 30), _rand((2, 3, 91, 128), F32, 31)
    O1, L1, raw = run_gpu(q, k, v, scale=0.1, token_major=True)
    O2, L2, _ = run_gpu(q, k, v, scale=0.1)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
    assert raw.stride() == (77 * 3 * 128, 128, 3 * 128, 1)


@pytest.mark.parametrize("B,Hq,Hkv,qL,kL,D,causal,kind", [
    (1, 4, 2, 1000, 700, 128, False, "none"),    # 8-wave work-groups, ragged last query tile
    (1, 4, 2, 333, 1111, 128, True, "bool"),
    (2, 16, 4, 600, 600, 64, True, "none"),      # grid resident at once: causal key halves
    (1, 6, 3, 777, 300, 64, False, "additive"),
    (1, 16, 4, 2000, 300, 256, False, "none"),   # D = 256 work-group kernel (256 query tiles)
    (1, 16, 8, 2047, 129, 256, True, "additive"),
], ids=lambda x: str(x))
def test_whole_line_output_stores(B, Hq, Hkv, qL, kL, D, causal, kind):
    """The unsplit epilogue passes O through LDS and stores whole lines of 8
    rows: token-major and head-major O, ragged query ranges (rows past qL
    are not written: the buffer's guard rows keep their sentinel), against
    the oracle and each other."""
    print(f"[case] whole-line O B={B} Hq={Hq} Hkv={Hkv} qL={qL} kL={kL} D={D} causal={causal} mask={kind}",
          flush=True)
    q, k, v = _rand((B, Hq, qL, D), BF16, 95), _rand((B, Hkv, kL, D), BF16, 96), _rand((B, Hkv, kL, D), BF16, 97)
    mask = None
    if kind != "none":
        rng = np.random.default_rng(98)
        masked = W.draw_masked(rng, (B, Hq, qL, kL), 0.3)
        if kind == "bool":
            mask = torch.from_numpy((~masked).astype(np.uint8))
        else:
            m = rng.standard_normal(masked.shape).astype(np.float32)
            m[masked] = -np.inf
            mask = torch.from_numpy(m).to(BF16)
    scale = 1 / math.sqrt(D)
    dev = torch.device("cuda:0")
    # token-major O inside a buffer with one guard row on each side
    buf = torch.full((B, qL + 2, Hq, D), 7.0, dtype=BF16, device=dev)
    out = buf[:, 1:qL + 1].transpose(1, 2)
    O1, L1, _ = run_gpu(q, k, v, mask, causal=causal, scale=scale, out=out)
    O2, L2, _ = run_gpu(q, k, v, mask, causal=causal, scale=scale)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
    g = buf.float().cpu()
    assert torch.all(g[:, 0] == 7.0) and torch.all(g[:, qL + 1] == 7.0)
    Oref, Lref = run_oracle(q, k, v, mask, causal=causal, scale=scale)
    assert_parity(O2, L2, Oref, Lref, "bf16", f"whole-line O qL={qL} kL={kL} D={D}")


def test_negative_and_zero_scale():
    q, k, v = _rand((1, 2, 64, 64), BF16, 32), _rand((1, 2, 80, 64), BF16, 33), _rand((1, 2, 80, 64), BF16, 34)
    for scale in (-0.2, 0.0):
        O, L, _ = run_gpu(q, k, v, scale=scale)
        Oref, Lref = run_oracle(q, k, v, scale=scale)
        assert_parity(O, L, Oref, Lref, "bf16", f"scale={scale}")


def test_strided_inputs():
    """q, k, v as strided views (a packed [B, L, 3, H, D] projection) give the same result."""
    B, Lx, H, D = 1, 150, 4, 64
    packed = _rand((B, Lx, 3, H, D), BF16, 35)
    q, k, v = (packed[:, :, i].transpose(1, 2) for i in range(3))
    O1, L1, _ = run_gpu(q, k, v, causal=True, scale=0.125)
    O2, L2, _ = run_gpu(q.contiguous(), k.contiguous(), v.contiguous(), causal=True, scale=0.125)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_repeat_calls_are_deterministic():
    w = W.C2
    q, k, v, _ = W.draw(w)
    O1, L1, _ = run_gpu(q, k, v, causal=True, scale=w.scale)
    O2, L2, _ = run_gpu(q, k, v, causal=True, scale=w.scale)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


@pytest.mark.parametrize("kL,causal", [(64, False), (320, True)], ids=["stream_kL64", "workgroup_kL320_causal"])
def test_tensors_past_2pow31_elements(kL, causal):
    """Maximum sizes: Q and O hold more than 2^31 elements each (byte offsets
    past 2^32), so every row offset must be computed in 64 bits.  Rows are
    sampled across the whole range, the very last row included, and checked
    against the oracle on that row's allowed keys (top-left causal: keys
    0..i); every row must be finite and inside the range of its head's V."""
    B, Hq, Hkv, D = 1, 32, 8, 128
    qL = (1 << 31) // (Hq * D) + 4096
    scale = 1 / math.sqrt(D)
    print(f"[case] large B={B} Hq={Hq} Hkv={Hkv} qL={qL} kL={kL} D={D} bf16 causal={causal} seed=31", flush=True)
    assert B * Hq * qL * D > (1 << 31)
    dev = torch.device("cuda:0")
    gq = torch.Generator(device=dev).manual_seed(31)
    q = torch.randn((B, Hq, qL, D), generator=gq, device=dev, dtype=torch.bfloat16)
    k = _rand((B, Hkv, kL, D), BF16, 32)
    v = _rand((B, Hkv, kL, D), BF16, 33)
    O, L = fa.fwd(q, k.to(dev), v.to(dev), causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(O).all()) and bool(torch.isfinite(L).all())
    grp = Hq // Hkv
    vmin, vmax = v.float().amin(dim=2), v.float().amax(dim=2)  # [B, Hkv, D]
    for h in range(Hq):
        oh = O[0, h].float()
        lo, hi = vmin[0, h // grp].to(dev), vmax[0, h // grp].to(dev)
        assert bool((oh >= lo - TOL_O["bf16"]).all()) and bool((oh <= hi + TOL_O["bf16"]).all()), f"head {h}"
        del oh
    rng = np.random.default_rng(34)
    picks = [(0, 0), (Hq - 1, qL - 1), (Hq - 1, qL - 2), (Hq // 2, qL // 2), (0, kL - 1), (0, min(kL, qL - 1))]
    picks += [(int(rng.integers(Hq)), int(rng.integers(qL))) for _ in range(40)]
    errs_o, errs_l = [], []
    for h, i in picks:
        n = min(i + 1, kL) if causal else kL
        qi = q[0, h, i].cpu().reshape(1, 1, 1, D)
        ki, vi = k[:, h // grp: h // grp + 1, :n], v[:, h // grp: h // grp + 1, :n]
        Oref, Lref = run_oracle(qi, ki, vi, causal=False, scale=scale)
        errs_o.append(max_err(O[0, h, i].double().cpu().numpy(), Oref.reshape(D)))
        errs_l.append(abs(float(L[0, h, i]) - float(Lref.reshape(()))))
    print(f"[parity] large kL={kL}: max|dO| = {max(errs_o):.3e}, max|dL| = {max(errs_l):.3e} over {len(picks)} rows",
          flush=True)
    assert max(errs_o) <= TOL_O["bf16"] and max(errs_l) <= TOL_L


@pytest.mark.parametrize("B,Hq,Hkv,qL,kL,D,kind,causal", [
    (1, 8, 2, 1, 4096, 128, "none", False),
    (1, 8, 2, 16, 4100, 128, "none", False),
    (2, 4, 4, 64, 3000, 64, "additive", False),
    (1, 8, 8, 16, 4096, 128, "bool", False),
    (1, 6, 3, 40, 5000, 96, "none", False),
    (1, 4, 2, 24, 3333, 16, "additive", False),
    (1, 2, 1, 2048, 2048, 128, "none", True),
    (1, 2, 2, 1500, 1600, 64, "bool", True),
    (1, 2, 2, 1024, 1100, 256, "bool", True),
    (1, 3, 1, 200, 2000, 256, "additive", False),
], ids=lambda x: str(x))
def test_key_range_split_over_work_groups(B, Hq, Hkv, qL, kL, D, kind, causal):
    """Small grids with long key ranges: the key range is split over
    work-groups and the partials merged (L = ln sum e^{L_s}).  Causal shapes
    leave later ranges partly or wholly above the diagonal (empty ranges
    weigh 0), and one row has no allowed key in any range."""
    print(f"[case] split B={B} Hq={Hq} Hkv={Hkv} qL={qL} kL={kL} D={D} mask={kind} causal={causal}", flush=True)
    q, k, v = _rand((B, Hq, qL, D), BF16, 41), _rand((B, Hkv, kL, D), BF16, 42), _rand((B, Hkv, kL, D), BF16, 43)
    mask = None
    if kind != "none":
        rng = np.random.default_rng(44)
        masked = W.draw_masked(rng, (B, Hq, qL, kL), 0.3)
        masked[0, Hq - 1, qL // 2, :] = True  # no allowed key in any range
        if kind == "bool":
            mask = torch.from_numpy((~masked).astype(np.uint8))
        else:
            m = rng.standard_normal(masked.shape).astype(np.float32)
            m[masked] = -np.inf
            mask = torch.from_numpy(m).to(BF16)
    scale = 1 / math.sqrt(D)
    O, L, _ = run_gpu(q, k, v, mask, causal=causal, scale=scale)
    Oref, Lref = run_oracle(q, k, v, mask, causal=causal, scale=scale)
    assert_parity(O, L, Oref, Lref, "bf16", f"split qL={qL} kL={kL} D={D} {kind} causal={causal}")
    if kind != "none":
        assert np.all(O[0, Hq - 1, qL // 2] == 0) and L[0, Hq - 1, qL // 2] == 0


@pytest.mark.parametrize("B,Hq,Hkv,qL,kL,D,kind,causal", [
    (1, 8, 2, 1, 4096, 128, "none", False),
    (1, 8, 2, 16, 4100, 128, "none", False),
    (2, 4, 4, 64, 3000, 64, "additive", False),
    (1, 8, 8, 16, 4096, 32, "bool", False),
    (1, 6, 3, 40, 5000, 96, "none", False),
    (1, 2, 1, 1024, 2048, 128, "none", True),
    (1, 2, 2, 1500, 1600, 80, "bool", True),
    (1, 3, 1, 100, 2000, 256, "additive", False),
], ids=lambda x: str(x))
def test_key_range_split_over_work_groups_f32(B, Hq, Hkv, qL, kL, D, kind, causal):
    """The fp32 kernel's key-range split: small grids with long key ranges,
    fp32 partials merged by L = ln sum e^{L_s}; empty causal ranges and a row
    with no allowed key in any range."""
    print(f"[case] f32 split B={B} Hq={Hq} Hkv={Hkv} qL={qL} kL={kL} D={D} mask={kind} causal={causal}", flush=True)
    q, k, v = _rand((B, Hq, qL, D), F32, 45), _rand((B, Hkv, kL, D), F32, 46), _rand((B, Hkv, kL, D), F32, 47)
    mask = None
    if kind != "none":
        rng = np.random.default_rng(48)
        masked = W.draw_masked(rng, (B, Hq, qL, kL), 0.3)
        masked[0, Hq - 1, qL // 2, :] = True  # no allowed key in any range
        if kind == "bool":
            mask = torch.from_numpy((~masked).astype(np.uint8))
        else:
            m = rng.standard_normal(masked.shape).astype(np.float32)
            m[masked] = -np.inf
            mask = torch.from_numpy(m)
    scale = 1 / math.sqrt(D)
    O, L, _ = run_gpu(q, k, v, mask, causal=causal, scale=scale)
    Oref, Lref = run_oracle(q, k, v, mask, causal=causal, scale=scale)
    assert_parity(O, L, Oref, Lref, "f32", f"f32 split qL={qL} kL={kL} D={D} {kind} causal={causal}")
    if kind != "none":
        assert np.all(O[0, Hq - 1, qL // 2] == 0) and L[0, Hq - 1, qL // 2] == 0


@pytest.mark.parametrize("B,Hq,Hkv,qL,kL,D,kind,causal", [
    (1, 8, 2, 1, 300, 64, "none", False),
    (2, 16, 2, 7, 5000, 128, "additive", False),
    (1, 8, 2, 16, 2048, 128, "bool", True),
    (1, 4, 1, 3, 777, 16, "none", False),
    (1, 12, 3, 16, 4096, 80, "additive", False),
    (1, 8, 2, 16, 4096, 256, "none", False),
    (1, 4, 1, 16, 9000, 128, "bool", False),
], ids=lambda x: str(x))
def test_packed_short_queries_f32(B, Hq, Hkv, qL, kL, D, kind, causal):
    """The fp32 kernel's packed shape (at most 16 query rows, GQA groups of a
    multiple of 4): a wave holds 16 rows of each of two heads, a work-group
    four heads of one group; split and unsplit key ranges, every mask kind,
    causal, and a row with no allowed key."""
    print(f"[case] f32 packed B={B} Hq={Hq} Hkv={Hkv} qL={qL} kL={kL} D={D} mask={kind} causal={causal}", flush=True)
    q, k, v = _rand((B, Hq, qL, D), F32, 55), _rand((B, Hkv, kL, D), F32, 56), _rand((B, Hkv, kL, D), F32, 57)
    mask = None
    if kind != "none":
        rng = np.random.default_rng(58)
        masked = W.draw_masked(rng, (B, Hq, qL, kL), 0.3)
        masked[0, Hq - 1, qL // 2, :] = True  # no allowed key
        if kind == "bool":
            mask = torch.from_numpy((~masked).astype(np.uint8))
        else:
            m = rng.standard_normal(masked.shape).astype(np.float32)
            m[masked] = -np.inf
            mask = torch.from_numpy(m)
    scale = 1 / math.sqrt(D)
    O, L, _ = run_gpu(q, k, v, mask, causal=causal, scale=scale)
    Oref, Lref = run_oracle(q, k, v, mask, causal=causal, scale=scale)
    assert_parity(O, L, Oref, Lref, "f32", f"f32 packed qL={qL} kL={kL} D={D} {kind} causal={causal}")
    if kind != "none":
        assert np.all(O[0, Hq - 1, qL // 2] == 0) and L[0, Hq - 1, qL // 2] == 0


@pytest.mark.parametrize("B,Hq,Hkv,qL,kL,D,kind,causal", [
    (1, 8, 2, 1, 300, 64, "none", False),
    (2, 16, 2, 7, 5000, 128, "additive", False),
    (1, 8, 2, 16, 2048, 128, "bool", True),
    (1, 4, 1, 3, 777, 16, "none", False),
    (1, 8, 1, 11, 1500, 32, "bool", False),
    (1, 4, 1, 16, 2100, 48, "additive", True),
    (1, 12, 3, 16, 4096, 80, "additive", False),
    (2, 8, 2, 9, 6000, 96, "none", False),
    (1, 8, 2, 16, 4096, 256, "none", False),
    (1, 8, 2, 5, 3001, 256, "bool", False),
    (1, 4, 1, 16, 9000, 128, "bool", False),
    (1, 32, 8, 16, 32768, 128, "none", False),
], ids=lambda x: str(x))
def test_packed_short_queries_bf16(B, Hq, Hkv, qL, kL, D, kind, causal):
    """The bf16 kernel's packed shape (at most 16 query rows, GQA groups of a
    multiple of 4): a wave holds 16 rows of each of two heads, a work-group
    four heads of one group; split and unsplit key ranges, every mask kind,
    causal, every head dimension, and a row with no allowed key."""
    print(f"[case] bf16 packed B={B} Hq={Hq} Hkv={Hkv} qL={qL} kL={kL} D={D} mask={kind} causal={causal}",
          flush=True)
    q, k, v = _rand((B, Hq, qL, D), BF16, 65), _rand((B, Hkv, kL, D), BF16, 66), _rand((B, Hkv, kL, D), BF16, 67)
    mask = None
    if kind != "none":
        rng = np.random.default_rng(68)
        masked = W.draw_masked(rng, (B, Hq, qL, kL), 0.3)
        masked[0, Hq - 1, qL // 2, :] = True  # no allowed key
        if kind == "bool":
            mask = torch.from_numpy((~masked).astype(np.uint8))
        else:
            m = rng.standard_normal(masked.shape).astype(np.float32)
            m[masked] = -np.inf
            mask = torch.from_numpy(m).to(BF16)
    scale = 1 / math.sqrt(D)
    O, L, _ = run_gpu(q, k, v, mask, causal=causal, scale=scale)
    Oref, Lref = run_oracle(q, k, v, mask, causal=causal, scale=scale)
    assert_parity(O, L, Oref, Lref, "bf16", f"bf16 packed qL={qL} kL={kL} D={D} {kind} causal={causal}")
    if kind != "none":
        assert np.all(O[0, Hq - 1, qL // 2] == 0) and L[0, Hq - 1, qL // 2] == 0


@pytest.mark.parametrize("Hq,Hkv,qL,kL,D,kind,causal", [
    (8, 4, 1, 4096, 128, "none", False),
    (8, 2, 17, 3000, 128, "additive", False),
    (9, 3, 32, 5000, 64, "none", False),
    (32, 4, 5, 2500, 96, "bool", False),
    (4, 2, 32, 100, 128, "none", False),
    (6, 2, 20, 333, 256, "additive", False),
    (4, 1, 32, 32, 64, "none", True),
    (8, 2, 24, 1000, 128, "bool", True),
], ids=lambda x: str(x))
def test_short_query_ranges_pack_gqa_heads(Hq, Hkv, qL, kL, D, kind, causal):
    """At most 32 query rows in a GQA group: one work-group takes the rows of
    two query heads of the group (one per wave; a group of odd size leaves a
    wave idle), with and without a split of the key range."""
    print(f"[case] pack Hq={Hq} Hkv={Hkv} qL={qL} kL={kL} D={D} mask={kind} causal={causal}", flush=True)
    q, k, v = _rand((2, Hq, qL, D), BF16, 51), _rand((2, Hkv, kL, D), BF16, 52), _rand((2, Hkv, kL, D), BF16, 53)
    mask = None
    if kind != "none":
        rng = np.random.default_rng(54)
        masked = W.draw_masked(rng, (2, Hq, qL, kL), 0.3)
        masked[1, Hq - 1, qL - 1, :] = True  # no allowed key
        if kind == "bool":
            mask = torch.from_numpy((~masked).astype(np.uint8))
        else:
            m = rng.standard_normal(masked.shape).astype(np.float32)
            m[masked] = -np.inf
            mask = torch.from_numpy(m).to(BF16)
    scale = 1 / math.sqrt(D)
    O, L, _ = run_gpu(q, k, v, mask, causal=causal, scale=scale)
    Oref, Lref = run_oracle(q, k, v, mask, causal=causal, scale=scale)
    assert_parity(O, L, Oref, Lref, "bf16", f"pack Hq={Hq}/{Hkv} qL={qL} kL={kL} D={D} {kind} causal={causal}")
    if kind != "none":
        assert np.all(O[1, Hq - 1, qL - 1] == 0) and L[1, Hq - 1, qL - 1] == 0


@pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "f32"])
@pytest.mark.parametrize("D", [16, 32, 48, 64, 80, 96, 128, 256])
@pytest.mark.parametrize("p", [0.0, 0.25, 1.0])
@pytest.mark.parametrize("B,Hq,Hkv,qL,kL,causal,kind", [
    (1, 2, 1, 130, 256, False, "none"),
    (2, 4, 2, 77, 203, True, "none"),
    (1, 2, 2, 64, 150, False, "bool"),
    (1, 4, 1, 16, 4096, False, "additive"),
], ids=lambda x: str(x))
def test_dropout_matches_the_oracle(D, p, B, Hq, Hkv, qL, kL, causal, kind, dtype):
    """Dropout on the attention weights: the keep mask is drawn from the same
    Philox-4x32-10 positions on both sides, so O matches element by element;
    L is the one without dropout.  kL = 203 and 150 put rows at offsets that
    are not multiples of 4 (two generator blocks per 4 keys); 16 rows over
    4096 keys split the key range over work-groups."""
    seed, offset = 0x9E3779B97F4A7C15, (1 << 33) + 5
    print(f"[case] dropout p={p} B={B} Hq={Hq} Hkv={Hkv} qL={qL} kL={kL} D={D} mask={kind} causal={causal} {dtype}",
          flush=True)
    q, k, v = _rand((B, Hq, qL, D), dtype, 61), _rand((B, Hkv, kL, D), dtype, 62), _rand((B, Hkv, kL, D), dtype, 63)
    mask = None
    if kind != "none":
        rng = np.random.default_rng(64)
        masked = W.draw_masked(rng, (B, Hq, qL, kL), 0.3)
        if kind == "bool":
            mask = torch.from_numpy((~masked).astype(np.uint8))
        else:
            m = rng.standard_normal(masked.shape).astype(np.float32)
            m[masked] = -np.inf
            mask = torch.from_numpy(m).to(dtype)
    scale = 1 / math.sqrt(D)
    dev = torch.device("cuda:0")
    Od, Ld = fa.fwd(q.to(dev), k.to(dev), v.to(dev), mask=None if mask is None else mask.to(dev), causal=causal,
                    scale=scale, dropout_p=p, seed=seed, offset=offset)
    torch.cuda.synchronize()
    Od, Ld = Od.double().cpu().numpy(), Ld.double().cpu().numpy()
    kindname = "none" if mask is None else ("bool" if kind == "bool" else "additive")
    m_np = None if mask is None else (mask.numpy() if kind == "bool" else mask.double().numpy())
    Oref, Lref = attention_fwd(q.double().numpy(), k.double().numpy(), v.double().numpy(), scale=scale, causal=causal,
                               mask=m_np, mask_kind=kindname, dropout_p=p, seed=seed, offset=offset)
    _, Lplain = run_oracle(q, k, v, mask, causal=causal, scale=scale)
    assert_parity(Od, Ld, Oref, Lref, "bf16" if dtype == BF16 else "f32",
                  f"dropout p={p} qL={qL} kL={kL} D={D} {kind} causal={causal}")
    assert np.max(np.abs(Ld - Lplain)) <= TOL_L
    if p == 1.0:
        assert np.all(Od == 0)


def test_dropout_rejects_bad_rates():
    dev = torch.device("cuda:0")
    q = torch.zeros((1, 1, 8, 64), dtype=BF16, device=dev)
    for bad in (-0.1, 1.5, float("nan")):
        with pytest.raises(fa.FaError):
            fa.fwd(q, q, q, dropout_p=bad)


def test_split_over_more_ranges_than_lanes():
    """One query tile of one head over 65536 keys: the key range splits over
    more work-groups than a wave has lanes (128 ranges), so the merge's
    per-lane loops over the ranges take several turns."""
    print("[case] split 1 head qL=16 kL=65536 D=128", flush=True)
    q, k, v = _rand((1, 1, 16, 128), BF16, 71), _rand((1, 1, 65536, 128), BF16, 72), _rand((1, 1, 65536, 128), BF16, 73)
    O, L, _ = run_gpu(q, k, v, scale=1 / math.sqrt(128))
    Oref, Lref = run_oracle(q, k, v, scale=1 / math.sqrt(128))
    assert_parity(O, L, Oref, Lref, "bf16", "split into 128 ranges")


@pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "f32"])
@pytest.mark.parametrize("D", [16, 64, 128, 256])
@pytest.mark.parametrize("kL", [2048, 4096, 8192, 16384, 40000])
def test_split_merge_range_counts(kL, D, dtype):
    """One head, one query tile: the number of key ranges grows with kL
    (about kL / 512 up to the GPU's fill), so the merge runs with one, two
    and four waves per row and with every lane layout of a partial row.  A
    bool mask leaves one query row a single allowed key near the end and
    another only keys of the first range, so most ranges weigh 0 there."""
    print(f"[case] merge kL={kL} D={D} {dtype}", flush=True)
    q, k, v = _rand((1, 1, 64, D), dtype, 91), _rand((1, 1, kL, D), dtype, 92), _rand((1, 1, kL, D), dtype, 93)
    allow = np.ones((1, 1, 64, kL), dtype=np.uint8)
    allow[0, 0, 5, :] = 0
    allow[0, 0, 5, kL - 3] = 1
    allow[0, 0, 9, 300:] = 0
    mask = torch.from_numpy(allow)
    scale = 1 / math.sqrt(D)
    O, L, _ = run_gpu(q, k, v, mask, scale=scale)
    Oref, Lref = run_oracle(q, k, v, mask, scale=scale)
    assert_parity(O, L, Oref, Lref, "bf16" if dtype == BF16 else "f32", f"merge kL={kL} D={D}")


@pytest.mark.parametrize("B,Hq,Hkv,qL,kL,D,window,kind", [
    (1, 4, 2, 1000, 1000, 128, 256, "none"),    # ragged, several tiles inside the window
    (1, 4, 4, 777, 900, 64, 1, "none"),         # the diagonal only
    (2, 4, 2, 520, 520, 64, 100, "none"),       # window edge inside tiles and waves
    (1, 2, 1, 300, 300, 256, 64, "none"),       # D = 256 (work-group kernel, never the key split)
    (1, 4, 2, 300, 333, 16, 33, "none"),
    (1, 4, 2, 600, 600, 96, 129, "none"),
    (1, 8, 2, 24, 4000, 128, 7, "none"),        # 32-row tiles packing GQA heads
    (1, 4, 2, 48, 48, 128, 10, "none"),         # 2-wave short-query shape
    (1, 2, 2, 100, 100, 128, 5, "none"),        # short keys (not the streaming kernel)
    (1, 4, 2, 1000, 300, 64, 40, "none"),       # rows past kL + window see no key
    (1, 4, 2, 400, 500, 64, 70, "additive"),
    (1, 2, 1, 333, 333, 128, 200, "bool"),
    (1, 2, 2, 257, 257, 80, 64, "bool"),
], ids=lambda x: str(x))
@pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "f32"])
def test_sliding_window_matches_the_oracle(B, Hq, Hkv, qL, kL, D, window, kind, dtype):
    """Causal sliding window (row i sees keys i - window + 1 .. i), element by
    element against the oracle; rows with no key give O = 0, L = 0 on both sides."""
    print(f"[case] window={window} B={B} Hq={Hq} Hkv={Hkv} qL={qL} kL={kL} D={D} mask={kind} {dtype}", flush=True)
    q, k, v = _rand((B, Hq, qL, D), dtype, 81), _rand((B, Hkv, kL, D), dtype, 82), _rand((B, Hkv, kL, D), dtype, 83)
    mask = None
    if kind != "none":
        rng = np.random.default_rng(84)
        masked = W.draw_masked(rng, (B, Hq, qL, kL), 0.3)
        if kind == "bool":
            mask = torch.from_numpy((~masked).astype(np.uint8))
        else:
            m = rng.standard_normal(masked.shape).astype(np.float32)
            m[masked] = -np.inf
            mask = torch.from_numpy(m).to(dtype)
    scale = 1 / math.sqrt(D)
    dev = torch.device("cuda:0")
    Od, Ld = fa.fwd(q.to(dev), k.to(dev), v.to(dev), mask=None if mask is None else mask.to(dev), causal=True,
                    scale=scale, window=window)
    torch.cuda.synchronize()
    Od, Ld = Od.double().cpu().numpy(), Ld.double().cpu().numpy()
    m_np = None if mask is None else (mask.numpy() if kind == "bool" else mask.double().numpy())
    Oref, Lref = attention_fwd(q.double().numpy(), k.double().numpy(), v.double().numpy(), scale=scale, causal=True,
                               mask=m_np, mask_kind=kind, window=window)
    assert_parity(Od, Ld, Oref, Lref, "bf16" if dtype == BF16 else "f32",
                  f"window={window} qL={qL} kL={kL} D={D} {kind}")
    empty = np.all(Oref == 0, axis=-1) & (Lref == 0)
    assert np.all(Od[empty] == 0) and np.all(Ld[empty] == 0)


@pytest.mark.parametrize("qL,D", [(2048, 128), (300, 64)])
def test_a_window_past_every_row_is_plain_causal(qL, D):
    """window >= qL + 32 takes no tile off the range and masks nothing more:
    the result is the plain causal one, bit for bit.  32 heads keep the grid
    large enough that the plain call does not split its key range over
    work-groups (a windowed call never does)."""
    dev = torch.device("cuda:0")
    q = _rand((1, 32, qL, D), BF16, 85).to(dev)
    k, v = (_rand((1, 8, qL, D), BF16, s).to(dev) for s in (86, 87))
    O0, L0 = fa.fwd(q, k, v, causal=True)
    O1, L1 = fa.fwd(q, k, v, causal=True, window=qL + 64)
    torch.cuda.synchronize()
    assert torch.equal(O0, O1) and torch.equal(L0, L1)


def test_window_rejects_bad_arguments():
    dev = torch.device("cuda:0")
    q = torch.zeros((1, 1, 8, 64), dtype=BF16, device=dev)
    with pytest.raises(fa.FaError, match="window"):
        fa.fwd(q, q, q, causal=True, window=0)
    with pytest.raises(fa.FaError, match="causal"):
        fa.fwd(q, q, q, causal=False, window=4)


def _default_pool_release_threshold():
    """The release threshold of the current device's default memory pool,
    read through the HIP runtime (hipDeviceGetDefaultMemPool,
    hipMemPoolGetAttribute with hipMemPoolAttrReleaseThreshold)."""
    import ctypes

    hip = ctypes.CDLL("libamdhip64.so")
    dev = ctypes.c_int(0)
    assert hip.hipGetDevice(ctypes.byref(dev)) == 0
    pool = ctypes.c_void_p()
    assert hip.hipDeviceGetDefaultMemPool(ctypes.byref(pool), dev) == 0
    value = ctypes.c_uint64(0)
    hip_mem_pool_attr_release_threshold = 4
    assert hip.hipMemPoolGetAttribute(pool, hip_mem_pool_attr_release_threshold, ctypes.byref(value)) == 0
    return value.value


def test_split_launch_leaves_the_default_pool_alone():
    """A split launch takes its partials from the library's own pool: the
    device's default pool keeps the release threshold the caller gave it."""
    torch.zeros(1, device="cuda:0")
    before = _default_pool_release_threshold()
    w = W.SPLIT_KV[0]
    q, k, v, _ = _draw(w)
    O, L, _ = run_gpu(q, k, v, None, causal=w.causal, scale=w.scale)
    assert np.all(np.isfinite(O))
    assert _default_pool_release_threshold() == before


def test_split_workspace_reuse_across_streams():
    """Split launches keep their partials in a workspace per (device, stream)
    that grows when a call needs more: calls of growing and shrinking size,
    bf16 and fp32, enqueued on two streams without synchronising in between,
    and calls on more streams than the library keeps workspaces for, match
    the same calls run one by one (bit for bit) and the oracle."""
    dev = torch.device("cuda:0")
    shapes = [(32, 8, 16, 8192, 128, BF16), (32, 8, 16, 32768, 128, BF16), (8, 2, 5, 3000, 64, F32),
              (16, 4, 16, 20000, 256, BF16), (32, 8, 1, 12000, 128, BF16), (8, 2, 16, 9000, 128, F32)]
    cases = []
    for i, (Hq, Hkv, qL, kL, D, dt) in enumerate(shapes):
        q, k, v = _rand((1, Hq, qL, D), dt, 300 + i), _rand((1, Hkv, kL, D), dt, 310 + i), _rand((1, Hkv, kL, D), dt, 320 + i)
        cases.append((q.to(dev), k.to(dev), v.to(dev), 1 / math.sqrt(D)))
    # one by one on the current stream
    ref = []
    for qd, kd, vd, sc in cases:
        O, L = fa.fwd(qd, kd, vd, scale=sc)
        torch.cuda.synchronize()
        ref.append((O.clone(), L.clone()))
    # interleaved on two streams, twice over, no synchronisation in between
    s1, s2 = torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)
    outs = []
    for rep in range(2):
        for i, (qd, kd, vd, sc) in enumerate(cases):
            st = s1 if (i + rep) % 2 == 0 else s2
            with torch.cuda.stream(st):
                outs.append(fa.fwd(qd, kd, vd, scale=sc, stream=st))
    torch.cuda.synchronize()
    for j, (O, L) in enumerate(outs):
        Or, Lr = ref[j % len(cases)]
        assert torch.equal(O, Or) and torch.equal(L, Lr), f"call {j} differs from the same call run alone"
    # more streams than the library keeps workspaces for: the rest take
    # their partials from the pool per call
    extra = [torch.cuda.Stream(device=dev) for _ in range(10)]
    outs = []
    for j, st in enumerate(extra):
        qd, kd, vd, sc = cases[j % len(cases)]
        with torch.cuda.stream(st):
            outs.append(fa.fwd(qd, kd, vd, scale=sc, stream=st))
    torch.cuda.synchronize()
    for j, (O, L) in enumerate(outs):
        Or, Lr = ref[j % len(cases)]
        assert torch.equal(O, Or) and torch.equal(L, Lr), f"extra-stream call {j} differs"
    # and the results themselves, against the oracle
    for (qd, kd, vd, sc), (Or, Lr) in zip(cases, ref):
        q, k, v = qd.cpu(), kd.cpu(), vd.cpu()
        Oref, Lref = run_oracle(q, k, v, scale=sc)
        assert_parity(Or.double().cpu().numpy(), Lr.double().cpu().numpy(), Oref, Lref, dtype_name(q),
                      f"workspace case qL={q.shape[2]} kL={k.shape[2]} D={q.shape[3]}")


@pytest.mark.parametrize("D", [16, 32, 48, 64])
@pytest.mark.parametrize("kind", ["none", "additive", "bool"])
@pytest.mark.parametrize("B,Hq,Hkv,qL,kL", [(1, 40, 8, 600, 600), (2, 24, 6, 700, 650), (1, 36, 4, 1100, 1025)],
                         ids=lambda x: str(x))
def test_causal_key_halves(D, kind, B, Hq, Hkv, qL, kL):
    """Causal grids that fit on the GPU at once but are too large to split over
    work-groups take the work-group kernel with its key range walked in two
    halves side by side, merged through LDS (odd tile counts leave half 1 one
    tile short, or empty on the first row block)."""
    print(f"[case] key halves B={B} Hq={Hq} Hkv={Hkv} qL={qL} kL={kL} D={D} mask={kind}", flush=True)
    q, k, v = _rand((B, Hq, qL, D), BF16, 51), _rand((B, Hkv, kL, D), BF16, 52), _rand((B, Hkv, kL, D), BF16, 53)
    mask = None
    if kind != "none":
        rng = np.random.default_rng(54)
        masked = W.draw_masked(rng, (B, Hq, qL, kL), 0.3)
        masked[0, Hq - 1, qL // 2, :] = True  # a row with no allowed key
        if kind == "bool":
            mask = torch.from_numpy((~masked).astype(np.uint8))
        else:
            m = rng.standard_normal(masked.shape).astype(np.float32)
            m[masked] = -np.inf
            mask = torch.from_numpy(m).to(BF16)
    scale = 1 / math.sqrt(D)
    O, L, _ = run_gpu(q, k, v, mask, causal=True, scale=scale)
    Oref, Lref = run_oracle(q, k, v, mask, causal=True, scale=scale)
    assert_parity(O, L, Oref, Lref, "bf16", f"key halves qL={qL} kL={kL} D={D} {kind}")
    if kind != "none":
        assert np.all(O[0, Hq - 1, qL // 2] == 0) and L[0, Hq - 1, qL // 2] == 0
