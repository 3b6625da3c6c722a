"""ctypes wrapper around fa_oracle.c (the fp64 CPU attention reference).

TEST INFRASTRUCTURE ONLY.  See fa_oracle.c for what is computed and which
passages of the pages each step follows.  This wrapper only converts arrays
to contiguous fp64, broadcasts a mask to its full [B, Hq, qL, kL] shape and
passes pointers; no attention arithmetic happens here.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fa_oracle.c")
LIB = os.path.join(HERE, "libfa_oracle.so")

MASK_KINDS = {"none": 0, "additive": 1, "bool": 2}


def build_oracle(src: str = SRC, out: str = LIB) -> str:
    """Compile the oracle with gcc (host only, OpenMP).  Returns the .so path."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O3", "-fopenmp", "-shared", "-fPIC", "-std=c99", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


class OracleLib:
    """One loaded copy of a compiled oracle (the tests also load planted mutants)."""

    def __init__(self, path: str = LIB):
        if path == LIB and not os.path.exists(path):
            build_oracle()
        self.path = path
        self.lib = ctypes.CDLL(path)
        f = self.lib.fa_oracle_fwd
        dp = ctypes.POINTER(ctypes.c_double)
        f.argtypes = [dp, dp, dp, dp, ctypes.c_int,
                      ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                      ctypes.c_int, ctypes.c_double, ctypes.c_int,
                      ctypes.POINTER(ctypes.c_int64), ctypes.c_int64, dp, dp]
        f.restype = ctypes.c_int
        fd = self.lib.fa_oracle_fwd_dropout
        fd.argtypes = list(f.argtypes) + [ctypes.c_float, ctypes.c_uint64, ctypes.c_uint64]
        fd.restype = ctypes.c_int
        fw = self.lib.fa_oracle_fwd_window
        fw.argtypes = list(f.argtypes) + [ctypes.c_int]
        fw.restype = ctypes.c_int
        u32p = ctypes.POINTER(ctypes.c_uint32)
        self.lib.fa_oracle_philox4x32_10.argtypes = [u32p, u32p, u32p]
        self.lib.fa_oracle_philox4x32_10.restype = None
        self.lib.fa_oracle_dropout_multiplier.argtypes = [ctypes.c_int64, ctypes.c_float, ctypes.c_uint64,
                                                          ctypes.c_uint64]
        self.lib.fa_oracle_dropout_multiplier.restype = ctypes.c_double
        self.lib.fa_oracle_threads.restype = ctypes.c_int
        fb = self.lib.fa_oracle_bwd
        i64p = ctypes.POINTER(ctypes.c_int64)
        fb.argtypes = [dp, dp, dp, dp, dp, ctypes.c_int,
                       ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                       ctypes.c_double, ctypes.c_int, i64p, ctypes.c_int64, i64p, ctypes.c_int64, dp, dp, dp]
        fb.restype = ctypes.c_int

    def threads(self) -> int:
        return int(self.lib.fa_oracle_threads())

    def philox4x32_10(self, ctr, key):
        """The Philox-4x32-10 block (4 words) for a 4-word counter and a 2-word key."""
        c = (ctypes.c_uint32 * 4)(*[int(x) & 0xFFFFFFFF for x in ctr])
        k = (ctypes.c_uint32 * 2)(*[int(x) & 0xFFFFFFFF for x in key])
        o = (ctypes.c_uint32 * 4)()
        self.lib.fa_oracle_philox4x32_10(c, k, o)
        return [int(x) for x in o]

    def dropout_multiplier(self, n, p, seed, offset=0):
        """k_n / (1 - p) for score position n (0 when dropped)."""
        return float(self.lib.fa_oracle_dropout_multiplier(int(n), float(p), int(seed), int(offset)))

    def fwd(self, q, k, v, *, scale, causal=False, mask=None, mask_kind="none", rows=None,
            dropout_p=None, seed=0, offset=0, window=None):
        """Attention forward in fp64.

        q [B,Hq,qL,D], k/v [B,Hkv,kL,D]; mask broadcastable to [B,Hq,qL,kL]
        (additive values, or bool/uint8 with nonzero = attend).
        Returns (O, L): O [B,Hq,qL,D] and L [B,Hq,qL], or O [n,D] and L [n]
        for the flat row indices `rows` (flat = (b*Hq + h)*qL + i).
        window (causal only): row i sees keys i - window + 1 .. i.
        """
        q = np.ascontiguousarray(q, dtype=np.float64)
        k = np.ascontiguousarray(k, dtype=np.float64)
        v = np.ascontiguousarray(v, dtype=np.float64)
        B, Hq, qL, D = q.shape
        Bk, Hkv, kL, Dk = k.shape
        if v.shape != k.shape or Bk != B or Dk != D:
            raise ValueError("oracle: q/k/v shapes disagree")
        kind = MASK_KINDS[mask_kind]
        mptr = None
        if kind != 0:
            if mask is None:
                raise ValueError("oracle: mask_kind needs a mask")
            m = np.asarray(mask)
            if kind == 2:
                m = (m != 0).astype(np.float64)
            m = np.ascontiguousarray(np.broadcast_to(m, (B, Hq, qL, kL)), dtype=np.float64)
            mptr = m.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
        elif mask is not None:
            raise ValueError("oracle: mask given with mask_kind='none'")
        if rows is None:
            n = B * Hq * qL
            rptr = None
        else:
            rows = np.ascontiguousarray(rows, dtype=np.int64)
            n = rows.size
            rptr = rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
        O = np.empty((n, D), dtype=np.float64)
        L = np.empty((n,), dtype=np.float64)
        dp = ctypes.POINTER(ctypes.c_double)
        args = (q.ctypes.data_as(dp), k.ctypes.data_as(dp), v.ctypes.data_as(dp),
                mptr, kind, B, Hq, Hkv, qL, kL, D, float(scale), int(bool(causal)),
                rptr, n, O.ctypes.data_as(dp), L.ctypes.data_as(dp))
        if window is not None and dropout_p is not None:
            raise ValueError("oracle: window and dropout are not combined")
        if window is not None:
            rc = self.lib.fa_oracle_fwd_window(*args, int(window))
        elif dropout_p is None:
            rc = self.lib.fa_oracle_fwd(*args)
        else:
            rc = self.lib.fa_oracle_fwd_dropout(*args, float(dropout_p), int(seed), int(offset))
        if rc != 0:
            raise ValueError("oracle: fa_oracle_fwd rejected its arguments")
        if rows is None:
            return O.reshape(B, Hq, qL, D), L.reshape(B, Hq, qL)
        return O, L


    def bwd(self, q, k, v, do, *, scale, causal=False, mask=None, mask_kind="none", qrows=None, krows=None):
        """Gradients of the attention forward pass in fp64 (fa_oracle_bwd).

        q, do [B,Hq,qL,D]; k, v [B,Hkv,kL,D]; mask as for fwd.  Returns
        (dQ, dK, dV) in the input shapes, or dQ [len(qrows), D] for the flat
        query rows (b*Hq + h)*qL + i and dK, dV [len(krows), D] for the flat
        key rows (b*Hkv + g)*kL + j when those are given.
        """
        q, k, v, do = (np.ascontiguousarray(x, dtype=np.float64) for x in (q, k, v, do))
        B, Hq, qL, D = q.shape
        Bk, Hkv, kL, Dk = k.shape
        if v.shape != k.shape or do.shape != q.shape or Bk != B or Dk != D:
            raise ValueError("oracle: q/k/v/do shapes disagree")
        kind = MASK_KINDS[mask_kind]
        mptr = None
        if kind != 0:
            m = np.asarray(mask)
            if kind == 2:
                m = (m != 0).astype(np.float64)
            m = np.ascontiguousarray(np.broadcast_to(m, (B, Hq, qL, kL)), dtype=np.float64)
            mptr = m.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
        elif mask is not None:
            raise ValueError("oracle: mask given with mask_kind='none'")
        i64p = ctypes.POINTER(ctypes.c_int64)
        dp = ctypes.POINTER(ctypes.c_double)

        def rows_arg(rows, total):
            if rows is None:
                return None, None, total
            rows = np.ascontiguousarray(rows, dtype=np.int64)
            return rows, rows.ctypes.data_as(i64p), rows.size

        qr, qptr, nq = rows_arg(qrows, B * Hq * qL)
        kr, kptr, nk = rows_arg(krows, B * Hkv * kL)
        dQ = np.empty((nq, D))
        dK = np.empty((nk, D))
        dV = np.empty((nk, D))
        rc = self.lib.fa_oracle_bwd(q.ctypes.data_as(dp), k.ctypes.data_as(dp), v.ctypes.data_as(dp),
                                    do.ctypes.data_as(dp), mptr, kind, B, Hq, Hkv, qL, kL, D, float(scale),
                                    int(bool(causal)), qptr, nq, kptr, nk, dQ.ctypes.data_as(dp),
                                    dK.ctypes.data_as(dp), dV.ctypes.data_as(dp))
        if rc != 0:
            raise ValueError("oracle: fa_oracle_bwd rejected its arguments")
        if qrows is None:
            dQ = dQ.reshape(B, Hq, qL, D)
        if krows is None:
            dK, dV = dK.reshape(B, Hkv, kL, D), dV.reshape(B, Hkv, kL, D)
        return dQ, dK, dV


_DEFAULT = None


def _default() -> OracleLib:
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = OracleLib()
    return _DEFAULT


def attention_fwd(q, k, v, *, scale, causal=False, mask=None, mask_kind="none", rows=None,
                  dropout_p=None, seed=0, offset=0, window=None):
    """fp64 attention forward with the default compiled oracle (see OracleLib.fwd).  With
    dropout_p set, each P V term is scaled by its keep decision / (1 - p) (L is unchanged);
    with window set (causal only), row i sees keys i - window + 1 .. i."""
    return _default().fwd(q, k, v, scale=scale, causal=causal, mask=mask, mask_kind=mask_kind, rows=rows,
                          dropout_p=dropout_p, seed=seed, offset=offset, window=window)


def philox4x32_10(ctr, key):
    return _default().philox4x32_10(ctr, key)


def dropout_multiplier(n, p, seed, offset=0):
    return _default().dropout_multiplier(n, p, seed, offset)


def oracle_threads() -> int:
    return _default().threads()


def attention_bwd(q, k, v, do, *, scale, causal=False, mask=None, mask_kind="none", qrows=None, krows=None):
    """fp64 gradients dQ, dK, dV of the attention forward pass for the upstream
    gradient do, with the default compiled oracle (see OracleLib.bwd)."""
    return _default().bwd(q, k, v, do, scale=scale, causal=causal, mask=mask, mask_kind=mask_kind, qrows=qrows,
                          krows=krows)
