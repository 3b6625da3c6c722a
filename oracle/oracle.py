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
        self.lib.fa_oracle_threads.restype = ctypes.c_int

    def threads(self) -> int:
        return int(self.lib.fa_oracle_threads())

    def fwd(self, q, k, v, *, scale, causal=False, mask=None, mask_kind="none", rows=None):
        """Attention forward in fp64.

        q [B,Hq,qL,D], k/v [B,Hkv,kL,D]; mask broadcastable to [B,Hq,qL,kL]
        (additive values, or bool/uint8 with nonzero = attend).
        Returns (O, L): O [B,Hq,qL,D] and L [B,Hq,qL], or O [n,D] and L [n]
        for the flat row indices `rows` (flat = (b*Hq + h)*qL + i).
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
        rc = self.lib.fa_oracle_fwd(q.ctypes.data_as(dp), k.ctypes.data_as(dp), v.ctypes.data_as(dp),
                                    mptr, kind, B, Hq, Hkv, qL, kL, D, float(scale), int(bool(causal)),
                                    rptr, n, O.ctypes.data_as(dp), L.ctypes.data_as(dp))
        if rc != 0:
            raise ValueError("oracle: fa_oracle_fwd rejected its arguments")
        if rows is None:
            return O.reshape(B, Hq, qL, D), L.reshape(B, Hq, qL)
        return O, L


_DEFAULT = None


def _default() -> OracleLib:
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = OracleLib()
    return _DEFAULT


def attention_fwd(q, k, v, *, scale, causal=False, mask=None, mask_kind="none", rows=None):
    """fp64 attention forward with the default compiled oracle (see OracleLib.fwd)."""
    return _default().fwd(q, k, v, scale=scale, causal=causal, mask=mask, mask_kind=mask_kind, rows=rows)


def oracle_threads() -> int:
    return _default().threads()
