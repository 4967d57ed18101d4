"""Python face of the CPU oracle (test infrastructure only).

The oracle is plain C (``msa_oracle.c``), compiled with gcc into
``libmsa_oracle.so`` next to this file and called through ctypes.  Only the
test suite, the smoke check and the benchmark's CPU-baseline leg use it; the
product path never imports this package.  It shares no code with the HIP
implementation.

All arrays crossing into the oracle are numpy arrays: bf16 tensors travel as
their uint16 bit patterns, results come back in fp64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import time

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msa_oracle.c")
_LIB = os.path.join(_HERE, "libmsa_oracle.so")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    if not force and os.path.exists(_LIB) and \
            os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB)
    return _LIB


class Dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64),
                ("N", ctypes.c_int64), ("Hq", ctypes.c_int32),
                ("G", ctypes.c_int32), ("d_h", ctypes.c_int32),
                ("d_I", ctypes.c_int32), ("Bk", ctypes.c_int32),
                ("k", ctypes.c_int32)]


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def bits(x) -> np.ndarray:
    """bf16 torch tensor (any device) -> contiguous uint16 numpy bit pattern."""
    import torch
    if isinstance(x, np.ndarray):
        assert x.dtype == np.uint16
        return np.ascontiguousarray(x)
    assert x.dtype == torch.bfloat16
    return x.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def codes(x) -> np.ndarray:
    """fp8 e4m3fn torch tensor (any device) or uint8 array -> contiguous uint8
    numpy codes."""
    import torch
    if isinstance(x, np.ndarray):
        assert x.dtype == np.uint8
        return np.ascontiguousarray(x)
    assert x.dtype == torch.float8_e4m3fn
    return x.detach().contiguous().view(torch.uint8).cpu().numpy()


def _rows(row_b, row_t):
    rb = np.ascontiguousarray(np.asarray(row_b, dtype=np.int64))
    rt = np.ascontiguousarray(np.asarray(row_t, dtype=np.int64))
    assert rb.shape == rt.shape and rb.ndim == 1
    return rb, rt


def dims_of(B, T, N, Hq, G, d_h, d_I, Bk, k) -> Dims:
    return Dims(B, T, N, Hq, G, d_h, d_I, Bk, k)


class OracleLib:
    """One loaded copy of the oracle library (the default build, or a copy
    compiled from a modified source by the pin tests' mutation check)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.msa_oracle_threads.restype = ctypes.c_int
        lib.msa_oracle_block_scores.argtypes = [ctypes.POINTER(Dims), i64, P, P, P, P, P]
        lib.msa_oracle_block_scores_fp8.argtypes = [ctypes.POINTER(Dims), i64, P, P, P, P, P]
        lib.msa_oracle_e4m3_values.argtypes = [P]
        lib.msa_oracle_select.argtypes = [ctypes.POINTER(Dims), i64, P, P, P]
        lib.msa_oracle_attend.argtypes = [ctypes.POINTER(Dims), i64, P, P, P, P, P, P, P, P]
        lib.msa_oracle_attend_backward.argtypes = [ctypes.POINTER(Dims), i64, P, P, P, P, P, P,
                                                   P, i64, i64, P, P, P]
        lib.msa_oracle_index_kl_backward.argtypes = [ctypes.POINTER(Dims), i64, P, P, P, P, P,
                                                     P, P, i64, i64, P, P, P]
        for f in (lib.msa_oracle_block_scores, lib.msa_oracle_block_scores_fp8,
                  lib.msa_oracle_e4m3_values, lib.msa_oracle_select, lib.msa_oracle_attend):
            f.restype = None
        self.lib = lib
        self.path = path

    def threads(self) -> int:
        return int(self.lib.msa_oracle_threads())

    def block_scores(self, d: Dims, row_b, row_t, qI_rows, kI) -> np.ndarray:
        """Stages 1+2.  qI_rows [n, G, d_I], kI [B, N, d_I] -> S [n, G, NB]."""
        rb, rt = _rows(row_b, row_t)
        q = bits(qI_rows)
        kk = bits(kI)
        n = rb.size
        NB = (d.N + d.Bk - 1) // d.Bk
        assert q.shape == (n, d.G, d.d_I), q.shape
        assert kk.shape == (d.B, d.N, d.d_I), kk.shape
        assert ((rt >= 0) & (rt < d.T) & (rb >= 0) & (rb < d.B)).all()
        S = np.empty((n, d.G, NB), dtype=np.float64)
        self.lib.msa_oracle_block_scores(ctypes.byref(d), n, _ptr(rb), _ptr(rt),
                                         _ptr(q), _ptr(kk), _ptr(S))
        return S

    def block_scores_fp8(self, d: Dims, row_b, row_t, qI_rows, kI) -> np.ndarray:
        """Stages 1+2 on fp8 E4M3 codes.  qI_rows [n, G, d_I], kI [B, N, d_I]
        (uint8 numpy arrays or float8_e4m3fn tensors) -> S [n, G, NB]."""
        rb, rt = _rows(row_b, row_t)
        q = codes(qI_rows)
        kk = codes(kI)
        n = rb.size
        NB = (d.N + d.Bk - 1) // d.Bk
        assert q.shape == (n, d.G, d.d_I), q.shape
        assert kk.shape == (d.B, d.N, d.d_I), kk.shape
        assert ((rt >= 0) & (rt < d.T) & (rb >= 0) & (rb < d.B)).all()
        S = np.empty((n, d.G, NB), dtype=np.float64)
        self.lib.msa_oracle_block_scores_fp8(ctypes.byref(d), n, _ptr(rb), _ptr(rt),
                                             _ptr(q), _ptr(kk), _ptr(S))
        return S

    def e4m3_values(self) -> np.ndarray:
        """The oracle's value of each of the 256 E4M3 codes."""
        out = np.empty(256, dtype=np.float64)
        self.lib.msa_oracle_e4m3_values(_ptr(out))
        return out

    def select(self, d: Dims, row_t, S) -> np.ndarray:
        """Stage 3.  S [n, G, NB] fp64 -> idx [n, G, k] int32."""
        rt = np.ascontiguousarray(np.asarray(row_t, dtype=np.int64))
        S = np.ascontiguousarray(S, dtype=np.float64)
        n = rt.size
        NB = (d.N + d.Bk - 1) // d.Bk
        assert S.shape == (n, d.G, NB), S.shape
        assert ((rt >= 0) & (rt < d.T)).all()
        idx = np.empty((n, d.G, d.k), dtype=np.int32)
        self.lib.msa_oracle_select(ctypes.byref(d), n, _ptr(rt), _ptr(S), _ptr(idx))
        return idx

    def attend(self, d: Dims, row_b, row_t, q_rows, K, V, idx):
        """Stage 4.  q_rows [n, Hq, d_h], K/V [B, G, N, d_h], idx [n, G, k]
        -> (O [n, Hq, d_h] fp64, lse [n, Hq] fp64)."""
        rb, rt = _rows(row_b, row_t)
        q = bits(q_rows)
        Kb = bits(K)
        Vb = bits(V)
        ix = np.ascontiguousarray(np.asarray(idx, dtype=np.int32))
        n = rb.size
        NB = (d.N + d.Bk - 1) // d.Bk
        assert q.shape == (n, d.Hq, d.d_h), q.shape
        assert Kb.shape == (d.B, d.G, d.N, d.d_h) and Vb.shape == Kb.shape
        assert ix.shape == (n, d.G, d.k)
        assert ((ix >= -1) & (ix < NB)).all()
        O = np.empty((n, d.Hq, d.d_h), dtype=np.float64)
        lse = np.empty((n, d.Hq), dtype=np.float64)
        self.lib.msa_oracle_attend(ctypes.byref(d), n, _ptr(rb), _ptr(rt), _ptr(q),
                                   _ptr(Kb), _ptr(Vb), _ptr(ix), _ptr(O), _ptr(lse))
        return O, lse

    def attend_backward(self, d: Dims, row_b, row_t, q_rows, dO_rows, K, V, idx, blk_lo=0,
                        nblk=None):
        """Stage 4 gradients for the listed rows, given their selection.
        q_rows, dO_rows [n, Hq, d_h]; K/V [B, G, N, d_h]; idx [n, G, k] ->
        (dq [n, Hq, d_h], dK, dV [B, G, nblk*Bk, d_h]) in fp64; dK and dV hold
        the listed rows' contributions to the keys of blocks
        blk_lo .. blk_lo+nblk-1 (all blocks by default)."""
        rb, rt = _rows(row_b, row_t)
        q = bits(q_rows)
        g = bits(dO_rows)
        Kb = bits(K)
        Vb = bits(V)
        ix = np.ascontiguousarray(np.asarray(idx, dtype=np.int32))
        n = rb.size
        NB = (d.N + d.Bk - 1) // d.Bk
        if nblk is None:
            nblk = NB - blk_lo
        assert 0 <= blk_lo and blk_lo + nblk <= NB and nblk >= 1
        assert q.shape == (n, d.Hq, d.d_h) and g.shape == q.shape, (q.shape, g.shape)
        assert Kb.shape == (d.B, d.G, d.N, d.d_h) and Vb.shape == Kb.shape
        assert ix.shape == (n, d.G, d.k)
        assert ((ix >= -1) & (ix < NB)).all()
        dq = np.empty((n, d.Hq, d.d_h), dtype=np.float64)
        dK = np.empty((d.B, d.G, nblk * d.Bk, d.d_h), dtype=np.float64)
        dV = np.empty_like(dK)
        self.lib.msa_oracle_attend_backward(ctypes.byref(d), n, _ptr(rb), _ptr(rt), _ptr(q),
                                            _ptr(g), _ptr(Kb), _ptr(Vb), _ptr(ix), blk_lo, nblk,
                                            _ptr(dq), _ptr(dK), _ptr(dV))
        return dq, dK, dV

    def index_kl_backward(self, d: Dims, row_b, row_t, qI_rows, kI, q_rows, K, idx, blk_lo=0,
                          nblk=None):
        """Index-branch KL alignment for the listed rows, given their
        selection.  qI_rows [n, G, d_I], kI [B, N, d_I], q_rows [n, Hq, d_h],
        K [B, G, N, d_h], idx [n, G, k] -> (dqI [n, G, d_I], dkI
        [B, nblk*Bk, d_I], kl [n, G]) in fp64; dkI holds the listed rows'
        contributions to the keys of blocks blk_lo .. blk_lo+nblk-1."""
        rb, rt = _rows(row_b, row_t)
        qi = bits(qI_rows)
        ki = bits(kI)
        q = bits(q_rows)
        Kb = bits(K)
        ix = np.ascontiguousarray(np.asarray(idx, dtype=np.int32))
        n = rb.size
        NB = (d.N + d.Bk - 1) // d.Bk
        if nblk is None:
            nblk = NB - blk_lo
        assert 0 <= blk_lo and blk_lo + nblk <= NB and nblk >= 1
        assert qi.shape == (n, d.G, d.d_I) and ki.shape == (d.B, d.N, d.d_I)
        assert q.shape == (n, d.Hq, d.d_h) and Kb.shape == (d.B, d.G, d.N, d.d_h)
        assert ix.shape == (n, d.G, d.k) and ((ix >= -1) & (ix < NB)).all()
        dqI = np.empty((n, d.G, d.d_I), dtype=np.float64)
        dkI = np.empty((d.B, nblk * d.Bk, d.d_I), dtype=np.float64)
        kl = np.empty((n, d.G), dtype=np.float64)
        self.lib.msa_oracle_index_kl_backward(ctypes.byref(d), n, _ptr(rb), _ptr(rt), _ptr(qi),
                                              _ptr(ki), _ptr(q), _ptr(Kb), _ptr(ix), blk_lo, nblk,
                                              _ptr(dqI), _ptr(dkI), _ptr(kl))
        return dqI, dkI, kl

    def forward(self, d: Dims, row_b, row_t, qI_rows, kI, q_rows, K, V):
        """All four stages for the listed rows; returns S, idx, O, lse and
        the wall time of each part."""
        t0 = time.perf_counter()
        S = self.block_scores(d, row_b, row_t, qI_rows, kI)
        t1 = time.perf_counter()
        idx = self.select(d, row_t, S)
        t2 = time.perf_counter()
        O, lse = self.attend(d, row_b, row_t, q_rows, K, V, idx)
        t3 = time.perf_counter()
        return dict(S=S, idx=idx, O=O, lse=lse,
                    seconds=dict(scores=t1 - t0, select=t2 - t1, attend=t3 - t2))


_default = None


def default() -> OracleLib:
    global _default
    if _default is None:
        _default = OracleLib(build(force=False))
    return _default


def threads() -> int:
    return default().threads()


def block_scores(*a, **kw):
    return default().block_scores(*a, **kw)


def select(*a, **kw):
    return default().select(*a, **kw)


def attend(*a, **kw):
    return default().attend(*a, **kw)


def attend_backward(*a, **kw):
    return default().attend_backward(*a, **kw)


def index_kl_backward(*a, **kw):
    return default().index_kl_backward(*a, **kw)


def forward(*a, **kw):
    return default().forward(*a, **kw)


def build_variant(source_text: str, out_dir: str, name: str, extra_flags=()) -> str:
    """Compile a copy of the oracle source, possibly modified (the tests that
    check that the pins catch planted mistakes) or with extra flags (the
    sanitizer build).  Returns the .so path."""
    src = os.path.join(out_dir, name + ".c")
    so = os.path.join(out_dir, name + ".so")
    with open(src, "w") as f:
        f.write(source_text)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC"] + list(extra_flags) +
                          ["-shared", src, "-o", so, "-lm"])
    return so


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


def s_as_fp32(S: np.ndarray) -> np.ndarray:
    """fp32 value of S as the HIP path reports it: the fp32 nearest to the
    exact score (numpy's round-to-nearest-even cast of the fp64 score)."""
    return S.astype(np.float32)


def block_scores_fp8(*a, **kw):
    return default().block_scores_fp8(*a, **kw)


def e4m3_values():
    return default().e4m3_values()
