"""Thin ctypes binding of libmsa.so (include/msa.h).

Every function here only marshals arguments: it checks shapes, dtypes and
contiguity of torch tensors, allocates outputs and scratch with torch, and
passes raw device pointers plus the current HIP stream to the C ABI.  All
arithmetic runs in the library's kernels.  If the library is missing the
first call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# MSA_LIB_PATH: another build of the same library (the sanitizer test loads a
# host-sanitized copy); there is no other implementation to fall back to.
LIB_PATH = os.environ.get("MSA_LIB_PATH") or os.path.join(_PKG, "libmsa.so")

MSA_OK = 0
OP_INDEX_SCORES = 0
OP_SELECT_BLOCKS = 1
OP_SELECT_FROM_SCORES = 2
OP_ATTN_PREFILL = 3
OP_ATTN_DECODE = 4
OP_ATTN_BACKWARD = 5
OP_INDEX_KL_BACKWARD = 6
OP_TRAIN_BACKWARD = 7
OP_PREFILL = 8
OP_DECODE = 9

# Every function the C header declares, with its ctypes signature.
_P = ctypes.c_void_p
_SIGS = {
    "msa_index_scores": (ctypes.c_int, [_P, _P, _P, _P, _P]),
    "msa_select_blocks": (ctypes.c_int, [_P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "msa_index_scores_fp8": (ctypes.c_int, [_P, _P, _P, _P, _P]),
    "msa_select_blocks_fp8": (ctypes.c_int, [_P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "msa_select_blocks_from_scores": (ctypes.c_int, [_P, _P, _P, _P]),
    "msa_sparse_attn_prefill": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P,
                                               ctypes.c_size_t, _P]),
    "msa_sparse_attn_decode": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P,
                                              ctypes.c_size_t, _P]),
    "msa_sparse_attn_decode_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P]),
    "msa_prefill": (ctypes.c_int, [_P] * 10 + [ctypes.c_size_t, _P, _P]),
    "msa_decode": (ctypes.c_int, [_P] * 10 + [ctypes.c_size_t, _P]),
    "msa_decode_fp8": (ctypes.c_int, [_P] * 10 + [ctypes.c_size_t, _P]),
    "msa_sparse_attn_backward": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                                _P, ctypes.c_size_t, _P]),
    "msa_train_backward": (ctypes.c_int, [_P] * 17 + [ctypes.c_size_t, _P]),
    "msa_index_kl_backward": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                             ctypes.c_size_t, _P]),
    "msa_select_blocks_paged": (ctypes.c_int, [_P, _P, _P, ctypes.c_int64, _P, _P, _P, _P,
                                               ctypes.c_size_t, _P]),
    "msa_select_blocks_paged_fp8": (ctypes.c_int, [_P, _P, _P, ctypes.c_int64, _P, _P, _P, _P,
                                                   ctypes.c_size_t, _P]),
    "msa_sparse_attn_decode_paged": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int64, _P, _P, _P,
                                                    _P, _P, _P, ctypes.c_size_t, _P]),
    "msa_decode_paged": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.c_int64, _P, _P, _P, _P,
                                        _P, _P, ctypes.c_size_t, _P]),
    "msa_decode_paged_fp8": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.c_int64, _P, _P, _P,
                                            _P, _P, _P, ctypes.c_size_t, _P]),
    "msa_timing_begin": (ctypes.c_int, [ctypes.c_int64]),
    "msa_timing_end": (ctypes.c_int, [_P, _P, ctypes.c_int]),
    "msa_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int, _P]),
    "msa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "msa_last_error": (ctypes.c_char_p, []),
}


class Dims(ctypes.Structure):
    """msa_dims_t"""
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64),
                ("N", ctypes.c_int64), ("Hq", ctypes.c_int32),
                ("G", ctypes.c_int32), ("d_h", ctypes.c_int32),
                ("d_I", ctypes.c_int32), ("Bk", ctypes.c_int32),
                ("k", ctypes.c_int32)]


def dims(B, T, N, Hq, G, k, d_h=128, d_I=128, Bk=128) -> Dims:
    return Dims(B, T, N, Hq, G, d_h, d_I, Bk, k)


class MSAError(RuntimeError):
    def __init__(self, code, where, text):
        super().__init__("%s failed (%d): %s" % (where, code, text))
        self.code = code


_lib = None


def lib():
    """The loaded library (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libmsa.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib


def _check(rc, where):
    if rc != MSA_OK:
        L = lib()
        text = "%s: %s" % (L.msa_status_string(rc).decode(), L.msa_last_error().decode())
        raise MSAError(rc, where, text)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype, shape=None):
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def workspace_bytes(op: int, d: Dims) -> int:
    return int(lib().msa_workspace_bytes(op, ctypes.byref(d)))


def _workspace(op, d, ws):
    need = workspace_bytes(op, d)
    if ws is None:
        if need == 0:
            return None, 0
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    return ws, ws.numel() * ws.element_size()


# The index branch takes bf16 or fp8 (OCP e4m3fn) q^I / k^I; the dtype picks
# the C entry point.
_INDEX_DTYPES = {torch.bfloat16: "", torch.float8_e4m3fn: "_fp8"}


def _index_inputs(qI, kI):
    if qI.dtype not in _INDEX_DTYPES:
        raise ValueError("qI must be bfloat16 or float8_e4m3fn, got %s" % qI.dtype)
    B, T, G, dI = qI.shape
    N = kI.shape[1]
    _need(qI, "qI", qI.dtype)
    _need(kI, "kI", qI.dtype, (B, N, dI))
    return B, T, G, dI, N, _INDEX_DTYPES[qI.dtype]


def index_scores(qI, kI, out=None, Bk=128):
    """Stages 1+2.  qI [B,T,G,128], kI [B,N,128] (both bf16 or both fp8
    e4m3fn) -> S [B,G,T,NB] fp32, NB = ceil(N / Bk)."""
    B, T, G, dI, N, sfx = _index_inputs(qI, kI)
    d = dims(B, T, N, G, G, 1, d_I=dI, Bk=Bk)
    NB = (N + d.Bk - 1) // d.Bk
    S = out if out is not None else torch.empty(B, G, T, NB, dtype=torch.float32, device=qI.device)
    _need(S, "S", torch.float32, (B, G, T, NB))
    name = "msa_index_scores" + sfx
    _check(getattr(lib(), name)(ctypes.byref(d), _ptr(qI), _ptr(kI), _ptr(S), _stream()), name)
    return S


def select_blocks(qI, kI, k, out=None, workspace=None, Bk=128):
    """Stages 1-3 fused (bf16 or fp8 e4m3fn inputs).  -> idx [B,G,T,k] int32
    (ascending, -1 padded)."""
    B, T, G, dI, N, sfx = _index_inputs(qI, kI)
    d = dims(B, T, N, G, G, k, d_I=dI, Bk=Bk)
    idx = out if out is not None else torch.empty(B, G, T, k, dtype=torch.int32, device=qI.device)
    _need(idx, "idx", torch.int32, (B, G, T, k))
    ws, nbytes = _workspace(OP_SELECT_BLOCKS, d, workspace)
    name = "msa_select_blocks" + sfx
    _check(getattr(lib(), name)(ctypes.byref(d), _ptr(qI), _ptr(kI), _ptr(idx), _ptr(ws),
                                nbytes, _stream()), name)
    return idx


def select_blocks_from_scores(S, k, N, out=None, Bk=128):
    """Stage 3 from S [B,G,T,NB] fp32 (query row t at position N - T + t)."""
    B, G, T, NB = S.shape
    _need(S, "S", torch.float32)
    d = dims(B, T, N, G, G, k, Bk=Bk)
    if NB != (N + d.Bk - 1) // d.Bk:
        raise ValueError("S has %d blocks, N=%d needs %d" % (NB, N, (N + d.Bk - 1) // d.Bk))
    idx = out if out is not None else torch.empty(B, G, T, k, dtype=torch.int32, device=S.device)
    _need(idx, "idx", torch.int32, (B, G, T, k))
    _check(lib().msa_select_blocks_from_scores(ctypes.byref(d), _ptr(S), _ptr(idx), _stream()),
           "msa_select_blocks_from_scores")
    return idx


# Kernel kinds of msa_timing_begin / msa_timing_end, in id order.
KERNEL_KINDS = ("select", "kv_outer", "combine", "invert", "decode_scan", "topk",
                "decode_attn", "decode_combine", "attn_backward", "index_kl", "decode_step")


def timing_begin(max_launches=65536):
    """Start timing every launch of the library's timed kernel kinds with HIP
    events on its own stream (msa_timing_begin)."""
    _check(lib().msa_timing_begin(int(max_launches)), "msa_timing_begin")


def timing_end():
    """Stop timing; {kind: (total ms, launches)} for the kinds that ran."""
    n = len(KERNEL_KINDS)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _check(lib().msa_timing_end(ms, cnt, n), "msa_timing_end")
    return {KERNEL_KINDS[i]: (ms[i], cnt[i]) for i in range(n) if cnt[i] > 0}


_side_streams = {}


def side_stream(device=None):
    """A second stream of the device (created once, default priority) for
    the attention windows of prefill()."""
    dev = torch.cuda.current_device() if device is None else device
    if dev not in _side_streams:
        _side_streams[dev] = torch.cuda.Stream(device=dev)
    return _side_streams[dev]


def prefill(qI, kI, q, K, V, k, return_lse=False, out=None, workspace=None, Bk=128,
            overlap=True):
    """Stages 1-4 in one call (msa_prefill): selection and attention of
    successive row windows overlapped on the current stream and a second
    one (overlap=False: all on the current stream).  Returns (idx, O) or
    (idx, O, lse); out = (idx, O) or (idx, O, lse) to write into."""
    B, T, G, dI = qI.shape
    _, _, Hq, dh = q.shape
    N = kI.shape[1]
    _index_inputs(qI, kI)
    if qI.dtype != torch.bfloat16:
        raise ValueError("prefill takes bf16 index inputs")
    _need(q, "q", torch.bfloat16, (B, T, Hq, dh))
    _need(K, "K", torch.bfloat16, (B, G, N, dh))
    _need(V, "V", torch.bfloat16, (B, G, N, dh))
    d = dims(B, T, N, Hq, G, k, d_h=dh, d_I=dI, Bk=Bk)
    if out is not None:
        idx, O = out[0], out[1]
        lse = out[2] if len(out) > 2 else None
    else:
        idx = torch.empty(B, G, T, k, dtype=torch.int32, device=q.device)
        O = torch.empty_like(q)
        lse = None
    if return_lse and lse is None:
        lse = torch.empty(B, Hq, T, dtype=torch.float32, device=q.device)
    _need(idx, "idx", torch.int32, (B, G, T, k))
    _need(O, "O", torch.bfloat16, q.shape)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, Hq, T))
    ws, nbytes = _workspace(OP_PREFILL, d, workspace)
    s2 = ctypes.c_void_p(side_stream(q.device.index).cuda_stream) if overlap else None
    _check(lib().msa_prefill(ctypes.byref(d), _ptr(qI), _ptr(kI), _ptr(q), _ptr(K), _ptr(V),
                             _ptr(idx), _ptr(O), _ptr(lse), _ptr(ws), nbytes, _stream(), s2),
           "msa_prefill")
    if ws is not None and workspace is None and overlap:
        # the side stream still reads the temporary workspace after this returns
        ws.record_stream(side_stream(q.device.index))
    return (idx, O, lse) if return_lse else (idx, O)


def sparse_attn_prefill(q, K, V, idx, return_lse=False, out=None, workspace=None, Bk=128):
    """Stage 4, KV-outer.  q [B,T,Hq,128], K/V [B,G,N,128] bf16, idx [B,G,T,k]
    -> O [B,T,Hq,128] bf16 (and lse [B,Hq,T] fp32)."""
    B, T, Hq, dh = q.shape
    _, G, N, _ = K.shape
    k = idx.shape[-1]
    _need(q, "q", torch.bfloat16)
    _need(K, "K", torch.bfloat16, (B, G, N, dh))
    _need(V, "V", torch.bfloat16, (B, G, N, dh))
    _need(idx, "idx", torch.int32, (B, G, T, k))
    d = dims(B, T, N, Hq, G, k, d_h=dh, Bk=Bk)
    O = out if out is not None else torch.empty_like(q)
    _need(O, "O", torch.bfloat16, q.shape)
    lse = torch.empty(B, Hq, T, dtype=torch.float32, device=q.device) if return_lse else None
    ws, nbytes = _workspace(OP_ATTN_PREFILL, d, workspace)
    _check(lib().msa_sparse_attn_prefill(ctypes.byref(d), _ptr(q), _ptr(K), _ptr(V), _ptr(idx),
                                         _ptr(O), _ptr(lse), _ptr(ws), nbytes, _stream()),
           "msa_sparse_attn_prefill")
    return (O, lse) if return_lse else O


def sparse_attn_backward(q, K, V, idx, O, lse, dO, out=None, workspace=None, Bk=128):
    """Stage 4 gradients (blocks of Bk keys).  q, O, dO [B,T,Hq,128] bf16, K/V
    [B,G,N,128] bf16, idx [B,G,T,k], lse [B,Hq,T] fp32 from the prefill ->
    (dq [B,T,Hq,128], dK, dV [B,G,N,128]), all fp32.  out: optional
    (dq, dK, dV) tensors to write."""
    B, T, Hq, dh = q.shape
    _, G, N, _ = K.shape
    k = idx.shape[-1]
    _need(q, "q", torch.bfloat16)
    _need(K, "K", torch.bfloat16, (B, G, N, dh))
    _need(V, "V", torch.bfloat16, (B, G, N, dh))
    _need(idx, "idx", torch.int32, (B, G, T, k))
    _need(O, "O", torch.bfloat16, q.shape)
    _need(dO, "dO", torch.bfloat16, q.shape)
    _need(lse, "lse", torch.float32, (B, Hq, T))
    d = dims(B, T, N, Hq, G, k, d_h=dh, Bk=Bk)
    if out is None:
        out = (torch.empty(q.shape, dtype=torch.float32, device=q.device),
               torch.empty(K.shape, dtype=torch.float32, device=q.device),
               torch.empty(K.shape, dtype=torch.float32, device=q.device))
    dq, dK, dV = out
    _need(dq, "dq", torch.float32, q.shape)
    _need(dK, "dK", torch.float32, K.shape)
    _need(dV, "dV", torch.float32, K.shape)
    ws, nbytes = _workspace(OP_ATTN_BACKWARD, d, workspace)
    _check(lib().msa_sparse_attn_backward(ctypes.byref(d), _ptr(q), _ptr(K), _ptr(V), _ptr(idx),
                                          _ptr(O), _ptr(lse), _ptr(dO), _ptr(dq), _ptr(dK),
                                          _ptr(dV), _ptr(ws), nbytes, _stream()),
           "msa_sparse_attn_backward")
    return dq, dK, dV


def index_kl_backward(qI, kI, q, K, idx, lse, return_loss=False, out=None, workspace=None,
                      Bk=128):
    """Index-branch KL alignment gradients (blocks of Bk keys).  qI [B,T,G,128],
    kI [B,N,128], q [B,T,Hq,128], K [B,G,N,128] bf16, idx [B,G,T,k], lse
    [B,Hq,T] fp32 (the prefill's) -> (dqI [B,T,G,128], dkI [B,N,128]) fp32,
    plus the loss kl [B,G,T] when return_loss."""
    B, T, G, dI = qI.shape
    _, N, _ = kI.shape
    Hq = q.shape[2]
    k = idx.shape[-1]
    _need(qI, "qI", torch.bfloat16)
    _need(kI, "kI", torch.bfloat16, (B, N, dI))
    _need(q, "q", torch.bfloat16, (B, T, Hq, q.shape[3]))
    _need(K, "K", torch.bfloat16, (B, G, N, q.shape[3]))
    _need(idx, "idx", torch.int32, (B, G, T, k))
    _need(lse, "lse", torch.float32, (B, Hq, T))
    d = dims(B, T, N, Hq, G, k, d_h=q.shape[3], d_I=dI, Bk=Bk)
    if out is None:
        out = (torch.empty(qI.shape, dtype=torch.float32, device=qI.device),
               torch.empty(kI.shape, dtype=torch.float32, device=qI.device))
    dqI, dkI = out
    _need(dqI, "dqI", torch.float32, qI.shape)
    _need(dkI, "dkI", torch.float32, kI.shape)
    kl = torch.empty(B, G, T, dtype=torch.float32, device=qI.device) if return_loss else None
    ws, nbytes = _workspace(OP_INDEX_KL_BACKWARD, d, workspace)
    _check(lib().msa_index_kl_backward(ctypes.byref(d), _ptr(qI), _ptr(kI), _ptr(q), _ptr(K),
                                       _ptr(idx), _ptr(lse), _ptr(dqI), _ptr(dkI), _ptr(kl),
                                       _ptr(ws), nbytes, _stream()),
           "msa_index_kl_backward")
    return (dqI, dkI, kl) if return_loss else (dqI, dkI)


def train_backward(q, K, V, qI, kI, idx, O, lse, dO, return_loss=False, out=None,
                   workspace=None, Bk=128):
    """Both training backwards in one call (msa_train_backward): the inputs
    of sparse_attn_backward and index_kl_backward together -> (dq, dK, dV,
    dqI, dkI), plus the loss kl [B,G,T] when return_loss.  out: optional
    (dq, dK, dV, dqI, dkI) tensors to write."""
    B, T, Hq, dh = q.shape
    _, G, N, _ = K.shape
    dI = qI.shape[3]
    k = idx.shape[-1]
    _need(q, "q", torch.bfloat16)
    _need(K, "K", torch.bfloat16, (B, G, N, dh))
    _need(V, "V", torch.bfloat16, (B, G, N, dh))
    _need(qI, "qI", torch.bfloat16, (B, T, G, dI))
    _need(kI, "kI", torch.bfloat16, (B, N, dI))
    _need(idx, "idx", torch.int32, (B, G, T, k))
    _need(O, "O", torch.bfloat16, q.shape)
    _need(dO, "dO", torch.bfloat16, q.shape)
    _need(lse, "lse", torch.float32, (B, Hq, T))
    d = dims(B, T, N, Hq, G, k, d_h=dh, d_I=dI, Bk=Bk)
    if out is None:
        dev = q.device
        out = (torch.empty(q.shape, dtype=torch.float32, device=dev),
               torch.empty(K.shape, dtype=torch.float32, device=dev),
               torch.empty(K.shape, dtype=torch.float32, device=dev),
               torch.empty(qI.shape, dtype=torch.float32, device=dev),
               torch.empty(kI.shape, dtype=torch.float32, device=dev))
    dq, dK, dV, dqI, dkI = out
    _need(dq, "dq", torch.float32, q.shape)
    _need(dK, "dK", torch.float32, K.shape)
    _need(dV, "dV", torch.float32, K.shape)
    _need(dqI, "dqI", torch.float32, qI.shape)
    _need(dkI, "dkI", torch.float32, kI.shape)
    kl = torch.empty(B, G, T, dtype=torch.float32, device=q.device) if return_loss else None
    ws, nbytes = _workspace(OP_TRAIN_BACKWARD, d, workspace)
    _check(lib().msa_train_backward(ctypes.byref(d), _ptr(q), _ptr(K), _ptr(V), _ptr(qI),
                                    _ptr(kI), _ptr(idx), _ptr(O), _ptr(lse), _ptr(dO), _ptr(dq),
                                    _ptr(dK), _ptr(dV), _ptr(dqI), _ptr(dkI), _ptr(kl), _ptr(ws),
                                    nbytes, _stream()),
           "msa_train_backward")
    return (dq, dK, dV, dqI, dkI, kl) if return_loss else (dq, dK, dV, dqI, dkI)


def sparse_attn_decode(q, K, V, idx, return_lse=False, out=None, workspace=None, Bk=128):
    """Stage 4 for one new token per sequence.  q [B,Hq,128], K/V [B,G,N,128],
    idx [B,G,1,k] -> O [B,Hq,128] bf16 (and lse [B,Hq] fp32)."""
    B, Hq, dh = q.shape
    _, G, N, _ = K.shape
    k = idx.shape[-1]
    _need(q, "q", torch.bfloat16)
    _need(K, "K", torch.bfloat16, (B, G, N, dh))
    _need(V, "V", torch.bfloat16, (B, G, N, dh))
    _need(idx, "idx", torch.int32, (B, G, 1, k))
    d = dims(B, 1, N, Hq, G, k, d_h=dh, Bk=Bk)
    O = out if out is not None else torch.empty_like(q)
    _need(O, "O", torch.bfloat16, q.shape)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=q.device) if return_lse else None
    ws, nbytes = _workspace(OP_ATTN_DECODE, d, workspace)
    _check(lib().msa_sparse_attn_decode(ctypes.byref(d), _ptr(q), _ptr(K), _ptr(V), _ptr(idx),
                                        _ptr(O), _ptr(lse), _ptr(ws), nbytes, _stream()),
           "msa_sparse_attn_decode")
    return (O, lse) if return_lse else O


def decode(qI, kI, q, K, V, k, return_lse=False, out=None, workspace=None, Bk=128):
    """Stages 1-4 of a decode step in one call (msa_decode, or msa_decode_fp8
    for float8_e4m3fn index inputs).  qI [B,1,G,128], kI [B,N,128] (both bf16
    or both fp8), q [B,Hq,128], K/V [B,G,N,128] -> (idx [B,G,1,k] int32,
    O [B,Hq,128] bf16) and lse [B,Hq] fp32 when return_lse.  out: optional
    (idx, O)."""
    B, Hq, dh = q.shape
    _, G, N, _ = K.shape
    if qI.dtype not in _INDEX_DTYPES:
        raise ValueError("qI must be bfloat16 or float8_e4m3fn, got %s" % qI.dtype)
    sfx = _INDEX_DTYPES[qI.dtype]
    _need(qI, "qI", qI.dtype, (B, 1, G, 128))
    _need(kI, "kI", qI.dtype, (B, N, 128))
    _need(q, "q", torch.bfloat16)
    _need(K, "K", torch.bfloat16, (B, G, N, dh))
    _need(V, "V", torch.bfloat16, (B, G, N, dh))
    d = dims(B, 1, N, Hq, G, k, d_h=dh, Bk=Bk)
    if out is None:
        idx = torch.empty(B, G, 1, k, dtype=torch.int32, device=q.device)
        O = torch.empty_like(q)
    else:
        idx, O = out
    _need(idx, "idx", torch.int32, (B, G, 1, k))
    _need(O, "O", torch.bfloat16, q.shape)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=q.device) if return_lse else None
    ws, nbytes = _workspace(OP_DECODE, d, workspace)
    name = "msa_decode" + sfx
    _check(getattr(lib(), name)(ctypes.byref(d), _ptr(qI), _ptr(kI), _ptr(q), _ptr(K), _ptr(V),
                                _ptr(idx), _ptr(O), _ptr(lse), _ptr(ws), nbytes, _stream()),
           name)
    return (idx, O, lse) if return_lse else (idx, O)


def sparse_attn_decode_noalloc(q, K, V, idx, return_lse=False, out=None, lse_out=None,
                               Bk=128):
    """msa_sparse_attn_decode_noalloc: the decode attention with the library's
    static scratch instead of a workspace (no device allocation by the
    library; pass out / lse_out to allocate nothing here either)."""
    B, Hq, dh = q.shape
    _, G, N, _ = K.shape
    k = idx.shape[-1]
    _need(q, "q", torch.bfloat16)
    _need(K, "K", torch.bfloat16, (B, G, N, dh))
    _need(V, "V", torch.bfloat16, (B, G, N, dh))
    _need(idx, "idx", torch.int32, (B, G, 1, k))
    d = dims(B, 1, N, Hq, G, k, d_h=dh, Bk=Bk)
    O = out if out is not None else torch.empty_like(q)
    _need(O, "O", torch.bfloat16, q.shape)
    lse = lse_out
    if lse is None and return_lse:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, Hq))
    _check(lib().msa_sparse_attn_decode_noalloc(ctypes.byref(d), _ptr(q), _ptr(K), _ptr(V),
                                                _ptr(idx), _ptr(O), _ptr(lse), _stream()),
           "msa_sparse_attn_decode_noalloc")
    return (O, lse) if (return_lse or lse_out is not None) else O


def forward(qI, kI, q, K, V, k, return_lse=False, Bk=128):
    """The whole path for prefill (T > 1) or decode (T == 1)."""
    idx = select_blocks(qI, kI, k, Bk=Bk)
    if qI.shape[1] == 1:
        res = sparse_attn_decode(q.reshape(q.shape[0], q.shape[2], q.shape[3]), K, V, idx,
                                 return_lse=return_lse, Bk=Bk)
    else:
        res = sparse_attn_prefill(q, K, V, idx, return_lse=return_lse, Bk=Bk)
    return idx, res


# ------------------------------------------------------------- paged decode
def _paged_args(block_table, seq_lens, B):
    _need(block_table, "block_table", torch.int32)
    _need(seq_lens, "seq_lens", torch.int64, (B,))
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, blocks], got %s" % (tuple(block_table.shape),))
    return block_table.shape[1] * 128  # capacity in tokens


def select_blocks_paged(qI, kI_pool, block_table, seq_lens, k, out=None, workspace=None):
    """Decode block selection over a paged index-key pool.  qI [B, G, 128]
    (bf16 or fp8 e4m3fn), kI_pool [pages, 128, 128] of the same dtype,
    block_table int32 [B, nb], seq_lens int64 [B] -> idx [B, G, 1, k]."""
    if qI.dtype not in _INDEX_DTYPES:
        raise ValueError("qI must be bfloat16 or float8_e4m3fn, got %s" % qI.dtype)
    B, G, dI = qI.shape
    _need(qI, "qI", qI.dtype)
    _need(kI_pool, "kI_pool", qI.dtype)
    if kI_pool.dim() != 3 or tuple(kI_pool.shape[1:]) != (128, dI):
        raise ValueError("kI_pool must be [pages, 128, %d], got %s" % (dI, tuple(kI_pool.shape)))
    N = _paged_args(block_table, seq_lens, B)
    d = dims(B, 1, N, G, G, k, d_I=dI)
    idx = out if out is not None else torch.empty(B, G, 1, k, dtype=torch.int32, device=qI.device)
    _need(idx, "idx", torch.int32, (B, G, 1, k))
    ws, nbytes = _workspace(OP_SELECT_BLOCKS, d, workspace)
    name = "msa_select_blocks_paged" + _INDEX_DTYPES[qI.dtype]
    _check(getattr(lib(), name)(ctypes.byref(d), _ptr(qI), _ptr(kI_pool), kI_pool.shape[0],
                                _ptr(block_table), _ptr(seq_lens), _ptr(idx), _ptr(ws), nbytes,
                                _stream()), name)
    return idx


def sparse_attn_decode_paged(q, K_pool, V_pool, block_table, seq_lens, idx, out=None,
                             lse=None, return_lse=False, workspace=None):
    """Decode attention over paged K/V pools.  q [B, Hq, 128] bf16, K_pool /
    V_pool [pages, G, 128, 128] bf16, block_table int32 [B, nb], seq_lens int64
    [B], idx [B, G, 1, k] -> O [B, Hq, 128] (and lse [B, Hq])."""
    B, Hq, dh = q.shape
    P, G = K_pool.shape[0], K_pool.shape[1]
    _need(q, "q", torch.bfloat16)
    _need(K_pool, "K_pool", torch.bfloat16, (P, G, 128, dh))
    _need(V_pool, "V_pool", torch.bfloat16, (P, G, 128, dh))
    k = idx.shape[-1]
    _need(idx, "idx", torch.int32, (B, G, 1, k))
    N = _paged_args(block_table, seq_lens, B)
    d = dims(B, 1, N, Hq, G, k, d_h=dh)
    O = out if out is not None else torch.empty_like(q)
    _need(O, "O", torch.bfloat16, (B, Hq, dh))
    if return_lse and lse is None:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, Hq))
    ws, nbytes = _workspace(OP_ATTN_DECODE, d, workspace)
    _check(lib().msa_sparse_attn_decode_paged(
        ctypes.byref(d), _ptr(q), _ptr(K_pool), _ptr(V_pool), P, _ptr(block_table),
        _ptr(seq_lens), _ptr(idx), _ptr(O), _ptr(lse), _ptr(ws), nbytes, _stream()),
        "msa_sparse_attn_decode_paged")
    return (O, lse) if return_lse else O


def decode_paged(qI, kI_pool, q, K_pool, V_pool, block_table, seq_lens, k, return_lse=False,
                 out=None, workspace=None):
    """A decode step over paged pools in one call (msa_decode_paged, or
    msa_decode_paged_fp8 for float8_e4m3fn index inputs).  qI [B, G, 128] and
    kI_pool [pages, 128, 128] (same dtype), q [B, Hq, 128] bf16, K_pool /
    V_pool [pages, G, 128, 128] bf16, block_table int32 [B, nb], seq_lens int64
    [B] -> (idx [B, G, 1, k], O [B, Hq, 128]) and lse [B, Hq] when return_lse.
    out: optional (idx, O)."""
    if qI.dtype not in _INDEX_DTYPES:
        raise ValueError("qI must be bfloat16 or float8_e4m3fn, got %s" % qI.dtype)
    B, G, dI = qI.shape
    _, Hq, dh = q.shape
    P = K_pool.shape[0]
    _need(qI, "qI", qI.dtype)
    _need(kI_pool, "kI_pool", qI.dtype, (P, 128, dI))
    _need(q, "q", torch.bfloat16, (B, Hq, dh))
    _need(K_pool, "K_pool", torch.bfloat16, (P, G, 128, dh))
    _need(V_pool, "V_pool", torch.bfloat16, (P, G, 128, dh))
    N = _paged_args(block_table, seq_lens, B)
    d = dims(B, 1, N, Hq, G, k, d_h=dh, d_I=dI)
    if out is None:
        idx = torch.empty(B, G, 1, k, dtype=torch.int32, device=q.device)
        O = torch.empty_like(q)
    else:
        idx, O = out
    _need(idx, "idx", torch.int32, (B, G, 1, k))
    _need(O, "O", torch.bfloat16, (B, Hq, dh))
    lse = torch.empty(B, Hq, dtype=torch.float32, device=q.device) if return_lse else None
    ws, nbytes = _workspace(OP_DECODE, d, workspace)
    name = "msa_decode_paged" + _INDEX_DTYPES[qI.dtype]
    _check(getattr(lib(), name)(ctypes.byref(d), _ptr(qI), _ptr(kI_pool), _ptr(q), _ptr(K_pool),
                                _ptr(V_pool), P, _ptr(block_table), _ptr(seq_lens), _ptr(idx),
                                _ptr(O), _ptr(lse), _ptr(ws), nbytes, _stream()), name)
    return (idx, O, lse) if return_lse else (idx, O)
