"""The C ABI without a GPU: the library loads, exports every function that
include/msa.h declares, and rejects bad arguments on the host (validation
runs before any HIP call, so these calls never touch a device)."""
import ctypes
import os
import re

import pytest

from block_sparse_long_index_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_\w+)\s*\(", text)))


def test_header_functions_are_exported():
    L = ops.lib()
    names = _declared()
    assert len(names) == 24, names
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(ops._SIGS)


def test_exports_match_nm():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", ops.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (msa_\w+)", out))
    assert set(_declared()) <= exported


def test_struct_layout():
    assert ctypes.sizeof(ops.Dims) == 48
    assert ops.Dims.k.offset == 44


def _rc(fn, *args):
    return fn(*args)


def _good(**kw):
    base = dict(B=1, T=256, N=256, Hq=8, G=2, k=4)
    base.update(kw)
    return ops.dims(**base)


FAKE = ctypes.c_void_p(0x1000)      # aligned, never dereferenced
MISALIGNED = ctypes.c_void_p(0x1004)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), -1), (dict(T=0), -1), (dict(T=300), -1), (dict(N=0, T=0), -1),
    (dict(Hq=7), -1), (dict(k=0), -1), (dict(G=3, Hq=9), -2), (dict(k=17), -2),
    (dict(d_h=64), -2), (dict(d_I=64), -2), (dict(Bk=96), -2), (dict(Bk=256), -2),
    (dict(Bk=64, k=33), -2), (dict(Bk=32, k=65), -2), (dict(Bk=32, N=600000, T=300), -2),
    (dict(Hq=64, G=2), -2),
])
def test_bad_dims(kw, code):
    L = ops.lib()
    d = _good(**kw)
    assert L.msa_index_scores(ctypes.byref(d), FAKE, FAKE, FAKE, None) == code
    assert L.msa_select_blocks(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == code
    assert L.msa_workspace_bytes(ops.OP_ATTN_PREFILL, ctypes.byref(d)) == 0
    assert len(L.msa_last_error()) > 0


def test_null_and_misaligned_pointers():
    L = ops.lib()
    d = _good()
    assert L.msa_index_scores(None, FAKE, FAKE, FAKE, None) == -1
    assert L.msa_index_scores(ctypes.byref(d), None, FAKE, FAKE, None) == -1
    assert b"qI" in L.msa_last_error()
    assert L.msa_index_scores(ctypes.byref(d), FAKE, MISALIGNED, FAKE, None) == -1
    assert b"aligned" in L.msa_last_error()
    assert L.msa_sparse_attn_prefill(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                     None, 1 << 30, None) == -1
    assert L.msa_sparse_attn_prefill(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE,
                                     MISALIGNED, FAKE, 1 << 30, None) == -1


def test_workspace_checks():
    L = ops.lib()
    d = _good()
    need = L.msa_workspace_bytes(ops.OP_ATTN_PREFILL, ctypes.byref(d))
    assert need > 0
    assert L.msa_sparse_attn_prefill(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                     FAKE, 16, None) == -3
    dd = _good(T=1)
    need_d = L.msa_workspace_bytes(ops.OP_ATTN_DECODE, ctypes.byref(dd))
    assert need_d > 0
    assert L.msa_sparse_attn_decode(ctypes.byref(dd), FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                    FAKE, need_d - 1, None) == -3
    # decode needs T == 1
    assert L.msa_sparse_attn_decode(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                    FAKE, 1 << 40, None) == -1
    need_s = L.msa_workspace_bytes(ops.OP_SELECT_BLOCKS, ctypes.byref(dd))
    assert need_s == 1 * 2 * 2 * 4  # B * G * NB floats
    assert L.msa_select_blocks(ctypes.byref(dd), FAKE, FAKE, FAKE, FAKE, need_s - 4, None) == -3
    assert L.msa_workspace_bytes(ops.OP_SELECT_BLOCKS, ctypes.byref(d)) == 0
    assert L.msa_workspace_bytes(99, ctypes.byref(d)) == 0


def test_workspace_is_bounded():
    """The prefill partials are held for one stage (rows of one group), not
    for all queries: at 1M tokens the whole workspace stays near a GB while
    the all-query partials would be ~280 GB."""
    L = ops.lib()
    big = L.msa_workspace_bytes(ops.OP_ATTN_PREFILL,
                                ctypes.byref(_good(T=1 << 20, N=1 << 20, Hq=64, G=8, k=16)))
    assert 0 < big < 2 * 2**30, big


def test_status_strings():
    L = ops.lib()
    for c in (0, -1, -2, -3, -4):
        assert L.msa_status_string(c)
    assert L.msa_status_string(12345) == b"unknown status"


def test_paged_argument_checks():
    L = ops.lib()
    d = _good(T=1)
    P = ctypes.c_int64
    good = dict(lens=ctypes.c_void_p(0x1008))
    # host-side rejections, before any HIP call (no call here may pass them:
    # it would launch kernels)
    dp = _good(T=2)
    assert L.msa_select_blocks_paged(ctypes.byref(dp), FAKE, FAKE, P(4), FAKE, good["lens"],
                                     FAKE, FAKE, 1 << 30, None) == -1
    assert b"decode only" in L.msa_last_error()
    assert L.msa_select_blocks_paged(ctypes.byref(d), FAKE, FAKE, P(0), FAKE, good["lens"],
                                     FAKE, FAKE, 1 << 30, None) == -1
    assert L.msa_select_blocks_paged(ctypes.byref(d), FAKE, FAKE, P(4), None, good["lens"],
                                     FAKE, FAKE, 1 << 30, None) == -1
    assert L.msa_select_blocks_paged_fp8(ctypes.byref(d), FAKE, FAKE, P(4), FAKE,
                                         ctypes.c_void_p(0x1004), FAKE, FAKE, 1 << 30, None) == -1
    assert b"seq_lens" in L.msa_last_error()
    assert L.msa_sparse_attn_decode_paged(ctypes.byref(d), FAKE, FAKE, FAKE, P(4), FAKE,
                                          good["lens"], FAKE, FAKE, None, FAKE, 16, None) == -3
    assert L.msa_sparse_attn_decode_paged(ctypes.byref(dp), FAKE, FAKE, FAKE, P(4), FAKE,
                                          good["lens"], FAKE, FAKE, None, FAKE, 1 << 30, None) == -1


def test_block_size_checks():
    """Blocks of 64 and 32 keys (k up to 32 and 64): the selection of a
    prefill materialises a window of block scores in the workspace; fp8 index
    inputs and paged caches take 128-key blocks only."""
    L = ops.lib()
    d64 = _good(Bk=64, k=32, N=1024, T=1024)
    need = L.msa_workspace_bytes(ops.OP_SELECT_BLOCKS, ctypes.byref(d64))
    assert need == 1024 * 2 * 16 * 4  # all rows: B * G * NB floats per row
    assert L.msa_select_blocks(ctypes.byref(d64), FAKE, FAKE, FAKE, FAKE, 2 * 16 * 4 - 4,
                               None) == -3
    assert L.msa_select_blocks_fp8(ctypes.byref(d64), FAKE, FAKE, FAKE, FAKE, need, None) == -2
    assert L.msa_index_scores_fp8(ctypes.byref(d64), FAKE, FAKE, FAKE, None) == -2
    d1 = _good(Bk=32, k=64, N=4096, T=1)
    assert L.msa_workspace_bytes(ops.OP_SELECT_BLOCKS, ctypes.byref(d1)) == 2 * 128 * 4
    P = ctypes.c_int64
    assert L.msa_select_blocks_paged(ctypes.byref(d1), FAKE, FAKE, P(4), FAKE,
                                     ctypes.c_void_p(0x1008), FAKE, FAKE, 1 << 30, None) == -2
    assert b"128-token pages" in L.msa_last_error()
    # decode and prefill attention workspaces grow with k
    assert (L.msa_workspace_bytes(ops.OP_ATTN_DECODE, ctypes.byref(d1)) >
            L.msa_workspace_bytes(ops.OP_ATTN_DECODE, ctypes.byref(_good(N=4096, T=1))))


def test_backward_argument_checks():
    """The backward validates before any HIP call: every pointer (lse is
    required), the block size, the workspace floor; its workspace is the
    prefill's plus one float per (row, head)."""
    L = ops.lib()
    d = _good()
    need = L.msa_workspace_bytes(ops.OP_ATTN_BACKWARD, ctypes.byref(d))
    assert need >= L.msa_workspace_bytes(ops.OP_ATTN_PREFILL, ctypes.byref(d)) + 256 * 8 * 4
    args = [FAKE] * 10
    for i in range(10):  # q K V idx O lse dO dq dK dV
        bad = list(args)
        bad[i] = None
        assert L.msa_sparse_attn_backward(ctypes.byref(d), *bad, FAKE, need, None) == -1
        bad[i] = MISALIGNED
        assert L.msa_sparse_attn_backward(ctypes.byref(d), *bad, FAKE, need, None) == -1
        assert b"aligned" in L.msa_last_error()
    assert L.msa_sparse_attn_backward(ctypes.byref(d), *args, None, need, None) == -1
    assert L.msa_sparse_attn_backward(ctypes.byref(d), *args, FAKE, 64, None) == -3
    # every supported block size has a workspace size; unsupported ones are refused
    for bk, k in ((64, 4), (32, 8)):
        assert L.msa_workspace_bytes(ops.OP_ATTN_BACKWARD, ctypes.byref(_good(Bk=bk, k=k))) > 0
    assert L.msa_sparse_attn_backward(ctypes.byref(_good(Bk=96)), *args, FAKE, 1 << 40,
                                      None) == -2


def test_index_kl_argument_checks():
    """Validation before any HIP call: every required pointer (kl may be
    NULL), the block size, the workspace floor."""
    L = ops.lib()
    d = _good()
    need = L.msa_workspace_bytes(ops.OP_INDEX_KL_BACKWARD, ctypes.byref(d))
    assert need >= L.msa_workspace_bytes(ops.OP_ATTN_PREFILL, ctypes.byref(d)) + 256 * 2 * 4
    args = [FAKE] * 9  # qI kI q K idx lse dqI dkI kl
    for i in range(8):
        bad = list(args)
        bad[i] = None
        assert L.msa_index_kl_backward(ctypes.byref(d), *bad, FAKE, need, None) == -1
        bad[i] = MISALIGNED
        assert L.msa_index_kl_backward(ctypes.byref(d), *bad, FAKE, need, None) == -1
    bad = list(args)
    bad[8] = MISALIGNED
    assert L.msa_index_kl_backward(ctypes.byref(d), *bad, FAKE, need, None) == -1
    assert L.msa_index_kl_backward(ctypes.byref(d), *args, None, need, None) == -1
    assert L.msa_index_kl_backward(ctypes.byref(d), *args, FAKE, 64, None) == -3
    for bk, k in ((64, 4), (32, 8)):
        assert L.msa_workspace_bytes(ops.OP_INDEX_KL_BACKWARD, ctypes.byref(_good(Bk=bk, k=k))) > 0
    assert L.msa_index_kl_backward(ctypes.byref(_good(Bk=96)), *args, FAKE, 1 << 40, None) == -2


def test_train_backward_argument_checks():
    """The fused training backward validates before any HIP call: every
    required pointer (kl may be NULL), the block size, the workspace floor;
    its workspace covers both separate calls' scratch plus one stage's
    teacher (fp32 per (row, slot, key))."""
    L = ops.lib()
    d = _good()
    need = L.msa_workspace_bytes(ops.OP_TRAIN_BACKWARD, ctypes.byref(d))
    prefill = L.msa_workspace_bytes(ops.OP_ATTN_PREFILL, ctypes.byref(d))
    assert need >= prefill + 256 * (8 + 2) * 4 + 256 * d.k * d.Bk * 4
    args = [FAKE] * 15  # q K V qI kI idx O lse dO dq dK dV dqI dkI kl
    for i in range(14):
        bad = list(args)
        bad[i] = None
        assert L.msa_train_backward(ctypes.byref(d), *bad, FAKE, need, None) == -1
        bad[i] = MISALIGNED
        assert L.msa_train_backward(ctypes.byref(d), *bad, FAKE, need, None) == -1
    bad = list(args)
    bad[14] = MISALIGNED
    assert L.msa_train_backward(ctypes.byref(d), *bad, FAKE, need, None) == -1
    assert L.msa_train_backward(ctypes.byref(d), *args, None, need, None) == -1
    assert L.msa_train_backward(ctypes.byref(d), *args, FAKE, 64, None) == -3
    for bk, k in ((64, 4), (32, 8)):
        assert L.msa_workspace_bytes(ops.OP_TRAIN_BACKWARD, ctypes.byref(_good(Bk=bk, k=k))) > 0
    assert L.msa_train_backward(ctypes.byref(_good(Bk=96)), *args, FAKE, 1 << 40, None) == -2


def test_noalloc_decode_rejects_on_host():
    """The no-allocation decode call validates like the workspace one and
    rejects a batch whose partials exceed its static scratch, all before any
    HIP call (fake pointers, no GPU)."""
    L = ops.lib()
    d = _good(T=1, N=4096, Hq=64, G=8, k=16, B=33)  # 33 * 64 * 16 > 32768 rows
    rc = L.msa_sparse_attn_decode_noalloc(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                          None)
    assert rc == -3 and b"scratch" in L.msa_last_error()
    d = _good(T=2, N=4096)
    assert L.msa_sparse_attn_decode_noalloc(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                            None) == -1
    d = _good(T=1, N=4096)
    assert L.msa_sparse_attn_decode_noalloc(ctypes.byref(d), FAKE, None, FAKE, FAKE, FAKE, None,
                                            None) == -1
    assert L.msa_sparse_attn_decode_noalloc(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, MISALIGNED,
                                            None, None) == -1


def test_timing_rejects_on_host():
    """The timing calls reject a bad pool size, a read without an open
    session and bad output arrays before any HIP call."""
    L = ops.lib()
    assert L.msa_timing_begin(0) == -1
    assert L.msa_timing_begin((1 << 20) + 1) == -1
    n = len(ops.KERNEL_KINDS)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    assert L.msa_timing_end(ms, cnt, n) == -1
    assert b"no timing session" in L.msa_last_error()
    assert L.msa_timing_end(None, cnt, n) == -1
    assert L.msa_timing_end(ms, cnt, n + 1) == -1
    assert n == 11  # MSA_KERNEL_KINDS


def test_decode_one_call_rejects_on_host():
    """msa_decode validates like the two decode calls, before any HIP call."""
    L = ops.lib()
    d = _good(T=2, N=4096)
    args = [FAKE] * 8
    assert L.msa_decode(ctypes.byref(d), *args, FAKE, 1 << 40, None) == -1  # T != 1
    d = _good(T=1, N=4096)
    assert L.msa_decode(ctypes.byref(d), FAKE, None, *([FAKE] * 6), FAKE, 1 << 40, None) == -1
    assert L.msa_decode(ctypes.byref(d), *([FAKE] * 6), MISALIGNED, None, FAKE, 1 << 40,
                        None) == -1  # O misaligned
    need = L.msa_workspace_bytes(ops.OP_DECODE, ctypes.byref(d))
    assert need > 0
    rc = L.msa_decode(ctypes.byref(d), *([FAKE] * 7), None, FAKE, need - 1, None)
    assert rc == -3
    assert L.msa_workspace_bytes(ops.OP_DECODE, ctypes.byref(_good(T=3, N=4096))) == 0
