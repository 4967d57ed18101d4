"""The 8-bit (E4M3) index branch on the GPU against the oracle.

The index inputs are integer-valued in [-4, 4], which E4M3 represents
exactly, and every dot product is an integer below 2^24, so the fp32 scores
are exact in any summation order: S must match the oracle's fp32 bit for bit
and idx exactly, at small sizes over all rows.  At full sizes the same fact
gives a property that holds at any size: the fp8 selection equals the bf16
selection on the same values.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from block_sparse_long_index_amd import ops
from msa_inputs import WORKLOADS, Workload, make_index_inputs, make_inputs

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    ops.lib()
    torch.cuda.set_device(0)


def to_fp8(x):
    return x.float().to(torch.float8_e4m3fn)


SMALL = [
    # name, B, T, N, G, k
    ("fp8_2k_g2", 1, 2048, 2048, 2, 4),
    ("fp8_ragged", 2, 1000, 1000, 2, 4),
    ("fp8_chunked", 1, 200, 1000, 4, 3),
    ("fp8_g8_k16", 1, 2304, 2304, 8, 16),
    ("fp8_g1", 1, 700, 700, 1, 5),
    ("fp8_g16", 1, 515, 515, 16, 8),
    ("fp8_tiny", 1, 5, 5, 2, 4),
    ("fp8_decode", 3, 1, 1000, 8, 16),
    ("fp8_decode_tail1", 2, 1, 129, 4, 16),
]


@pytest.mark.parametrize("name,B,T,N,G,k", SMALL, ids=[s[0] for s in SMALL])
def test_fp8_small_all_rows(name, B, T, N, G, k):
    w = Workload(name, B=B, T=T, N=N, Hq=G, G=G, k=k, seed=41 + len(name))
    say("case", name)
    qI, kI, _ = make_index_inputs(w, device="cuda")
    q8, k8 = to_fp8(qI), to_fp8(kI)
    assert torch.equal(q8.float(), qI.float()) and torch.equal(k8.float(), kI.float())
    S = ops.index_scores(q8, k8)
    idx = ops.select_blocks(q8, k8, k)
    torch.cuda.synchronize()
    d = oracle.dims_of(B, T, N, G, G, 128, 128, 128, k)
    rb, rt = np.repeat(np.arange(B), T), np.tile(np.arange(T), B)
    S_ref = oracle.block_scores_fp8(d, rb, rt, q8.cpu()[rb, rt], k8.cpu())
    idx_ref = oracle.select(d, rt, S_ref)
    got_S = S.permute(0, 2, 1, 3).reshape(B * T, G, -1).cpu().numpy()
    assert np.array_equal(got_S.view(np.uint32), oracle.s_as_fp32(S_ref).view(np.uint32))
    got_idx = idx.permute(0, 2, 1, 3).reshape(B * T, G, k).cpu().numpy()
    assert np.array_equal(got_idx, idx_ref)


@pytest.mark.parametrize("name", ["prefill_32k", "prefill_128k", "decode_256k_b16"])
def test_fp8_full_equals_bf16(name):
    """At the full sizes: the fp8 and bf16 selections agree exactly (integer
    inputs), and so do the decode block scores."""
    w = WORKLOADS[name]
    say("case", name)
    qI, kI, _ = make_index_inputs(w, device="cuda")
    idx16 = ops.select_blocks(qI, kI, w.k)
    idx8 = ops.select_blocks(to_fp8(qI), to_fp8(kI), w.k)
    torch.cuda.synchronize()
    assert torch.equal(idx16, idx8)
    if w.T == 1:
        assert torch.equal(ops.index_scores(qI, kI), ops.index_scores(to_fp8(qI), to_fp8(kI)))


@pytest.mark.parametrize("B,N,Hq,G,k", [
    (16, 5000, 64, 8, 16),   # 128 rows: the one-workgroup-per-row step
    (3, 5000, 64, 8, 16),    # 24 rows: the separate top-k, attention and combine
    (16, 129, 16, 8, 4),     # one key in the last block
])
def test_fp8_decode_one_call(B, N, Hq, G, k):
    """msa_decode_fp8: on integer-valued index inputs the fp8 scan gives the
    bf16 scan's scores, so idx, O and lse equal msa_decode's bit for bit."""
    w = Workload("fp8_decode1", B=B, T=1, N=N, Hq=Hq, G=G, k=k, seed=21 + N + B)
    inp = make_inputs(w, device="cuda")
    q = inp["q"][:, 0].contiguous()
    idx, O, lse = ops.decode(inp["qI"], inp["kI"], q, inp["K"], inp["V"], k, return_lse=True)
    idx8, O8, lse8 = ops.decode(to_fp8(inp["qI"]), to_fp8(inp["kI"]), q, inp["K"], inp["V"], k,
                                return_lse=True)
    idx_s = ops.select_blocks(to_fp8(inp["qI"]), to_fp8(inp["kI"]), k)
    torch.cuda.synchronize()
    assert torch.equal(idx8, idx_s), "idx differs from msa_select_blocks_fp8"
    assert torch.equal(idx8, idx) and torch.equal(O8, O) and torch.equal(lse8, lse)


def test_fp8_decode_needs_bk128():
    w = Workload("fp8_decode_bk", B=2, T=1, N=1000, Hq=16, G=2, k=8, Bk=64, seed=4)
    inp = make_inputs(w, device="cuda")
    q = inp["q"][:, 0].contiguous()
    with pytest.raises(ops.MSAError):
        ops.decode(to_fp8(inp["qI"]), to_fp8(inp["kI"]), q, inp["K"], inp["V"], w.k, Bk=64)


def test_fp8_rejects_mixed_dtypes():
    qI = torch.zeros(1, 4, 2, 128, dtype=torch.float8_e4m3fn, device="cuda")
    kI = torch.zeros(1, 4, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        ops.select_blocks(qI, kI, 4)
