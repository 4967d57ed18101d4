"""GPU parity of the one-call prefill (msa_prefill: selection and attention
of successive row windows overlapped on two streams).

It runs the same kernels as msa_select_blocks followed by
msa_sparse_attn_prefill, only scheduled window by window, and a partial result
does not depend on which other rows share its chunk, so idx, O and lse must
equal the two calls' outputs bit for bit; a sample of rows is also compared
with the oracle to the usual bar (idx and S exact, O max-abs 2e-2 and mean-abs
2e-3, lse 1e-3).  Small shapes (ragged, chunked T < N, B > 1, every block
size, several windows), then the 32K and 128K workloads in the benchmark's
configuration.
"""
import sys

import numpy as np
import pytest
import torch

from block_sparse_long_index_amd import ops
from msa_inputs import WORKLOADS, Workload, make_inputs, sample_rows
from test_parity_gpu import check_invariants, check_needles, compare_rows

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    ops.lib()
    torch.cuda.set_device(0)


def two_calls(w, inp):
    idx = ops.select_blocks(inp["qI"], inp["kI"], w.k, Bk=w.Bk)
    O, lse = ops.sparse_attn_prefill(inp["q"], inp["K"], inp["V"], idx, return_lse=True,
                                     Bk=w.Bk)
    return idx, O, lse


CASES = [
    # name, B, T, N, Hq, G, k, Bk
    ("c2k", 1, 2048, 2048, 8, 2, 4, 128),
    ("ragged_b2", 2, 9000, 9000, 16, 4, 8, 128),
    ("chunked", 1, 5000, 12000, 64, 8, 16, 128),
    ("one_window", 1, 40000, 40000, 64, 8, 16, 128),   # < 4 windows: one window
    ("windows", 1, 70000, 70000, 16, 4, 8, 128),       # 5 windows, the last one halved
    ("bk64", 1, 10000, 10000, 32, 8, 32, 64),
    ("bk64_windows", 1, 66000, 66000, 16, 4, 32, 64),  # 4 windows of 64-key blocks
    ("bk32_b2", 2, 6000, 6500, 16, 2, 64, 32),
    ("hg16", 1, 3333, 3333, 64, 4, 3, 128),
    ("two_rows", 3, 2, 130, 8, 2, 4, 128),
]


@pytest.mark.parametrize("overlap", [True, False], ids=["two_streams", "one_stream"])
@pytest.mark.parametrize("name,B,T,N,Hq,G,k,Bk", CASES, ids=[c[0] for c in CASES])
def test_prefill_equals_two_calls(name, B, T, N, Hq, G, k, Bk, overlap):
    w = Workload(name, B=B, T=T, N=N, Hq=Hq, G=G, k=k, Bk=Bk, seed=300 + T)
    say("case", w, "overlap", overlap)
    inp = make_inputs(w, device="cuda")
    idx, O, lse = ops.prefill(inp["qI"], inp["kI"], inp["q"], inp["K"], inp["V"], k,
                              return_lse=True, Bk=Bk, overlap=overlap)
    idx2, O2, lse2 = two_calls(w, inp)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2), "idx"
    assert torch.equal(O, O2), "O"
    assert torch.equal(lse, lse2), "lse"
    check_invariants(w, idx)
    rb, rt = sample_rows(w, 64)
    compare_rows(w, inp, idx, O, lse, rb.numpy(), rt.numpy(), tag=name)


def test_prefill_repeat_and_stream_order():
    """Two calls in a row on the same outputs, and a consumer on the caller's
    stream right after: it must see the finished results."""
    w = Workload("rep", B=1, T=70000, N=70000, Hq=16, G=4, k=8, seed=5)  # 5 windows
    inp = make_inputs(w, device="cuda")
    out = (torch.empty(1, w.G, w.T, w.k, dtype=torch.int32, device="cuda"),
           torch.empty_like(inp["q"]))
    ops.prefill(inp["qI"], inp["kI"], inp["q"], inp["K"], inp["V"], w.k, out=out)
    a = out[1].float().sum()  # enqueued on the caller's stream after the call
    ops.prefill(inp["qI"], inp["kI"], inp["q"], inp["K"], inp["V"], w.k, out=out)
    b = out[1].float().sum()
    idx2, O2, _ = two_calls(w, inp)
    torch.cuda.synchronize()
    assert torch.equal(out[0], idx2) and torch.equal(out[1], O2)
    assert a.item() == b.item() == O2.float().sum().item()


@pytest.mark.parametrize("name", ["prefill_32k", "prefill_128k"])
def test_prefill_full(name):
    w = WORKLOADS[name]
    say("workload", name, "generating")
    inp = make_inputs(w, device="cuda")
    idx, O, lse = ops.prefill(inp["qI"], inp["kI"], inp["q"], inp["K"], inp["V"], w.k,
                              return_lse=True)
    idx2, O2, lse2 = two_calls(w, inp)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(O, O2) and torch.equal(lse, lse2)
    check_invariants(w, idx)
    check_needles(w, inp, idx)
    rb, rt = sample_rows(w, 48)
    compare_rows(w, inp, idx, O, lse, rb.numpy(), rt.numpy(), tag=name)
