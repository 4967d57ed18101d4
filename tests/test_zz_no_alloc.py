"""The decode attention entry point that allocates nothing
(msa_sparse_attn_decode_noalloc, partials in the library's static scratch)
against the workspace entry point (msa_sparse_attn_decode) on the same
inputs: outputs bitwise equal, on two calls in a row with the second smaller
(the scratch keeps the first call's contents), and at the largest size the
scratch takes."""
import sys

import numpy as np
import pytest
import torch

from block_sparse_long_index_amd import ops
from msa_inputs import Workload, make_inputs

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    ops.lib()
    torch.cuda.set_device(0)


def _both(w):
    inp = make_inputs(w, device="cuda")
    q = inp["q"][:, 0].contiguous()
    idx = ops.select_blocks(inp["qI"], inp["kI"], w.k)
    O_ws, lse_ws = ops.sparse_attn_decode(q, inp["K"], inp["V"], idx, return_lse=True)
    O_na, lse_na = ops.sparse_attn_decode_noalloc(q, inp["K"], inp["V"], idx, return_lse=True)
    torch.cuda.synchronize()
    return O_ws, lse_ws, O_na, lse_na


def test_noalloc_two_calls_second_smaller():
    big = Workload("noalloc_big", B=16, T=1, N=40000, Hq=64, G=8, k=16, seed=91)
    small = Workload("noalloc_small", B=3, T=1, N=3000, Hq=16, G=4, k=8, seed=92)
    for w in (big, small):
        say("case", w)
        O_ws, lse_ws, O_na, lse_na = _both(w)
        assert torch.equal(O_ws, O_na), w.name
        assert torch.equal(lse_ws, lse_na), w.name


def test_noalloc_largest():
    """B * Hq * k = 32768 partial rows, the scratch's capacity; then a call one
    row group past it is rejected on the host."""
    w = Workload("noalloc_max", B=32, T=1, N=5000, Hq=64, G=8, k=16, seed=93)
    O_ws, lse_ws, O_na, lse_na = _both(w)
    assert torch.equal(O_ws, O_na) and torch.equal(lse_ws, lse_na)
    w2 = w.replace(B=33)
    inp = make_inputs(w2, device="cuda")
    q = inp["q"][:, 0].contiguous()
    idx = torch.zeros(w2.B, w2.G, 1, w2.k, dtype=torch.int32, device="cuda")
    with pytest.raises(ops.MSAError) as e:
        ops.sparse_attn_decode_noalloc(q, inp["K"], inp["V"], idx)
    assert e.value.code == -3
