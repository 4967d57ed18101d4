"""GPU test of the library's per-kernel timing (msa_timing_begin / _end):
outputs are the same bits with timing on and off, every kernel kind the
calls launch is reported with its launch count and a positive duration, and
a pool too small for the launches is reported as an error after the arrays
are filled."""
import sys

import pytest
import torch

from block_sparse_long_index_amd import ops
from msa_inputs import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    ops.lib()
    torch.cuda.set_device(0)


def test_timing_prefill_and_decode():
    w = WORKLOADS["prefill_2k"]
    say("timing: prefill", w)
    inp = make_inputs(w, device="cuda")
    idx = ops.select_blocks(inp["qI"], inp["kI"], w.k)
    O = ops.sparse_attn_prefill(inp["q"], inp["K"], inp["V"], idx)
    torch.cuda.synchronize()
    ops.timing_begin(1024)
    idx_t = ops.select_blocks(inp["qI"], inp["kI"], w.k)
    O_t = ops.sparse_attn_prefill(inp["q"], inp["K"], inp["V"], idx_t)
    torch.cuda.synchronize()
    t = ops.timing_end()
    say(t)
    assert torch.equal(idx, idx_t) and torch.equal(O, O_t)
    for kind in ("select", "kv_outer", "combine", "invert"):
        assert kind in t and t[kind][1] >= 1 and t[kind][0] > 0, (kind, t)
    assert t["select"][1] == 1
    assert t["kv_outer"][1] == t["combine"][1]

    wd = Workload("dec", B=3, T=1, N=5000, Hq=8, G=2, k=4, seed=5)
    say("timing: decode", wd)
    di = make_inputs(wd, device="cuda")
    q = di["q"][:, 0].contiguous()
    ix = ops.select_blocks(di["qI"], di["kI"], wd.k)
    Od = ops.sparse_attn_decode(q, di["K"], di["V"], ix)
    torch.cuda.synchronize()
    ops.timing_begin(16)
    ix_t = ops.select_blocks(di["qI"], di["kI"], wd.k)
    Od_t = ops.sparse_attn_decode(q, di["K"], di["V"], ix_t)
    torch.cuda.synchronize()
    t = ops.timing_end()
    say(t)
    assert torch.equal(ix, ix_t) and torch.equal(Od, Od_t)
    for kind in ("decode_scan", "topk", "decode_attn", "decode_combine"):
        assert kind in t and t[kind][1] == 1 and t[kind][0] > 0, (kind, t)


def test_timing_pool_too_small():
    w = WORKLOADS["prefill_2k"]
    inp = make_inputs(w, device="cuda")
    idx = ops.select_blocks(inp["qI"], inp["kI"], w.k)
    torch.cuda.synchronize()
    ops.timing_begin(1)
    ops.sparse_attn_prefill(inp["q"], inp["K"], inp["V"], idx)
    torch.cuda.synchronize()
    with pytest.raises(RuntimeError, match="not timed"):
        ops.timing_end()
    # the session is closed: a new one opens
    ops.timing_begin(4)
    ops.timing_end()
