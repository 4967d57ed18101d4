"""GPU parity of the fused training backward (msa_train_backward): dq, dK, dV
of the main branch and dq^I, dk^I and the loss of the index branch's KL
alignment from one call, the teacher formed by the main backward.

Against the CPU oracle, with the tolerances of the two separate calls (same
arithmetic: bf16 weights in the products, bf16 partials summed in slot order):
every row and key of small shapes, all block sizes; sampled rows of the 32K
workload.  Against the separate calls on the same inputs: dq bit for bit (the
same kernel and partials), dq^I and the loss within the rounding of the
teacher's head sum (summed in another order), dK, dV and dk^I within fp32
atomic-order noise; the 128K workload included.
"""
import numpy as np
import pytest
import torch

from block_sparse_long_index_amd import ops
from msa_inputs import WORKLOADS, Workload, make_grad_output, make_inputs, sample_rows
import test_backward_gpu as tb
import test_index_kl_gpu as tk

pytestmark = pytest.mark.gpu

say = tb.say


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    ops.lib()
    torch.cuda.set_device(0)


def forward(w, inp):
    idx = ops.select_blocks(inp["qI"], inp["kI"], w.k, Bk=w.Bk)
    O, lse = ops.sparse_attn_prefill(inp["q"], inp["K"], inp["V"], idx, return_lse=True, Bk=w.Bk)
    return idx, O, lse


def fused(w, inp, idx, O, lse, dO, workspace=None):
    return ops.train_backward(inp["q"], inp["K"], inp["V"], inp["qI"], inp["kI"], idx, O, lse,
                              dO, return_loss=True, workspace=workspace, Bk=w.Bk)


def separate(w, inp, idx, O, lse, dO):
    dq, dK, dV = ops.sparse_attn_backward(inp["q"], inp["K"], inp["V"], idx, O, lse, dO, Bk=w.Bk)
    dqI, dkI, kl = ops.index_kl_backward(inp["qI"], inp["kI"], inp["q"], inp["K"], idx, lse,
                                         return_loss=True, Bk=w.Bk)
    return dq, dK, dV, dqI, dkI, kl


def near(tag, a, b, rel):
    err = (a.double() - b.double()).abs().max().item()
    scale = max(b.double().abs().max().item(), 1e-3)
    say("%s fused vs separate: max err %.3e of max %.3e" % (tag, err, scale))
    assert err <= rel * scale, (tag, err, scale)


def against_separate(w, inp, idx, O, lse, dO, out):
    ref = separate(w, inp, idx, O, lse, dO)
    torch.cuda.synchronize()
    dq, dK, dV, dqI, dkI, kl = out
    assert torch.equal(dq, ref[0]), "dq differs from the separate backward"
    near("dK", dK, ref[1], 1e-5)
    near("dV", dV, ref[2], 1e-5)
    # the teacher's head sum in another order: a few fp32 ulps of each weight,
    # which reach dq^I through bf16 rounding of dz (one bf16 ulp at most)
    near("dqI", dqI, ref[3], 1e-2)
    near("dkI", dkI, ref[4], 1e-3)
    near("kl", kl, ref[5], 1e-4)


SMALL = [
    # name, B, T, N, Hq, G, k, Bk
    ("prefill_2k", 1, 2048, 2048, 8, 2, 4, 128),
    ("ragged", 2, 1000, 1000, 8, 2, 4, 128),
    ("chunked", 1, 300, 1100, 16, 4, 3, 128),
    ("k16_g8", 1, 2304, 2304, 64, 8, 16, 128),
    ("g1_hg1", 1, 700, 700, 1, 1, 5, 128),
    ("g16_hg2", 1, 515, 515, 32, 16, 8, 128),
    ("hg4", 1, 450, 450, 16, 4, 6, 128),
    ("hg16", 1, 333, 333, 64, 4, 2, 128),
    ("tiny", 1, 5, 5, 8, 2, 4, 128),
    ("two_rows", 3, 2, 130, 8, 2, 4, 128),
    ("bk64_k32", 1, 2100, 2100, 64, 8, 32, 64),
    ("bk32_k64", 1, 2500, 2500, 64, 8, 64, 32),
    ("bk32_g16", 1, 700, 700, 32, 16, 12, 32),
    ("bk64_hg16", 1, 500, 500, 64, 4, 5, 64),
]


@pytest.mark.parametrize("name,B,T,N,Hq,G,k,Bk", SMALL, ids=[s[0] for s in SMALL])
def test_train_backward_small_all(name, B, T, N, Hq, G, k, Bk):
    w = Workload(name, B=B, T=T, N=N, Hq=Hq, G=G, k=k, Bk=Bk, seed=71 + N)
    say("case", w)
    inp = make_inputs(w, device="cuda")
    dO = make_grad_output(w, device="cuda")
    idx, O, lse = forward(w, inp)
    out = fused(w, inp, idx, O, lse, dO)
    torch.cuda.synchronize()
    dq, dK, dV, dqI, dkI, kl = out
    rb = np.repeat(np.arange(B), T)
    rt = np.tile(np.arange(T), B)
    ref_idx = tb.oracle_selection(w, inp, rb, rt)
    assert np.array_equal(tb.gpu_rows(idx, rb, rt), ref_idx), "selection"
    rdq, rdK, rdV = tb.oracle_backward(w, inp, dO, rb, rt, ref_idx)
    ex_dq, ex_dk = tb.bound_extras(w, inp, dO, rb, rt, ref_idx)
    tb.close(name + " dq", dq.cpu().reshape(B * T, Hq, -1), rdq, ex_dq)
    tb.close(name + " dK", dK.cpu(), rdK[:, :, :N], ex_dk[:, :, :N])
    tb.close(name + " dV", dV.cpu(), rdV[:, :, :N])
    rdqI, rdkI, rkl = tk.oracle_kl(w, inp, rb, rt, ref_idx)
    tk.close(name + " dqI", dqI.cpu().reshape(B * T, G, -1), rdqI)
    tk.close(name + " dkI", dkI.cpu(), rdkI[:, :N])
    tk.close_kl(name, kl.permute(0, 2, 1).reshape(B * T, G).cpu(), rkl)
    tb.check_sums(w, inp, dO, dK, dV)
    tk.check_sum(w, inp, dkI)
    against_separate(w, inp, idx, O, lse, dO, out)


@pytest.mark.parametrize("B,T,N,Hq,G,k,Bk", tb._random_cases(12, 2027))
def test_train_backward_random_shapes(B, T, N, Hq, G, k, Bk):
    """Seeded random shapes (block sizes, chunked rows, group layouts, k):
    every row and key of all six outputs against the oracle, and the
    separate calls on the same inputs."""
    w = Workload("rand", B=B, T=T, N=N, Hq=Hq, G=G, k=k, Bk=Bk, seed=N * 5 + T)
    say("case", w)
    inp = make_inputs(w, device="cuda")
    dO = make_grad_output(w, device="cuda")
    idx, O, lse = forward(w, inp)
    out = fused(w, inp, idx, O, lse, dO)
    torch.cuda.synchronize()
    dq, dK, dV, dqI, dkI, kl = out
    rb = np.repeat(np.arange(B), T)
    rt = np.tile(np.arange(T), B)
    ref_idx = tb.oracle_selection(w, inp, rb, rt)
    assert np.array_equal(tb.gpu_rows(idx, rb, rt), ref_idx), "selection"
    rdq, rdK, rdV = tb.oracle_backward(w, inp, dO, rb, rt, ref_idx)
    ex_dq, ex_dk = tb.bound_extras(w, inp, dO, rb, rt, ref_idx)
    tb.close("rand dq", dq.cpu().reshape(B * T, Hq, -1), rdq, ex_dq)
    tb.close("rand dK", dK.cpu(), rdK[:, :, :N], ex_dk[:, :, :N])
    tb.close("rand dV", dV.cpu(), rdV[:, :, :N])
    rdqI, rdkI, rkl = tk.oracle_kl(w, inp, rb, rt, ref_idx)
    tk.close("rand dqI", dqI.cpu().reshape(B * T, G, -1), rdqI)
    tk.close("rand dkI", dkI.cpu(), rdkI[:, :N])
    tk.close_kl("rand", kl.permute(0, 2, 1).reshape(B * T, G).cpu(), rkl)
    against_separate(w, inp, idx, O, lse, dO, out)


def test_train_backward_windows_and_repeat():
    """A workspace of a few rows per window (several inversions, and stages
    of fewer rows) and a repeat: dq, dq^I and the loss bit for bit, dK, dV
    and dk^I within fp32 atomic-order noise."""
    w = Workload("win", B=2, T=900, N=900, Hq=16, G=4, k=6, seed=8)
    inp = make_inputs(w, device="cuda")
    dO = make_grad_output(w, device="cuda")
    idx, O, lse = forward(w, inp)
    a = fused(w, inp, idx, O, lse, dO)
    d = ops.dims(w.B, w.T, w.N, w.Hq, w.G, w.k)
    ws = torch.empty(ops.workspace_bytes(ops.OP_TRAIN_BACKWARD, d) // 3, dtype=torch.uint8,
                     device="cuda")
    b = fused(w, inp, idx, O, lse, dO, workspace=ws)
    c = fused(w, inp, idx, O, lse, dO)
    torch.cuda.synchronize()
    for x in (b, c):
        for i in (0, 3, 5):
            assert torch.equal(a[i], x[i]), i
        for i in (1, 2, 4):
            assert (a[i] - x[i]).abs().max().item() <= 1e-5 * a[i].abs().max().item(), i


def _full(name, n_rows, oracle_rows):
    w = WORKLOADS[name]
    say("workload", name, "generating")
    inp = make_inputs(w, device="cuda")
    dO = make_grad_output(w, device="cuda")
    say("workload", name, "forward + fused training backward")
    idx, O, lse = forward(w, inp)
    out = fused(w, inp, idx, O, lse, dO)
    torch.cuda.synchronize()
    dq, dK, dV, dqI, dkI, kl = out
    tb.check_sums(w, inp, dO, dK, dV)
    tk.check_sum(w, inp, dkI)
    if oracle_rows:
        rb, rt = sample_rows(w, n_rows)
        rb, rt = rb.numpy(), rt.numpy()
        say("workload", name, "oracle on", len(rb), "rows")
        ref_idx = tb.oracle_selection(w, inp, rb, rt)
        assert np.array_equal(tb.gpu_rows(idx, rb, rt), ref_idx), "selection"
        rdq, _, _ = tb.oracle_backward(w, inp, dO, rb, rt, ref_idx, blk_lo=w.NB - 1, nblk=1)
        sel = (torch.as_tensor(rb, device="cuda"), torch.as_tensor(rt, device="cuda"))
        tb.close(name + " dq rows", dq[sel].cpu(), rdq,
                 tb.dq_bound_extra(w, inp, dO, rb, rt, ref_idx))
        rdqI, _, rkl = tk.oracle_kl(w, inp, rb, rt, ref_idx, blk_lo=w.NB - 1, nblk=1)
        tk.close(name + " dqI rows", dqI[sel].cpu(), rdqI)
        tk.close_kl(name, kl.permute(0, 2, 1)[sel].cpu(), rkl)
    say("workload", name, "separate calls")
    against_separate(w, inp, idx, O, lse, dO, out)


def test_train_backward_full_32k():
    _full("prefill_32k", 32, True)


def test_train_backward_full_128k():
    _full("prefill_128k", 0, False)
