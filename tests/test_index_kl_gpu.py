"""GPU parity of the index branch's KL alignment backward (dq^I, dk^I and
the loss) against the CPU oracle.

The GPU path runs the product calls: the fused selection, the prefill (for the
main lse), then msa_index_kl_backward.  The oracle recomputes the selection of
the rows it checks (equal to the GPU's bit for bit) and the teacher, the proxy,
the loss and the gradients from the definition in fp64.

Tolerance, element by element (tests/grad_tol.py, derived from the bf16
roundings of dz = p_x - p_t and of the per-slot dq^I partials):
|got - ref| <= 4u |ref| + 6u rms(vector) + 1e-5 max|ref|, u = 2^-8, over each
(row, group) dq^I vector and each key's dk^I vector.  The loss is summed in
fp32 from fp32 logarithms: relative 2e-3, absolute 1e-4.

Small shapes: every row's dq^I and loss and every key's dk^I.  The 32K and
128K workloads: sampled rows' dq^I and loss, and dk^I exactly on the last two
blocks (only rows from the first of them on can select them), plus
sum_j dk^I_j = 0 over all keys (the weight differences of a row sum to zero),
within 4u/sqrt(d_I) * sum |q^I|.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from block_sparse_long_index_amd import ops
from grad_tol import close_grad
from msa_inputs import WORKLOADS, Workload, make_inputs, sample_rows

pytestmark = pytest.mark.gpu

KL_RTOL, KL_ATOL = 2e-3, 1e-4


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    ops.lib()
    torch.cuda.set_device(0)


def odims(w):
    return oracle.dims_of(w.B, w.T, w.N, w.Hq, w.G, w.d_h, w.d_I, w.Bk, w.k)


def close(tag, got, ref):
    close_grad(tag, got, ref)


def close_kl(tag, got, ref):
    err = np.abs(np.asarray(got, np.float64) - ref)
    say("%s loss max err %.3e (max %.3e)" % (tag, err.max(), np.abs(ref).max()))
    assert (err <= KL_RTOL * np.abs(ref) + KL_ATOL).all(), (tag, err.max())


def run_gpu(w, inp):
    idx = ops.select_blocks(inp["qI"], inp["kI"], w.k, Bk=w.Bk)
    _, lse = ops.sparse_attn_prefill(inp["q"], inp["K"], inp["V"], idx, return_lse=True, Bk=w.Bk)
    dqI, dkI, kl = ops.index_kl_backward(inp["qI"], inp["kI"], inp["q"], inp["K"], idx, lse,
                                         return_loss=True, Bk=w.Bk)
    torch.cuda.synchronize()
    return idx, dqI, dkI, kl


def oracle_selection(w, inp, rb, rt):
    rb_t = torch.as_tensor(rb, device=inp["qI"].device)
    rt_t = torch.as_tensor(rt, device=inp["qI"].device)
    S = oracle.block_scores(odims(w), rb, rt, inp["qI"][rb_t, rt_t].cpu(), inp["kI"].cpu())
    return oracle.select(odims(w), rt, S)


def gpu_rows(x, rb, rt):
    return x.permute(0, 2, 1, 3)[torch.as_tensor(rb, device=x.device),
                                 torch.as_tensor(rt, device=x.device)].cpu().numpy()


def oracle_kl(w, inp, rb, rt, ref_idx, blk_lo=0, nblk=None):
    rb_t = torch.as_tensor(rb, device=inp["q"].device)
    rt_t = torch.as_tensor(rt, device=inp["q"].device)
    return oracle.index_kl_backward(odims(w), rb, rt, inp["qI"][rb_t, rt_t].cpu(),
                                    inp["kI"].cpu(), inp["q"][rb_t, rt_t].cpu(), inp["K"].cpu(),
                                    ref_idx, blk_lo=blk_lo, nblk=nblk)


def check_sum(w, inp, dkI):
    u = 2.0 ** -8
    err = dkI.double().sum(dim=1).abs()                                   # [B, d]
    bound = 4 * u / w.d_I ** 0.5 * inp["qI"].double().abs().sum(dim=(1, 2))
    r = (err / bound.clamp(min=1e-30)).max().item()
    say("sum of dk^I: %.3e of its bound" % r)
    assert bool((err <= bound + 1e-6).all())  # (a dim where every q^I is 0 has bound 0)


SMALL = [
    # name, B, T, N, Hq, G, k
    ("prefill_2k", 1, 2048, 2048, 8, 2, 4),
    ("ragged", 2, 1000, 1000, 8, 2, 4),
    ("chunked", 1, 300, 1100, 16, 4, 3),
    ("k16_g8", 1, 2304, 2304, 64, 8, 16),
    ("g1_hg1", 1, 700, 700, 1, 1, 5),
    ("g16_hg2", 1, 515, 515, 32, 16, 8),
    ("hg16", 1, 333, 333, 64, 4, 2),
    ("hg4", 1, 450, 450, 16, 4, 6),
    ("k1", 1, 400, 400, 8, 2, 1),
    ("dense", 1, 600, 600, 8, 2, 16),
    ("tiny", 1, 5, 5, 8, 2, 4),
    ("one", 1, 1, 1, 8, 2, 4),
    ("two_rows", 3, 2, 130, 8, 2, 4),
]


@pytest.mark.parametrize("name,B,T,N,Hq,G,k", SMALL, ids=[s[0] for s in SMALL])
def test_index_kl_small_all(name, B, T, N, Hq, G, k):
    w = Workload(name, B=B, T=T, N=N, Hq=Hq, G=G, k=k, seed=61 + N)
    say("case", w)
    inp = make_inputs(w, device="cuda")
    idx, dqI, dkI, kl = run_gpu(w, inp)
    rb = np.repeat(np.arange(B), T)
    rt = np.tile(np.arange(T), B)
    ref_idx = oracle_selection(w, inp, rb, rt)
    assert np.array_equal(gpu_rows(idx, rb, rt), ref_idx), "selection"
    rdq, rdk, rkl = oracle_kl(w, inp, rb, rt, ref_idx)
    close(name + " dqI", dqI.cpu().reshape(B * T, G, -1), rdq)
    close(name + " dkI", dkI.cpu(), rdk[:, :N])
    close_kl(name, kl.permute(0, 2, 1).reshape(B * T, G).cpu(), rkl)
    check_sum(w, inp, dkI)


def test_index_kl_windows_and_repeat():
    """A workspace of a few rows per window and a repeat give the same dq^I
    and loss bit for bit and dk^I within fp32 atomic-order noise."""
    w = Workload("win", B=2, T=900, N=900, Hq=16, G=4, k=6, seed=8)
    inp = make_inputs(w, device="cuda")
    idx, dqI, dkI, kl = run_gpu(w, inp)
    _, lse = ops.sparse_attn_prefill(inp["q"], inp["K"], inp["V"], idx, return_lse=True)
    d = ops.dims(w.B, w.T, w.N, w.Hq, w.G, w.k)
    ws = torch.empty(ops.workspace_bytes(ops.OP_INDEX_KL_BACKWARD, d) // 3, dtype=torch.uint8,
                     device="cuda")
    dq2, dk2, kl2 = ops.index_kl_backward(inp["qI"], inp["kI"], inp["q"], inp["K"], idx, lse,
                                          return_loss=True, workspace=ws)
    dq3, dk3, kl3 = ops.index_kl_backward(inp["qI"], inp["kI"], inp["q"], inp["K"], idx, lse,
                                          return_loss=True)
    torch.cuda.synchronize()
    assert torch.equal(dqI, dq2) and torch.equal(dqI, dq3)
    assert torch.equal(kl, kl2) and torch.equal(kl, kl3)
    for x in (dk2, dk3):
        assert (x - dkI).abs().max().item() <= 1e-5 * dkI.abs().max().item()


def _full(name, n_rows):
    w = WORKLOADS[name]
    say("workload", name, "generating")
    inp = make_inputs(w, device="cuda")
    say("workload", name, "select, prefill, index KL backward")
    idx, dqI, dkI, kl = run_gpu(w, inp)
    check_sum(w, inp, dkI)
    rb, rt = sample_rows(w, n_rows)
    rb, rt = rb.numpy(), rt.numpy()
    say("workload", name, "oracle on", len(rb), "rows")
    ref_idx = oracle_selection(w, inp, rb, rt)
    assert np.array_equal(gpu_rows(idx, rb, rt), ref_idx), "selection"
    rdq, _, rkl = oracle_kl(w, inp, rb, rt, ref_idx, blk_lo=w.NB - 1, nblk=1)
    got = dqI[torch.as_tensor(rb, device="cuda"), torch.as_tensor(rt, device="cuda")].cpu()
    close(name + " dqI rows", got, rdq)
    gkl = kl.permute(0, 2, 1)[torch.as_tensor(rb, device="cuda"),
                              torch.as_tensor(rt, device="cuda")].cpu()
    close_kl(name, gkl, rkl)
    lo = w.NB - 2
    tl = np.arange(lo * w.Bk - (w.N - w.T), w.T)
    tb = np.repeat(np.arange(w.B), tl.size)
    tt = np.tile(tl, w.B)
    say("workload", name, "oracle dk^I of the last two blocks from", tt.size, "rows")
    tail_idx = oracle_selection(w, inp, tb, tt)
    assert np.array_equal(gpu_rows(idx, tb, tt), tail_idx), "tail selection"
    _, rdk, _ = oracle_kl(w, inp, tb, tt, tail_idx, blk_lo=lo, nblk=2)
    n_in = w.N - lo * w.Bk
    close(name + " dkI tail", dkI[:, lo * w.Bk:].cpu(), rdk[:, :n_in])


def test_index_kl_full_32k():
    _full("prefill_32k", 48)


def test_index_kl_full_128k():
    _full("prefill_128k", 24)


def _random_cases(n, seed):
    g = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        G = int(g.choice([1, 2, 4, 8, 16]))
        hg = int(g.choice([1, 2, 4, 8, 16]))
        if G * hg > 64:
            continue
        Bk = int(g.choice([32, 64, 128]))
        k = int(g.integers(1, 2048 // Bk + 1))
        N = int(g.integers(1, 2600))
        T = int(g.choice([N, int(g.integers(1, N + 1))]))
        B = int(g.integers(1, 4))
        cases.append((B, T, N, G * hg, G, k, Bk))
    return cases


@pytest.mark.parametrize("B,T,N,Hq,G,k,Bk", _random_cases(12, 78))
def test_index_kl_random_shapes(B, T, N, Hq, G, k, Bk):
    """Seeded random shapes (block sizes too): every row's dq^I and loss and
    every key's dk^I against the oracle."""
    w = Workload("rand", B=B, T=T, N=N, Hq=Hq, G=G, k=k, Bk=Bk, seed=N * 5 + T)
    say("case", w)
    inp = make_inputs(w, device="cuda")
    idx, dqI, dkI, kl = run_gpu(w, inp)
    rb = np.repeat(np.arange(B), T)
    rt = np.tile(np.arange(T), B)
    ref_idx = oracle_selection(w, inp, rb, rt)
    assert np.array_equal(gpu_rows(idx, rb, rt), ref_idx), "selection"
    rdq, rdk, rkl = oracle_kl(w, inp, rb, rt, ref_idx)
    close("rand dqI", dqI.cpu().reshape(B * T, G, -1), rdq)
    close("rand dkI", dkI.cpu(), rdk[:, :N])
    close_kl("rand", kl.permute(0, 2, 1).reshape(B * T, G).cpu(), rkl)


BK_CASES = [
    ("bk64_k32", 1, 2100, 2100, 64, 8, 32, 64),
    ("bk32_k64", 1, 2500, 2500, 64, 8, 64, 32),
    ("bk64_chunked", 2, 300, 900, 32, 8, 20, 64),
    ("bk32_g16", 1, 700, 700, 32, 16, 12, 32),
    ("bk32_tiny", 1, 5, 5, 8, 2, 4, 32),
]


@pytest.mark.parametrize("name,B,T,N,Hq,G,k,Bk", BK_CASES, ids=[c[0] for c in BK_CASES])
def test_index_kl_block_sizes(name, B, T, N, Hq, G, k, Bk):
    """Blocks of 64 and 32 keys: every row's dq^I and loss, every key's dk^I."""
    w = Workload(name, B=B, T=T, N=N, Hq=Hq, G=G, k=k, Bk=Bk, seed=93 + N)
    say("case", w)
    inp = make_inputs(w, device="cuda")
    idx, dqI, dkI, kl = run_gpu(w, inp)
    rb = np.repeat(np.arange(B), T)
    rt = np.tile(np.arange(T), B)
    ref_idx = oracle_selection(w, inp, rb, rt)
    assert np.array_equal(gpu_rows(idx, rb, rt), ref_idx), "selection"
    rdq, rdk, rkl = oracle_kl(w, inp, rb, rt, ref_idx)
    close(name + " dqI", dqI.cpu().reshape(B * T, G, -1), rdq)
    close(name + " dkI", dkI.cpu(), rdk[:, :N])
    close_kl(name, kl.permute(0, 2, 1).reshape(B * T, G).cpu(), rkl)
    check_sum(w, inp, dkI)
