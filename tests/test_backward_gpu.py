"""GPU parity of the stage-4 backward (dq, dK, dV) against the CPU oracle.

The GPU path runs the product calls: the fused selection, the prefill (O and
lse), then msa_sparse_attn_backward on O, lse and a seeded dO.  The oracle
recomputes the selection of the rows it checks (which must equal the GPU's
bit for bit) and the gradients from the definition in fp64; nothing it uses
comes from the HIP path.

Tolerance, element by element (tests/grad_tol.py, derived from the bf16
roundings of P, dS, the per-slot dq partials and the forward O):
|got - ref| <= 4u |ref| + 6u rms(vector) + 1e-5 max|ref|, u = 2^-8, over each
(row, head) dq vector and each key's dK and dV vectors.

Small shapes: every row's dq and every key's dK / dV.  The 32K and 128K
workloads, in the configuration the benchmark times: dq on sampled rows, and
dK / dV exactly on the last two blocks, which only the rows from the first of
them on can select (so the oracle needs only those rows); plus, on all keys,
the identities sum_j dV_j = sum of dO over the group's rows and heads and
sum_j dK_j = 0 (softmax weights sum to one).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from block_sparse_long_index_amd import ops
from grad_tol import close_grad, d_shift, dq_extra
from msa_inputs import WORKLOADS, Workload, make_grad_output, make_inputs, sample_rows

pytestmark = pytest.mark.gpu



def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    ops.lib()
    torch.cuda.set_device(0)


def odims(w):
    return oracle.dims_of(w.B, w.T, w.N, w.Hq, w.G, w.d_h, w.d_I, w.Bk, w.k)


def close(tag, got, ref, extra=None):
    close_grad(tag, got, ref, extra)


def bound_extras(w, inp, dO, rb, rt, ref_idx, blk_lo=0, nblk=None):
    """The element-wise bound's D terms (tests/grad_tol.py) for the dq of the
    listed rows and for the dK of blocks blk_lo .. blk_lo + nblk - 1 from
    those rows: the rows' exact forward output (the oracle's), max |K| per
    (sequence, group, dim), and the oracle's dV for the upstream gradient
    dD |q| / sqrt(d_h) (rounded up to bf16)."""
    rb_t = torch.as_tensor(rb, device=inp["q"].device)
    rt_t = torch.as_tensor(rt, device=inp["q"].device)
    q_rows = inp["q"][rb_t, rt_t].cpu()
    K, V = inp["K"].cpu(), inp["V"].cpu()
    O_ref, _ = oracle.attend(odims(w), rb, rt, q_rows, K, V, ref_idx)
    dD = d_shift(dO[rb_t, rt_t].float().cpu().numpy(), O_ref)
    kmax = inp["K"].float().abs().amax(dim=2).cpu().numpy()          # [B, G, d]
    heads_g = np.arange(w.Hq) // w.hg
    ex_dq = dq_extra(dD, kmax[np.asarray(rb)][:, heads_g], w.d_h)
    # scaled up by 2^-7 before the bf16 rounding (relative error <= 2^-8),
    # so that every rounded value is still >= the exact term
    g = torch.from_numpy(dD * q_rows.float().abs().numpy() * ((1 + 2.0 ** -7) / w.d_h ** 0.5))
    _, _, ex_dk = oracle.attend_backward(odims(w), rb, rt, q_rows, g.to(torch.bfloat16), K, V,
                                         ref_idx, blk_lo=blk_lo, nblk=nblk)
    return ex_dq, ex_dk


def dq_bound_extra(w, inp, dO, rb, rt, ref_idx):
    return bound_extras(w, inp, dO, rb, rt, ref_idx, blk_lo=w.NB - 1, nblk=1)[0]


def run_gpu(w, inp, dO):
    idx = ops.select_blocks(inp["qI"], inp["kI"], w.k, Bk=w.Bk)
    O, lse = ops.sparse_attn_prefill(inp["q"], inp["K"], inp["V"], idx, return_lse=True, Bk=w.Bk)
    dq, dK, dV = ops.sparse_attn_backward(inp["q"], inp["K"], inp["V"], idx, O, lse, dO, Bk=w.Bk)
    torch.cuda.synchronize()
    return idx, dq, dK, dV


def oracle_selection(w, inp, rb, rt):
    rb_t = torch.as_tensor(rb, device=inp["qI"].device)
    rt_t = torch.as_tensor(rt, device=inp["qI"].device)
    S = oracle.block_scores(odims(w), rb, rt, inp["qI"][rb_t, rt_t].cpu(), inp["kI"].cpu())
    return oracle.select(odims(w), rt, S)


def gpu_rows(x, rb, rt):
    """[B, G, T, k] -> [n, G, k] for the listed rows."""
    return x.permute(0, 2, 1, 3)[torch.as_tensor(rb, device=x.device),
                                 torch.as_tensor(rt, device=x.device)].cpu().numpy()


def oracle_backward(w, inp, dO, rb, rt, ref_idx, blk_lo=0, nblk=None):
    rb_t = torch.as_tensor(rb, device=inp["q"].device)
    rt_t = torch.as_tensor(rt, device=inp["q"].device)
    return oracle.attend_backward(odims(w), rb, rt, inp["q"][rb_t, rt_t].cpu(),
                                  dO[rb_t, rt_t].cpu(), inp["K"].cpu(), inp["V"].cpu(),
                                  ref_idx, blk_lo=blk_lo, nblk=nblk)


def check_sums(w, inp, dO, dK, dV):
    """Identities over all keys of every (sequence, group), with bounds from
    the bf16 rounding (unit roundoff u = 2^-8) of the weights the kernels
    multiply with:
      sum_j dV_j = sum of dO over the group's rows and heads, up to
        u * sum |dO| (the rounded weights of a row sum to 1 within u);
      sum_j dK_j = 0, up to 4u/sqrt(d) * max|V_j| * sum |q| |dO| (per row,
        the rounded dS_j sum to zero within u * sum_j |dS_j| <=
        2u |dO| max|V_j|, and D = dO . O is off by at most u |dO| |O|)."""
    u = 2.0 ** -8
    go = dO.double().view(w.B, w.T, w.G, w.hg, w.d_h)
    err_v = (dV.double().sum(dim=2) - go.sum(dim=(1, 3))).abs()          # [B, G, d]
    bound_v = u * go.abs().sum(dim=(1, 3))
    q = inp["q"].double().view(w.B, w.T, w.G, w.hg, w.d_h)
    vmax = inp["V"].double().norm(dim=-1).amax(dim=2)                       # [B, G]
    gnorm = go.norm(dim=-1, keepdim=True)                                   # [B, T, G, hg, 1]
    bound_k = 4 * u / w.d_h ** 0.5 * vmax.unsqueeze(-1) * (q.abs() * gnorm).sum(dim=(1, 3))
    err_k = dK.double().sum(dim=2).abs()
    rv = (err_v / bound_v).max().item()
    rk = (err_k / bound_k).max().item()
    say("sums: dV error %.3e of its bound, dK %.3e of its bound" % (rv, rk))
    assert rv <= 1.0 and rk <= 1.0


SMALL = [
    # name, B, T, N, Hq, G, k
    ("prefill_2k", 1, 2048, 2048, 8, 2, 4),
    ("ragged", 2, 1000, 1000, 8, 2, 4),
    ("chunked", 1, 300, 1100, 16, 4, 3),
    ("k16_g8", 1, 2304, 2304, 64, 8, 16),
    ("g1_hg1", 1, 700, 700, 1, 1, 5),
    ("g16_hg2", 1, 515, 515, 32, 16, 8),
    ("hg16", 1, 333, 333, 64, 4, 2),
    ("k1", 1, 400, 400, 8, 2, 1),
    ("dense", 1, 600, 600, 8, 2, 16),
    ("tiny", 1, 5, 5, 8, 2, 4),
    ("one", 1, 1, 1, 8, 2, 4),
    ("two_rows", 3, 2, 130, 8, 2, 4),
]


@pytest.mark.parametrize("name,B,T,N,Hq,G,k", SMALL, ids=[s[0] for s in SMALL])
def test_backward_small_all(name, B, T, N, Hq, G, k):
    w = Workload(name, B=B, T=T, N=N, Hq=Hq, G=G, k=k, seed=41 + N)
    say("case", w)
    inp = make_inputs(w, device="cuda")
    dO = make_grad_output(w, device="cuda")
    idx, dq, dK, dV = run_gpu(w, inp, dO)
    rb = np.repeat(np.arange(B), T)
    rt = np.tile(np.arange(T), B)
    ref_idx = oracle_selection(w, inp, rb, rt)
    assert np.array_equal(gpu_rows(idx, rb, rt), ref_idx), "selection"
    rdq, rdK, rdV = oracle_backward(w, inp, dO, rb, rt, ref_idx)
    ex_dq, ex_dk = bound_extras(w, inp, dO, rb, rt, ref_idx)
    close(name + " dq", dq.cpu().reshape(B * T, Hq, -1), rdq, ex_dq)
    close(name + " dK", dK.cpu(), rdK[:, :, :N], ex_dk[:, :, :N])
    close(name + " dV", dV.cpu(), rdV[:, :, :N])
    check_sums(w, inp, dO, dK, dV)


def test_backward_windows_and_repeat():
    """A workspace of a few rows per window gives the same dq bit for bit and
    dK / dV within fp32 atomic-order noise; two calls in a row agree."""
    w = Workload("win", B=2, T=900, N=900, Hq=16, G=4, k=6, seed=8)
    inp = make_inputs(w, device="cuda")
    dO = make_grad_output(w, device="cuda")
    idx, dq, dK, dV = run_gpu(w, inp, dO)
    O, lse = ops.sparse_attn_prefill(inp["q"], inp["K"], inp["V"], idx, return_lse=True)
    d = ops.dims(w.B, w.T, w.N, w.Hq, w.G, w.k)
    full = ops.workspace_bytes(ops.OP_ATTN_BACKWARD, d)
    ws = torch.empty(full // 3, dtype=torch.uint8, device="cuda")
    dq2, dK2, dV2 = ops.sparse_attn_backward(inp["q"], inp["K"], inp["V"], idx, O, lse, dO,
                                             workspace=ws)
    dq3, dK3, dV3 = ops.sparse_attn_backward(inp["q"], inp["K"], inp["V"], idx, O, lse, dO)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dq, dq3)
    for a, b in ((dK, dK2), (dV, dV2), (dK, dK3), (dV, dV3)):
        assert (a - b).abs().max().item() <= 1e-5 * a.abs().max().item()


def _full(name, n_rows):
    w = WORKLOADS[name]
    say("workload", name, "generating")
    inp = make_inputs(w, device="cuda")
    dO = make_grad_output(w, device="cuda")
    say("workload", name, "forward + backward")
    idx, dq, dK, dV = run_gpu(w, inp, dO)
    say("workload", name, "sums")
    check_sums(w, inp, dO, dK, dV)
    rb, rt = sample_rows(w, n_rows)
    rb, rt = rb.numpy(), rt.numpy()
    say("workload", name, "oracle dq on", len(rb), "rows")
    ref_idx = oracle_selection(w, inp, rb, rt)
    assert np.array_equal(gpu_rows(idx, rb, rt), ref_idx), "selection"
    rdq, _, _ = oracle_backward(w, inp, dO, rb, rt, ref_idx, blk_lo=w.NB - 1, nblk=1)
    got = dq[torch.as_tensor(rb, device="cuda"), torch.as_tensor(rt, device="cuda")].cpu()
    close(name + " dq rows", got, rdq, dq_bound_extra(w, inp, dO, rb, rt, ref_idx))
    # the last two blocks: only rows at positions >= 128 * (NB - 2) select them
    lo = w.NB - 2
    tl = np.arange(lo * w.Bk - (w.N - w.T), w.T)
    tb = np.repeat(np.arange(w.B), tl.size)
    tt = np.tile(tl, w.B)
    say("workload", name, "oracle dK/dV of the last two blocks from", tt.size, "rows")
    tail_idx = oracle_selection(w, inp, tb, tt)
    assert np.array_equal(gpu_rows(idx, tb, tt), tail_idx), "tail selection"
    _, rdK, rdV = oracle_backward(w, inp, dO, tb, tt, tail_idx, blk_lo=lo, nblk=2)
    keys = slice(lo * w.Bk, w.N)
    n_in = w.N - lo * w.Bk
    _, ex_dk = bound_extras(w, inp, dO, tb, tt, tail_idx, blk_lo=lo, nblk=2)
    close(name + " dK tail", dK[:, :, keys].cpu(), rdK[:, :, :n_in], ex_dk[:, :, :n_in])
    close(name + " dV tail", dV[:, :, keys].cpu(), rdV[:, :, :n_in])


def test_backward_full_32k():
    _full("prefill_32k", 48)


def test_backward_full_128k():
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


@pytest.mark.parametrize("B,T,N,Hq,G,k,Bk", _random_cases(12, 77))
def test_backward_random_shapes(B, T, N, Hq, G, k, Bk):
    """Seeded random shapes (block sizes, chunked rows, group layouts, k):
    every row's dq and every key's dK / dV against the oracle."""
    w = Workload("rand", B=B, T=T, N=N, Hq=Hq, G=G, k=k, Bk=Bk, seed=N * 3 + T)
    say("case", w)
    inp = make_inputs(w, device="cuda")
    dO = make_grad_output(w, device="cuda")
    idx, dq, dK, dV = run_gpu(w, inp, dO)
    rb = np.repeat(np.arange(B), T)
    rt = np.tile(np.arange(T), B)
    ref_idx = oracle_selection(w, inp, rb, rt)
    assert np.array_equal(gpu_rows(idx, rb, rt), ref_idx), "selection"
    rdq, rdK, rdV = oracle_backward(w, inp, dO, rb, rt, ref_idx)
    ex_dq, ex_dk = bound_extras(w, inp, dO, rb, rt, ref_idx)
    close("rand dq", dq.cpu().reshape(B * T, Hq, -1), rdq, ex_dq)
    close("rand dK", dK.cpu(), rdK[:, :, :N], ex_dk[:, :, :N])
    close("rand dV", dV.cpu(), rdV[:, :, :N])


BK_CASES = [
    # name, B, T, N, Hq, G, k, Bk  (k * Bk <= 2048)
    ("bk64_k32", 1, 2100, 2100, 64, 8, 32, 64),
    ("bk32_k64", 1, 2500, 2500, 64, 8, 64, 32),
    ("bk64_chunked", 2, 300, 900, 32, 8, 20, 64),
    ("bk32_g16", 1, 700, 700, 32, 16, 12, 32),
    ("bk32_tiny", 1, 5, 5, 8, 2, 4, 32),
]


@pytest.mark.parametrize("name,B,T,N,Hq,G,k,Bk", BK_CASES, ids=[c[0] for c in BK_CASES])
def test_backward_block_sizes(name, B, T, N, Hq, G, k, Bk):
    """Blocks of 64 and 32 keys: every row's dq and every key's dK / dV."""
    w = Workload(name, B=B, T=T, N=N, Hq=Hq, G=G, k=k, Bk=Bk, seed=91 + N)
    say("case", w)
    inp = make_inputs(w, device="cuda")
    dO = make_grad_output(w, device="cuda")
    idx, dq, dK, dV = run_gpu(w, inp, dO)
    rb = np.repeat(np.arange(B), T)
    rt = np.tile(np.arange(T), B)
    ref_idx = oracle_selection(w, inp, rb, rt)
    assert np.array_equal(gpu_rows(idx, rb, rt), ref_idx), "selection"
    rdq, rdK, rdV = oracle_backward(w, inp, dO, rb, rt, ref_idx)
    ex_dq, ex_dk = bound_extras(w, inp, dO, rb, rt, ref_idx)
    close(name + " dq", dq.cpu().reshape(B * T, Hq, -1), rdq, ex_dq)
    close(name + " dK", dK.cpu(), rdK[:, :, :N], ex_dk[:, :, :N])
    close(name + " dV", dV.cpu(), rdV[:, :, :N])
    check_sums(w, inp, dO, dK, dV)
