"""Decode over paged caches on the GPU against the oracle.

A paged decode of sequence b is, by definition, the contiguous decode of the
cache that its block table describes: the oracle runs on each sequence's own
contiguous inputs (length seq_lens[b]), and the GPU runs on the same data
scattered into shuffled pages of one shared pool.  Unused rows and pages of
the pools hold values that would change the result if any kernel read them
(index keys of all 4s, K rows of 300s, V rows of 1000s).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from block_sparse_long_index_amd import ops

pytestmark = pytest.mark.gpu

O_MAX, O_MEAN, LSE_TOL = 2e-2, 2e-3, 1e-3


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    ops.lib()
    torch.cuda.set_device(0)


def make_case(lens, Hq, G, k, seed, extra_pages=5):
    g = torch.Generator().manual_seed(seed)
    B = len(lens)
    nb = max(-(-L // 128) for L in lens)
    need = sum(-(-L // 128) for L in lens)
    P = need + extra_pages
    perm = torch.randperm(P, generator=g)
    kI_pool = torch.full((P, 128, 128), 4.0).to(torch.bfloat16)
    K_pool = torch.full((P, G, 128, 128), 300.0).to(torch.bfloat16)
    V_pool = torch.full((P, G, 128, 128), 1000.0).to(torch.bfloat16)
    table = torch.full((B, nb), -7, dtype=torch.int32)  # never read past a sequence's end
    seqs = []
    used = 0
    for b, L in enumerate(lens):
        kI = torch.randint(-4, 5, (L, 128), generator=g).to(torch.bfloat16)
        K = torch.randn(G, L, 128, generator=g).to(torch.bfloat16)
        V = torch.randn(G, L, 128, generator=g).to(torch.bfloat16)
        qI = torch.randint(-4, 5, (G, 128), generator=g).to(torch.bfloat16)
        q = torch.randn(Hq, 128, generator=g).to(torch.bfloat16)
        for j in range(-(-L // 128)):
            pg = int(perm[used])
            used += 1
            table[b, j] = pg
            r0, r1 = j * 128, min(L, (j + 1) * 128)
            kI_pool[pg, : r1 - r0] = kI[r0:r1]
            K_pool[pg, :, : r1 - r0] = K[:, r0:r1]
            V_pool[pg, :, : r1 - r0] = V[:, r0:r1]
        seqs.append(dict(kI=kI, K=K, V=V, qI=qI, q=q, L=L))
    return seqs, kI_pool, K_pool, V_pool, table, nb


def oracle_seq(sq, Hq, G, k):
    L = sq["L"]
    d = oracle.dims_of(1, 1, L, Hq, G, 128, 128, 128, k)
    z = np.zeros(1, dtype=np.int64)
    return oracle.forward(d, z, z, sq["qI"].unsqueeze(0), sq["kI"].unsqueeze(0),
                          sq["q"].unsqueeze(0), sq["K"].unsqueeze(0), sq["V"].unsqueeze(0))


CASES = [
    # name, lens, Hq, G, k
    ("mixed", [1000, 129, 3000, 1], 64, 8, 16),
    ("block_edges", [128, 256, 127, 255, 2048], 16, 4, 4),
    ("hg16_g1", [700, 5], 16, 1, 8),
    # 32 sequences x 4 groups: enough (sequence, group) pairs for the one-pass
    # decode attention (one workgroup per pair)
    ("many_seqs", [1 + (i * 977) % 3100 for i in range(32)], 32, 4, 16),
]


@pytest.mark.parametrize("name,lens,Hq,G,k", CASES, ids=[c[0] for c in CASES])
def test_paged_decode(name, lens, Hq, G, k):
    say("case", name)
    seqs, kI_pool, K_pool, V_pool, table, nb = make_case(lens, Hq, G, k, seed=len(name) * 7)
    B = len(lens)
    dev = "cuda"
    qI = torch.stack([s["qI"] for s in seqs]).to(dev)
    q = torch.stack([s["q"] for s in seqs]).to(dev)
    lens_t = torch.tensor(lens, dtype=torch.int64, device=dev)
    table_d = table.to(dev)
    kI_d, K_d, V_d = kI_pool.to(dev), K_pool.to(dev), V_pool.to(dev)
    idx = ops.select_blocks_paged(qI, kI_d, table_d, lens_t, k)
    idx8 = ops.select_blocks_paged(qI.float().to(torch.float8_e4m3fn),
                                   kI_d.float().to(torch.float8_e4m3fn), table_d, lens_t, k)
    O, lse = ops.sparse_attn_decode_paged(q, K_d, V_d, table_d, lens_t, idx, return_lse=True)
    # the one call (msa_decode_paged, and on the same integer values with
    # 8-bit index keys: the same scores, so the same bits)
    idx1, O1, lse1 = ops.decode_paged(qI, kI_d, q, K_d, V_d, table_d, lens_t, k, return_lse=True)
    idx18, O18, lse18 = ops.decode_paged(qI.float().to(torch.float8_e4m3fn),
                                         kI_d.float().to(torch.float8_e4m3fn), q, K_d, V_d,
                                         table_d, lens_t, k, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx8), "fp8 paged selection differs from bf16"
    assert torch.equal(idx1, idx), "one-call paged selection differs"
    assert torch.equal(idx18, idx1) and torch.equal(O18, O1) and torch.equal(lse18, lse1)
    assert (O1.float() - O.float()).abs().max().item() <= 1e-2
    assert (lse1 - lse).abs().max().item() <= 1e-3
    for b, sq in enumerate(seqs):
        ref = oracle_seq(sq, Hq, G, k)
        got_idx = idx[b, :, 0].cpu().numpy()
        assert np.array_equal(got_idx, ref["idx"][0]), (name, b, got_idx, ref["idx"][0])
        err = np.abs(O[b].float().cpu().numpy() - ref["O"][0])
        say("%s seq %d (L=%d) O err max %.3e mean %.3e" % (name, b, sq["L"], err.max(), err.mean()))
        assert err.max() <= O_MAX and err.mean() <= O_MEAN
        assert np.abs(lse[b].cpu().numpy() - ref["lse"][0]).max() <= LSE_TOL
        err1 = np.abs(O1[b].float().cpu().numpy() - ref["O"][0])
        assert err1.max() <= O_MAX and err1.mean() <= O_MEAN, (name, b, "one call")
        assert np.abs(lse1[b].cpu().numpy() - ref["lse"][0]).max() <= LSE_TOL


def test_paged_equals_contiguous_full_256k():
    """The full decode shape (16 x 256K) with an identity-like page table
    (page = b * nb + j) must give exactly the contiguous path's selection and
    output: the same kernels, only the addressing differs."""
    from msa_inputs import WORKLOADS, make_inputs
    w = WORKLOADS["decode_256k_b16"]
    inp = make_inputs(w, device="cuda")
    qI, kI, K, V = inp["qI"][:, 0].contiguous(), inp["kI"], inp["K"], inp["V"]
    q = inp["q"][:, 0].contiguous()
    nb = w.N // 128
    # pools laid out page-major: page p = (b, j)
    kI_pool = kI.view(w.B * nb, 128, 128)
    K_pool = K.view(w.B, w.G, nb, 128, 128).permute(0, 2, 1, 3, 4).reshape(w.B * nb, w.G, 128, 128)
    V_pool = V.view(w.B, w.G, nb, 128, 128).permute(0, 2, 1, 3, 4).reshape(w.B * nb, w.G, 128, 128)
    table = torch.arange(w.B * nb, dtype=torch.int32, device="cuda").view(w.B, nb)
    lens = torch.full((w.B,), w.N, dtype=torch.int64, device="cuda")
    idx_c = ops.select_blocks(inp["qI"], kI, w.k)
    idx_p = ops.select_blocks_paged(qI, kI_pool, table, lens, w.k)
    O_c = ops.sparse_attn_decode(q, K, V, idx_c)
    O_p = ops.sparse_attn_decode_paged(q, K_pool.contiguous(), V_pool.contiguous(), table, lens,
                                       idx_p)
    idx_c1, O_c1 = ops.decode(inp["qI"], kI, q, K, V, w.k)
    idx_p1, O_p1 = ops.decode_paged(qI, kI_pool, q, K_pool.contiguous(), V_pool.contiguous(),
                                    table, lens, w.k)
    torch.cuda.synchronize()
    assert torch.equal(idx_c, idx_p)
    assert torch.equal(O_c, O_p)
    assert torch.equal(idx_p1, idx_c1) and torch.equal(O_p1, O_c1)
