"""Algorithmic work counts for the MSA forward path (host logic, no GPU).

These are the figures the benchmark divides by measured time.  They count
what the method has to do by its definition, not what a kernel happens to
execute:

* index scoring (stages 1+2): one d_I-long dot per (query, group, visible
  key): 2 * G * d_I * sum_t (p_t + 1) FLOP;
* main branch (stage 4): QK^T and PV over the n_sel(t) support keys of every
  query head: 4 * Hq * d_h * sum_t n_sel(t) FLOP, where
  n_sel(t) = min(local(t), k - 1) * Bk + (p_t mod Bk) + 1;
* decode bytes: the whole index-key cache (B * L * d_I * 2 B), the selected
  K and V blocks, and the small q, q^I, O and idx tensors;
* standalone top-k bytes: the visible candidate block scores (fp32) of every
  row plus the written indices.

Sources: the MSA study-notes page (dimensionstp.github.io/study-concept/msa)
section 2-3 (index score over the whole causal context, main-branch budget
k * Bk) and section 5-3 (per-token compute reduction); the llama.cpp analysis
page (velog.io/@sleekydevzero86/...) section 2 (256 B of index key per token,
decode traffic of dense vs MSA).
"""
from __future__ import annotations

import numpy as np


def positions(N: int, T: int) -> np.ndarray:
    return np.arange(N - T, N, dtype=np.int64)


def causal_pairs(N: int, T: int, B: int = 1) -> int:
    p = positions(N, T)
    return int(B * (p + 1).sum())


def support_tokens(N: int, T: int, Bk: int, k: int, B: int = 1) -> int:
    p = positions(N, T)
    L = p // Bk
    n = np.minimum(L, k - 1) * Bk + (p % Bk) + 1
    return int(B * n.sum())


def index_flops(N, T, G, d_I, B=1) -> int:
    return 2 * G * d_I * causal_pairs(N, T, B)


def candidate_flops(N, T, G, d_I, Bk, B=1) -> int:
    """Scores of the candidate blocks only (the local block excluded): the
    work a fused select does, since the local block is forced."""
    p = positions(N, T)
    return int(2 * G * d_I * B * ((p // Bk) * Bk).sum())


def main_flops(N, T, Hq, d_h, Bk, k, B=1) -> int:
    return 4 * Hq * d_h * support_tokens(N, T, Bk, k, B)


def backward_flops(N, T, Hq, d_h, Bk, k, B=1) -> int:
    """Stage-4 backward over the same supports: five products of the
    forward's per-product size (S = q K^T recomputed, dP = dO V^T,
    dV += P^T dO, dK += dS^T q, dq = dS K), against the forward's two."""
    return 10 * Hq * d_h * support_tokens(N, T, Bk, k, B)


def index_kl_flops(N, T, Hq, G, d_h, d_I, Bk, k, B=1) -> int:
    """Index-branch KL backward over the same supports: the teacher's main
    scores for every head (2 d_h per (row, head, key)), the index scores twice
    (proxy lse pass, gradient pass) and the two gradient products dq^I, dk^I
    (2 d_I each per (row, group, key))."""
    n = support_tokens(N, T, Bk, k, B)
    return 2 * Hq * d_h * n + 8 * G * d_I * n


def train_flops(N, T, Hq, G, d_h, d_I, Bk, k, B=1) -> int:
    """Fused training backward: the stage-4 backward's five products plus the
    index branch's four (index scores for the proxy lse and for the gradient
    pass, dq^I, dk^I); the teacher comes from the backward's own weights, so
    the main scores are not counted twice."""
    n = support_tokens(N, T, Bk, k, B)
    return 10 * Hq * d_h * n + 8 * G * d_I * n


def prefill_flops(w) -> dict:
    idx = index_flops(w.N, w.T, w.G, w.d_I, w.B)
    main = main_flops(w.N, w.T, w.Hq, w.d_h, w.Bk, w.k, w.B)
    return dict(index=idx, main=main, total=idx + main,
                candidates=candidate_flops(w.N, w.T, w.G, w.d_I, w.Bk, w.B))


def decode_bytes(w, index_bytes: int = 2) -> dict:
    """Bytes one decode step must move: T == 1, cache length N; the index
    branch's q^I / k^I take index_bytes per value (2: bf16, 1: fp8)."""
    kI = w.B * w.N * w.d_I * index_bytes
    nsel_blocks = w.B * w.G * min(w.k, (w.N - 1) // w.Bk + 1)
    kv = nsel_blocks * w.Bk * w.d_h * 2 * 2
    small = (w.B * w.Hq * w.d_h * 2 * 2          # q in, O out
             + w.B * w.G * w.d_I * index_bytes   # q^I
             + w.B * w.G * w.k * 4)              # idx
    return dict(index_keys=kI, kv=kv, small=small, total=kI + kv + small)


def stage4_bytes(w) -> dict:
    """Bytes stage 4 must move at least: q, K, V and idx read once, O (bf16)
    and lse (fp32) written once."""
    q = w.B * w.T * w.Hq * w.d_h * 2
    kv = 2 * w.B * w.G * w.N * w.d_h * 2
    idx = w.B * w.G * w.T * w.k * 4
    out = q + w.B * w.T * w.Hq * 4
    return dict(q=q, kv=kv, idx=idx, out=out, total=q + kv + idx + out)


def partial_bytes(w) -> dict:
    """Bytes of the per-(row, slot) partial results a split over key blocks
    produces for every query head: the bf16 unnormalised output (2 d_h B) and
    its (max, sum) pair (8 B), for the support slots of every row.  A KV-outer
    schedule writes them once and its combine reads them once; the combine
    also reads idx and writes O and lse."""
    p = positions(w.N, w.T)
    slots = np.minimum(p // w.Bk + 1, w.k)
    entries = int(w.B * w.Hq * slots.sum())
    part = entries * (2 * w.d_h + 8)
    comb = part + w.B * w.G * w.T * w.k * 4 + w.B * w.T * w.Hq * (2 * w.d_h + 4)
    return dict(entries=entries, partials=part, combine=comb)


def decode_flops(w) -> int:
    return (2 * w.G * w.d_I * w.B * w.N
            + 4 * w.Hq * w.d_h * support_tokens(w.N, 1, w.Bk, w.k, w.B))


def topk_bytes(w) -> dict:
    p = positions(w.N, w.T)
    L = p // w.Bk
    read = int(w.B * w.G * 4 * L.sum())
    write = w.B * w.G * w.T * w.k * 4
    return dict(read=read, write=write, total=read + write)


def dense_over_msa_per_token(N, Hq, G, d_h, d_I, Bk, k, fixed_budget=True) -> float:
    """Attention compute per token, dense causal GQA over MSA (index branch
    plus main branch), averaged over the positions of an N-token context.

    fixed_budget=True charges every token the full k * Bk main-branch keys
    (the fixed budget the study notes state in section 2-3); False charges
    the exact support n_sel(t), which is smaller for the partial local block
    and for early tokens."""
    dense = 4 * Hq * d_h * causal_pairs(N, N)
    if fixed_budget:
        main = 4 * Hq * d_h * N * k * Bk
    else:
        main = main_flops(N, N, Hq, d_h, Bk, k)
    return dense / (index_flops(N, N, G, d_I) + main)


def dense_decode_kv_bytes(context, kv_heads, d_h, bytes_per_elem, layers) -> int:
    """K and V read per generated token by dense attention."""
    return 2 * kv_heads * d_h * bytes_per_elem * layers * context


def index_key_bytes_per_token(d_I, bytes_per_elem=2) -> int:
    return d_I * bytes_per_elem
