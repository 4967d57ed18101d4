"""Seeded synthetic inputs for the MiniMax Sparse Attention (MSA) forward path.

This module holds the workload shapes and the seeded random generators, and
nothing else: it does none of the method's arithmetic (no scores, no pooling,
no selection, no attention).  Both the CPU oracle side (tests, bench baseline)
and the HIP side draw their inputs from here; the oracle always receives copies
of the very tensors the GPU path consumed.

Value distributions follow the workloads the MSA pages describe:

* main-branch q, K, V: standard normal, rounded to bf16;
* index-branch q^I, k^I: integers drawn uniformly from {-4, ..., 4}, stored as
  bf16 (exact), so every index dot product is an integer of magnitude at most
  128 * 16 = 2048 and is exact in fp32 in any summation order;
* "needle" blocks: one key token of a chosen block gets k^I = u, a random
  {-4, +4}^128 sign vector (self dot 2048); a quarter of the later query rows of
  the owning group copy u into q^I with a quarter of the coordinates redrawn,
  so those rows score the needle block near 1536 while random block maxima sit
  near 200-340.  This gives the selection a content dependence like the
  retrieval evaluations on the study-notes page (section 5, RULER) without
  using any item of such a suite.

Layouts (all contiguous, row-major):
  qI [B, T, G, d_I]   kI [B, N, d_I]
  q  [B, T, Hq, d_h]  K, V [B, G, N, d_h]
  dO [B, T, Hq, d_h]  (the backward's upstream gradient, ~N(0,1) bf16)
Query row t of sequence b sits at absolute position p = N - T + t.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    N: int
    Hq: int
    G: int
    d_h: int = 128
    d_I: int = 128
    Bk: int = 128
    k: int = 16
    needles: Optional[str] = None  # None | "per_group_8" | "per_64k"
    seed: int = 1234

    @property
    def NB(self) -> int:
        return (self.N + self.Bk - 1) // self.Bk

    @property
    def hg(self) -> int:
        return self.Hq // self.G

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads of the measurement plan, in order; seeds are 1234 + order.
WORKLOADS = {
    "prefill_2k": Workload("prefill_2k", B=1, T=2048, N=2048, Hq=8, G=2, k=4,
                           needles=None, seed=1234),
    "prefill_32k": Workload("prefill_32k", B=1, T=32768, N=32768, Hq=64, G=8,
                            k=16, needles="per_group_8", seed=1235),
    "prefill_128k": Workload("prefill_128k", B=1, T=131072, N=131072, Hq=64,
                             G=8, k=16, needles="per_group_8", seed=1236),
    "decode_256k_b16": Workload("decode_256k_b16", B=16, T=1, N=262144,
                                Hq=64, G=8, k=16, needles=None, seed=1237),
    "prefill_1m": Workload("prefill_1m", B=1, T=1048576, N=1048576, Hq=64,
                           G=8, k=16, needles="per_64k", seed=1238),
}


def _randint_bf16(gen, shape, device, lo=-4, hi=4):
    return torch.randint(lo, hi + 1, shape, generator=gen, device=device,
                         dtype=torch.int16).to(torch.bfloat16)


def _randn_bf16(gen, shape, device, chunk=1 << 27):
    """Standard normal values rounded to bf16, drawn in chunks so that the
    fp32 temporary stays small for the 1M-token workload."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        flat[s:e] = torch.randn(e - s, generator=gen, device=device,
                                dtype=torch.float32).to(torch.bfloat16)
    return out


def _needle_blocks(w: Workload, gen, device):
    """Needle block ids per group: a list of G 1-D int64 tensors (sorted)."""
    NB = w.NB
    if w.needles == "per_group_8":
        per = 8
        if NB - 1 < per * w.G:
            raise ValueError("too few blocks for 8 disjoint needles per group")
        perm = torch.randperm(NB - 1, generator=gen, device=device)[: per * w.G]
        blocks = perm.view(w.G, per)
        return [torch.sort(blocks[g]).values for g in range(w.G)]
    if w.needles == "per_64k":
        seg = 65536
        nseg = max(1, w.N // seg)
        bps = seg // w.Bk
        offs = torch.randint(0, bps, (nseg,), generator=gen, device=device)
        blocks = torch.arange(nseg, device=device) * bps + offs
        blocks = torch.clamp(blocks, max=NB - 2)
        owner = torch.arange(nseg, device=device) % w.G
        return [torch.sort(blocks[owner == g]).values for g in range(w.G)]
    raise ValueError(w.needles)


def make_index_inputs(w: Workload, device="cpu", gen=None):
    """q^I [B,T,G,d_I] and k^I [B,N,d_I] (bf16, integer-valued), with needles
    planted when the workload asks for them."""
    if gen is None:
        gen = torch.Generator(device=device)
        gen.manual_seed(w.seed)
    kI = _randint_bf16(gen, (w.B, w.N, w.d_I), device)
    qI = _randint_bf16(gen, (w.B, w.T, w.G, w.d_I), device)
    meta = {}
    if w.needles is not None:
        blocks = _needle_blocks(w, gen, device)
        meta["needle_blocks"] = [b.cpu() for b in blocks]
        # per group: the query rows that copied a needle and that needle's block
        meta["needle_rows"] = []
        pos = torch.arange(w.T, device=device) + (w.N - w.T)
        local = torch.div(pos, w.Bk, rounding_mode="floor")
        for g in range(w.G):
            nb = blocks[g]
            n = nb.numel()
            if n == 0:
                meta["needle_rows"].append((torch.zeros(0, dtype=torch.int64),
                                            torch.zeros(0, dtype=torch.int64)))
                continue
            signs = torch.randint(0, 2, (n, w.d_I), generator=gen, device=device)
            u = (signs * 8 - 4).to(torch.bfloat16)  # {-4, +4}
            tok = nb * w.Bk + torch.randint(0, w.Bk, (n,), generator=gen, device=device)
            kI[:, tok, :] = u.unsqueeze(0)
            # rows whose local block lies strictly after a needle block
            eligible = torch.searchsorted(nb.contiguous(), local.contiguous())
            pick = torch.rand(w.T, generator=gen, device=device)
            which = torch.floor(torch.rand(w.T, generator=gen, device=device)
                                * eligible.clamp(min=1).float()).long()
            which = torch.minimum(which, (eligible - 1).clamp(min=0))
            assign = (pick < 0.25) & (eligible > 0)
            redraw = torch.rand(w.T, w.d_I, generator=gen, device=device) < 0.25
            fresh = _randint_bf16(gen, (w.T, w.d_I), device)
            planted = torch.where(redraw, fresh, u[which])
            for b in range(w.B):
                row = qI[b, :, g, :]
                row[assign] = planted[assign]
            rows = torch.nonzero(assign).view(-1)
            meta["needle_rows"].append((rows.cpu(), nb[which[rows]].cpu()))
        meta["needle_rows_fraction"] = 0.25
    return qI, kI, meta


def make_main_inputs(w: Workload, device="cpu", gen=None):
    """q [B,T,Hq,d_h], K [B,G,N,d_h], V [B,G,N,d_h] (bf16, ~N(0,1))."""
    if gen is None:
        gen = torch.Generator(device=device)
        gen.manual_seed(w.seed + 100000)
    q = _randn_bf16(gen, (w.B, w.T, w.Hq, w.d_h), device)
    K = _randn_bf16(gen, (w.B, w.G, w.N, w.d_h), device)
    V = _randn_bf16(gen, (w.B, w.G, w.N, w.d_h), device)
    return q, K, V


def make_grad_output(w: Workload, device="cpu"):
    """dO [B,T,Hq,d_h] (bf16, ~N(0,1)): the upstream gradient of the
    attention output for the backward."""
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed + 200000)
    return _randn_bf16(gen, (w.B, w.T, w.Hq, w.d_h), device)


def make_inputs(w: Workload, device="cpu"):
    qI, kI, meta = make_index_inputs(w, device)
    q, K, V = make_main_inputs(w, device)
    return dict(qI=qI, kI=kI, q=q, K=K, V=V, meta=meta)


def sample_rows(w: Workload, n: int, seed: int = 99):
    """A fixed sample of (b, t) query rows: the edge positions the method has
    (p = 0, Bk-1, Bk, (k-1)*Bk +- 1, N-1, block boundaries) plus uniform rows.
    Returns two int64 tensors (b, t)."""
    edge_pos = {0, w.Bk - 1, w.Bk, (w.k - 1) * w.Bk - 1, (w.k - 1) * w.Bk,
                (w.k - 1) * w.Bk + 1, w.k * w.Bk, w.N - 1, w.N - 2,
                w.N - w.Bk, w.N - w.Bk - 1}
    t_edge = sorted(p - (w.N - w.T) for p in edge_pos if 0 <= p - (w.N - w.T) < w.T)
    g = torch.Generator().manual_seed(seed)
    n_rand = max(0, n - len(t_edge) * w.B)
    tb = torch.randint(0, w.B, (n_rand,), generator=g)
    tt = torch.randint(0, w.T, (n_rand,), generator=g)
    b = torch.cat([torch.arange(w.B).repeat_interleave(len(t_edge)), tb])
    t = torch.cat([torch.tensor(t_edge, dtype=torch.int64).repeat(w.B), tt])
    return b[:max(n, len(t_edge) * w.B)], t[:max(n, len(t_edge) * w.B)]
