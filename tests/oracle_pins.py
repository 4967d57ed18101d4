"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each pin takes an ``oracle.OracleLib`` and raises AssertionError when the
oracle disagrees with what the MSA pages and the mathematics fix:

* brute force on tiny inputs (a dense score matrix with a causal mask, cut
  into blocks and max-reduced; exhaustive enumeration of block subsets);
* closed forms (zero keys, one-hot keys with a linear ramp, all-ties
  selection, constant values, zero queries);
* special cases that reduce to a library routine (dense causal GQA attention
  via torch's scaled_dot_product_attention when k*Bk covers the context,
  a masked SDPA for any selection, numpy.lexsort ranking);
* the invariants the pages state (local block always selected, budget of at
  most k*Bk keys, heads of a group share the selection).

The same functions run against deliberately broken copies of the oracle in
test_oracle_pins.py to show that each plausible mistake is caught.
"""
from __future__ import annotations

import itertools
import math

import numpy as np
import torch
import torch.nn.functional as F

from oracle import dims_of


def _gen(seed):
    return torch.Generator().manual_seed(seed)


def _int_bf16(g, shape, lo=-4, hi=4):
    return torch.randint(lo, hi + 1, shape, generator=g).to(torch.bfloat16)


def _randn_bf16(g, shape):
    return torch.randn(shape, generator=g).to(torch.bfloat16)


def _all_rows(B, T):
    return np.repeat(np.arange(B), T), np.tile(np.arange(T), B)


def _brute_block_scores(qI, kI, T, N, Bk):
    """Dense reference for stages 1+2 on one sequence: qI [T,G,dI], kI [N,dI]
    -> [T, G, NB] with the full score matrix built by einsum and masked."""
    q = qI.double().numpy()
    k = kI.double().numpy()
    dI = q.shape[-1]
    s = np.einsum("tgc,jc->tgj", q, k) / math.sqrt(dI)
    pos = (N - T) + np.arange(T)
    future = np.arange(N)[None, :] > pos[:, None]
    s = np.where(future[:, None, :], -np.inf, s)
    NB = -(-N // Bk)
    pad = np.full((T, s.shape[1], NB * Bk - N), -np.inf)
    s = np.concatenate([s, pad], axis=2).reshape(T, s.shape[1], NB, Bk)
    return s.max(axis=3)


# ----------------------------------------------------------------- stages 1+2
def pin_scores_brute_force(orc):
    cases = [  # B, T, N, G, dI, Bk, integer-valued?
        (2, 23, 23, 3, 8, 4, True),
        (1, 7, 30, 2, 16, 8, True),
        (2, 19, 19, 1, 4, 5, False),
        (1, 1, 13, 2, 8, 4, False),
        (1, 40, 40, 2, 32, 128, True),
    ]
    for ci, (B, T, N, G, dI, Bk, integer) in enumerate(cases):
        g = _gen(10 + ci)
        mk = _int_bf16 if integer else _randn_bf16
        qI = mk(g, (B, T, G, dI))
        kI = mk(g, (B, N, dI))
        d = dims_of(B, T, N, G, G, 128, dI, Bk, 4)
        rb, rt = _all_rows(B, T)
        S = orc.block_scores(d, rb, rt, qI.reshape(B * T, G, dI), kI)
        for b in range(B):
            ref = _brute_block_scores(qI[b], kI[b], T, N, Bk)
            got = S[b * T:(b + 1) * T]
            assert np.array_equal(np.isneginf(got), np.isneginf(ref)), ci
            fin = np.isfinite(ref)
            if integer:
                assert np.array_equal(got[fin], ref[fin]), ci
            else:
                assert np.allclose(got[fin], ref[fin], rtol=1e-12, atol=1e-12), ci


def pin_scores_zero_keys(orc):
    B, T, N, G, dI, Bk = 1, 33, 33, 2, 8, 8
    g = _gen(1)
    qI = _int_bf16(g, (B, T, G, dI))
    kI = torch.zeros(B, N, dI, dtype=torch.bfloat16)
    d = dims_of(B, T, N, G, G, 128, dI, Bk, 4)
    rb, rt = _all_rows(B, T)
    S = orc.block_scores(d, rb, rt, qI.reshape(B * T, G, dI), kI)
    NB = -(-N // Bk)
    for t in range(T):
        vis = t // Bk  # last visible block (T == N)
        for blk in range(NB):
            want = 0.0 if blk <= vis else -np.inf
            assert (S[t, :, blk] == want).all(), (t, blk)


def pin_scores_ramp_closed_form(orc):
    """q^I = c * e_0 and k^I[j] = j * e_0 give s_j = c * j / sqrt(d_I); the
    block max is the last visible key for c > 0 and the first key for c < 0.
    Uses T < N so that the bottom-right causal alignment is pinned too."""
    B, T, N, G, dI, Bk = 1, 9, 50, 2, 4, 8
    qI = torch.zeros(B, T, G, dI)
    qI[..., 0, 0] = 2.0
    qI[..., 1, 0] = -3.0
    kI = torch.zeros(B, N, dI)
    kI[0, :, 0] = torch.arange(N, dtype=torch.float32)
    d = dims_of(B, T, N, G, G, 128, dI, Bk, 4)
    rb, rt = _all_rows(B, T)
    S = orc.block_scores(d, rb, rt, qI.to(torch.bfloat16).reshape(T, G, dI),
                         kI.to(torch.bfloat16))
    NB = -(-N // Bk)
    for t in range(T):
        p = N - T + t
        for blk in range(NB):
            lo = blk * Bk
            if lo > p:
                assert S[t, 0, blk] == -np.inf and S[t, 1, blk] == -np.inf
                continue
            hi = min(lo + Bk - 1, p)
            assert S[t, 0, blk] == 2.0 * hi / 2.0, (t, blk)
            assert S[t, 1, blk] == -3.0 * lo / 2.0, (t, blk)


# ------------------------------------------------------------------- stage 3
def _expected_ties(p, Bk, k):
    L = p // Bk
    m = min(k - 1, L)
    return list(range(m)) + [L] + [-1] * (k - m - 1)


def pin_select_all_ties(orc):
    """Zero index queries make every visible block score 0: the selection is
    the lowest min(k-1, L) blocks plus the local block L."""
    for (B, T, N, G, Bk, k) in [(2, 70, 70, 2, 8, 4), (1, 5, 90, 3, 8, 6),
                                (1, 300, 300, 1, 16, 16)]:
        g = _gen(3)
        qI = torch.zeros(B, T, G, 8, dtype=torch.bfloat16)
        kI = _int_bf16(g, (B, N, 8))
        d = dims_of(B, T, N, G, G, 128, 8, Bk, k)
        rb, rt = _all_rows(B, T)
        S = orc.block_scores(d, rb, rt, qI.reshape(B * T, G, 8), kI)
        idx = orc.select(d, rt, S)
        for r in range(B * T):
            want = _expected_ties(N - T + rt[r], Bk, k)
            for gg in range(G):
                assert idx[r, gg].tolist() == want, (r, gg, idx[r, gg], want)


def _best_subset_brute(scores, L, m):
    """The unique m-subset of 0..L-1 whose every member beats every
    non-member under (score desc, block asc), found by enumeration."""
    found = []
    for A in itertools.combinations(range(L), m):
        Aset = set(A)
        ok = True
        for a in A:
            for c in range(L):
                if c in Aset:
                    continue
                if not (scores[a] > scores[c] or (scores[a] == scores[c] and a < c)):
                    ok = False
                    break
            if not ok:
                break
        if ok:
            found.append(A)
    assert len(found) == 1
    return list(found[0])


def pin_select_exhaustive(orc):
    g = np.random.default_rng(5)
    Bk = 4
    for (NB, k, lo, hi) in [(12, 4, -3, 3), (11, 5, 0, 1), (9, 9, -50, 50), (12, 1, 0, 2)]:
        N = NB * Bk - 1
        T = N
        d = dims_of(1, T, N, 2, 2, 128, 8, Bk, k)
        rt = np.arange(T)
        S = g.integers(lo, hi + 1, size=(T, 2, NB)).astype(np.float64)
        idx = orc.select(d, rt, S)
        for t in range(T):
            L = t // Bk
            m = min(k - 1, L)
            for gg in range(2):
                best = _best_subset_brute(S[t, gg], L, m)
                want = sorted(best) + [L] + [-1] * (k - m - 1)
                assert idx[t, gg].tolist() == want, (t, gg)


def pin_select_lexsort(orc):
    g = np.random.default_rng(6)
    # (Bk, k, NB): 128-key-style k = 16, and the 2048-token budget at Bk = 32 (k = 64)
    for Bk, k, NB in ((16, 16, 200), (32, 64, 90)):
        N = T = NB * Bk
        d = dims_of(1, T, N, 3, 3, 128, 8, Bk, k)
        rt = g.integers(0, T, size=300)
        S = np.round(g.normal(size=(rt.size, 3, NB)) * 4)  # many ties
        idx = orc.select(d, rt, S)
        for r in range(rt.size):
            L = rt[r] // Bk
            m = min(k - 1, L)
            for gg in range(3):
                cand = np.arange(L)
                order = np.lexsort((cand, -S[r, gg, :L]))[:m]
                want = sorted(cand[order].tolist()) + [L] + [-1] * (k - m - 1)
                assert idx[r, gg].tolist() == want


def pin_select_needle(orc):
    """A key whose index vector equals the query's wins its block's place in
    every later query's selection."""
    B, N, G, dI, Bk, k = 1, 512, 2, 16, 16, 3
    T = N
    g = _gen(8)
    kI = _int_bf16(g, (B, N, dI), -1, 1)
    qI = _int_bf16(g, (B, T, G, dI), -1, 1)
    u = torch.full((dI,), 4.0)
    u[::2] = -4.0
    kI[0, 77] = u.to(torch.bfloat16)  # block 4
    qI[0, :, 1] = u.to(torch.bfloat16)
    d = dims_of(B, T, N, G, G, 128, dI, Bk, k)
    rb, rt = _all_rows(B, T)
    S = orc.block_scores(d, rb, rt, qI.reshape(T, G, dI), kI)
    idx = orc.select(d, rt, S)
    for t in range(5 * Bk, T):
        assert 4 in idx[t, 1].tolist(), t


def pin_select_invariants(orc):
    g = _gen(9)
    B, T, N, G, dI, Bk, k = 2, 200, 200, 3, 8, 8, 5
    qI = _int_bf16(g, (B, T, G, dI))
    kI = _int_bf16(g, (B, N, dI))
    d = dims_of(B, T, N, G, G, 128, dI, Bk, k)
    rb, rt = _all_rows(B, T)
    S = orc.block_scores(d, rb, rt, qI.reshape(B * T, G, dI), kI)
    idx = orc.select(d, rt, S)
    for r in range(B * T):
        p = rt[r]
        L = p // Bk
        for gg in range(G):
            sel = [x for x in idx[r, gg].tolist() if x >= 0]
            assert sel == sorted(set(sel))
            assert sel[-1] == L
            assert len(sel) == min(k, L + 1)
            assert all(x <= L for x in sel)
            n_keys = sum(min(Bk, p - x * Bk + 1) for x in sel)
            assert n_keys <= k * Bk
            pad = idx[r, gg].tolist()[len(sel):]
            assert all(x == -1 for x in pad)


# ------------------------------------------------------------------- stage 4
def _sdpa_reference(q, K, V, mask, hg):
    """torch SDPA in fp64 with the K/V heads repeated for GQA.
    q [T,Hq,dh], K/V [G,N,dh], mask [G or 1, T, N] bool (True = attend)."""
    qq = q.double().permute(1, 0, 2)  # [Hq, T, dh]
    kk = K.double().repeat_interleave(hg, dim=0)
    vv = V.double().repeat_interleave(hg, dim=0)
    mm = mask.repeat_interleave(hg, dim=0) if mask.shape[0] > 1 else mask
    out = F.scaled_dot_product_attention(qq.unsqueeze(0), kk.unsqueeze(0),
                                         vv.unsqueeze(0), attn_mask=mm.unsqueeze(0))
    scores = (qq @ kk.transpose(1, 2)) / math.sqrt(qq.shape[-1])
    scores = scores.masked_fill(~mm, -math.inf)
    lse = torch.logsumexp(scores, dim=-1)  # [Hq, T]
    return out[0].permute(1, 0, 2).numpy(), lse.permute(1, 0).numpy()


def _mask_from_idx(idx, T, N, Bk, G):
    """[G, T, N] bool: key j visible (j <= p) and in a selected block."""
    m = torch.zeros(G, T, N, dtype=torch.bool)
    for t in range(T):
        p = N - T + t
        for g in range(G):
            for blk in idx[t, g].tolist():
                if blk < 0:
                    continue
                lo = blk * Bk
                hi = min(lo + Bk, p + 1)
                if hi > lo:
                    m[g, t, lo:hi] = True
    return m


def _attend_case(orc, B, T, N, Hq, G, dh, Bk, k, seed, idx_maker):
    g = _gen(seed)
    q = _randn_bf16(g, (B, T, Hq, dh))
    K = _randn_bf16(g, (B, G, N, dh))
    V = _randn_bf16(g, (B, G, N, dh))
    d = dims_of(B, T, N, Hq, G, dh, 8, Bk, k)
    rb, rt = _all_rows(B, T)
    idx = idx_maker(d, rb, rt, g)
    O, lse = orc.attend(d, rb, rt, q.reshape(B * T, Hq, dh), K, V, idx)
    return q, K, V, idx, O.reshape(B, T, Hq, dh), lse.reshape(B, T, Hq)


def pin_attend_dense_equivalence(orc):
    """k*Bk covering the context makes MSA dense causal GQA attention."""
    for (B, T, N, Hq, G, dh, Bk) in [(1, 40, 40, 4, 2, 16, 8),
                                     (2, 11, 37, 6, 3, 8, 4),
                                     (1, 130, 130, 2, 1, 32, 16)]:
        NB = -(-N // Bk)
        k = NB + 1

        def all_blocks(d, rb, rt, g):
            idx = np.full((rb.size, d.G, d.k), -1, dtype=np.int32)
            for r in range(rb.size):
                L = (N - T + rt[r]) // Bk
                idx[r, :, :L + 1] = np.arange(L + 1)
            return idx

        q, K, V, idx, O, lse = _attend_case(orc, B, T, N, Hq, G, dh, Bk, k, 21,
                                            all_blocks)
        pos = (N - T) + torch.arange(T)
        causal = (torch.arange(N)[None, :] <= pos[:, None]).unsqueeze(0)
        for b in range(B):
            refO, refL = _sdpa_reference(q[b], K[b], V[b], causal, Hq // G)
            assert np.allclose(O[b], refO, rtol=1e-10, atol=1e-10)
            assert np.allclose(lse[b], refL, rtol=1e-10, atol=1e-10)


def pin_attend_masked_sdpa(orc):
    """Any selection: attention over the support equals SDPA with the
    support's boolean mask (also with more than 16 slots)."""
    for (B, T, N, Hq, G, dh, Bk, k) in ((1, 64, 64, 6, 3, 16, 4, 4),
                                        (1, 200, 200, 4, 2, 8, 2, 40)):

        def random_sel(d, rb, rt, g):
            S = torch.randn(rb.size, d.G, -(-N // Bk), generator=g).double().numpy()
            return orc.select(d, rt, S)

        q, K, V, idx, O, lse = _attend_case(orc, B, T, N, Hq, G, dh, Bk, k, 22,
                                            random_sel)
        mask = _mask_from_idx(idx, T, N, Bk, G)
        refO, refL = _sdpa_reference(q[0], K[0], V[0], mask, Hq // G)
        assert np.allclose(O[0], refO, rtol=1e-10, atol=1e-10)
        assert np.allclose(lse[0], refL, rtol=1e-10, atol=1e-10)


def pin_attend_k1_block_diagonal(orc):
    """k = 1 keeps only the local block: block-diagonal causal attention."""
    B, T, N, Hq, G, dh, Bk = 1, 45, 45, 4, 2, 8, 8

    def local_only(d, rb, rt, g):
        idx = np.zeros((rb.size, d.G, 1), dtype=np.int32)
        idx[:, :, 0] = ((N - T + rt) // Bk)[:, None]
        return idx

    q, K, V, idx, O, lse = _attend_case(orc, B, T, N, Hq, G, dh, Bk, 1, 23,
                                        local_only)
    j = torch.arange(N)
    pos = (N - T) + torch.arange(T)
    mask = ((j[None, :] // Bk) == (pos[:, None] // Bk)) & (j[None, :] <= pos[:, None])
    refO, refL = _sdpa_reference(q[0], K[0], V[0], mask.unsqueeze(0), Hq // G)
    assert np.allclose(O[0], refO, rtol=1e-10, atol=1e-10)
    assert np.allclose(lse[0], refL, rtol=1e-10, atol=1e-10)


def pin_attend_closed_forms(orc):
    """Zero queries: uniform weights, lse = ln(number of support keys) and O
    the mean of V over the support.  Constant V: O equals that constant."""
    B, T, N, Hq, G, dh, Bk, k = 1, 50, 50, 4, 2, 8, 8, 3
    g = _gen(24)
    q = torch.zeros(B, T, Hq, dh, dtype=torch.bfloat16)
    K = _randn_bf16(g, (B, G, N, dh))
    V = _randn_bf16(g, (B, G, N, dh))
    d = dims_of(B, T, N, Hq, G, dh, 8, Bk, k)
    rb, rt = _all_rows(B, T)
    S = torch.randn(T, G, -(-N // Bk), generator=g).double().numpy()
    idx = orc.select(d, rt, S)
    O, lse = orc.attend(d, rb, rt, q.reshape(T, Hq, dh), K, V, idx)
    for t in range(T):
        for h in range(Hq):
            gg = h // (Hq // G)
            keys = []
            for blk in idx[t, gg].tolist():
                if blk >= 0:
                    keys += list(range(blk * Bk, min(blk * Bk + Bk, t + 1)))
            assert abs(lse[t, h] - math.log(len(keys))) < 1e-12
            mean = V[0, gg, keys].double().mean(0).numpy()
            assert np.allclose(O[t, h], mean, atol=1e-12)
    Vc = torch.full((B, G, N, dh), 1.5, dtype=torch.bfloat16)
    q2 = _randn_bf16(g, (B, T, Hq, dh))
    O2, _ = orc.attend(d, rb, rt, q2.reshape(T, Hq, dh), K, Vc, idx)
    assert np.allclose(O2, 1.5, atol=1e-12)


def pin_decode_is_last_prefill_row(orc):
    """A single new token at the end of a cache of length L is the last row
    of the prefill over the same L tokens."""
    B, N, Hq, G, dh, dI, Bk, k = 2, 77, 4, 2, 16, 8, 8, 3
    g = _gen(25)
    qI = _int_bf16(g, (B, N, G, dI))
    kI = _int_bf16(g, (B, N, dI))
    q = _randn_bf16(g, (B, N, Hq, dh))
    K = _randn_bf16(g, (B, G, N, dh))
    V = _randn_bf16(g, (B, G, N, dh))
    dp = dims_of(B, N, N, Hq, G, dh, dI, Bk, k)
    dd = dims_of(B, 1, N, Hq, G, dh, dI, Bk, k)
    rb = np.arange(B)
    full = orc.forward(dp, rb, np.full(B, N - 1), qI[:, N - 1], kI, q[:, N - 1], K, V)
    dec = orc.forward(dd, rb, np.zeros(B, dtype=np.int64), qI[:, N - 1], kI,
                      q[:, N - 1], K, V)
    assert np.array_equal(full["idx"], dec["idx"])
    assert np.array_equal(full["S"], dec["S"])
    assert np.array_equal(full["O"], dec["O"])


def pin_e4m3_codes(orc):
    """The 8-bit E4M3 decoder against torch's float8_e4m3fn conversion for all
    256 codes (a library routine), and a few codes checked by hand from the
    format: 0x38 = 1, 0xB8 = -1, 0x7E = 448 (largest finite), 0x08 = 2^-6
    (smallest normal), 0x01 = 2^-9 (smallest subnormal), 0x7F / 0xFF NaN."""
    vals = orc.e4m3_values()
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    ref = ref.to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(vals), nan)
    assert np.array_equal(vals[~nan], ref[~nan])
    hand = {0x38: 1.0, 0xB8: -1.0, 0x7E: 448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9,
            0x00: 0.0, 0x40: 2.0, 0x44: 3.0, 0x48: 4.0, 0xC8: -4.0}
    for c, v in hand.items():
        assert vals[c] == v, (hex(c), vals[c], v)
    assert np.isnan(vals[0x7F]) and np.isnan(vals[0xFF])


def pin_fp8_scores_match_bf16_on_integers(orc):
    """Integers in [-4, 4] are exact in both bf16 and E4M3, so the 8-bit
    index branch must give the same block scores as the bf16 one."""
    B, T, N, G, dI, Bk = 2, 45, 70, 3, 16, 8
    g = _gen(31)
    qI = _int_bf16(g, (B, T, G, dI))
    kI = _int_bf16(g, (B, N, dI))
    d = dims_of(B, T, N, G, G, 16, dI, Bk, 4)
    rb, rt = _all_rows(B, T)
    S16 = orc.block_scores(d, rb, rt, qI[rb, rt], kI)
    S8 = orc.block_scores_fp8(d, rb, rt, qI.float().to(torch.float8_e4m3fn)[rb, rt],
                              kI.float().to(torch.float8_e4m3fn))
    assert np.array_equal(S16, S8)



# ------------------------------------------------------------ stage 4 backward
def _bwd_case(orc, B, T, N, Hq, G, dh, Bk, k, seed, dense=False):
    """Random q, K, V, dO and a selection made by the oracle's own ranking
    of random block scores (or every visible block when dense)."""
    g = _gen(seed)
    q = _randn_bf16(g, (B, T, Hq, dh))
    K = _randn_bf16(g, (B, G, N, dh))
    V = _randn_bf16(g, (B, G, N, dh))
    dO = _randn_bf16(g, (B, T, Hq, dh))
    d = dims_of(B, T, N, Hq, G, dh, 8, Bk, k)
    rb, rt = _all_rows(B, T)
    NB = -(-N // Bk)
    if dense:
        idx = np.full((rb.size, G, k), -1, dtype=np.int32)
        for r in range(rb.size):
            L = (N - T + rt[r]) // Bk
            idx[r, :, :L + 1] = np.arange(L + 1)
    else:
        S = torch.randn(rb.size, G, NB, generator=g).double().numpy()
        idx = orc.select(d, rt, S)
    return d, rb, rt, q, K, V, dO, idx


def _autograd_reference(q, K, V, dO, mask, hg):
    """Gradients of sum(dO * O) for softmax attention under a boolean mask,
    by torch autograd in fp64.  q/dO [T,Hq,dh], K/V [G,N,dh], mask [G,T,N]."""
    qq = q.double().permute(1, 0, 2).clone().requires_grad_(True)  # [Hq,T,dh]
    kk = K.double().clone().requires_grad_(True)
    vv = V.double().clone().requires_grad_(True)
    ke = kk.repeat_interleave(hg, dim=0)
    ve = vv.repeat_interleave(hg, dim=0)
    mm = mask.repeat_interleave(hg, dim=0)
    sc = (qq @ ke.transpose(1, 2)) / math.sqrt(qq.shape[-1])
    sc = sc.masked_fill(~mm, -math.inf)
    out = torch.softmax(sc, dim=-1) @ ve
    (out * dO.double().permute(1, 0, 2)).sum().backward()
    return qq.grad.permute(1, 0, 2).numpy(), kk.grad.numpy(), vv.grad.numpy()


def pin_backward_autograd(orc):
    """dq, dK, dV equal torch autograd through masked softmax attention (the
    support's mask), GQA heads summed into their group; a window of blocks
    equals the same slice of the full result."""
    for (B, T, N, Hq, G, dh, Bk, k) in ((1, 60, 60, 6, 3, 16, 4, 4),
                                        (2, 23, 41, 4, 2, 8, 4, 3),
                                        (1, 150, 150, 4, 1, 8, 2, 40)):
        d, rb, rt, q, K, V, dO, idx = _bwd_case(orc, B, T, N, Hq, G, dh, Bk, k, 31)
        dq, dK, dV = orc.attend_backward(d, rb, rt, q.reshape(-1, Hq, dh),
                                         dO.reshape(-1, Hq, dh), K, V, idx)
        dq = dq.reshape(B, T, Hq, dh)
        assert not dK[:, :, N:].any() and not dV[:, :, N:].any()  # keys past N
        dK, dV = dK[:, :, :N], dV[:, :, :N]
        ix = idx.reshape(B, T, G, k)
        for b in range(B):
            mask = _mask_from_idx(ix[b], T, N, Bk, G)
            rq, rk, rv = _autograd_reference(q[b], K[b], V[b], dO[b], mask, Hq // G)
            assert np.allclose(dq[b], rq, rtol=1e-10, atol=1e-10)
            assert np.allclose(dK[b], rk, rtol=1e-10, atol=1e-10)
            assert np.allclose(dV[b], rv, rtol=1e-10, atol=1e-10)
        NB = -(-N // Bk)
        lo, nb = NB // 3, 2
        _, wK, wV = orc.attend_backward(d, rb, rt, q.reshape(-1, Hq, dh),
                                        dO.reshape(-1, Hq, dh), K, V, idx, blk_lo=lo, nblk=nb)
        keys = slice(lo * Bk, min((lo + nb) * Bk, N))
        n_in = keys.stop - keys.start
        assert np.array_equal(wK[:, :, :n_in], dK[:, :, keys])
        assert np.array_equal(wV[:, :, :n_in], dV[:, :, keys])


def pin_backward_dense_sdpa(orc):
    """Every visible block selected: the gradients of dense causal GQA
    attention, through torch's scaled_dot_product_attention."""
    B, T, N, Hq, G, dh, Bk = 1, 37, 45, 4, 2, 8, 4
    NB = -(-N // Bk)
    d, rb, rt, q, K, V, dO, idx = _bwd_case(orc, B, T, N, Hq, G, dh, Bk, NB + 1, 32, dense=True)
    dq, dK, dV = orc.attend_backward(d, rb, rt, q.reshape(-1, Hq, dh), dO.reshape(-1, Hq, dh),
                                     K, V, idx)
    hg = Hq // G
    qq = q[0].double().permute(1, 0, 2).clone().requires_grad_(True)
    kk = K[0].double().clone().requires_grad_(True)
    vv = V[0].double().clone().requires_grad_(True)
    pos = (N - T) + torch.arange(T)
    causal = torch.arange(N)[None, :] <= pos[:, None]
    out = F.scaled_dot_product_attention(qq.unsqueeze(0), kk.repeat_interleave(hg, 0).unsqueeze(0),
                                         vv.repeat_interleave(hg, 0).unsqueeze(0),
                                         attn_mask=causal)
    (out[0] * dO[0].double().permute(1, 0, 2)).sum().backward()
    assert np.allclose(dq.reshape(T, Hq, dh), qq.grad.permute(1, 0, 2).numpy(), atol=1e-10)
    assert np.allclose(dK[0, :, :N], kk.grad.numpy(), atol=1e-10)
    assert np.allclose(dV[0, :, :N], vv.grad.numpy(), atol=1e-10)


def _bf16_value(x):
    return torch.tensor([x], dtype=torch.bfloat16)[0]


def pin_backward_finite_differences(orc):
    """Central differences of L = sum(dO . O) through the oracle's forward:
    a coordinate is set to 1.5 and moved to 1.5 +- 2^-7 (all exact in bf16),
    for coordinates of q, of K and V in a selected block, and of K in a block
    no row of the group selects (zero gradient)."""
    B, T, N, Hq, G, dh, Bk, k = 1, 24, 24, 4, 2, 8, 4, 2
    d, rb, rt, q, K, V, dO, idx = _bwd_case(orc, B, T, N, Hq, G, dh, Bk, k, 33)
    hg = Hq // G
    step = 2.0 ** -7

    def loss(qx, Kx, Vx):
        O, _ = orc.attend(d, rb, rt, qx.reshape(-1, Hq, dh), Kx, Vx, idx)
        return float((O * dO.reshape(-1, Hq, dh).double().numpy()).sum())

    def fd(tensor, where):
        plus, minus = tensor.clone(), tensor.clone()
        plus[where] = _bf16_value(1.5 + step)
        minus[where] = _bf16_value(1.5 - step)
        base = tensor.clone()
        base[where] = _bf16_value(1.5)
        return base, plus, minus

    chosen = set(int(x) for x in idx[:, 0].ravel() if x >= 0)
    unused = [blk for blk in range(-(-N // Bk)) if blk not in chosen]
    sel_blk = sorted(chosen)[0]
    cases = [("q", (0, 20, 1, 3)), ("q", (0, 7, 3, 0)),
             ("K", (0, 0, sel_blk * Bk + 1, 5)), ("V", (0, 0, sel_blk * Bk + 2, 6)),
             ("V", (0, 1, N - 1, 0))]
    if unused:
        cases.append(("K", (0, 0, unused[0] * Bk, 2)))
    for name, where in cases:
        src = {"q": q, "K": K, "V": V}[name]
        base, plus, minus = fd(src, where)
        def with_(t):
            a = {"q": q, "K": K, "V": V}
            a[name] = t
            return loss(a["q"], a["K"], a["V"])
        num = (with_(plus) - with_(minus)) / (2 * step)
        a = {"q": q, "K": K, "V": V}
        a[name] = base
        dq, dK, dV = orc.attend_backward(d, rb, rt, a["q"].reshape(-1, Hq, dh),
                                         dO.reshape(-1, Hq, dh), a["K"], a["V"], idx)
        if name == "q":
            ana = dq.reshape(B, T, Hq, dh)[where]
        else:
            ana = (dK if name == "K" else dV)[where]
        assert abs(num - ana) <= 2e-3 * max(1.0, abs(ana)), (name, where, num, ana)
        assert name == "K" and where[2] // Bk in unused or abs(ana) > 1e-3, (name, where, ana)
        if name == "K" and where[2] // Bk in unused:
            assert ana == 0.0 and num == 0.0


def pin_backward_closed_forms(orc):
    """Softmax weights sum to one, so over all keys of a group sum(dV) is the
    sum of dO over the group's rows and heads and sum(dK) is zero; dO = 0
    gives zero gradients; a constant V gives dq = 0 and dK = 0."""
    B, T, N, Hq, G, dh, Bk, k = 2, 40, 52, 6, 2, 8, 4, 4
    d, rb, rt, q, K, V, dO, idx = _bwd_case(orc, B, T, N, Hq, G, dh, Bk, k, 34)
    hg = Hq // G
    dq, dK, dV = orc.attend_backward(d, rb, rt, q.reshape(-1, Hq, dh), dO.reshape(-1, Hq, dh),
                                     K, V, idx)
    go = dO.double().numpy().reshape(B, T, G, hg, dh)
    assert np.allclose(dV.sum(axis=2), go.sum(axis=(1, 3)), atol=1e-10)
    assert np.allclose(dK.sum(axis=2), 0.0, atol=1e-10)
    z = torch.zeros_like(dO)
    dq0, dK0, dV0 = orc.attend_backward(d, rb, rt, q.reshape(-1, Hq, dh), z.reshape(-1, Hq, dh),
                                        K, V, idx)
    assert not dq0.any() and not dK0.any() and not dV0.any()
    Vc = torch.full_like(V, -0.75)
    dqc, dKc, dVc = orc.attend_backward(d, rb, rt, q.reshape(-1, Hq, dh),
                                        dO.reshape(-1, Hq, dh), K, Vc, idx)
    assert np.abs(dqc).max() < 1e-12 and np.abs(dKc).max() < 1e-12
    assert np.allclose(dVc, dV, atol=1e-10)  # dV does not depend on V



# ------------------------------------------------- index-branch KL alignment
def _kl_case(orc, B, T, N, Hq, G, dh, dI, Bk, k, seed, zero_q=False, zero_qI=False):
    g = _gen(seed)
    q = _randn_bf16(g, (B, T, Hq, dh))
    K = _randn_bf16(g, (B, G, N, dh))
    qI = _randn_bf16(g, (B, T, G, dI))
    kI = _randn_bf16(g, (B, N, dI))
    if zero_q:
        q = torch.zeros_like(q)
    if zero_qI:
        qI = torch.zeros_like(qI)
    d = dims_of(B, T, N, Hq, G, dh, dI, Bk, k)
    rb, rt = _all_rows(B, T)
    S = torch.randn(rb.size, G, -(-N // Bk), generator=g).double().numpy()
    idx = orc.select(d, rt, S)
    return d, rb, rt, q, K, qI, kI, idx


def _kl_call(orc, d, rb, rt, q, K, qI, kI, idx):
    B, T, Hq, dh = q.shape
    return orc.index_kl_backward(d, rb, rt, qI.reshape(B * T, d.G, -1), kI,
                                 q.reshape(B * T, Hq, dh), K, idx)


def pin_index_kl_autograd(orc):
    """dq^I, dk^I and the loss equal torch autograd of
    sum KL(teacher || softmax(s)) over masked dense scores in fp64, with the
    teacher (mean of the group's heads' attention weights) detached."""
    for (B, T, N, Hq, G, dh, dI, Bk, k) in ((1, 50, 50, 6, 3, 8, 16, 4, 4),
                                            (2, 19, 33, 4, 2, 8, 8, 4, 3)):
        d, rb, rt, q, K, qI, kI, idx = _kl_case(orc, B, T, N, Hq, G, dh, dI, Bk, k, 51)
        dqI, dkI, kl = _kl_call(orc, d, rb, rt, q, K, qI, kI, idx)
        assert not dkI[:, N:].any()
        hg = Hq // G
        ix = idx.reshape(B, T, G, k)
        for b in range(B):
            mask = _mask_from_idx(ix[b], T, N, Bk, G)                  # [G, T, N]
            qq = q[b].double().permute(1, 0, 2)                          # [Hq, T, dh]
            sc = (qq @ K[b].double().repeat_interleave(hg, 0).transpose(1, 2)) / math.sqrt(dh)
            sc = sc.masked_fill(~mask.repeat_interleave(hg, 0), -math.inf)
            teacher = torch.softmax(sc, -1).view(G, hg, T, N).mean(1)    # [G, T, N]
            qi = qI[b].double().permute(1, 0, 2).clone().requires_grad_(True)  # [G, T, dI]
            ki = kI[b].double().clone().requires_grad_(True)
            s = (qi @ ki.T) / math.sqrt(dI)
            logp = torch.log_softmax(s.masked_fill(~mask, -math.inf), -1)
            logp = logp.masked_fill(~mask, 0.0)
            per_row = (torch.xlogy(teacher, teacher) - teacher * logp).sum(-1)  # [G, T]
            per_row.sum().backward()
            assert np.allclose(kl.reshape(B, T, G)[b], per_row.detach().T.numpy(), atol=1e-10)
            assert np.allclose(dqI.reshape(B, T, G, dI)[b], qi.grad.permute(1, 0, 2).numpy(),
                               atol=1e-10)
            assert np.allclose(dkI[b, :N], ki.grad.numpy(), atol=1e-10)


def pin_index_kl_finite_differences(orc):
    """Central differences of sum KL (the oracle's own loss values) in a
    q^I and a k^I coordinate set to 1.5 and moved by +-2^-7 (exact in
    bf16) match dq^I and dk^I."""
    B, T, N, Hq, G, dh, dI, Bk, k = 1, 24, 24, 4, 2, 8, 8, 4, 3
    d, rb, rt, q, K, qI, kI, idx = _kl_case(orc, B, T, N, Hq, G, dh, dI, Bk, k, 52)
    step = 2.0 ** -7
    for name, where in (("qI", (0, 21, 1, 2)), ("qI", (0, 9, 0, 5)), ("kI", (0, 3, 4)),
                        ("kI", (0, 17, 0))):
        src = qI if name == "qI" else kI
        vals = []
        for v in (1.5 + step, 1.5 - step, 1.5):
            t = src.clone()
            t[where] = _bf16_value(v)
            a = (t, kI) if name == "qI" else (qI, t)
            vals.append(_kl_call(orc, d, rb, rt, q, K, a[0], a[1], idx))
        num = (vals[0][2].sum() - vals[1][2].sum()) / (2 * step)
        dqI, dkI, _ = vals[2]
        ana = dqI.reshape(B, T, G, dI)[where] if name == "qI" else dkI[where]
        assert abs(num - ana) <= 2e-3 * max(1.0, abs(ana)), (name, where, num, ana)
        assert abs(ana) > 1e-4, (name, where, ana)


def pin_index_kl_closed_forms(orc):
    """Zero q and zero q^I make teacher and proxy both uniform on the
    support: zero loss and zero gradients.  Equal index keys give dq^I = 0
    (the weights' differences sum to zero).  The loss is never negative."""
    B, T, N, Hq, G, dh, dI, Bk, k = 1, 40, 40, 4, 2, 8, 8, 4, 3
    d, rb, rt, q, K, qI, kI, idx = _kl_case(orc, B, T, N, Hq, G, dh, dI, Bk, k, 53,
                                            zero_q=True, zero_qI=True)
    dqI, dkI, kl = _kl_call(orc, d, rb, rt, q, K, qI, kI, idx)
    assert np.abs(kl).max() < 1e-12 and np.abs(dqI).max() < 1e-12 and np.abs(dkI).max() < 1e-12
    d, rb, rt, q, K, qI, kI, idx = _kl_case(orc, B, T, N, Hq, G, dh, dI, Bk, k, 54)
    kI_eq = kI[:, :1].expand_as(kI).contiguous()
    dqI, _, kl = _kl_call(orc, d, rb, rt, q, K, qI, kI_eq, idx)
    assert np.abs(dqI).max() < 1e-12
    _, _, kl = _kl_call(orc, d, rb, rt, q, K, qI, kI, idx)
    assert kl.min() >= -1e-12 and kl.max() > 1e-3


ALL_PINS = [
    pin_scores_brute_force,
    pin_scores_zero_keys,
    pin_scores_ramp_closed_form,
    pin_select_all_ties,
    pin_select_exhaustive,
    pin_select_lexsort,
    pin_select_needle,
    pin_select_invariants,
    pin_attend_dense_equivalence,
    pin_attend_masked_sdpa,
    pin_attend_k1_block_diagonal,
    pin_attend_closed_forms,
    pin_decode_is_last_prefill_row,
    pin_e4m3_codes,
    pin_fp8_scores_match_bf16_on_integers,
    pin_backward_autograd,
    pin_backward_dense_sdpa,
    pin_backward_finite_differences,
    pin_backward_closed_forms,
    pin_index_kl_autograd,
    pin_index_kl_finite_differences,
    pin_index_kl_closed_forms,
]
