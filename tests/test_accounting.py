"""Host-side work accounting pinned to the figures the MSA pages print
(tests/golden/page_figures.json) and to closed forms.  No GPU needed."""
import json
import os

import numpy as np

from block_sparse_long_index_amd import accounting as acc
from msa_inputs import WORKLOADS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def _fig():
    with open(GOLDEN) as f:
        return json.load(f)


def test_compute_reduction_matches_page():
    f = _fig()["attention_compute_reduction"]
    bb, sel = f["backbone"], f["selection"]
    r = acc.dense_over_msa_per_token(f["context_tokens"], bb["Hq"], bb["G"],
                                     bb["d_h"], f["index_key_width"],
                                     sel["Bk"], sel["k"])
    assert abs(r - f["value"]) < 0.05, r
    # charging the exact (slightly smaller) support moves it by under 1%
    r2 = acc.dense_over_msa_per_token(f["context_tokens"], bb["Hq"], bb["G"],
                                      bb["d_h"], f["index_key_width"],
                                      sel["Bk"], sel["k"], fixed_budget=False)
    assert f["value"] < r2 < f["value"] * 1.01, r2


def test_token_budget():
    f = _fig()["token_budget"]
    assert f["Bk"] * f["k"] == f["value"]
    # no query ever exceeds the budget, and the long-context mean approaches it
    n = acc.support_tokens(1 << 20, 1 << 20, f["Bk"], f["k"])
    assert n <= f["value"] * (1 << 20)
    assert n / (1 << 20) > 0.99 * (f["value"] - f["Bk"] / 2)


def test_index_key_bytes_and_fraction():
    f = _fig()
    assert acc.index_key_bytes_per_token(128) == f["index_key_bytes_per_token"]["value"]
    fr = f["index_cache_fraction_of_main_cache"]
    main = 2 * fr["kv_heads"] * fr["d_h"] * fr["bytes_per_elem"]
    assert abs(256 / main - fr["value"]) < 0.005


def test_dense_decode_bytes_match_page():
    f = _fig()["dense_decode_bytes_per_token"]
    for pt in f["points"]:
        b = acc.dense_decode_kv_bytes(pt["context"], f["kv_heads"], f["d_h"],
                                      f["bytes_per_elem"], f["layers"])
        assert abs(b / 2**30 - pt["gigabytes"]) / pt["gigabytes"] < 0.05, (pt, b)


def test_closed_form_sums():
    # sum over p of (p+1) for T == N is N(N+1)/2
    for N in (1, 127, 128, 2048, 131072):
        assert acc.causal_pairs(N, N) == N * (N + 1) // 2
    # brute force n_sel on a small case
    N, Bk, k = 1000, 16, 5
    brute = 0
    for p in range(N):
        L = p // Bk
        brute += min(L, k - 1) * Bk + (p - L * Bk) + 1
    assert acc.support_tokens(N, N, Bk, k) == brute


def test_workload_totals():
    """The per-workload totals quoted in the measurement plan."""
    w = WORKLOADS["prefill_128k"]
    fl = acc.prefill_flops(w)
    assert abs(fl["index"] / 1e12 - 17.59) < 0.01
    assert abs(fl["main"] / 1e12 - 8.46) < 0.01
    assert acc.support_tokens(w.N, w.T, w.Bk, w.k) == 258146304
    d = acc.decode_bytes(WORKLOADS["decode_256k_b16"])
    assert abs(d["index_keys"] / 1e9 - 1.0737) < 1e-3
    assert abs(d["kv"] / 1e6 - 134.2) < 0.1
    tk = acc.topk_bytes(w)
    assert abs(tk["read"] / 1e9 - 2.145) < 0.01
    # backward: five products of the forward's per-product size
    assert acc.backward_flops(w.N, w.T, w.Hq, w.d_h, w.Bk, w.k) * 2 == fl["main"] * 5
    assert abs(acc.backward_flops(w.N, w.T, w.Hq, w.d_h, w.Bk, w.k) / 1e12 - 21.15) < 0.01
    # index KL backward: the teacher's scores (half a forward) + 4 index products
    kl = acc.index_kl_flops(w.N, w.T, w.Hq, w.G, w.d_h, w.d_I, w.Bk, w.k)
    assert kl * 2 == fl["main"] + 8 * w.G * w.d_I * acc.support_tokens(w.N, w.T, w.Bk, w.k) * 2
    assert abs(kl / 1e12 - 6.344) < 0.01
    # fused training backward: the backward's five products + the 4 index products
    tr = acc.train_flops(w.N, w.T, w.Hq, w.G, w.d_h, w.d_I, w.Bk, w.k)
    assert tr * 2 == fl["main"] * 5 + 8 * w.G * w.d_I * acc.support_tokens(w.N, w.T, w.Bk, w.k) * 2
    assert abs(tr / 1e12 - 23.26) < 0.01
    w0 = WORKLOADS["prefill_2k"]
    assert acc.support_tokens(w0.N, w0.T, w0.Bk, w0.k) == 820224
    assert np.isclose(acc.prefill_flops(w0)["index"], 1.074e9, rtol=1e-3)


def test_fp32_score_rounding_identity():
    """The kernels report S as fp32(fp64(dot) * fp64(1/sqrt(128))) with the
    dot accumulated exactly; the oracle reports dot / sqrt(128) in fp64 and
    the tests round it to fp32.  For every integer dot an index score can
    take (|dot| <= 128 * 16) the two roundings agree bit for bit."""
    inv = np.float64(0.088388347648318440550)  # the constant the kernels use
    d = np.arange(-2048, 2049, dtype=np.float64)
    kernel = (d * inv).astype(np.float32)
    oracle_side = (d / np.sqrt(np.float64(128.0))).astype(np.float32)
    assert np.array_equal(kernel.view(np.uint32), oracle_side.view(np.uint32))
