"""The CPU oracle against its pins, and the pins against planted mistakes.

No GPU needed.  The mutation check compiles modified copies of the oracle
source (each with one plausible mistake) and requires that at least one pin
fails for every copy; each copy runs in a child process so that a mistake
that crashes the oracle counts as caught without taking pytest down.
"""
import os
import subprocess
import sys

import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def orc():
    return oracle.OracleLib(oracle.build(force=False))


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


# (name, text in the oracle source, replacement) -- one plausible mistake each
MUTATIONS = [
    ("score_drops_own_key", "for (int64_t j = 0; j <= p; ++j) {",
     "for (int64_t j = 0; j < p; ++j) {"),
    ("score_scale_inverted", "const double s = dot / root;",
     "const double s = dot * root;"),
    ("score_top_left_causal", "return d->N - d->T + t;", "return t;"),
    ("score_block_of_key_wrong", "const int64_t blk = j / d->Bk;",
     "const int64_t blk = (j + 1) / d->Bk < block_count(d) ? (j + 1) / d->Bk : j / d->Bk;"),
    ("select_ties_to_higher_index", "if (best < 0 || sc[c] > sc[best])",
     "if (best < 0 || sc[c] >= sc[best])"),
    ("select_local_outside_budget",
     "const int64_t want = (k - 1 < local) ? k - 1 : local;",
     "const int64_t want = (k < local) ? k : local;"),
    ("select_wrong_local", "out[want] = (int32_t)local;",
     "out[want] = (int32_t)(local > 0 ? local - 1 : 0);"),
    ("select_not_sorted", "while (z >= 0 && chosen[z] > v) {",
     "while (z >= 0 && chosen[z] < v) {"),
    ("select_lowest_score", "if (best < 0 || sc[c] > sc[best])",
     "if (best < 0 || sc[c] < sc[best])"),
    ("attend_interleaved_heads", "const int64_t g = h / hg;",
     "const int64_t g = h % G;"),
    ("attend_no_causal_mask_in_local_block",
     "j < (blk + 1) * d->Bk && j <= p; ++j)", "j < (blk + 1) * d->Bk && j < d->N; ++j)"),
    ("attend_missing_scale", "z[i] = dot / root;", "z[i] = dot;"),
    ("attend_lse_without_max", "lse[r * Hq + h] = m + log(l);",
     "lse[r * Hq + h] = log(l);"),
    ("attend_unnormalised", "o[c] /= l;", "o[c] /= 1.0;"),
    ("attend_drops_first_block", "if (blk < 0)\n                continue;",
     "if (blk <= 0)\n                continue;"),
    ("widen_wrong_shift", "uint32_t u = (uint32_t)bits << 16;",
     "uint32_t u = (uint32_t)bits << 15;"),
    ("e4m3_wrong_bias", "v = ldexp(1.0 + m / 8.0, e - 7);", "v = ldexp(1.0 + m / 8.0, e - 8);"),
    ("e4m3_subnormal_as_normal", "v = ldexp((double)m, -9);", "v = ldexp(1.0 + m / 8.0, -7);"),
    ("e4m3_mantissa_halved", "v = ldexp(1.0 + m / 8.0, e - 7);",
     "v = ldexp(1.0 + m / 16.0, e - 7);"),
    ("e4m3_sign_dropped", "return sign ? -v : v;", "return v;"),
    ("bwd_no_softmax_jacobian_term", "const double dz = z[i] * (dp[i] - pdp);",
     "const double dz = z[i] * dp[i];"),
    ("bwd_dq_unscaled", "dqr[c] += dz * widen_bf16(kv[c]) / root;",
     "dqr[c] += dz * widen_bf16(kv[c]);"),
    ("bwd_dv_weighted_by_dz", "myv[kw * dh + c] += z[i] * go[c];",
     "myv[kw * dh + c] += dz * go[c];"),
    ("bwd_dk_sign", "myk[kw * dh + c] += dz * qd[c] / root;",
     "myk[kw * dh + c] -= dz * qd[c] / root;"),
    ("bwd_unnormalised_weights", "                z[i] /= l;\n", "                z[i] /= 1.0;\n"),
    ("bwd_heads_interleaved", "const int64_t b = bh / Hq, h = bh % Hq, g = h / hg;",
     "const int64_t b = bh / Hq, h = bh % Hq, g = h % G;"),
    ("bwd_no_causal_mask", "j < (blk + 1) * Bk && j <= p; ++j)",
     "j < (blk + 1) * Bk && j < d->N; ++j)"),
    ("bwd_window_offset_dropped", "const int64_t kw = key[i] - key_lo;",
     "const int64_t kw = key[i];"),
    ("kl_teacher_summed_not_averaged", "pt[i] += z[i] / l / (double)hg;", "pt[i] += z[i] / l;"),
    ("kl_teacher_first_head_only", "for (int64_t h = g * hg; h < (g + 1) * hg; ++h) {\n                for (int64_t c = 0; c < dh; ++c)\n                    qh[c]",
     "for (int64_t h = g * hg; h < g * hg + 1; ++h) {\n                for (int64_t c = 0; c < dh; ++c)\n                    qh[c]"),
    ("kl_gradient_sign", "const double dz = exp(logx) - pt[i];", "const double dz = pt[i] - exp(logx);"),
    ("kl_dqI_unscaled", "dq[c] += dz * widen_bf16(kv[c]) / root_i;", "dq[c] += dz * widen_bf16(kv[c]);"),
    ("kl_dkI_first_group_only", "        for (int64_t g = 0; g < G; ++g) {\n            const double *sg",
     "        for (int64_t g = 0; g < 1; ++g) {\n            const double *sg"),
    ("kl_proxy_unnormalised", "const double lse = m + log(l);", "const double lse = m;"),
    ("kl_loss_direction", "loss += pt[i] * (log(pt[i]) - logx);", "loss += exp(logx) * (logx - log(pt[i]));"),
    ("fp8_scores_use_bf16_decoder", "block_scores(d, nrows, row_b, row_t, qI_rows, kI, 1, S);",
     "block_scores(d, nrows, row_b, row_t, qI_rows, kI, 0, S);"),
]

_RUNNER = r"""
import sys
sys.path[:0] = [%r, %r]
import oracle, oracle_pins
orc = oracle.OracleLib(%r)
failed = []
for pin in oracle_pins.ALL_PINS:
    try:
        pin(orc)
    except AssertionError:
        failed.append(pin.__name__)
print("FAILED_PINS", ",".join(failed))
sys.exit(3 if failed else 0)
"""


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new):
    src = oracle.source_text()
    assert src.count(old) >= 1, "mutation anchor vanished: " + name
    mutated = src.replace(old, new, 1)
    so = oracle.build_variant(mutated, str(tmp_path), name)
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    here = os.path.dirname(os.path.abspath(__file__))
    code = _RUNNER % (root, here, so)
    env = dict(os.environ, OMP_NUM_THREADS="2")
    res = subprocess.run([sys.executable, "-c", code], capture_output=True,
                         text=True, timeout=300, env=env)
    # exit 3: some pin failed; any other non-zero: the mutant crashed
    assert res.returncode != 0, (name, res.stdout[-2000:], res.stderr[-2000:])
