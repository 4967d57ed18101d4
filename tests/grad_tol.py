"""Element-wise tolerance for the gradients of the training calls.

Every gradient value is a sum of many products over a row's support (dq, dq^I)
or over the rows that selected a key (dK, dV, dk^I).  On the GPU each product
carries at most three bf16 roundings (unit roundoff u = 2^-8): the weight it
multiplies with (P, dS or dz = p_proxy - p_teacher rounded before the MFMA),
the per-slot partial sum (dq, dq^I are summed from bf16 partials) and, through
D = dO . O, the bf16 forward output.  Round-to-nearest errors are independent
with zero mean, so a value's error behaves like a sum of independent terms
whose spread is at most about u * sqrt(sum of the squared products); the value
itself is the signed sum of the same products, so that root sum of squares is
of the order of the typical magnitude of the vector the value belongs to (its
root mean square over the vector's d = 128 values).  Where the products do not
cancel (a row with few keys) the errors add up instead: at most 3u relative.

Bound per element of a vector v (last axis of the arrays, 128 values):

    |got - ref| <= A * |ref| + B * rms(ref_v) + F

with A = 4u (three roundings and margin), B = 6u (six standard deviations of
the independent-rounding error) and F = 1e-5 * max |ref| + 1e-6 (vectors that
are exactly zero in exact arithmetic, e.g. a row whose support is one key,
where the GPU returns fp32 rounding noise of order 1e-7).  The relative Frobenius error of the whole
tensor is also checked (<= 1e-2).

dq has one more source: D = dO . O is formed from the forward's output, which
the backward receives in bf16 and which carries the forward's own rounding
(P rounded before its PV product): |O_gpu - O| <= 2u (|O| + rms(O)) per value.
The resulting |dD| moves every dS_j = P_j (dP_j - D) of the row by P_j dD, so
dq_d moves by at most dD * max_j |K_jd| / sqrt(d_h) (the weights sum to one);
that term is passed as `extra`.  It does not cancel with the row's other
errors and matters in rows of a few keys, where dP_j - D cancels.  dK_j gets
the same shift from every row and head that reaches key j:
sum over them of P_j dD |q_d| / sqrt(d_h); that is exactly the dV the oracle
returns for the upstream gradient dD |q| / sqrt(d_h) (non-negative terms), so
the tests take it from the oracle.
"""
import sys

import numpy as np

U = 2.0 ** -8
A_REL, B_RMS, F_ABS, F_NOISE, REL_FRO = 4 * U, 6 * U, 1e-5, 1e-6, 1e-2


def close_grad(tag, got, ref, extra=None):
    """extra: an additional per-element bound of an error source that is not
    a rounding of the gradient's own terms (same shape as ref)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (tag, got.shape, ref.shape)
    if ref.size == 0:
        return
    err = np.abs(got - ref)
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
    floor = F_ABS * np.abs(ref).max() + F_NOISE
    bound = A_REL * np.abs(ref) + B_RMS * rms + floor
    if extra is not None:
        bound = bound + np.asarray(extra, dtype=np.float64)
    ratio = err / bound
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    fro = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    print("%s rel fro %.3e; worst element %s: err %.3e, |ref| %.3e, vector rms %.3e, "
          "%.3f of its bound" % (tag, fro, tuple(int(i) for i in worst), err[worst],
                                 abs(ref[worst]), rms[worst[:-1]][0], ratio[worst]),
          file=sys.stderr, flush=True)
    assert ratio[worst] <= 1.0, (tag, "element-wise bound", ratio[worst], worst)
    assert fro <= REL_FRO or np.linalg.norm(ref) < floor * ref.size ** 0.5, (tag, fro)


def d_shift(dO_rows, O_rows):
    """Bound of |dD| per (row, head) [n, H, 1]: dO_rows, O_rows [n, H, d] (O:
    the oracle's exact forward output of the rows)."""
    dO_rows = np.asarray(dO_rows, dtype=np.float64)
    O_rows = np.asarray(O_rows, dtype=np.float64)
    o_rms = np.sqrt(np.mean(O_rows * O_rows, axis=-1, keepdims=True))
    return 2 * U * np.sum(np.abs(dO_rows) * (np.abs(O_rows) + o_rms), axis=-1, keepdims=True)


def dq_extra(dD, kmax_rows, d_h=128):
    """The dq D term above; kmax_rows [n, H, d]: max |K_jd| over the keys of
    the row's group."""
    return dD * np.asarray(kmax_rows, dtype=np.float64) / d_h ** 0.5
