"""Oracle for the nested parent producer: the MatGPTQ scale search and the
cross-width code choice, with no calibration data (identity Hessian).

TEST INFRASTRUCTURE ONLY.  A plain, slow CPU definition that the HIP producer
is checked against.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import it; the library never calls it and
shares no code with it.

What it computes ("MatGPTQ: Efficient and Accurate Inference over Nested
Quantized Models", section 3.2 "The MatGPTQ Algorithm", points 1 and 2, and
Appendix A.2 "MatGPTQ adaptation", Algorithms 1 and 2):

* Scale search (point 1, Algorithm 1).  Per group of ``group`` consecutive
  input indices of one output row, each candidate pair (s, z) is scored by the
  error of the weights it reconstructs at every target width r in R, weighted
  by lambda_r, and the best candidate is kept.  The pages give no grid; the
  reading taken here is the usual range-shrinking search over the min-max
  range [min(0, min w), max(0, max w)]: candidate i (i = 0 .. n_grid - 1)
  shrinks the range by p_i = 1 - i / grid_den, takes the fp16 scale of the
  shrunk range over 2^c - 1 levels and the integer zero point that puts the
  shrunk minimum on code 0.  Each weight is coded to the nearest c-bit code
  under the candidate (round half to even, clamped), sliced at every r, and
  dequantized with the shared (s, z).
* Code choice (point 2, Algorithm 2).  With the chosen (s, z), every c-bit
  code q in [0, 2^c - 1] is a candidate for each weight; its error is the
  lambda-weighted sum over r of the squared distance between the weight and
  the r-bit reconstruction of q (equation 5 of the pages); the code with the
  smallest error is stored.  The pages do this one column at a time, holding
  a 2^c x d_row error matrix in FP32 (4 MB for a 4096-row column).

Decisions are taken in fp32, the precision the pages store the error matrix
in, with every operation rounded on its own (no fused multiply-add) in this
order: d = w - w_hat, t = lambda_r * (d * d), running sum over the widths in
the order R is given; in the scale search the running sum is over the
group's weights in index order, widths innermost.  Ties go to the first
candidate (smallest i, smallest q).  w_hat itself is exact in fp32 (fp16
scale, integer zero point, half-integer slice value), so only these rounded
sums and products need a fixed order.

The slice and its reconstruction are those of ``mq_oracle`` (true prefix with
delta_r, MatQuant's rounded slice, or the unclamped one).
"""
from __future__ import annotations

import numpy as np

from .mq_oracle import C_BITS, sliced_value

F32 = np.float32


def candidate_shrink(i: int, grid_den: int) -> np.float32:
    """p_i = 1 - i / grid_den, each operation rounded to fp32."""
    return F32(1) - F32(i) / F32(grid_den)


def candidate_scale_zero(lo: np.ndarray, hi: np.ndarray, p: np.float32, c: int = C_BITS):
    """fp16 scale and integer zero point of the range [p*lo, p*hi] (lo <= 0 <= hi,
    fp32).  A scale that rounds to zero in fp16 is replaced by 1; the zero
    point is a non-negative integer (+0, never -0)."""
    qmax = F32(2 ** c - 1)
    lo_p = (p * lo).astype(F32)
    hi_p = (p * hi).astype(F32)
    s16 = ((hi_p - lo_p) / qmax).astype(F32).astype(np.float16)
    s16 = np.where(s16 == 0, np.float16(1), s16)
    s = s16.astype(F32)
    # + 0 turns the -0 of an all-positive group (lo = 0) into the integer 0
    z = np.clip(np.rint(-lo_p / s), 0, qmax).astype(F32) + F32(0)
    return s16, s, z


def nearest_code(w: np.ndarray, s: np.ndarray, z: np.ndarray, c: int = C_BITS) -> np.ndarray:
    """clamp(rint(w / s) + z, 0, 2^c - 1) in fp32 (round half to even), as int64."""
    qmax = F32(2 ** c - 1)
    return np.clip(np.rint((w / s).astype(F32)) + z, 0, qmax).astype(np.int64)


def reconstruct(q: np.ndarray, s: np.ndarray, z: np.ndarray, r: int, rule: str) -> np.ndarray:
    """w_hat_r(q) = s * (v_r(q) - z) as fp32; exact (asserted), so the
    evaluation order does not matter."""
    v = sliced_value(q, r, rule)
    exact = np.asarray(s, dtype=np.float64) * (v - np.asarray(z, dtype=np.float64))
    w32 = exact.astype(F32)
    if not np.array_equal(w32.astype(np.float64), exact):
        raise AssertionError("reconstruction not exact in fp32")
    return w32


def weighted_term(w: np.ndarray, w_hat: np.ndarray, lam: np.float32) -> np.ndarray:
    d = (w - w_hat).astype(F32)
    return (F32(lam) * (d * d).astype(F32)).astype(F32)


def _check(widths, lambdas, group, k):
    widths = [int(r) for r in widths]
    lambdas = [F32(v) for v in lambdas]
    if not widths or len(widths) != len(lambdas) or len(set(widths)) != len(widths):
        raise ValueError("widths and lambdas must be non-empty, of equal length, widths distinct")
    if any(not 1 <= r <= C_BITS for r in widths):
        raise ValueError("width out of range")
    if k % group:
        raise ValueError("k must be a multiple of group")
    return widths, lambdas


def search_scale_zero(w, group: int, widths, lambdas, rule: str, n_grid: int = 80,
                      grid_den: int = 100, return_errors: bool = False):
    """Algorithm 1 (identity Hessian).  w: fp32 [n, k].  Returns fp16 scales and
    zero points [n, k/group] (and, optionally, the fp32 error of every
    candidate, [n_grid, n, k/group])."""
    w = np.ascontiguousarray(w, dtype=F32)
    n, k = w.shape
    widths, lambdas = _check(widths, lambdas, group, k)
    if not 1 <= n_grid <= grid_den:
        raise ValueError("need 1 <= n_grid <= grid_den")
    wg = w.reshape(n, k // group, group)
    lo = np.minimum(wg.min(axis=-1), F32(0))
    hi = np.maximum(wg.max(axis=-1), F32(0))
    errs = np.empty((n_grid, n, k // group), dtype=F32)
    cand = []
    for i in range(n_grid):
        s16, s, z = candidate_scale_zero(lo, hi, candidate_shrink(i, grid_den))
        cand.append((s16, z))
        acc = np.zeros((n, k // group), dtype=F32)
        for j in range(group):
            wj = wg[:, :, j]
            q = nearest_code(wj, s, z)
            for r, lam in zip(widths, lambdas):
                acc = (acc + weighted_term(wj, reconstruct(q, s, z, r, rule), lam)).astype(F32)
        errs[i] = acc
    best = np.argmin(errs, axis=0)              # first minimum
    s_out = np.empty((n, k // group), dtype=np.float16)
    z_out = np.empty((n, k // group), dtype=np.float16)
    for i in range(n_grid):
        sel = best == i
        s_out[sel] = cand[i][0][sel]
        z_out[sel] = cand[i][1][sel].astype(np.float16)
    if return_errors:
        return s_out, z_out, errs
    return s_out, z_out


def column_errors(w_col, s_col, z_col, widths, lambdas, rule: str, c: int = C_BITS) -> np.ndarray:
    """The 2^c x d_row fp32 error matrix of one column (Algorithm 2): entry
    [q, i] is sum_r lambda_r (w[i] - w_hat_r(q))^2, summed in the order of R."""
    w_col = np.asarray(w_col, dtype=F32)[None, :]
    s = np.asarray(s_col, dtype=np.float16).astype(F32)[None, :]
    z = np.asarray(z_col, dtype=np.float16).astype(F32)[None, :]
    q = np.arange(2 ** c, dtype=np.int64)[:, None]
    err = np.zeros((2 ** c, w_col.shape[1]), dtype=F32)
    for r, lam in zip(widths, lambdas):
        err = (err + weighted_term(w_col, reconstruct(q, s, z, r, rule), lam)).astype(F32)
    return err


def choose_codes(w, scales, zeros, group: int, widths, lambdas, rule: str) -> np.ndarray:
    """Algorithm 2: per weight, the c-bit code with the smallest weighted error
    over the widths (first minimum).  One column at a time.  uint8 [n, k]."""
    w = np.ascontiguousarray(w, dtype=F32)
    n, k = w.shape
    widths, lambdas = _check(widths, lambdas, group, k)
    scales = np.asarray(scales, dtype=np.float16)
    zeros = np.asarray(zeros, dtype=np.float16)
    if scales.shape != (n, k // group) or zeros.shape != (n, k // group):
        raise ValueError("scales and zeros must be [n, k/group]")
    q = np.empty((n, k), dtype=np.uint8)
    for col in range(k):
        g = col // group
        err = column_errors(w[:, col], scales[:, g], zeros[:, g], widths, lambdas, rule)
        q[:, col] = np.argmin(err, axis=0)
    return q


def produce_parent(w, group: int, widths, lambdas, rule: str, n_grid: int = 80, grid_den: int = 100):
    """Scale search, then code choice: (codes uint8 [n,k], scales fp16, zeros fp16)."""
    s, z = search_scale_zero(w, group, widths, lambdas, rule, n_grid, grid_den)
    return choose_codes(w, s, z, group, widths, lambdas, rule), s, z
