"""Oracle for the sliced-precision quantized linear layer  Y = X . dequant(slice_r(Q_c))^T.

TEST INFRASTRUCTURE ONLY.  This is the plain, slow, obviously correct CPU
definition that the HIP library is checked against.  Only the tests, the
package smoke check and the benchmark's CPU-baseline leg may import it; the
library never calls it and shares no code, tables or constants with it.

Everything is integer or float64 numpy, written from the definitions on the
pages rather than from the GPU's bit tricks:

* MatQuant slice ("Matryoshka Quantization | Summary", section 3.2 "MatQuant"):
  for a c-bit code q and 0 < r < c, S(q, r) = clamp(round(q / 2^(c-r)), 0,
  2^r - 1) * 2^(c-r).  Appendix A of that summary and Appendix A.1 of
  "MatGPTQ: Efficient and Accurate Inference over Nested Quantized Models"
  state that the rounding is decided by the (r+1)-th most significant bit, so a
  tie (q exactly halfway between two cells) rounds upward.
* MatGPTQ true-prefix slice (same MatGPTQ page, Appendix A.1 "Improved nested
  representation"): keep the r most significant bits (right shift), map them
  back into the c-bit code space (left shift), then add delta_r, which moves
  the value from the lower edge to the centre of its cell.  The centre of the
  2^(c-r) integer codes that share a prefix is delta_r = (2^(c-r) - 1) / 2.
* Shared-scale asymmetric dequant (MatQuant summary section 3.1; MatGPTQ
  section 1 and section 3.2): one scale s and integer zero point z per group
  of consecutive input indices, shared by every width r:  w_hat = s * (v - z).
* Contraction (MatGPTQ section 4 "Fast Matryoshka Kernels"): Y = X W_D with
  the nn.Linear orientation, i.e. Y[m, n] = sum_k X[m, k] * w_hat[n, k],
  here in float64.
* Extra-Precision MatQuant (MatQuant summary section 7 "Errata"): the
  rounded slice without the clamp, S(q, r) = round(q / 2^(c-r)) * 2^(c-r),
  which keeps 2^r + 1 values (unsigned 234 at r = 2 gives 256).
* Mix'n'Match (MatQuant summary section 4.3): every layer matrix is sliced at
  its own width; the oracle applies the single-layer definition per call.

Readings where the pages are silent (each is a keyword argument so the
alternative can be tried without touching the GPU path): ties round upward
(``tie="up"``; ``"even"`` is numpy's half-to-even); delta_r is the centre of
the integer cell (``delta="centre"``; ``"half_cell"`` = 2^(c-r-1)); at r = c
both rules are the identity.
"""
from __future__ import annotations

import numpy as np

C_BITS = 8
PREFIX = "prefix"   # MatGPTQ true-prefix slice (+ delta_r)
ROUND = "round"     # MatQuant rounded and clamped slice
EXTRA = "extra"     # Extra-Precision MatQuant: rounded, not clamped (2^r + 1 levels)


# ----------------------------------------------------------------------------
# slicing (integer arithmetic)
# ----------------------------------------------------------------------------
def cell_width(r: int, c: int = C_BITS) -> int:
    """Number of c-bit codes that share one r-bit prefix: 2^(c - r)."""
    return 2 ** (c - r)


def _codes(q) -> np.ndarray:
    q = np.asarray(q, dtype=np.int64)
    if q.size and (q.min() < 0 or q.max() > 255):
        raise ValueError("parent codes are unsigned 8-bit")
    return q


def slice_prefix(q, r: int, c: int = C_BITS) -> np.ndarray:
    """True-prefix r-bit code: the quotient of q by the cell width (the r most
    significant bits of q)."""
    q = _codes(q)
    return q // cell_width(r, c)


def slice_round_unclamped(q, r: int, c: int = C_BITS, tie: str = "up") -> np.ndarray:
    """round(q / 2^(c-r)) before the clamp.  Can reach 2^r (the extra level of
    the unclamped variant, MatQuant summary section 7 "Errata")."""
    q = _codes(q)
    if r == c:
        return q.copy()
    m = cell_width(r, c)
    if tie == "up":
        # floor(q/m + 1/2) computed exactly as floor((2q + m) / 2m)
        return (2 * q + m) // (2 * m)
    if tie == "even":
        return np.round(q / m).astype(np.int64)
    raise ValueError(tie)


def slice_round(q, r: int, c: int = C_BITS, tie: str = "up") -> np.ndarray:
    """MatQuant r-bit code: clamp(round(q / 2^(c-r)), 0, 2^r - 1)."""
    pre = slice_round_unclamped(q, r, c, tie)
    return np.clip(pre, 0, 2 ** r - 1)


def slice_code(q, r: int, rule: str, c: int = C_BITS, tie: str = "up") -> np.ndarray:
    if not 1 <= r <= c:
        raise ValueError("width out of range")
    if rule == PREFIX:
        return slice_prefix(q, r, c)
    if rule == ROUND:
        return slice_round(q, r, c, tie)
    if rule == EXTRA:
        # MatQuant summary section 7 "Errata": the slice without the clamp keeps
        # the extra value 2^r (2^r + 1 levels in all)
        return slice_round_unclamped(q, r, c, tie)
    raise ValueError(rule)


def delta_r(r: int, c: int = C_BITS, delta: str = "centre") -> float:
    """Offset that moves a truncated value from the lower edge of its cell to
    its centre.  ``centre``: mean of the 2^(c-r) integer codes in the cell."""
    m = cell_width(r, c)
    if delta == "centre":
        return (m - 1) / 2.0
    if delta == "half_cell":
        return m / 2.0 if r < c else 0.0
    raise ValueError(delta)


def sliced_value(q, r: int, rule: str, c: int = C_BITS, tie: str = "up",
                 delta: str = "centre") -> np.ndarray:
    """Reconstructed value in the c-bit code space (float64)."""
    code = slice_code(q, r, rule, c, tie).astype(np.float64)
    v = code * cell_width(r, c)
    if rule == PREFIX:
        v = v + delta_r(r, c, delta)
    return v


# ----------------------------------------------------------------------------
# dequantization and exports
# ----------------------------------------------------------------------------
def expand_groups(a: np.ndarray, group: int) -> np.ndarray:
    """[n, k/group] -> [n, k]: every group covers ``group`` consecutive k."""
    return np.repeat(np.asarray(a, dtype=np.float64), group, axis=1)


def dequant(q, scales, zeros, r: int, rule: str, group: int, c: int = C_BITS,
            tie: str = "up", delta: str = "centre") -> np.ndarray:
    """w_hat = s * (v - z), exact in float64.  [n, k] float64."""
    q = _codes(q)
    n, k = q.shape
    scales = np.asarray(scales)
    zeros = np.asarray(zeros)
    if k % group or scales.shape != (n, k // group) or zeros.shape != (n, k // group):
        raise ValueError("scale/zero shape must be [n, k/group]")
    v = sliced_value(q, r, rule, c, tie, delta)
    return expand_groups(scales, group) * (v - expand_groups(zeros, group))


def export_f32(w64: np.ndarray) -> np.ndarray:
    """fp32 image of the exact dequantized weights.  With an fp16 scale and an
    integer zero point the exact value needs at most 21 significant bits, so
    the conversion must be lossless; this is asserted."""
    w32 = w64.astype(np.float32)
    if not np.array_equal(w32.astype(np.float64), w64):
        raise AssertionError("dequantized weight not exactly representable in fp32")
    return w32


def export_f16(w64: np.ndarray) -> np.ndarray:
    """One IEEE round-to-nearest-even from the exact value."""
    return export_f32(w64).astype(np.float16)


def f32_to_bf16_bits(a32: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16, as uint16 bit patterns (finite inputs)."""
    u = np.ascontiguousarray(a32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def export_bf16_bits(w64: np.ndarray) -> np.ndarray:
    return f32_to_bf16_bits(export_f32(w64))


# ----------------------------------------------------------------------------
# the layer
# ----------------------------------------------------------------------------
def linear(x, q, scales, zeros, r: int, rule: str, group: int, **kw) -> np.ndarray:
    """Y64[m, n] = sum_k X[m, k] * w_hat[n, k] in float64.  ``x`` is any array
    convertible to float64 with shape [m, k]."""
    x64 = np.asarray(x, dtype=np.float64)
    w64 = dequant(q, scales, zeros, r, rule, group, **kw)
    if x64.ndim != 2 or x64.shape[1] != w64.shape[1]:
        raise ValueError("x must be [m, k]")
    return x64 @ w64.T


def linear_rows(x, q, scales, zeros, r: int, rule: str, group: int, rows, **kw) -> np.ndarray:
    """Y64[:, rows] only (dequantizes just those output rows), for sampled
    checks at full size."""
    rows = np.asarray(rows)
    return linear(x, np.asarray(q)[rows], np.asarray(scales)[rows],
                  np.asarray(zeros)[rows], r, rule, group, **kw)


def normalized_error(y, y_ref, x, w64) -> float:
    """max_{m,n} |y - y_ref| / (||X[m,:]||_2 * ||w_hat[n,:]||_2).  By
    Cauchy-Schwarz |y_ref| is at most the denominator."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    xn = np.linalg.norm(np.asarray(x, dtype=np.float64), axis=1)
    wn = np.linalg.norm(np.asarray(w64, dtype=np.float64), axis=1)
    den = xn[:, None] * wn[None, :]
    num = np.abs(y - y_ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(den > 0, num / np.where(den > 0, den, 1.0), np.where(num > 0, np.inf, 0.0))
    return float(rel.max()) if rel.size else 0.0


def linear_mixed(calls) -> list:
    """Each call is a dict with keys x, q, scales, zeros, r, rule, group; the
    single-layer definition applied to each with its own width."""
    return [linear(c["x"], c["q"], c["scales"], c["zeros"], c["r"], c["rule"], c["group"])
            for c in calls]
