"""Pins for the CPU oracle: each check ties the oracle to something other than
itself -- values printed on the pages, hand-worked values, bit-level readings,
closed forms, library routines and brute force.  CPU only."""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import mq_oracle as O
from nested_integer_weight_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "slice_worked_examples.txt")
ALLQ = np.arange(256)
WIDTHS = [1, 2, 3, 4, 5, 6, 7, 8]


def _golden_rows():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            q, r, rule, code, pre, value, src = line.split()
            rows.append((int(q), int(r), rule, int(code), None if pre == "-" else int(pre),
                         float(value), src))
    return rows


@pytest.mark.parametrize("row", _golden_rows(), ids=lambda t: f"q{t[0]}r{t[1]}{t[2]}")
def test_worked_examples(row):
    q, r, rule, code, pre, value, _ = row
    assert int(O.slice_code(q, r, rule)) == code
    assert float(O.sliced_value(q, r, rule)) == value
    if pre is not None:
        assert int(O.slice_round_unclamped(q, r)) == pre


def test_errata_unclamped_value_256():
    # "Matryoshka Quantization | Summary", section 7 "Errata": without the clamp,
    # 234 sliced to int2 reconstructs to 256.
    assert int(O.slice_round_unclamped(234, 2)) * O.cell_width(2) == 256


def test_int2_value_set_constant_spacing():
    # MatQuant summary, section 5.5: int2 values extracted from int8 are 0, 64,
    # 128 and 192 with constant spacing 64.
    vals = sorted(set(O.sliced_value(ALLQ, 2, O.ROUND).tolist()))
    assert vals == [0.0, 64.0, 128.0, 192.0]


def _bits(q):
    return format(int(q), "08b")


@pytest.mark.parametrize("r", WIDTHS)
def test_prefix_is_top_r_bits(r):
    # The true prefix is the r most significant bits (MatGPTQ App. A.1; the
    # 2-bit model is "the top-2 MSBs", MatQuant rebuttal page).
    for q in ALLQ:
        assert int(O.slice_prefix(q, r)) == int(_bits(q)[:r], 2)


@pytest.mark.parametrize("r", WIDTHS[:-1])
def test_round_uses_r_plus_1_th_bit(r):
    # MatGPTQ App. A.1: extract the r MSBs, use the (r+1)-th bit for rounding,
    # clamp on overflow.
    for q in ALLQ:
        b = _bits(q)
        pre = int(b[:r], 2) + int(b[r])
        assert int(O.slice_round_unclamped(q, r)) == pre
        assert int(O.slice_round(q, r)) == min(pre, 2 ** r - 1)


@pytest.mark.parametrize("r", WIDTHS[:-1])
def test_round_reads_exactly_r_plus_1_bits(r):
    # MatGPTQ section 1: an r-bit MatQuant model needs r+1 bits of the parent.
    keep = ~((1 << (8 - r - 1)) - 1) & 0xFF
    full = O.slice_round(ALLQ, r)
    assert np.array_equal(full, O.slice_round(ALLQ & keep, r))
    keep_r = ~((1 << (8 - r)) - 1) & 0xFF
    assert not np.array_equal(full, O.slice_round(ALLQ & keep_r, r))
    assert np.array_equal(O.slice_prefix(ALLQ, r), O.slice_prefix(ALLQ & keep_r, r))


@pytest.mark.parametrize("r", WIDTHS[:-1])
def test_extra_is_the_round_slice_without_clamp(r):
    # MatQuant summary section 7 "Errata": the unclamped variant keeps the value
    # 2^r that the clamp removes; read off the binary digits: top r digits plus
    # the (r+1)-th digit, no clamp.  2^r + 1 levels, the top one 2^c.
    for q in ALLQ:
        b = _bits(q)
        pre = int(b[:r], 2) + int(b[r])
        assert int(O.slice_code(q, r, O.EXTRA)) == pre
        assert float(O.sliced_value(q, r, O.EXTRA)) == pre * 2 ** (8 - r)
    vals = sorted(set(O.sliced_value(ALLQ, r, O.EXTRA).tolist()))
    assert len(vals) == 2 ** r + 1 and vals[0] == 0.0 and vals[-1] == 256.0
    differ = O.slice_code(ALLQ, r, O.EXTRA) != O.slice_code(ALLQ, r, O.ROUND)
    assert np.all(O.slice_code(ALLQ, r, O.EXTRA)[differ] == 2 ** r)


@pytest.mark.parametrize("rule", [O.PREFIX, O.ROUND, O.EXTRA])
def test_identity_at_full_width(rule):
    assert np.array_equal(O.slice_code(ALLQ, 8, rule), ALLQ)
    assert np.array_equal(O.sliced_value(ALLQ, 8, rule), ALLQ.astype(float))


@pytest.mark.parametrize("r", WIDTHS[:-1])
def test_level_counts(r):
    # 2^r levels for both strict rules; the unclamped slice has 2^r + 1 levels
    # (Errata) and its top level is 2^c.
    for rule in (O.PREFIX, O.ROUND):
        assert len(set(O.sliced_value(ALLQ, r, rule).tolist())) == 2 ** r
    unc = O.slice_round_unclamped(ALLQ, r) * O.cell_width(r)
    assert len(set(unc.tolist())) == 2 ** r + 1
    assert unc.max() == 256


@pytest.mark.parametrize("r", WIDTHS)
def test_nesting_and_monotonicity(r):
    for r2 in range(1, r + 1):
        assert np.array_equal(O.slice_prefix(O.slice_prefix(ALLQ, r) << (8 - r), r2),
                              O.slice_prefix(ALLQ, r2))
    for rule in (O.PREFIX, O.ROUND, O.EXTRA):
        v = O.sliced_value(ALLQ, r, rule)
        assert np.all(np.diff(v) >= 0)


def _rms(err):
    return float(np.sqrt(np.mean(np.square(err))))


@pytest.mark.parametrize("r", [2, 3, 4, 6])
def test_delta_centres_cells_and_minimises_rms(r):
    # MatGPTQ App. A.1: truncation lands on the lower edge of each cell; adding
    # delta_r centres it, which minimises the RMS error for the fixed nested
    # partition.  Closed forms over uniform q (m = cell width):
    #   truncation RMS = sqrt((m-1)(2m-1)/6), centred RMS = sqrt((m^2-1)/12).
    m = O.cell_width(r)
    trunc = O.slice_prefix(ALLQ, r) * m
    cen = O.sliced_value(ALLQ, r, O.PREFIX)
    assert _rms(trunc - ALLQ) == pytest.approx(np.sqrt((m - 1) * (2 * m - 1) / 6), rel=1e-12)
    assert _rms(cen - ALLQ) == pytest.approx(np.sqrt((m * m - 1) / 12), rel=1e-12)
    shifts = np.arange(0, 4 * m + 1) / 4.0
    best = min(shifts, key=lambda t: _rms(trunc + t - ALLQ))
    assert best == O.delta_r(r)
    rnd = O.sliced_value(ALLQ, r, O.ROUND)
    assert _rms(trunc - ALLQ) > _rms(rnd - ALLQ) > _rms(cen - ALLQ)


def test_tie_reading_alternative_differs_only_on_ties():
    for r in (2, 3, 4, 6):
        m = O.cell_width(r)
        differ = np.nonzero(O.slice_round(ALLQ, r, tie="up") != O.slice_round(ALLQ, r, tie="even"))[0]
        assert len(differ) > 0
        assert np.all(ALLQ[differ] % m == m // 2)


def test_bf16_export_matches_library_rne():
    rng = np.random.default_rng(1)
    a = rng.standard_normal(100000).astype(np.float32) * np.float32(3e-3)
    # exact ties between two bf16 values, both parities of the kept LSB
    ties = (np.arange(2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    a = np.concatenate([a, ties, -ties])
    ours = O.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_fp16_export_matches_library_rne():
    lay = synth.all_codes_layer(64, 512, 64)
    w = O.dequant(lay.q, lay.scales, lay.zeros, 3, O.PREFIX, 64)
    ref = torch.from_numpy(w).to(torch.float16).numpy()
    assert np.array_equal(O.export_f16(w).view(np.uint16), ref.view(np.uint16))


@pytest.mark.parametrize("rule", [O.PREFIX, O.ROUND, O.EXTRA])
@pytest.mark.parametrize("r", [2, 3, 4, 6, 8])
def test_dequant_exact_in_fp32(r, rule):
    lay = synth.all_codes_layer(96, 1024, 128)
    w = O.dequant(lay.q, lay.scales, lay.zeros, r, rule, 128)
    O.export_f32(w)  # raises if any value is not exactly representable


@pytest.mark.parametrize("r,rule", [(8, O.PREFIX), (4, O.PREFIX), (2, O.PREFIX), (4, O.ROUND), (2, O.ROUND)])
def test_dequant_reconstructs_minmax_weights(r, rule):
    # Independent of the oracle's formula: the parent was made from W by the
    # min-max quantizer with groups along k, so s*(v - z) must sit within the
    # slice's cell error of W.  At r = 8 that is half a step (one step where the
    # rounded range was clamped).
    lay = synth.make_layer(cfg_id=1, tensor_id=7, n=64, k=512, m=0, group=64)
    w_hat = O.dequant(lay.q, lay.scales, lay.zeros, r, rule, 64)
    s = O.expand_groups(lay.scales, 64)
    m = O.cell_width(r)
    err = np.abs(w_hat - lay.w.astype(np.float64)) / s
    if r == 8:
        assert np.quantile(err, 0.999) <= 0.5 + 1e-3
        assert err.max() <= 1.0 + 1e-3
    elif rule == O.PREFIX:
        assert err.max() <= m / 2 + 1.0 + 1e-3
    else:
        assert err.max() <= m - 0.5 + 1.0 + 1e-3
    # the error is centred: its mean is small against the cell width
    assert abs(np.mean((w_hat - lay.w) / s)) < 0.1 * m


def test_linear_matches_nn_linear_orientation():
    lay = synth.make_layer(cfg_id=1, tensor_id=8, n=48, k=256, m=5, group=64)
    x64 = lay.x.double().numpy()
    w64 = O.dequant(lay.q, lay.scales, lay.zeros, 3, O.PREFIX, 64)
    y = O.linear(x64, lay.q, lay.scales, lay.zeros, 3, O.PREFIX, 64)
    ref = torch.nn.functional.linear(torch.from_numpy(x64), torch.from_numpy(w64)).numpy()
    assert y.shape == (5, 48)
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-15)


def test_linear_brute_force_exact_rationals():
    lay = synth.make_layer(cfg_id=1, tensor_id=9, n=3, k=128, m=2, group=64)
    q, s, z = lay.q, lay.scales, lay.zeros
    x = lay.x.double().numpy()
    r = 3
    y = O.linear(x, q, s, z, r, O.PREFIX, 64)
    for mi in range(2):
        for ni in range(3):
            acc = Fraction(0)
            for ki in range(128):
                code = int(q[ni, ki]) >> (8 - r)                       # top r bits
                val = Fraction(code * 32) + Fraction(31, 2)           # centre of the 32-code cell
                sc = Fraction(float(s[ni, ki // 64]))
                zz = Fraction(float(z[ni, ki // 64]))
                acc += Fraction(float(x[mi, ki])) * sc * (val - zz)
            assert abs(float(acc) - y[mi, ni]) <= 1e-12 * max(1.0, abs(float(acc)))


def test_linear_rows_is_a_column_subset():
    lay = synth.make_layer(cfg_id=1, tensor_id=10, n=40, k=256, m=3, group=128)
    x = lay.x.double().numpy()
    full = O.linear(x, lay.q, lay.scales, lay.zeros, 4, O.ROUND, 128)
    rows = [0, 7, 39]
    np.testing.assert_array_equal(O.linear_rows(x, lay.q, lay.scales, lay.zeros, 4, O.ROUND, 128, rows),
                                  full[:, rows])


def test_normalized_error_metric():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 64))
    w = rng.standard_normal((5, 64))
    y = x @ w.T
    # Cauchy-Schwarz: a zero output is at most 1 away in this metric
    assert O.normalized_error(np.zeros_like(y), y, x, w) <= 1.0 + 1e-12
    den = np.linalg.norm(x[2]) * np.linalg.norm(w[3])
    y2 = y.copy()
    y2[2, 3] += 1e-3 * den
    assert O.normalized_error(y2, y, x, w) == pytest.approx(1e-3, rel=1e-9)
    assert O.normalized_error(y, y, x, w) == 0.0


def test_mixnmatch_recipe_and_mixed_definition():
    widths = synth.mixnmatch_widths()
    assert len(widths) == 42 and sum(widths) == 3 * 42
    assert sorted(set(widths)) == [2, 3, 4]
    calls = []
    for i, r in enumerate(widths[:3]):
        lay = synth.make_layer(cfg_id=5, tensor_id=i, n=32, k=256, m=1, group=128)
        calls.append(dict(x=lay.x.double().numpy(), q=lay.q, scales=lay.scales, zeros=lay.zeros,
                          r=r, rule=O.PREFIX, group=128))
    outs = O.linear_mixed(calls)
    assert [y.shape for y in outs] == [(1, 32)] * 3


def _exact_value(q, r, rule):
    """Reconstructed code-space value read off the binary digits of q, as a
    Fraction: the top r digits, then (rounded slice) plus the (r+1)-th digit
    with a clamp at the largest r-bit code, or (true prefix) plus the centre
    of the 2^(8-r) codes that share the prefix."""
    b = format(int(q), "08b")
    top = int(b[:r], 2)
    if r == 8:
        return Fraction(top)
    if rule == O.ROUND:
        return Fraction(min(top + int(b[r]), 2 ** r - 1) * 2 ** (8 - r))
    return Fraction(top * 2 ** (8 - r)) + Fraction(2 ** (8 - r) - 1, 2)


def test_linear_mixed_brute_force_exact_rationals():
    # Mix'n'Match (MatQuant summary section 4.3): each layer matrix at its own
    # width and rule.  Every output is recomputed as an exact rational from the
    # bit-level definitions, independently of the oracle's arithmetic.
    specs = [(2, O.ROUND, 64), (6, O.PREFIX, 128), (8, O.ROUND, 64), (3, O.PREFIX, 64), (4, O.ROUND, 128)]
    calls = []
    for i, (r, rule, g) in enumerate(specs):
        lay = synth.make_layer(cfg_id=1, tensor_id=20 + i, n=3, k=128, m=2, group=g, outlier_frac=0.02)
        calls.append(dict(x=lay.x.double().numpy(), q=lay.q, scales=lay.scales, zeros=lay.zeros,
                          r=r, rule=rule, group=g))
    outs = O.linear_mixed(calls)
    assert len(outs) == len(calls)
    for c, y in zip(calls, outs):
        assert y.shape == (2, 3)
        for mi in range(2):
            for ni in range(3):
                acc = Fraction(0)
                for ki in range(128):
                    gi = ki // c["group"]
                    v = _exact_value(c["q"][ni, ki], c["r"], c["rule"])
                    acc += (Fraction(float(c["x"][mi, ki])) * Fraction(float(c["scales"][ni, gi]))
                            * (v - Fraction(float(c["zeros"][ni, gi]))))
                assert abs(float(acc) - y[mi, ni]) <= 1e-12 * max(1.0, abs(float(acc)))


def test_synth_is_deterministic_and_minmax_in_range():
    a = synth.make_layer(cfg_id=2, tensor_id=0, n=16, k=256, m=1, group=128, outlier_frac=1e-3)
    b = synth.make_layer(cfg_id=2, tensor_id=0, n=16, k=256, m=1, group=128, outlier_frac=1e-3)
    assert np.array_equal(a.q, b.q) and torch.equal(a.x, b.x)
    assert np.all(a.zeros.astype(np.float64) == np.rint(a.zeros.astype(np.float64)))
    assert a.zeros.min() >= 0 and a.zeros.max() <= 255
    assert np.all(a.scales > 0)
