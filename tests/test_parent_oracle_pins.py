"""Pins of the parent-producer oracle (oracle/mq_parent_oracle.py) against
facts that do not come from the oracle itself.

* Single candidate: the scale search with one candidate (no shrinking) must
  return the plain min-max quantizer's scale and zero point, here taken from
  the input generator's own, separately written, min-max parent
  ("Matryoshka Quantization | Summary", section 3.1, MinMax quantizer).
* Reductions to textbook rounding: with R = {8} the code choice is the
  nearest code (round to nearest), with R = {2} it is the nearest of the four
  2-bit levels, reached by the first code of that cell.
* Exact minimum: the fp32 decisions agree with the minimum of the exact
  (float64) weighted error, up to the rounding of the fp32 sums.
* Scale invariance: multiplying every lambda by a power of two changes no
  decision.
* The "4 MB" figure ("MatGPTQ: Efficient and Accurate Inference over Nested
  Quantized Models", Appendix A.2, runtime and memory considerations): one
  4096-row column's error matrix over the 2^8 candidates is 256 x 4096 fp32.
* Planted mistakes (a dropped width, a lambda applied to the wrong width, the
  last instead of the first minimum, no clamp) each fail one of the checks.
"""
from __future__ import annotations

import numpy as np
import pytest

from nested_integer_weight_amd import synth
from oracle import mq_oracle as O
from oracle import mq_parent_oracle as P

WIDTHS = [3, 4, 8]
LAMS = [1.0, 1.0, 1.0]


def _layer(n=24, k=256, seed=1, outliers=1e-2):
    return synth.gaussian_weights(synth.rng_for(31, seed), n, k, outlier_frac=outliers)


def exact_errors(w, s16, z16, group, widths, lambdas, rule):
    """float64 weighted error of every code for every weight: [256, n, k].
    Written directly from equation 5: sum_r lambda_r (w - s (v_r(q) - z))^2."""
    w64 = np.asarray(w, dtype=np.float64)
    s = O.expand_groups(np.asarray(s16, dtype=np.float64), group)
    z = O.expand_groups(np.asarray(z16, dtype=np.float64), group)
    q = np.arange(256)
    out = np.zeros((256,) + w64.shape)
    for r, lam in zip(widths, lambdas):
        v = O.sliced_value(q, r, rule)[:, None, None]
        out += float(np.float32(lam)) * (w64[None] - s[None] * (v - z[None])) ** 2
    return out


def check_choice_is_exact_minimum(w, s, z, q, group, widths, lambdas, rule):
    e = exact_errors(w, s, z, group, widths, lambdas, rule)
    chosen = np.take_along_axis(e, np.asarray(q, dtype=np.int64)[None], axis=0)[0]
    best = e.min(axis=0)
    assert np.all(chosen <= best * (1 + 4e-6) + 1e-30), "a chosen code is not the minimum"
    agree = np.mean(np.asarray(q) == e.argmin(axis=0))
    assert agree > 0.999, agree


def check_search_is_exact_minimum(w, group, widths, lambdas, rule, n_grid, grid_den, s, z):
    """Every candidate re-scored in float64 from its own (s, z): the chosen one
    is the minimum up to the fp32 rounding of the sums."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    wg = w.reshape(n, k // group, group).astype(np.float64)
    lo = np.minimum(w.reshape(n, k // group, group).min(-1), np.float32(0))
    hi = np.maximum(w.reshape(n, k // group, group).max(-1), np.float32(0))
    errs, cands = [], []
    for i in range(n_grid):
        s16, s32, z32 = P.candidate_scale_zero(lo, hi, P.candidate_shrink(i, grid_den))
        sc = s32.astype(np.float64)[..., None]
        zc = z32.astype(np.float64)[..., None]
        # the candidate's codes: nearest c-bit code, decided in fp32 as defined
        x = np.rint(w.reshape(n, k // group, group) / s32[..., None]) + z32[..., None]
        q = np.clip(x, 0, 255).astype(np.int64)
        e = np.zeros((n, k // group))
        for r, lam in zip(widths, lambdas):
            v = O.sliced_value(q, r, rule)
            e += float(np.float32(lam)) * ((wg - sc * (v - zc)) ** 2).sum(-1)
        errs.append(e)
        cands.append((s16, z32))
    errs = np.stack(errs)
    pick = np.full((n, k // group), -1)
    for i, (s16, z32) in enumerate(cands):
        hit = (s16 == s) & (z32.astype(np.float16) == z) & (pick < 0)
        pick[hit] = i
    assert np.all(pick >= 0), "chosen (s, z) is not one of the candidates"
    chosen = np.take_along_axis(errs, pick[None], axis=0)[0]
    assert np.all(chosen <= errs.min(axis=0) * (1 + 1e-5) + 1e-30)
    # never worse than the unshrunk min-max candidate
    assert np.all(chosen <= errs[0] * (1 + 1e-5) + 1e-30)


# ----------------------------------------------------------------------------
def test_single_candidate_is_minmax():
    w = _layer(32, 512, seed=2)
    for group in (64, 128):
        s, z = P.search_scale_zero(w, group, WIDTHS, LAMS, O.PREFIX, n_grid=1)
        _, s_ref, z_ref = synth.minmax_parent(w, group)
        assert np.array_equal(s.view(np.uint16), s_ref.view(np.uint16))
        assert np.array_equal(z, z_ref)


def test_width8_choice_is_nearest_code():
    w = _layer(32, 256, seed=3)
    q_ref, s, z = synth.minmax_parent(w, 64)
    q = P.choose_codes(w, s, z, 64, [8], [1.0], O.PREFIX)
    check_choice_is_exact_minimum(w, s, z, q, 64, [8], [1.0], O.PREFIX)
    # away from exact half-way points it is round-to-nearest, as the min-max parent rounds
    x = w.astype(np.float64) / O.expand_groups(s, 64) + O.expand_groups(z, 64)
    far = np.abs(x - np.floor(x) - 0.5) > 1e-3
    assert np.array_equal(q[far], q_ref[far])


@pytest.mark.parametrize("rule", [O.PREFIX, O.ROUND])
def test_width2_choice_is_nearest_level_first_code(rule):
    w = _layer(32, 256, seed=4)
    _, s, z = synth.minmax_parent(w, 64)
    q = P.choose_codes(w, s, z, 64, [2], [1.0], rule).astype(np.int64)
    codes = np.arange(256)
    levels = O.sliced_value(codes, 2, rule)                  # value of every code at r = 2
    distinct = np.unique(levels)
    assert distinct.size == 4
    sw = O.expand_groups(s, 64)
    zw = O.expand_groups(z, 64)
    dist = np.abs(w[None].astype(np.float64) - sw[None] * (distinct[:, None, None] - zw[None]))
    best_level = distinct[dist.argmin(axis=0)]
    assert np.array_equal(O.sliced_value(q, 2, rule), best_level)
    # the first code whose slice is that level
    first = {lv: int(codes[levels == lv].min()) for lv in distinct}
    assert np.array_equal(q, np.vectorize(first.get)(best_level))


@pytest.mark.parametrize("rule", [O.PREFIX, O.ROUND, O.EXTRA])
def test_cross_width_choice_is_exact_minimum(rule):
    w = _layer(24, 256, seed=5)
    lams = [0.5, 0.25, 1.0]
    s, z = P.search_scale_zero(w, 64, WIDTHS, lams, rule, n_grid=20)
    q = P.choose_codes(w, s, z, 64, WIDTHS, lams, rule)
    check_choice_is_exact_minimum(w, s, z, q, 64, WIDTHS, lams, rule)


@pytest.mark.parametrize("widths,lams", [([3, 4, 8], [1.0, 1.0, 1.0]), ([2, 4, 8], [1.0, 0.1, 0.1]),
                                         ([2, 3, 4, 6, 8], [1, 1, 1, 1, 1])])
def test_scale_search_is_exact_minimum(widths, lams):
    w = _layer(16, 256, seed=6)
    s, z = P.search_scale_zero(w, 64, widths, lams, O.PREFIX, n_grid=40)
    check_search_is_exact_minimum(w, 64, widths, lams, O.PREFIX, 40, 100, s, z)


def test_power_of_two_lambda_scaling_changes_nothing():
    w = _layer(16, 256, seed=7)
    a = P.produce_parent(w, 64, WIDTHS, [0.3, 0.7, 1.1], O.PREFIX, n_grid=30)
    b = P.produce_parent(w, 64, WIDTHS, [1.2, 2.8, 4.4], O.PREFIX, n_grid=30)   # x 4, exact
    for u, v in zip(a, b):
        assert np.array_equal(np.asarray(u).view(np.uint8), np.asarray(v).view(np.uint8))


def test_zero_group_and_constant_group():
    w = _layer(4, 256, seed=8)
    w[0, :64] = 0.0                      # all-zero group: scale 1, zero 0, code 0
    w[1, 64:128] = np.float32(0.0125)   # constant positive group
    s, z = P.search_scale_zero(w, 64, WIDTHS, LAMS, O.PREFIX)
    q = P.choose_codes(w, s, z, 64, WIDTHS, LAMS, O.PREFIX)
    assert s[0, 0] == 1 and z[0, 0] == 0 and np.all(q[0, :64] == 0)
    check_choice_is_exact_minimum(w, s, z, q, 64, WIDTHS, LAMS, O.PREFIX)


def test_column_error_matrix_is_4_mb():
    # one 4096-row column: 2^8 candidates x 4096 rows of fp32
    w = _layer(4096, 64, seed=9, outliers=0.0)
    _, s, z = synth.minmax_parent(w, 64)
    e = P.column_errors(w[:, 0], s[:, 0], z[:, 0], WIDTHS, LAMS, O.PREFIX)
    assert e.shape == (256, 4096) and e.dtype == np.float32
    assert e.nbytes == 256 * 4096 * 4 == 4 * 2 ** 20


# ----------------------------------------------------------------------------
# planted mistakes: each one must fail a check above
# ----------------------------------------------------------------------------
def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def test_planted_mistakes_are_caught(monkeypatch):
    w = _layer(32, 256, seed=10)
    _, s, z = synth.minmax_parent(w, 64)
    # MatQuant's rounded slice: there the cross-width choice moves a few percent
    # of the codes away from plain rounding (with the centred true prefix the
    # nearest code is already the best one at every width), so a wrong term shows
    widths, lams = [2, 4, 8], [1.0, 0.1, 0.1]

    def run_choice(rule=O.ROUND):
        q = P.choose_codes(w, s, z, 64, widths, lams, rule)
        check_choice_is_exact_minimum(w, s, z, q, 64, widths, lams, rule)

    def run_search(rule=O.PREFIX):
        s2, z2 = P.search_scale_zero(w[:8], 64, WIDTHS, LAMS, rule, n_grid=40)
        check_search_is_exact_minimum(w[:8], 64, WIDTHS, LAMS, rule, 40, 100, s2, z2)

    run_choice()
    run_search()   # the unmodified oracle passes both

    real_cols, real_rec, real_nearest = P.column_errors, P.reconstruct, P.nearest_code
    mutations = {
        # a dropped width in the weighted sum
        "dropped width": ("column_errors", lambda wc, sc, zc, wd, lm, rule: real_cols(wc, sc, zc, wd[1:], lm[1:], rule),
                          run_choice),
        # the lambdas applied to the wrong widths
        "lambdas reversed": ("column_errors", lambda wc, sc, zc, wd, lm, rule: real_cols(wc, sc, zc, wd, lm[::-1], rule),
                             run_choice),
        # the zero point added instead of subtracted
        "zero sign": ("reconstruct", lambda q, s_, z_, r, rule: real_rec(q, s_, -np.asarray(z_), r, rule), run_choice),
        # a width index off by one in the search (r = 3 reconstructed as r = 4)
        "width index": ("reconstruct", lambda q, s_, z_, r, rule: real_rec(q, s_, z_, 4 if r == 3 else r, rule),
                        run_search),
        # the nearest-code step of the search without its clamp (codes wrap)
        "no clamp": ("nearest_code",
                     lambda w_, s_, z_, c=8: (np.rint((w_ / s_).astype(np.float32)) + z_).astype(np.int64) % 256,
                     run_search),
    }
    for name, (attr, bad, check) in mutations.items():
        monkeypatch.setattr(P, attr, bad)
        assert _fails(check), name
        monkeypatch.setattr(P, attr, {"column_errors": real_cols, "reconstruct": real_rec,
                                      "nearest_code": real_nearest}[attr])

    # the last instead of the first minimum: ties inside a 2-bit cell
    real_choose = P.choose_codes

    def last_min(w_, s_, z_, g, wd, lm, rule):
        out = np.empty(w_.shape, dtype=np.uint8)
        for col in range(w_.shape[1]):
            e = P.column_errors(w_[:, col], s_[:, col // g], z_[:, col // g], wd, lm, rule)
            out[:, col] = 255 - np.argmin(e[::-1], axis=0)
        return out
    monkeypatch.setattr(P, "choose_codes", last_min)
    assert _fails(lambda: test_width2_choice_is_nearest_level_first_code(O.PREFIX))
    monkeypatch.setattr(P, "choose_codes", real_choose)


@pytest.mark.parametrize("widths,lams", [([3, 4, 8], [1.0, 1.0, 1.0]), ([2, 4, 8], [1.0, 0.1, 0.1]),
                                         ([2, 3, 4, 6, 8], [1, 1, 1, 1, 1])])
def test_centred_prefix_choice_is_the_nearest_code(widths, lams):
    """With the centred true prefix each r-bit cell's value is the centre of
    the cell's code interval, so the cell that holds the nearest code also has
    the nearest centre: the cross-width choice is plain rounding, except where
    a weight sits (within rounding) halfway between two codes."""
    w = _layer(32, 256, seed=11)
    q_ref, s, z = synth.minmax_parent(w, 64)
    q = P.choose_codes(w, s, z, 64, widths, lams, O.PREFIX)
    x = w.astype(np.float64) / O.expand_groups(s, 64) + O.expand_groups(z, 64)
    far = np.abs(x - np.floor(x) - 0.5) > 1e-3
    assert np.array_equal(q[far], q_ref[far])
    assert np.all(np.abs(q.astype(int) - q_ref.astype(int)) <= 1)


def test_zero_points_are_non_negative_integers():
    """An all-positive group has lo = 0, so -lo * p is -0; the stored zero
    point must be the integer 0 (+0)."""
    w = np.abs(_layer(8, 256, seed=12))
    s, z = P.search_scale_zero(w, 64, WIDTHS, LAMS, O.PREFIX, n_grid=10)
    zb = z.view(np.uint16)
    assert np.all(zb == 0)     # every group all positive -> zero point +0
    assert np.all(z == np.rint(z)) and np.all(z >= 0)
