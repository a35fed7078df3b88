"""CPU tests of the float64 oracle against its pins, plus planted-mistake checks.

The planted mistakes replace the oracle's per-row kernel with a copy carrying
one plausible slip (a dropped term, a wrong sign, a transposed operand, a
wrong axis, a wrong log base ...).  Every such copy must fail at least one pin,
which shows the pins constrain every step of the definition.
"""

import numpy as np
import pytest

import oracle.attention as oa
from oracle import attention_forward, attention_rows
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(attention_forward)


def test_rows_api_matches_full_forward():
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal((2, 3, 70, 16)) for _ in range(3))
    o, lse = attention_forward(q, k, v, 0.25, row_block=16)
    rows = [0, 5, 33, 69]
    o_r, l_r = attention_rows(q, k, v, 0.25, 1, 2, rows)
    np.testing.assert_allclose(o_r, o[1, 2, rows], rtol=0, atol=1e-13)
    np.testing.assert_allclose(l_r, lse[1, 2, rows], rtol=0, atol=1e-13)


def _rows_match_full_forward(rows_fn):
    """attention_rows with a causal mask against the matching rows of the pinned full
    forward: offsets 0, -7 and 13, queries fewer and more than keys, scattered
    rows that include rows without any visible key (O = 0, LSE = -inf)."""
    rng = np.random.default_rng(5)
    for Sq, Skv in [(40, 40), (40, 57), (57, 23)]:
        q = rng.standard_normal((2, 2, Sq, 8))
        k, v = (rng.standard_normal((2, 2, Skv, 8)) for _ in range(2))
        for off in (0, -7, 13):
            o, lse = attention_forward(q, k, v, 0.3, row_block=16, causal_offset=off)
            rows = [Sq - 1, 0, 3, 6, 7, 11, 20, Sq // 2, Sq - 2]
            for (b, h) in [(0, 1), (1, 0)]:
                o_r, l_r = rows_fn(q, k, v, 0.3, b, h, rows, causal_offset=off)
                np.testing.assert_allclose(o_r, o[b, h, rows], rtol=0, atol=1e-13)
                np.testing.assert_array_equal(np.isneginf(l_r), np.isneginf(lse[b, h, rows]))
                fin = np.isfinite(lse[b, h, rows])
                np.testing.assert_allclose(l_r[fin], lse[b, h, rows][fin], rtol=0, atol=1e-13)
            if off == -7:   # rows 0..6 see no key: the keyless branch is exercised
                assert np.isneginf(lse[:, :, :7]).all() and not np.isneginf(lse[:, :, 7:]).any()


def test_rows_api_causal_matches_full_forward():
    _rows_match_full_forward(attention_rows)


def _r_row_positions(q, k, v, scale, b, h, rows, causal_offset=None):
    # slip: the mask built for positions 0..len(rows)-1 instead of the rows asked for
    rows = np.asarray(rows, dtype=np.int64)
    qh = np.asarray(q[b, h], dtype=np.float64)[rows]
    kh, vh = np.asarray(k[b, h], dtype=np.float64), np.asarray(v[b, h], dtype=np.float64)
    mask = None if causal_offset is None else oa.causal_mask(range(len(rows)), kh.shape[0],
                                                             causal_offset)
    return oa._rows(qh, kh, vh, scale, mask)


def _r_offset_ignored(q, k, v, scale, b, h, rows, causal_offset=None):
    # slip: the offset dropped (mask j <= i)
    return attention_rows(q, k, v, scale, b, h, rows, None if causal_offset is None else 0)


def _r_wrong_head(q, k, v, scale, b, h, rows, causal_offset=None):
    # slip: keys and values of the head with the indices swapped
    return attention_rows(q, k, v, scale, h, b, rows, causal_offset)


@pytest.mark.parametrize("mutant", [_r_row_positions, _r_offset_ignored, _r_wrong_head],
                         ids=lambda f: f.__name__)
def test_planted_rows_mistake_fails_rows_pin(mutant):
    with pytest.raises(AssertionError):
        _rows_match_full_forward(mutant)


def test_row_blocking_does_not_change_result():
    rng = np.random.default_rng(4)
    q, k, v = (rng.standard_normal((1, 2, 130, 8)) for _ in range(3))
    a = attention_forward(q, k, v, 0.5, row_block=7)
    b = attention_forward(q, k, v, 0.5, row_block=4096)
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(a[1], b[1], rtol=0, atol=1e-14)


def test_rejects_mismatched_shapes():
    with pytest.raises(ValueError):   # k and v lengths differ
        attention_forward(np.zeros((1, 1, 4, 2)), np.zeros((1, 1, 5, 2)), np.zeros((1, 1, 6, 2)), 1.0)
    with pytest.raises(ValueError):   # head dimension differs
        attention_forward(np.zeros((1, 1, 4, 2)), np.zeros((1, 1, 5, 3)), np.zeros((1, 1, 5, 3)), 1.0)
    with pytest.raises(ValueError):   # no keys
        attention_forward(np.zeros((1, 1, 4, 2)), np.zeros((1, 1, 0, 2)), np.zeros((1, 1, 0, 2)), 1.0)


# --- planted mistakes -------------------------------------------------------

def _m_transposed_scores(qh, kh, vh, scale, mask=None):
    s = scale * (kh @ qh.T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    return (e @ vh) / l, m[:, 0] + np.log(l[:, 0])


def _m_no_scale(qh, kh, vh, scale, mask=None):
    return oa.__dict__["_orig_rows"](qh, kh, vh, 1.0, mask)


def _m_sign(qh, kh, vh, scale, mask=None):
    return oa.__dict__["_orig_rows"](qh, kh, vh, -scale, mask)


def _m_wrong_axis(qh, kh, vh, scale, mask=None):
    s = scale * (qh @ kh.T)
    m = s.max(axis=0, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=0, keepdims=True)
    o = (e / l) @ vh
    return o, np.log(np.exp(s).sum(axis=1))


def _m_no_max_subtraction(qh, kh, vh, scale, mask=None):
    s = scale * (qh @ kh.T)
    e = np.exp(s)
    l = e.sum(axis=1, keepdims=True)
    return (e @ vh) / l, np.log(l[:, 0])


def _m_lse_without_max(qh, kh, vh, scale, mask=None):
    o, lse = oa.__dict__["_orig_rows"](qh, kh, vh, scale, mask)
    m = (scale * (qh @ kh.T)).max(axis=1)
    return o, lse - m


def _m_lse_base2(qh, kh, vh, scale, mask=None):
    o, lse = oa.__dict__["_orig_rows"](qh, kh, vh, scale, mask)
    return o, lse / np.log(2.0)


def _m_no_normalisation(qh, kh, vh, scale, mask=None):
    s = scale * (qh @ kh.T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    return e @ vh, m[:, 0] + np.log(l[:, 0])


def _m_dropped_last_key_in_sum(qh, kh, vh, scale, mask=None):
    s = scale * (qh @ kh.T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e[:, :-1].sum(axis=1, keepdims=True) if e.shape[1] > 1 else e.sum(axis=1, keepdims=True)
    return (e @ vh) / l, m[:, 0] + np.log(l[:, 0])


def _m_reversed_values(qh, kh, vh, scale, mask=None):
    return oa.__dict__["_orig_rows"](qh, kh, vh[::-1], scale, mask)


def _m_keys_used_as_values(qh, kh, vh, scale, mask=None):
    return oa.__dict__["_orig_rows"](qh, kh, kh, scale, mask)


def _m_off_by_one_key(qh, kh, vh, scale, mask=None):
    s = scale * (qh @ np.roll(kh, 1, axis=0).T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    return (e @ vh) / l, m[:, 0] + np.log(l[:, 0])


def _m_exp2_instead_of_exp(qh, kh, vh, scale, mask=None):
    s = scale * (qh @ kh.T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp2(s - m)
    l = e.sum(axis=1, keepdims=True)
    return (e @ vh) / l, m[:, 0] + np.log(l[:, 0])


MUTANTS = [_m_transposed_scores, _m_no_scale, _m_sign, _m_wrong_axis, _m_no_max_subtraction,
           _m_lse_without_max, _m_lse_base2, _m_no_normalisation, _m_dropped_last_key_in_sum,
           _m_reversed_values, _m_keys_used_as_values, _m_off_by_one_key, _m_exp2_instead_of_exp]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda f: f.__name__)
def test_planted_mistake_fails_some_pin(mutant, monkeypatch):
    monkeypatch.setitem(oa.__dict__, "_orig_rows", oa._rows)
    monkeypatch.setattr(oa, "_rows", mutant)
    failed = []
    with np.errstate(all="ignore"):
        for pin in P.ALL_PINS:
            try:
                pin(oa.attention_forward)
            except (AssertionError, ValueError, FloatingPointError):
                failed.append(pin.__name__)
    assert failed, f"planted mistake {mutant.__name__} passed every pin"


# --- planted mistakes in the causal mask ---------------------------------------------

def _c_strict(rows, Skv, offset):          # j < i + offset: the diagonal key dropped
    rows = np.asarray(rows)
    return np.arange(Skv)[None, :] < rows[:, None] + offset


def _c_top_left(rows, Skv, offset):        # alignment ignored: j <= i
    rows = np.asarray(rows)
    return np.arange(Skv)[None, :] <= rows[:, None]


def _c_transposed(rows, Skv, offset):      # j >= i + offset
    rows = np.asarray(rows)
    return np.arange(Skv)[None, :] >= rows[:, None] + offset


def _c_none(rows, Skv, offset):            # mask ignored
    return np.ones((len(np.asarray(rows)), Skv), dtype=bool)


CAUSAL_MUTANTS = [_c_strict, _c_top_left, _c_transposed, _c_none]


@pytest.mark.parametrize("mutant", CAUSAL_MUTANTS, ids=lambda f: f.__name__)
def test_planted_causal_mistake_fails_some_pin(mutant, monkeypatch):
    monkeypatch.setattr(oa, "causal_mask", mutant)
    failed = []
    with np.errstate(all="ignore"):
        for pin in P.ALL_PINS:
            try:
                pin(oa.attention_forward)
            except (AssertionError, ValueError, FloatingPointError):
                failed.append(pin.__name__)
    assert failed, f"planted mistake {mutant.__name__} passed every pin"
