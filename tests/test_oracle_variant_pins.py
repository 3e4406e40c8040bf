"""Pins for the oracle's codec variants (FP4 and INT4 tables, block constants
without double quantization, centered double quantization), on the CPU.

Each check ties the oracle to something outside itself: the facts in
tests/golden/codec_variant_facts.json, brute-force nearest levels in exact
rational arithmetic, the textbook absmax integer quantizer, exact sums, and
bounds that follow from the definitions.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import codec_variants as cv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "codec_variant_facts.json")


def _facts():
    with open(GOLDEN) as f:
        return json.load(f)


def _f32(x):
    return np.float32(x)


# ---------------------------------------------------------------------------
# Level tables
# ---------------------------------------------------------------------------

def test_fp4_table_is_e2m1_over_its_max():
    mags = _facts()["e2m1_magnitudes"]["value"]
    vals = sorted({Fraction(m).limit_denominator(4) for m in mags}
                  | {-Fraction(m).limit_denominator(4) for m in mags})
    # 15 distinct values (+0 and -0 coincide) plus the second zero
    assert len(vals) == 15
    top = max(vals)
    expect = []
    for v in vals:
        expect.append(v / top)
        if v == 0:
            expect.append(Fraction(0))
    lv = cv.fp4_levels()
    assert lv.dtype == np.float32 and lv.shape == (16,)
    for got, want in zip(lv, expect):
        assert got == _f32(float(want))
    assert not np.signbit(lv[lv == 0]).any()       # both zeros are +0
    assert lv[0] == -1.0 and lv[-1] == 1.0


def test_int4_table_is_the_page_range_over_seven():
    lo, hi = _facts()["int4_range"]["value"]
    lv = cv.int4_levels()
    assert lv.shape == (hi - lo + 1,)
    for k, got in zip(range(lo, hi + 1), lv):
        exact = Fraction(k, 7)
        # got is the float32 nearest to k/7
        up = np.nextafter(got, np.float32(np.inf))
        dn = np.nextafter(got, np.float32(-np.inf))
        err = abs(Fraction(float(got)) - exact)
        assert err <= abs(Fraction(float(up)) - exact)
        assert err <= abs(Fraction(float(dn)) - exact)
    assert lv[8] == 0.0 and lv[15] == 1.0


@pytest.mark.parametrize("code", [cv.CODE_FP4, cv.CODE_INT4, cv.CODE_NF4])
def test_thresholds_are_sorted_midpoints(code):
    lv, t = cv.levels(code), cv.thresholds(code)
    assert np.all(np.diff(lv.astype(np.float64)) >= 0)
    for j in range(15):
        mid = (Fraction(float(lv[j])) + Fraction(float(lv[j + 1]))) / 2
        assert abs(Fraction(float(t[j])) - mid) <= abs(mid) * Fraction(1, 2 ** 24)


def _nearest_code_brute(n, lv):
    """Index of the nearest level in exact arithmetic, ties to the lower
    index, equal levels resolved to the lower index."""
    fn = Fraction(float(n))
    best, best_d = None, None
    for j, L in enumerate(lv):
        d = abs(fn - Fraction(float(L)))
        if best_d is None or d < best_d:
            best, best_d = j, d
    return best


def _probe_values(code, rng):
    t = cv.thresholds(code)
    vals = list(rng.uniform(-1, 1, 400).astype(np.float32))
    for x in t:
        vals += [x, np.nextafter(x, np.float32(2)), np.nextafter(x, np.float32(-2))]
    vals += [np.float32(-1), np.float32(1), np.float32(0)]
    return np.array(vals, dtype=np.float32)


@pytest.mark.parametrize("code", [cv.CODE_FP4, cv.CODE_INT4])
def test_codes_are_nearest_level_with_ties_low(code):
    rng = np.random.default_rng(71)
    n = _probe_values(code, rng)
    lv = cv.levels(code)
    # c = 1 so the oracle's division is the identity
    got = oracle.nf4_codes(n, np.ones(-(-n.size // 64), np.float32),
                           cv.thresholds(code))
    t = cv.thresholds(code)
    for x, g in zip(n, got):
        want = _nearest_code_brute(x, lv)
        if lv[g] == lv[want]:
            continue          # same level (the two FP4 zeros)
        # otherwise x must lie between the exact midpoint of the two adjacent
        # levels and its fp32 rounding t_j, on the side the rule puts it
        j = min(int(g), want)
        assert abs(int(g) - want) == 1, (code, float(x), int(g), want)
        mid = (Fraction(float(lv[j])) + Fraction(float(lv[j + 1]))) / 2
        fx, ft = Fraction(float(x)), Fraction(float(t[j]))
        assert min(mid, ft) <= fx <= max(mid, ft), (code, float(x), int(g), want)
        assert (int(g) == j + 1) == (fx > ft)


def test_int4_codes_are_the_absmax_integer_quantizer():
    # textbook absmax quantizer: q = round(7 * w / absmax), away from ties
    rng = np.random.default_rng(72)
    w = rng.standard_normal(64 * 300).astype(np.float32)
    c = oracle.block_absmax(w)
    codes = oracle.nf4_codes(w, c, cv.thresholds(cv.CODE_INT4)).astype(np.int64)
    n = (w / c[np.arange(w.size) // 64]).astype(np.float32).astype(np.float64)
    scaled = 7.0 * n
    frac = np.abs(scaled - np.floor(scaled) - 0.5)
    keep = frac > 1e-5
    assert keep.mean() > 0.99
    assert np.array_equal(codes[keep] - 8, np.rint(scaled[keep]).astype(np.int64))
    assert codes.min() >= 1  # -8 (code 0) lies beyond -1 and is never chosen


@pytest.mark.parametrize("code", [cv.CODE_NF4, cv.CODE_FP4, cv.CODE_INT4])
def test_zero_weight_code_and_pad_nibble(code):
    z = cv.zero_code(code)
    assert cv.levels(code)[z] == 0.0
    w = np.zeros(129, np.float32)
    w[:64] = np.linspace(-1, 1, 64, dtype=np.float32)
    packed, consts, gs, gm = cv.quantize(w, code, cv.DQ_NONE)
    assert packed.size == 65
    assert packed[-1] & 0x0F == z and packed[-1] >> 4 == z   # element 128 + pad
    out = cv.dequantize(packed, consts, gs, gm, w.size, code, cv.DQ_NONE)
    assert np.all(out[64:] == 0)                                 # +0 bits


# ---------------------------------------------------------------------------
# Block-constant storage
# ---------------------------------------------------------------------------

def test_bits_per_weight_match_the_pages():
    f = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "page_facts.json")))
    no_dq = _facts()["no_dq_constant_bits_per_weight"]["value"]
    assert cv.bits_per_weight(cv.DQ_NONE) == f["bits_per_weight_code"]["value"] + no_dq
    saving = cv.bits_per_weight(cv.DQ_NONE) - cv.bits_per_weight(cv.DQ_U8)
    assert abs(saving - f["dq_saving_bits_per_param"]["value"]) <= \
        f["dq_saving_bits_per_param"]["tolerance"]
    assert cv.bits_per_weight(cv.DQ_CENTERED) > cv.bits_per_weight(cv.DQ_U8)


def test_no_dq_dequant_is_level_times_exact_absmax():
    rng = np.random.default_rng(73)
    w = (rng.standard_normal(64 * 40) * 0.02).astype(np.float32)
    for code in (cv.CODE_NF4, cv.CODE_FP4, cv.CODE_INT4):
        packed, consts, gs, gm = cv.quantize(w, code, cv.DQ_NONE)
        c = np.abs(w.reshape(-1, 64)).max(axis=1)
        assert np.array_equal(consts, c)
        out = cv.dequantize(packed, consts, gs, gm, w.size, code, cv.DQ_NONE)
        codes = oracle.unpack_nibbles(packed, w.size)
        prod = cv.levels(code)[codes].astype(np.float64) * np.repeat(c, 64)
        # one fp32 rounding then one bf16 rounding of the exact product
        vals = oracle.bf16_bits_to_f64(out)
        assert np.all(np.abs(vals - prod) <= np.abs(prod) * (2.0 ** -8 + 2.0 ** -24))


def test_variant_nf4_u8_is_the_nf4_codec():
    rng = np.random.default_rng(74)
    w = (rng.standard_normal(64 * 300 + 17) * 0.02).astype(np.float32)
    p0, q0, d0 = oracle.nf4_quantize(w)
    p1, q1, d1, _ = cv.quantize(w, cv.CODE_NF4, cv.DQ_U8)
    assert np.array_equal(p0, p1) and np.array_equal(q0, q1)
    assert np.array_equal(d0.view(np.uint32), d1.view(np.uint32))
    a = oracle.nf4_dequantize(p0, q0, d0, w.size)
    b = cv.dequantize(p1, q1, d1, np.zeros(0, np.float32), w.size, cv.CODE_NF4, cv.DQ_U8)
    assert np.array_equal(a, b)


def test_pairwise_mean_is_close_to_the_exact_mean():
    rng = np.random.default_rng(75)
    for n in (1, 2, 3, 255, 256):
        c = (rng.random(n) * 0.1).astype(np.float32)
        s = cv.pairwise_sum_f32(c)
        exact = sum(Fraction(float(x)) for x in c)
        # depth-8 pairwise tree: |error| <= 8 u sum|c| with u = 2^-24
        assert abs(Fraction(float(s)) - exact) <= 8 * Fraction(1, 2 ** 24) * exact
        # exact for small integers
        ci = rng.integers(0, 1000, n).astype(np.float32)
        assert float(cv.pairwise_sum_f32(ci)) == float(sum(int(x) for x in ci))


def test_pairwise_sum_pairs_adjacent_values():
    # 1 + 2^-24 + 2^-24 + ... : adjacent pairing keeps the small terms
    # together (2^-23 each pair), a left-to-right sum would drop them all
    x = np.full(256, 2.0 ** -24, np.float32)
    x[0] = 1.0
    s = cv.pairwise_sum_f32(x)
    exact = 1.0 + 255 * 2.0 ** -24
    assert abs(float(s) - exact) <= 2.0 ** -23
    left = np.float32(0)
    for v in x:
        left = np.float32(left + v)
    assert float(left) == 1.0


def test_centered_dq_bounds_and_extremes():
    rng = np.random.default_rng(76)
    c = (np.abs(rng.standard_normal(256 * 3 + 40)) * 0.05 + 0.01).astype(np.float32)
    c[5] = 0.9   # an outlier constant
    q, d, mu = cv.centered_quantize(c)
    assert q.dtype == np.int8 and q.min() >= -127 and q.max() <= 127
    cp = cv.block_constants(q, d, mu, c.size, cv.DQ_CENTERED)
    for g in range(d.size):
        s, e = 256 * g, min(256 * g + 256, c.size)
        exact_mean = sum(Fraction(float(x)) for x in c[s:e]) / (e - s)
        assert abs(Fraction(float(mu[g])) - exact_mean) <= \
            10 * Fraction(1, 2 ** 24) * abs(exact_mean)
        dev = c[s:e].astype(np.float64) - float(mu[g])
        j = int(np.argmax(np.abs(dev)))
        assert abs(int(q[s + j])) == 127            # the extreme maps to +-127
        # decoded constant within half a step (plus fp32 rounding) of c
        err = np.abs(cp[s:e].astype(np.float64) - c[s:e].astype(np.float64))
        slack = 2.0 ** -21 * (np.abs(c[s:e]) + abs(float(mu[g])) + np.abs(dev).max())
        assert np.all(err <= float(d[g]) / 2 * (1 + 2 ** -20) + slack)
    # the mean is added back: constants far from zero decode near themselves
    assert np.all(np.abs(cp - c) < 0.01)


def test_centered_dq_degenerate_groups():
    # all equal -> mean exact, d = 0, q = 0, c' = c exactly
    c = np.full(256 + 1, 0.3, np.float32)
    c[256] = 0.7   # a one-constant tail group: its own mean, d = 0
    q, d, mu = cv.centered_quantize(c)
    assert np.all(q == 0) and np.all(d == 0)
    assert mu[0] == np.float32(0.3) and mu[1] == np.float32(0.7)
    cp = cv.block_constants(q, d, mu, c.size, cv.DQ_CENTERED)
    assert np.array_equal(cp, c)
    # an all-zero group
    q, d, mu = cv.centered_quantize(np.zeros(300, np.float32))
    assert np.all(q == 0) and np.all(d == 0) and np.all(mu == 0)


def test_centered_decode_rounds_twice():
    # c' = fp32(fp32(q d) + mu) with q = 3, d = 1 + 2^-23, mu = -3:
    # q d = 3 + 1.5 * 2^-22 rounds (tie, to even) to 3 + 2^-21, so the sum
    # is 2^-21; a fused multiply-add would give the exact 3 * 2^-23
    q = np.array([3], np.int8)
    d = np.array([1.0 + 2.0 ** -23], np.float32)
    mu = np.array([-3.0], np.float32)
    cp = cv.block_constants(q, d, mu, 1, cv.DQ_CENTERED)
    assert float(cp[0]) == 2.0 ** -21
    assert float(cp[0]) != 3 * 2.0 ** -23


# ---------------------------------------------------------------------------
# The pages' comparison: NF4 against FP4 and INT4
# ---------------------------------------------------------------------------

def test_nf4_has_lower_error_than_fp4_and_int4_on_normal_weights():
    assert _facts()["nf4_beats_fp4_and_int4"]["value"] is True
    rng = np.random.default_rng(77)
    w = (rng.standard_normal(64 * 4096) * 0.02).astype(np.float32)
    mse = {}
    for code in (cv.CODE_NF4, cv.CODE_FP4, cv.CODE_INT4):
        packed, consts, gs, gm = cv.quantize(w, code, cv.DQ_NONE)
        out = oracle.bf16_bits_to_f64(
            cv.dequantize(packed, consts, gs, gm, w.size, code, cv.DQ_NONE))
        mse[code] = float(np.mean((out - w.astype(np.float64)) ** 2))
    assert mse[cv.CODE_NF4] < mse[cv.CODE_FP4]
    assert mse[cv.CODE_NF4] < mse[cv.CODE_INT4]


def test_dq_modes_order_their_constant_error():
    # the constant error of each storage mode is bounded by its step:
    # none 0, centered d/2 (d = max|c - mu|/127), u8 d/2 (d = max c/255)
    rng = np.random.default_rng(78)
    w = (rng.standard_normal(64 * 256 * 4) * 0.02).astype(np.float32)
    c = oracle.block_absmax(w)
    q8, d8 = oracle.double_quantize(c)
    qc, dc, mu = cv.centered_quantize(c)
    e8 = np.abs(cv.block_constants(q8, d8, None, c.size, cv.DQ_U8) - c).max()
    ec = np.abs(cv.block_constants(qc, dc, mu, c.size, cv.DQ_CENTERED) - c).max()
    assert ec <= dc.max() / 2 * 1.001 + 1e-9
    assert e8 <= d8.max() / 2 * 1.001 + 1e-9
    assert ec < e8
