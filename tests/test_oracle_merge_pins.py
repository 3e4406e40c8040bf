"""Pins of the oracle's dequantize-and-merge (CPU): the single float64 ->
bf16 rounding against exact rational arithmetic and a brute-force search
over bf16 neighbours, hand-made tie cases, and the reductions a merge must
satisfy (B = 0 leaves the dequantized base unchanged; one rank reproduces a
hand-computed outer product)."""

from fractions import Fraction

import numpy as np

import oracle


def _bf16_value(bits: int) -> Fraction:
    """Exact rational value of a finite bf16 bit pattern."""
    f32 = np.array([bits << 16], dtype=np.uint32).view(np.float32)[0]
    return Fraction(float(f32))


def _nearest_bf16_bruteforce(x: Fraction) -> int:
    """bf16 bits nearest to x, ties to the even pattern, by scanning every
    finite bf16 value of x's sign (the candidates are checked exactly)."""
    best, best_d = None, None
    signs = [0x0000] if x > 0 else ([0x8000] if x < 0 else [0x0000])
    for sign in signs:
        for mag in range(0x7F80):              # all finite magnitudes
            bits = sign | mag
            d = abs(_bf16_value(bits) - x)
            if best is None or d < best_d or (d == best_d and bits % 2 == 0):
                best, best_d = bits, d
    return best


def test_rne_from_f64_matches_bruteforce_on_samples():
    rng = np.random.default_rng(11)
    vals = np.concatenate([
        rng.standard_normal(12) * 0.02,
        rng.standard_normal(6) * 3.0,
        np.ldexp(rng.random(4) + 0.5, rng.integers(-130, -120, 4)),   # near subnormal
    ])
    got = oracle.bf16_rne_from_f64(vals)
    for v, g in zip(vals, got):
        assert int(g) == _nearest_bf16_bruteforce(Fraction(float(v))), v


def test_rne_from_f64_ties_and_near_ties():
    one = 1.0
    cases = {
        one: 0x3F80,
        one + 2.0 ** -8: 0x3F80,                     # tie -> even (1.0)
        one + 2.0 ** -7 + 2.0 ** -8: 0x3F82,         # tie -> even (odd below)
        one + 2.0 ** -8 + 2.0 ** -40: 0x3F81,        # just past the tie
        one + 2.0 ** -8 - 2.0 ** -40: 0x3F80,        # just before the tie
        -(one + 2.0 ** -7 + 2.0 ** -8): 0xBF82,
        2.0 ** -134: 0x0000,                         # half of the least subnormal
        1.5 * 2.0 ** -133: 0x0002,
    }
    v = np.array(list(cases), dtype=np.float64)
    assert [int(b) for b in oracle.bf16_rne_from_f64(v)] == list(cases.values())


def test_rne_from_f64_agrees_with_fp32_path_on_fp32_values():
    # a value that is exactly an fp32 number is rounded once either way
    rng = np.random.default_rng(3)
    f = (rng.standard_normal(4096) * 0.1).astype(np.float32)
    assert np.array_equal(oracle.bf16_rne_from_f64(f.astype(np.float64)),
                          oracle.bf16_rne_bits(f))


def _bits(a):
    return oracle.bf16_rne_bits(np.asarray(a, dtype=np.float32))


def test_merge_zero_update_is_the_dequantized_base():
    rng = np.random.default_rng(5)
    w = _bits(rng.standard_normal((8, 64)) * 0.02)
    a = _bits(rng.standard_normal((3, 64)))
    b = np.zeros((8, 3), dtype=np.uint16)
    merged, v = oracle.merge_f64(w, a, b, 2.0)
    assert np.array_equal(merged, w)


def test_merge_rank_one_by_hand():
    # W' = [[1, 1.25], [-2, 0]], B = [[0.5], [0.25]], A = [[0.25, -1]], s = 2
    w = _bits([[1.0, 1.25], [-2.0, 0.0]])
    b = _bits([[0.5], [0.25]])
    a = _bits([[0.25, -1.0]])
    merged, v = oracle.merge_f64(w, a, b, 2.0)
    exp = np.array([[1.25, 0.25], [-1.875, -0.5]])
    assert np.array_equal(v, exp)
    assert np.array_equal(merged, _bits(exp))
    # B A = 2^-9: s = 1 stays below half an ulp of 1 (2^-8); s = 2 lands on
    # the midpoints exactly and rounds to the even neighbour
    w = _bits([[1.0, 1.0 + 2.0 ** -7]])
    b = _bits([[2.0 ** -5]])
    a = _bits([[2.0 ** -4, 2.0 ** -4]])
    merged, v = oracle.merge_f64(w, a, b, 1.0)       # adds 2^-9 each
    assert int(merged[0, 0]) == 0x3F80 and int(merged[0, 1]) == 0x3F81
    merged, v = oracle.merge_f64(w, a, b, 2.0)       # adds 2^-8 each: ties
    assert int(merged[0, 0]) == 0x3F80 and int(merged[0, 1]) == 0x3F82


def test_merge_matches_exact_rationals_on_tiny_input():
    rng = np.random.default_rng(9)
    n, k, r, s = 3, 5, 4, 0.75
    w = _bits(rng.standard_normal((n, k)) * 0.5)
    a = _bits(rng.standard_normal((r, k)))
    b = _bits(rng.standard_normal((n, r)) * 0.1)
    merged, _ = oracle.merge_f64(w, a, b, s)
    for i in range(n):
        for j in range(k):
            x = _bf16_value(int(w[i, j])) + Fraction(s) * sum(
                _bf16_value(int(b[i, t])) * _bf16_value(int(a[t, j])) for t in range(r))
            assert int(merged[i, j]) == _nearest_bf16_bruteforce(x), (i, j)
