"""Pins for the oracle's LoRA dropout (oracle/dropout.py), on the CPU.

Philox4x32-10 against its published known-answer vectors; the mask's keep
rate and independence against the binomial law; inverted dropout's
unbiasedness; p = 0 reducing to the layer without dropout; and the
backward against torch autograd of the same forward.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import dropout as dr

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox_kat.json")


def _facts():
    with open(GOLDEN) as f:
        return json.load(f)


def test_philox_known_answers():
    for v in _facts()["vectors"]:
        ctr = [int(c, 16) for c in v["ctr"]]
        key = [int(c, 16) for c in v["key"]]
        out = dr.philox4x32_10(ctr, key)
        assert [f"{int(o):08x}" for o in out] == v["out"]


def test_philox_vectorised_equals_scalar_calls():
    rng = np.random.default_rng(601)
    ctr = [rng.integers(0, 2 ** 32, 50, dtype=np.uint64) for _ in range(4)]
    key = (0x12345678, 0x9ABCDEF0)
    vec = dr.philox4x32_10(ctr, key)
    for i in range(50):
        one = dr.philox4x32_10([int(c[i]) for c in ctr], key)
        assert [int(o) for o in one] == [int(v[i]) for v in vec]


@pytest.mark.parametrize("p", _facts()["lora_dropout_values"]["values"] + [0.5])
def test_keep_rate_is_binomial(p):
    M, K = 512, 1024
    keep = dr.keep_mask(M, K, p, seed=1234567890123)
    n = M * K
    kept = int(keep.sum())
    mean, sd = n * (1 - p), math.sqrt(n * p * (1 - p))
    assert abs(kept - mean) < 5 * sd
    # every row and column of a large mask is near the rate as well
    rows = keep.mean(axis=1)
    assert np.all(np.abs(rows - (1 - p)) < 6 * math.sqrt(p * (1 - p) / K))


def test_mask_has_no_neighbour_correlation():
    p = 0.5
    keep = dr.keep_mask(1024, 1024, p, seed=42).astype(np.float64) - 0.5
    n = keep.size
    for a, b in ((keep[1:], keep[:-1]), (keep[:, 1:], keep[:, :-1]),
                 (keep[4:], keep[:-4])):
        corr = float(np.mean(a * b)) / 0.25
        assert abs(corr) < 5 / math.sqrt(n)


def test_seeds_give_different_masks_and_same_seed_the_same():
    a = dr.keep_mask(64, 256, 0.1, seed=1)
    b = dr.keep_mask(64, 256, 0.1, seed=2)
    c = dr.keep_mask(64, 256, 0.1, seed=1)
    assert np.array_equal(a, c) and not np.array_equal(a, b)
    # the key uses both halves of a 64-bit seed
    d = dr.keep_mask(64, 256, 0.1, seed=1 + (1 << 32))
    assert not np.array_equal(a, d)


def test_inverted_dropout_is_unbiased():
    rng = np.random.default_rng(602)
    x = oracle.bf16_rne_bits(rng.standard_normal((256, 512)).astype(np.float32))
    xv = oracle.bf16_bits_to_f64(x)
    acc = np.zeros_like(xv)
    trials = 64
    for s in range(trials):
        acc += oracle.bf16_bits_to_f64(dr.dropout_x_bits(x, 0.1, seed=1000 + s))
    # E[X_d] = X up to the bf16 rounding of x / 0.9 (relative 2^-9)
    err = np.abs(acc / trials - xv)
    sd = np.abs(xv) * math.sqrt(0.1 / 0.9 / trials)
    assert np.mean(err <= 5 * sd + np.abs(xv) * 2.0 ** -8) > 0.999


def test_p_zero_is_the_layer_without_dropout():
    rng = np.random.default_rng(603)
    M, N, K, r = 24, 40, 128, 8
    bits = lambda a: oracle.bf16_rne_bits(a.astype(np.float32))
    x, w = bits(rng.standard_normal((M, K))), bits(rng.standard_normal((N, K)) * 0.02)
    a, b = bits(rng.standard_normal((r, K)) * 0.1), bits(rng.standard_normal((N, r)) * 0.1)
    dy = bits(rng.standard_normal((M, N)))
    assert np.array_equal(dr.dropout_x_bits(x, 0.0, 7), x)
    y0, t0 = oracle.qlora_forward(x, w, a, b, 16.0, r)
    y1, t1 = dr.qlora_forward_dropout(x, w, a, b, 16.0, r, 0.0, 7)
    assert np.array_equal(y0, y1) and np.array_equal(t0, t1)
    g0 = oracle.qlora_backward(dy, x, w, a, b, 16.0, r, t0)
    g1 = dr.qlora_backward_dropout(dy, x, w, a, b, 16.0, r, 0.0, 7, t1)
    for u, v in zip(g0, g1):
        assert np.allclose(u, v, rtol=0, atol=1e-12)


def test_backward_matches_autograd_of_the_dropout_forward():
    rng = np.random.default_rng(604)
    M, N, K, r, p, seed, alpha = 20, 24, 64, 4, 0.3, 99, 8.0
    bits = lambda a: oracle.bf16_rne_bits(a.astype(np.float32))
    x, w = bits(rng.standard_normal((M, K))), bits(rng.standard_normal((N, K)))
    a, b = bits(rng.standard_normal((r, K))), bits(rng.standard_normal((N, r)))
    dy = bits(rng.standard_normal((M, N)))
    f = oracle.bf16_bits_to_f64
    keep = dr.keep_mask(M, K, p, seed)
    ms = torch.from_numpy(np.where(keep, float(dr.keep_scale(p)), 0.0))
    X = torch.from_numpy(f(x)).requires_grad_()
    A = torch.from_numpy(f(a)).requires_grad_()
    B = torch.from_numpy(f(b)).requires_grad_()
    W = torch.from_numpy(f(w))
    s = alpha / r
    # the same forward with the rounding of X_d left out (straight through)
    Y = X @ W.T + s * ((X * ms) @ A.T) @ B.T
    Y.backward(torch.from_numpy(f(dy)))
    _, t = dr.qlora_forward_dropout(x, w, a, b, alpha, r, p, seed)
    dx, da, db = dr.qlora_backward_dropout(dy, x, w, a, b, alpha, r, p, seed, t)
    assert np.allclose(dx, X.grad.numpy(), rtol=1e-12, atol=1e-10)
    # dA and dB use X_d with its bf16 rounding: within 2^-8 relative of the
    # unrounded autograd values
    assert np.max(np.abs(da - A.grad.numpy())) <= 2 ** -7 * np.max(np.abs(A.grad.numpy()))
    assert np.max(np.abs(db - B.grad.numpy())) <= 2 ** -7 * np.max(np.abs(B.grad.numpy()))


def test_dropped_elements_are_zero_and_kept_are_scaled():
    rng = np.random.default_rng(605)
    x = oracle.bf16_rne_bits(rng.standard_normal((33, 70)).astype(np.float32))
    xd = dr.dropout_x_bits(x, 0.25, seed=5)
    keep = dr.keep_mask(33, 70, 0.25, seed=5)
    assert np.all(xd[~keep] == 0)
    ratio = oracle.bf16_bits_to_f64(xd[keep]) / oracle.bf16_bits_to_f64(x[keep])
    ok = np.isfinite(ratio)
    assert np.all(np.abs(ratio[ok] - 1 / 0.75) <= (1 / 0.75) * 2.0 ** -8)
