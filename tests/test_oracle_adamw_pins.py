"""Pins for the oracle's 8-bit AdamW step (oracle/adamw8.py), on the CPU.

E4M3 encoding and decoding against torch's float8_e4m3fn conversion and the
OCP format facts in tests/golden/adamw8_facts.json; the AdamW algebra
against torch.optim.AdamW; closed forms of the first step; bounds of the
blockwise state codec; and the 8-bit optimizer tracking the 32-bit one.
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import adamw8 as aw

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "adamw8_facts.json")


def _facts():
    with open(GOLDEN) as f:
        return json.load(f)


def test_e4m3_format_facts():
    e = _facts()["e4m3"]
    for val, code in ((e["max_finite"], e["max_finite_code"]),
                      (e["min_normal"], e["min_normal_code"]),
                      (e["min_subnormal"], e["min_subnormal_code"]),
                      (1.0, e["one_code"])):
        assert aw.e4m3_encode(np.float32(val)) == code
        assert aw.e4m3_value(np.uint8(code)) == val
        assert aw.e4m3_encode(np.float32(-val)) == code | 0x80


def test_e4m3_decode_matches_torch():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(aw.e4m3_value(codes), ref)


def test_e4m3_encode_matches_torch():
    rng = np.random.default_rng(81)
    parts = [rng.uniform(-448, 448, 4000), rng.standard_normal(4000),
             rng.standard_normal(4000) * 2.0 ** -7,     # subnormal range
             rng.standard_normal(4000) * 2.0 ** -11]    # below the smallest
    # every value and every midpoint between neighbouring codes (ties)
    vals = np.unique(aw.e4m3_value(np.arange(0, 0x7F, dtype=np.uint8)))
    mids = (vals[:-1] + vals[1:]) / 2
    parts += [vals, -vals, mids, -mids]
    x = np.concatenate(parts).astype(np.float32)
    got = aw.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ref = np.where(ref == 0x80, 0, ref)          # this codec stores no -0
    assert np.array_equal(got, ref)


def test_e4m3_clamps_above_448():
    x = np.array([448.0, 450.0, 463.9, 1e4, -1e4], np.float32)
    assert list(aw.e4m3_encode(x)) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE]


def test_state_block_maps_its_absmax_to_448():
    rng = np.random.default_rng(82)
    x = (rng.standard_normal(256 * 5 + 17) * 1e-3).astype(np.float32)
    codes, scales = aw.quantize_state(x)
    for b in range(scales.size):
        s, e = 256 * b, min(256 * b + 256, x.size)
        j = s + int(np.argmax(np.abs(x[s:e])))
        assert codes[j] & 0x7F == 0x7E
        assert scales[b] == np.float32(np.abs(x[s:e]).max()) / np.float32(448)


def test_state_roundtrip_within_half_an_e4m3_step():
    rng = np.random.default_rng(83)
    x = (rng.standard_normal(256 * 40) * np.exp(rng.uniform(-8, 0, 256 * 40))).astype(np.float32)
    x[:256] = 0
    codes, scales = aw.quantize_state(x)
    y = aw.dequantize_state(codes, scales).astype(np.float64)
    sc = np.repeat(scales, 256)[: x.size].astype(np.float64)
    # relative step 2^-3 for normals (half: 2^-4), absolute 2^-9 * scale
    # below the normal range (half: 2^-10 * scale), plus fp32 roundings
    bound = np.maximum(np.abs(x) * 2.0 ** -4, sc * 2.0 ** -10) * (1 + 2 ** -20) \
        + np.abs(x) * 2.0 ** -22
    assert np.all(np.abs(y - x) <= bound)
    assert np.all(y[:256] == 0) and np.all(codes[:256] == 0) and scales[0] == 0


def test_adamw_f32_matches_torch_adamw():
    rng = np.random.default_rng(84)
    n = 1000
    p0 = rng.standard_normal(n).astype(np.float32)
    hp = aw.HParams(lr=1e-2, beta1=0.9, beta2=0.99, eps=1e-6, weight_decay=0.1)
    tp = torch.nn.Parameter(torch.from_numpy(p0.astype(np.float64)))
    opt = torch.optim.AdamW([tp], lr=hp.lr, betas=(hp.beta1, hp.beta2),
                            eps=hp.eps, weight_decay=hp.weight_decay)
    p, m, v = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    for t in range(1, 8):
        g = rng.standard_normal(n).astype(np.float32)
        tp.grad = torch.from_numpy(g.astype(np.float64))
        opt.step()
        p, m, v = aw.adamw_step_f32(p, g, m, v, hp, t)
        ref = tp.detach().numpy()
        assert np.max(np.abs(p - ref)) <= 1e-5 * np.max(np.abs(ref))


def test_first_step_moves_each_weight_by_lr_sign_g():
    # zero state: m = (1-b1) g, v = (1-b2) g^2, so m/(1-b1) / sqrt(v/(1-b2))
    # = sign(g); the first step is p - lr sign(g) (for |g| >> eps)
    rng = np.random.default_rng(85)
    n = 300
    p = oracle.bf16_rne_bits(rng.standard_normal(n).astype(np.float32))
    g = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    hp = aw.HParams(lr=2e-4)
    p1, st = aw.adamw8_step(p, g, aw.State8.zeros(n), hp, 1)
    p0 = oracle.bf16_bits_to_f64(p)
    want = p0 - hp.lr * np.sign(g)
    got = oracle.bf16_bits_to_f64(p1)
    ulp = np.abs(want) * 2.0 ** -8
    assert np.all(np.abs(got - want) <= ulp)
    # and the stored state decodes to those moments
    m = aw.dequantize_state(st.m_codes, st.m_scales)
    assert np.allclose(m, 0.1 * g, rtol=2 ** -4)


def test_weight_decay_is_decoupled():
    # zero gradient, zero state: only the decay acts, p -> p (1 - lr wd)
    n = 256
    p = oracle.bf16_rne_bits(np.linspace(-2, 2, n).astype(np.float32))
    hp = aw.HParams(lr=0.05, weight_decay=0.5)
    p1, _ = aw.adamw8_step(p, np.zeros(n, np.float32), aw.State8.zeros(n), hp, 1)
    want = oracle.bf16_rne_bits((oracle.bf16_bits_to_f64(p) * np.float32(1 - 0.025)).astype(np.float32))
    assert np.array_equal(p1, want)


def test_sqrt_domain_keeps_small_second_moments():
    # one large gradient in a block: second moments down to ~1e-10 of the
    # largest stay nonzero in the square-root domain
    g = np.full(256, 1e-5, np.float32)
    g[0] = 1.0
    _, st = aw.adamw8_step(np.zeros(256, np.uint16), g, aw.State8.zeros(256),
                           aw.HParams(), 1)
    r = aw.dequantize_state(st.r_codes, st.r_scales)
    assert np.all(r[1:] > 0)


def test_adamw8_tracks_adamw32_on_a_quadratic():
    # f(p) = 1/2 sum a_i (p_i - c_i)^2; 200 steps of both optimizers
    rng = np.random.default_rng(86)
    n = 2048
    a = np.exp(rng.uniform(-3, 1, n)).astype(np.float32)
    c = rng.standard_normal(n).astype(np.float32)
    hp = aw.HParams(lr=1e-2, weight_decay=0.0)
    pb = oracle.bf16_rne_bits(np.zeros(n, np.float32))
    st = aw.State8.zeros(n)
    p32, m, v = np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.float32)
    f0 = 0.5 * np.sum(a * c.astype(np.float64) ** 2)
    for t in range(1, 201):
        p8 = oracle.bf16_bits_to_f64(pb).astype(np.float32)
        pb, st = aw.adamw8_step(pb, (a * (p8 - c)).astype(np.float32), st, hp, t)
        p32, m, v = aw.adamw_step_f32(p32, (a * (p32 - c)).astype(np.float32), m, v, hp, t)
    p8 = oracle.bf16_bits_to_f64(pb)
    f8 = 0.5 * np.sum(a * (p8 - c) ** 2)
    f32 = 0.5 * np.sum(a * (p32.astype(np.float64) - c) ** 2)
    assert f8 < 0.05 * f0 and f32 < 0.05 * f0
    assert abs(f8 - f32) < 0.3 * f32
    # the bf16 parameters and 8-bit moments stay within a few percent of
    # the 32-bit trajectory (measured 6.7%)
    rel = np.linalg.norm(p8 - p32) / np.linalg.norm(p32)
    assert rel < 0.15
