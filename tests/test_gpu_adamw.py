"""GPU parity of the 8-bit AdamW step (resident and paged) against the CPU
oracle in oracle/adamw8.py.

The new bf16 parameters, the E4M3 state codes and the fp32 state scales
are all decided by fp32 arithmetic that both sides perform in the same
order, so every comparison is bit-exact.  Calls go through the C ABI.
"""

import numpy as np
import pytest
import torch

from oracle import adamw8 as aw
from bit_nf4_quantized_14_amd import capi

from gpu_util import DEV, bits_host

pytestmark = pytest.mark.gpu

HP = dict(lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01,
          grad_scale=0.7)


def _oracle_hp():
    return aw.HParams(lr=HP["lr"], beta1=HP["beta1"], beta2=HP["beta2"],
                      eps=HP["eps"], weight_decay=HP["weight_decay"],
                      grad_scale=HP["grad_scale"])


def _grads(rng, n, step):
    """Gradients whose magnitude varies by block (a few blocks tiny, one
    block zero, an outlier), like adapter gradients of different layers."""
    g = rng.standard_normal(n).astype(np.float32)
    nb = -(-n // 256)
    scale = np.exp(rng.uniform(-12, 0, nb)).astype(np.float32)
    g *= np.repeat(scale, 256)[:n]
    if nb > 2:
        g[256:512] = 0.0
    g[rng.integers(0, n)] *= 100.0
    return g


def _host_state(st: capi.AdamW8State) -> aw.State8:
    return aw.State8(st.m_codes.cpu().numpy(), st.m_scale.cpu().numpy(),
                     st.r_codes.cpu().numpy(), st.r_scale.cpu().numpy())


def _assert_state_equal(a: aw.State8, b: aw.State8):
    assert np.array_equal(a.m_codes, b.m_codes)
    assert np.array_equal(a.r_codes, b.r_codes)
    assert np.array_equal(a.m_scales.view(np.uint32), b.m_scales.view(np.uint32))
    assert np.array_equal(a.r_scales.view(np.uint32), b.r_scales.view(np.uint32))


@pytest.mark.parametrize("n", [1, 255, 256, 1000, 256 * 37 + 11, 65536])
def test_adamw8_matches_oracle_over_steps(n):
    print(f"[adamw] n={n}", flush=True)
    rng = np.random.default_rng(500 + n)
    p_bits = rng.standard_normal(n).astype(np.float32) * 0.01
    p_bits = torch.from_numpy(p_bits).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    p = torch.from_numpy(p_bits.view(np.int16).copy()).to(DEV).view(torch.bfloat16)
    st = capi.AdamW8State.zeros(n)
    ref_p, ref_st = p_bits.copy(), aw.State8.zeros(n)
    for t in range(1, 5):
        g = _grads(rng, n, t)
        capi.qn_adamw8_step(p, torch.from_numpy(g).to(DEV), st, t, **HP)
        torch.cuda.synchronize()
        ref_p, ref_st = aw.adamw8_step(ref_p, g, ref_st, _oracle_hp(), t)
        assert np.array_equal(bits_host(p), ref_p), f"step {t}"
        _assert_state_equal(_host_state(st), ref_st)


def test_adamw8_large_sampled_blocks():
    """16M parameters on the GPU (two steps); 64 sampled state blocks
    (independent 256-element units) checked against the oracle."""
    n = 1 << 24
    rng = np.random.default_rng(510)
    p0 = torch.from_numpy((rng.standard_normal(n) * 0.01).astype(np.float32)).to(torch.bfloat16)
    p = p0.to(DEV)
    st = capi.AdamW8State.zeros(n)
    g1, g2 = _grads(rng, n, 1), _grads(rng, n, 2)
    capi.qn_adamw8_step(p, torch.from_numpy(g1).to(DEV), st, 1, **HP)
    torch.cuda.synchronize()
    mid_p, mid_st = bits_host(p), _host_state(st)
    capi.qn_adamw8_step(p, torch.from_numpy(g2).to(DEV), st, 2, **HP)
    torch.cuda.synchronize()
    out_p, out_st = bits_host(p), _host_state(st)
    blocks = sorted(set(rng.integers(0, n // 256, 62).tolist()) | {0, n // 256 - 1})
    for b in blocks:
        s = slice(256 * b, 256 * b + 256)
        sub = aw.State8(mid_st.m_codes[s], mid_st.m_scales[b:b + 1],
                        mid_st.r_codes[s], mid_st.r_scales[b:b + 1])
        rp, rst = aw.adamw8_step(mid_p[s], g2[s], sub, _oracle_hp(), 2)
        assert np.array_equal(out_p[s], rp)
        _assert_state_equal(aw.State8(out_st.m_codes[s], out_st.m_scales[b:b + 1],
                                      out_st.r_codes[s], out_st.r_scales[b:b + 1]), rst)


@pytest.mark.parametrize("streams", ["separate", "one"])
def test_adamw8_paged_equals_resident(streams):
    n, chunk = 3 * 8192 + 1000, 8192           # four pages, the last short
    rng = np.random.default_rng(520)
    p0 = torch.from_numpy((rng.standard_normal(n) * 0.01).astype(np.float32)).to(torch.bfloat16)
    p_res, p_pag = p0.to(DEV), p0.to(DEV)
    st_res = capi.AdamW8State.zeros(n)
    st_host = capi.AdamW8State.zeros(n, device="cpu", pin_memory=True)
    staging = torch.empty(capi.qn_adamw8_staging_bytes(chunk), dtype=torch.uint8, device=DEV)
    h2d = torch.cuda.Stream() if streams == "separate" else None
    d2h = torch.cuda.Stream() if streams == "separate" else None
    for t in range(1, 4):
        g = torch.from_numpy(_grads(rng, n, t)).to(DEV)
        capi.qn_adamw8_step(p_res, g, st_res, t, **HP)
        capi.qn_adamw8_paged_step(p_pag, g, st_host, staging, chunk, t,
                                  h2d_stream=h2d, d2h_stream=d2h, **HP)
        torch.cuda.synchronize()
        assert torch.equal(p_res.view(torch.int16), p_pag.view(torch.int16)), f"step {t}"
        _assert_state_equal(_host_state(st_res), _host_state(st_host))


def test_adamw8_e4m3_rounding_at_ties():
    """With beta1 = beta2 = 0 and grad_scale 1 the stored codes are those of
    g / s and |g| / s (c1 = 1, sqrt(g^2) = |g| for these short mantissas).
    Each block's largest |g| is 448 * 2^-10, so s = 2^-10 exactly and every
    E4M3 value and every midpoint between neighbours (ties, subnormal ones
    included) reaches the encoder exactly."""
    vals = np.unique(aw.e4m3_value(np.arange(0, 0x7F, dtype=np.uint8)))
    mids = (vals[:-1] + vals[1:]) / 2
    body = np.concatenate([vals, mids, -vals, -mids, [2.0 ** -11, -2.0 ** -11]])
    n_blk = -(-body.size // 255)
    g = np.zeros(256 * n_blk, np.float64)
    for b in range(n_blk):
        part = body[255 * b:255 * (b + 1)]
        g[256 * b] = 448.0
        g[256 * b + 1:256 * b + 1 + part.size] = part
    g = (g * 2.0 ** -10).astype(np.float32)
    assert np.all(g.astype(np.float64) == g)           # exact in fp32
    n = g.size
    hp = dict(lr=1e-3, beta1=0.0, beta2=0.0, eps=1e-8, weight_decay=0.0,
              grad_scale=1.0)
    p = torch.zeros(n, dtype=torch.bfloat16, device=DEV)
    st = capi.AdamW8State.zeros(n)
    capi.qn_adamw8_step(p, torch.from_numpy(g).to(DEV), st, 1, **hp)
    torch.cuda.synchronize()
    ref_p, ref_st = aw.adamw8_step(np.zeros(n, np.uint16), g, aw.State8.zeros(n),
                                   aw.HParams(**hp), 1)
    got = _host_state(st)
    assert np.all(ref_st.m_scales == np.float32(2.0 ** -10))
    # the oracle's codes are the nearest-even E4M3 codes of body (pinned
    # against torch on the CPU); the GPU must give the same bytes
    assert np.array_equal(got.m_codes, ref_st.m_codes)
    assert np.array_equal(got.r_codes, ref_st.r_codes)
    _assert_state_equal(got, ref_st)
    assert np.array_equal(bits_host(p), ref_p)


def test_adamw8_benchmark_size_sampled_blocks():
    """The benchmarked buffer: r = 16 adapters of all 7 projections of 80
    layers of a 70B-class model, 207,093,760 parameters; two steps, 64
    sampled state blocks of the second checked against the oracle."""
    n = 80 * 16 * (2 * 8192 + 2 * (1024 + 8192) + 2 * 8192 + 3 * (28672 + 8192))
    assert n == 207093760
    rng = np.random.default_rng(530)
    p0 = torch.from_numpy((rng.standard_normal(n, dtype=np.float32) * 0.01)).to(torch.bfloat16)
    p = p0.to(DEV)
    del p0
    st = capi.AdamW8State.zeros(n)
    g1 = _grads(rng, n, 1)
    capi.qn_adamw8_step(p, torch.from_numpy(g1).to(DEV), st, 1, **HP)
    del g1
    torch.cuda.synchronize()
    mid_p, mid_st = bits_host(p), _host_state(st)
    g2 = _grads(rng, n, 2)
    capi.qn_adamw8_step(p, torch.from_numpy(g2).to(DEV), st, 2, **HP)
    torch.cuda.synchronize()
    out_p, out_st = bits_host(p), _host_state(st)
    nb = -(-n // 256)
    blocks = sorted(set(rng.integers(0, nb, 62).tolist()) | {0, nb - 1})
    for b in blocks:
        s = slice(256 * b, min(256 * b + 256, n))
        sub = aw.State8(mid_st.m_codes[s], mid_st.m_scales[b:b + 1],
                        mid_st.r_codes[s], mid_st.r_scales[b:b + 1])
        rp, rst = aw.adamw8_step(mid_p[s], g2[s], sub, _oracle_hp(), 2)
        assert np.array_equal(out_p[s], rp)
        _assert_state_equal(aw.State8(out_st.m_codes[s], out_st.m_scales[b:b + 1],
                                      out_st.r_codes[s], out_st.r_scales[b:b + 1]), rst)
