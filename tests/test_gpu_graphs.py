"""The library's calls captured in HIP graphs (as the benchmark replays
them): each graph is replayed several times with eager work and
synchronisations in between, and every replay must reproduce the eager
result bit for bit (all kernels are deterministic).  Calls go through the
C ABI."""

import numpy as np
import pytest
import torch

from bit_nf4_quantized_14_amd import capi
from bit_nf4_quantized_14_amd import workloads as wl

from gpu_util import bf16_dev, f32_dev

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def _eager_noise():
    # unrelated eager work between replays
    a = torch.randn(1 << 20, device="cuda")
    (a * 2.0 + 1.0).sum().item()
    torch.cuda.synchronize()


def _same(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def _check_replays(fn, outs):
    """fn() writes the tensors in outs; compare graph replays with eager."""
    fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    for o in outs:
        o.zero_()
    g = _capture(fn)
    for rep in range(REPLAYS):
        for o in outs:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, ref)):
            assert _same(o, r), f"replay {rep}, output {i}"
        _eager_noise()


def _problem(m, n, k, r):
    wk = wl.workload("tiny")
    w = wl.weight(wk, 0, rows=n, cols=k)
    x = bf16_dev(wl.activations(wk, 0, m=m, k=k))
    a = bf16_dev(wl.lora_a(wk, 0, r=r, k=k))
    b = bf16_dev(wl.lora_b(wk, 0, r=r, n=n))
    dy = bf16_dev(wl.grad_out(wk, 0, m=m, n=n))
    t = capi.nf4_quantize(f32_dev(w).view(n, k))
    return t, x, a, b, dy


def test_graph_dequantize_batch():
    wk = wl.workload("tiny")
    ts = [capi.nf4_quantize(f32_dev(wl.weight(wk, 0, rows=n, cols=k)).view(n, k))
          for n, k in ((256, 512), (300, 1000), (64, 4160))]
    outs = [torch.empty((t.rows, t.cols), dtype=torch.bfloat16, device="cuda") for t in ts]
    _check_replays(lambda: capi.nf4_dequantize_batch(ts, outs), outs)


@pytest.mark.parametrize("m", [8, 300])
def test_graph_linear_fwd_bwd(m):
    n, k, r = 264, 512, 16
    t, x, a, b, dy = _problem(m, n, k, r)
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    ts = torch.empty((m, r), dtype=torch.float32, device="cuda")
    dx = torch.empty((m, k), dtype=torch.bfloat16, device="cuda")
    da = torch.empty((r, k), dtype=torch.float32, device="cuda")
    db = torch.empty((n, r), dtype=torch.float32, device="cuda")
    wsf = torch.empty(capi.qlora_workspace_bytes(m, n, k, r, capi.QN_FWD),
                      dtype=torch.uint8, device="cuda")
    wsb = torch.empty(capi.qlora_workspace_bytes(m, n, k, r, capi.QN_BWD),
                      dtype=torch.uint8, device="cuda")

    def step():
        capi.qlora_linear_fwd(x, t, a, b, r, 32.0, y=y, t_save=ts, ws=wsf)
        capi.qlora_linear_bwd(dy, x, t, a, b, r, 32.0, ts, dx=dx,
                              dx_dtype=capi.QN_BF16, dA=da, dB=db, ws=wsb)
    _check_replays(step, [y, ts, dx, da, db])


def test_graph_linear_with_dropout():
    m, n, k, r = 130, 136, 320, 8
    t, x, a, b, dy = _problem(m, n, k, r)
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    ts = torch.empty((m, r), dtype=torch.float32, device="cuda")
    dx = torch.empty((m, k), dtype=torch.float32, device="cuda")
    da = torch.empty((r, k), dtype=torch.float32, device="cuda")
    db = torch.empty((n, r), dtype=torch.float32, device="cuda")
    wsf = torch.empty(capi.qlora_workspace_bytes(m, n, k, r, capi.QN_FWD_DROPOUT),
                      dtype=torch.uint8, device="cuda")
    wsb = torch.empty(capi.qlora_workspace_bytes(m, n, k, r, capi.QN_BWD),
                      dtype=torch.uint8, device="cuda")

    def step():
        capi.qlora_linear_fwd_dropout(x, t, a, b, r, 16.0, 0.1, 99, y=y,
                                      t_save=ts, ws=wsf)
        capi.qlora_linear_bwd_dropout(dy, x, t, a, b, r, 16.0, ts, 0.1, 99,
                                      dx=dx, dA=da, dB=db, ws=wsb)
    _check_replays(step, [y, ts, dx, da, db])


def test_graph_merge():
    n, k, r = 200, 1024, 16
    t, _, a, b, _ = _problem(8, n, k, r)
    out = torch.empty((n, k), dtype=torch.bfloat16, device="cuda")
    _check_replays(lambda: capi.nf4_merge(t, a, b, r, 32.0, out), [out])


def test_graph_adamw8_steps_match_eager_steps():
    """The step mutates its state, so replay i is compared with eager step
    i run on a copy."""
    n = 256 * 40 + 17
    rng = np.random.default_rng(808)
    p0 = torch.from_numpy((rng.standard_normal(n) * 0.01).astype(np.float32)).to(torch.bfloat16)
    g = torch.from_numpy((rng.standard_normal(n) * 1e-3).astype(np.float32)).cuda()
    pe, pg = p0.cuda(), p0.cuda()
    se, sg = capi.AdamW8State.zeros(n), capi.AdamW8State.zeros(n)
    # one eager step on both so the state is non-zero, then capture step 2
    capi.qn_adamw8_step(pe, g, se, 1, weight_decay=0.01)
    capi.qn_adamw8_step(pg, g, sg, 1, weight_decay=0.01)
    torch.cuda.synchronize()
    graph = _capture(lambda: capi.qn_adamw8_step(pg, g, sg, 2, weight_decay=0.01))
    # capturing does not run the step: pg/sg are still after step 1
    for rep in range(REPLAYS):
        graph.replay()
        capi.qn_adamw8_step(pe, g, se, 2, weight_decay=0.01)
        torch.cuda.synchronize()
        assert _same(pg, pe), f"replay {rep}"
        for u, v in ((sg.m_codes, se.m_codes), (sg.m_scale, se.m_scale),
                     (sg.r_codes, se.r_codes), (sg.r_scale, se.r_scale)):
            assert _same(u, v), f"replay {rep}"
        _eager_noise()
