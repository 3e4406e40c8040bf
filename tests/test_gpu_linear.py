"""GPU parity of the fused QLoRA linear forward/backward against the oracle.

Gate: max|gpu - ref| / max|ref| <= 2e-3 per output tensor for fp32 outputs
(Y, T, dX, dA, dB), and 2^-8 + 2e-3 where Y/dX are emitted in bf16.  The
oracle runs in float64 on the exact bf16 inputs and on the oracle's own
dequantized weight.  Calls go through the C ABI.
"""

import numpy as np
import pytest
import torch

import oracle
from bit_nf4_quantized_14_amd import capi
from bit_nf4_quantized_14_amd import workloads as wl

from gpu_util import (TOL, TOL_BF16, bf16_dev, f64_host, nf4_host,
                      quantize_dev, rel_err)

pytestmark = pytest.mark.gpu


def _inputs(wk, proj, m=None, n=None, k=None, r=None):
    w = wl.weight(wk, proj, rows=n, cols=k)
    n, k = w.shape
    r = wk.r if r is None else r
    m = wk.m if m is None else m
    x = wl.activations(wk, proj, m=m, k=k)
    a = wl.lora_a(wk, proj, r=r, k=k)
    b = wl.lora_b(wk, proj, r=r, n=n)
    dy = wl.grad_out(wk, proj, m=m, n=n)
    return w, x, a, b, dy, r


def _run(w, x, a, b, dy, r, alpha, out_dtype=capi.QN_F32, backward=True):
    print(f"[linear] M={x.shape[0]} N={w.shape[0]} K={w.shape[1]} r={r} "
          f"alpha={alpha} dtype={out_dtype}", flush=True)
    t, status = quantize_dev(w)
    X, A, B, DY = bf16_dev(x), bf16_dev(a), bf16_dev(b), bf16_dev(dy)
    y, ts = capi.qlora_linear_fwd(X, t, A, B, r, alpha, y_dtype=out_dtype)
    res = {"y": y, "t": ts, "nf4": t}
    if backward:
        dx, da, db = capi.qlora_linear_bwd(DY, X, t, A, B, r, alpha, ts,
                                           dx_dtype=out_dtype)
        res.update(dx=dx, da=da, db=db)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    return res


def _oracle_w(res, numel):
    packed, q, d = nf4_host(res["nf4"])
    return oracle.nf4_dequantize(packed, q, d, numel)


def _compare_full(w, x, a, b, dy, r, alpha, out_dtype=capi.QN_F32):
    res = _run(w, x, a, b, dy, r, alpha, out_dtype)
    n, k = w.shape
    # the codec itself is checked bit-exact in test_gpu_codec; here the
    # oracle's own quantization feeds the reference
    rp, rq, rd = oracle.nf4_quantize(w)
    wbits = oracle.nf4_dequantize(rp, rq, rd, w.size).reshape(n, k)
    y, t = oracle.qlora_forward(x, wbits, a, b, alpha, r)
    dx, da, db = oracle.qlora_backward(dy, x, wbits, a, b, alpha, r, t)
    tol = TOL if out_dtype == capi.QN_F32 else TOL_BF16
    errs = {
        "y": rel_err(f64_host(res["y"]), y),
        "t": rel_err(f64_host(res["t"]), t),
        "dx": rel_err(f64_host(res["dx"]), dx),
        "da": rel_err(f64_host(res["da"]), da),
        "db": rel_err(f64_host(res["db"]), db),
    }
    print(f"[linear] rel errors {errs}", flush=True)
    assert errs["y"] <= tol and errs["dx"] <= tol
    assert errs["t"] <= TOL and errs["da"] <= TOL and errs["db"] <= TOL
    return errs


def test_tiny_workload_fp32():
    wk = wl.workload("tiny")
    errs = _compare_full(*_inputs(wk, 0), alpha=wk.alpha)
    assert max(errs.values()) < 1e-5      # fp32 accumulation of exact products


def test_tiny_workload_bf16_outputs():
    wk = wl.workload("tiny")
    _compare_full(*_inputs(wk, 0), alpha=wk.alpha, out_dtype=capi.QN_BF16)


@pytest.mark.parametrize("m,n,k,r,alpha", [
    (37, 200, 192, 5, 7.0),      # ragged M and N tiles, odd rank
    (1, 8, 64, 1, 1.0),          # smallest legal problem
    (130, 136, 320, 64, 16.0),   # r = 64, N and M just past a tile
    (300, 264, 128, 17, 3.0),    # rank just past a 16-wide tile
    (300, 264, 256, 48, 3.0),    # r = 48: two 256-row blocks of the rank
                                 # streams, the second ragged
    (64, 128, 256, 256, 512.0),  # maximum rank
    (1024, 2048, 2112, 256, 64.0),  # maximum rank, two or three stages per
                                    # rank-stream workgroup (two-buffer
                                    # pipeline), a ragged last one
    (257, 1024, 576, 16, 32.0),  # M spans two split-M chunks
    (8, 200, 320, 5, 3.0),       # skinny path: N % 16 != 0, K % 256 != 0
    (13, 1032, 2368, 33, 8.0),   # skinny path: several K slices, r > 32
    (16, 64, 4160, 256, 64.0),   # skinny path at the largest M and rank
    (17, 136, 192, 8, 16.0),     # just above the skinny threshold
])
def test_ragged_shapes(m, n, k, r, alpha):
    wk = wl.workload("tiny")
    _compare_full(*_inputs(wk, 0, m=m, n=n, k=k, r=r), alpha=alpha)


@pytest.mark.parametrize("m,n,k", [
    (2048, 8448, 1024),   # forward: 264 output tiles, a ragged second wave
    (2048, 1024, 8448),   # backward dX: 264 tiles
    # 256 x 256 tiles with ragged edges: forward M and N ragged and an odd
    # number of 64-wide steps (17); backward M and K ragged and a partial
    # last step (N = 1032)
    (2050, 8200, 1088),
    (2050, 1032, 8256),
])
def test_more_than_one_wave_of_tiles(m, n, k):
    """256 x 256 tiles over more than one wave of workgroups (a ragged last
    wave), and with ragged tile edges: full element-wise comparison with
    the oracle."""
    wk = wl.workload("tiny")
    _compare_full(*_inputs(wk, 0, m=m, n=n, k=k, r=16), alpha=32.0)


def test_zero_adapter_matches_hipblaslt_on_dequantized_weight():
    """With B = 0 the layer is X W'^T: compare with torch.matmul (hipBLASLt,
    a black-box library) on the GPU-dequantized W'."""
    wk = wl.workload("tiny")
    w, x, a, b, dy, r = _inputs(wk, 0, m=64, n=512, k=1024)
    b0 = np.zeros_like(b)
    res = _run(w, x, a, b0, dy, r, wk.alpha, backward=False)
    wq = capi.nf4_dequantize(res["nf4"]).float()
    ref = torch.matmul(bf16_dev(x).float(), wq.t().contiguous())
    torch.cuda.synchronize()
    assert rel_err(f64_host(res["y"]), ref.double().cpu().numpy()) <= 1e-5


def test_linear_deterministic():
    wk = wl.workload("tiny")
    w, x, a, b, dy, r = _inputs(wk, 0, m=300, n=264, k=256, r=16)
    r1 = _run(w, x, a, b, dy, r, 32.0)
    r2 = _run(w, x, a, b, dy, r, 32.0)
    for key in ("y", "t", "dx", "da", "db"):
        assert torch.equal(r1[key], r2[key]), key


@pytest.mark.parametrize("m,n,k", [(2048, 8448, 1024), (2050, 1032, 8256)])
def test_split_last_wave_repeatable(m, n, k):
    """Shapes whose last wave of 256 x 256 tiles is split into two
    reduction halves per tile (forward: 264 tiles; backward: 297 tiles):
    three calls in a row give bit-identical results, whichever half of a
    tile finishes first and with the counters the halves leave behind."""
    wk = wl.workload("tiny")
    w, x, a, b, dy, r = _inputs(wk, 0, m=m, n=n, k=k, r=16)
    runs = [_run(w, x, a, b, dy, r, 32.0) for _ in range(3)]
    for res in runs[1:]:
        for key in ("y", "t", "dx", "da", "db"):
            assert torch.equal(runs[0][key], res[key]), key


def _full_check(w, x, a, b, dy, r, alpha, res, out_dtype):
    """Every element of Y, T, dX, dA and dB against oracle.forward_f64 /
    oracle.backward_f64 on the exact bf16 inputs and the oracle's
    dequantization of the GPU's NF4 tensor (bit-exact to the oracle's own,
    test_gpu_codec)."""
    n, k = w.shape
    W = oracle.bf16_bits_to_f64(_oracle_w(res, w.size).reshape(n, k))
    X, A, B, DY = (oracle.bf16_bits_to_f64(v) for v in (x, a, b, dy))
    s = alpha / r
    y_ref, t_ref = oracle.forward_f64(X, W, A, B, s)
    errs = {"y": rel_err(f64_host(res["y"]), y_ref),
            "t": rel_err(f64_host(res["t"]), t_ref)}
    del y_ref
    dx_ref, da_ref, db_ref = oracle.backward_f64(DY, X, W, A, B, s, t_ref)
    errs.update(dx=rel_err(f64_host(res["dx"]), dx_ref),
                da=rel_err(f64_host(res["da"]), da_ref),
                db=rel_err(f64_host(res["db"]), db_ref))
    tol = TOL if out_dtype == capi.QN_F32 else TOL_BF16
    print(f"[linear] full-size rel errors {errs}", flush=True)
    assert errs["y"] <= tol and errs["dx"] <= tol
    assert errs["t"] <= TOL and errs["da"] <= TOL and errs["db"] <= TOL


@pytest.mark.parametrize("out_dtype", [capi.QN_F32, capi.QN_BF16])
def test_gate7b_full_size(out_dtype):
    """7B gate projection, M=4096, r=16 (the benchmarked step, both output
    types): every element against the oracle."""
    wk = wl.workload("gate7b")
    w, x, a, b, dy, r = _inputs(wk, 0)
    res = _run(w, x, a, b, dy, r, wk.alpha, out_dtype)
    _full_check(w, x, a, b, dy, r, wk.alpha, res, out_dtype)


@pytest.mark.parametrize("proj", [0, 1, 3, 4, 6])
def test_layer70b_projection_full_size(proj):
    """70B-layer projections q and o (8192x8192), k (1024x8192), gate
    (28672x8192; its forward GEMM splits the last 128 of 896 tiles) and down
    (8192x28672; its dX GEMM splits) at M=2048, r=64, alpha=16: every
    element against the oracle."""
    wk = wl.workload("layer70b")
    w, x, a, b, dy, r = _inputs(wk, proj)
    res = _run(w, x, a, b, dy, r, wk.alpha, capi.QN_F32)
    _full_check(w, x, a, b, dy, r, wk.alpha, res, capi.QN_F32)


@pytest.mark.parametrize("proj", [0, 4, 6])
def test_skinny70b_forward_full_size(proj):
    """M = 8 tokens through 70B-layer projections (q, gate, down)."""
    wk = wl.workload("skinny70b")
    w, x, a, b, dy, r = _inputs(wk, proj)
    res = _run(w, x, a, b, dy, r, wk.alpha, capi.QN_F32, backward=False)
    n, k = w.shape
    W = oracle.bf16_bits_to_f64(_oracle_w(res, w.size).reshape(n, k))
    X, A, B = (oracle.bf16_bits_to_f64(v) for v in (x, a, b))
    y, t = oracle.forward_f64(X, W, A, B, wk.alpha / r)
    ey, et = rel_err(f64_host(res["y"]), y), rel_err(f64_host(res["t"]), t)
    print(f"[skinny] proj={proj} y={ey} t={et}", flush=True)
    assert ey <= TOL and et <= TOL


@pytest.mark.parametrize("m,n,k", [(2048, 8448, 1024), (2050, 1032, 8256)])
def test_split_status_word_with_garbage_workspace(m, n, k):
    """The split area (status word, counters, partial tiles) sits at the
    start of the workspace.  Workspaces filled with 0xFF bytes before the
    call: the call zeroes the status word and the counters itself, the
    status word reads QN_OK afterwards, and the results equal those of a
    call on a fresh workspace."""
    wk = wl.workload("tiny")
    w, x, a, b, dy, r = _inputs(wk, 0, m=m, n=n, k=k, r=16)
    t, _ = quantize_dev(w)
    X, A, B, DY = bf16_dev(x), bf16_dev(a), bf16_dev(b), bf16_dev(dy)
    fb = capi.qlora_workspace_bytes(m, n, k, r, capi.QN_FWD)
    bb = capi.qlora_workspace_bytes(m, n, k, r, capi.QN_BWD)
    wsf = torch.full((fb,), 0xFF, dtype=torch.uint8, device="cuda")
    wsb = torch.full((bb,), 0xFF, dtype=torch.uint8, device="cuda")
    y, ts = capi.qlora_linear_fwd(X, t, A, B, r, 32.0, ws=wsf)
    dx, da, db = capi.qlora_linear_bwd(DY, X, t, A, B, r, 32.0, ts, ws=wsb)
    y2, ts2 = capi.qlora_linear_fwd(X, t, A, B, r, 32.0)
    dx2, _, _ = capi.qlora_linear_bwd(DY, X, t, A, B, r, 32.0, ts2)
    torch.cuda.synchronize()
    assert int(wsf[:4].view(torch.int32).item()) == capi.QN_OK
    assert int(wsb[:4].view(torch.int32).item()) == capi.QN_OK
    assert torch.equal(y, y2) and torch.equal(dx, dx2)
