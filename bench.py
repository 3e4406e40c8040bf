#!/usr/bin/env python3
"""Benchmark of the QLoRA linear layer on one MI355X.

One step = qlora_linear_fwd + qlora_linear_bwd of the Llama-7B gate
projection (W 11008x4096 NF4 + double quant, X 4096 tokens, r=16, alpha=32,
bf16 Y and dX).  The NF4 weight is dequantized on the fly inside the fused
kernels every step.  ``value`` is fwd+bwd TFLOP/s counting only algorithmic
matmul flops 4MNK + 6Mr(K+N).

The same JSON line also reports, each timed on its own:
  dequant7b  nf4_dequantize over the 7 projections of a 7B-class layer, HBM
             GB/s over 2.516 B/param (packed + block codes + group scales in,
             bf16 out)
  quantize7b nf4_quantize over the same projections, 4.516 B/param
  skinny70b  qlora_linear_fwd with M=8 over the 7 projections of a
             70B-class layer, GB/s over NF4 + adapters + X + Y bytes
  layer70b   fwd+bwd over the 7 70B-class projections, M=2048, r=64
and the roofline of the dominant kernel from per-launch HIP events recorded
on the library's stream, plus the CPU oracle timed on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 flop/clk (dense)
METRIC = "fused QLoRA linear fwd+bwd TFLOP/s (7B shapes) + NF4 dequant HBM GB/s"


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def linear_flops(m, n, k, r, backward=True):
    fwd = 2 * m * n * k + 2 * m * r * (k + n)
    bwd = 2 * m * n * k + 4 * m * r * (k + n)
    return fwd + (bwd if backward else 0)


class Problem:
    """Device inputs of one projection: NF4 weight + bf16 X, A, B, dY."""

    def __init__(self, wk, proj, backward=True, y_dtype=None, dropout=None):
        import numpy as np
        import torch
        from bit_nf4_quantized_14_amd import capi
        from bit_nf4_quantized_14_amd import workloads as wl

        self.capi = capi
        _, self.n, self.k = wk.projections[proj]
        self.m, self.r, self.alpha = wk.m, wk.r, wk.alpha
        dev = "cuda"

        def up(bits):
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

        w = torch.from_numpy(wl.weight(wk, proj)).to(dev)
        self.w = capi.nf4_quantize(w)
        del w
        self.x = up(wl.activations(wk, proj))
        self.a = up(wl.lora_a(wk, proj))
        self.b = up(wl.lora_b(wk, proj))
        self.dy = up(wl.grad_out(wk, proj)) if backward else None
        ydt = capi.QN_BF16 if y_dtype is None else y_dtype
        self.ydt = ydt
        tdt = torch.bfloat16 if ydt == capi.QN_BF16 else torch.float32
        self.y = torch.empty((self.m, self.n), dtype=tdt, device=dev)
        self.t = torch.empty((self.m, self.r), dtype=torch.float32, device=dev)
        # dropout: (p, seed) of LoRA dropout on the adapter input, or None
        self.dropout = dropout
        fb = capi.qlora_workspace_bytes(
            self.m, self.n, self.k, self.r,
            capi.QN_FWD if dropout is None else capi.QN_FWD_DROPOUT)
        self.wsf = torch.empty(max(fb, 1), dtype=torch.uint8, device=dev)
        if backward:
            self.dx = torch.empty((self.m, self.k), dtype=tdt, device=dev)
            self.da = torch.empty((self.r, self.k), dtype=torch.float32, device=dev)
            self.db = torch.empty((self.n, self.r), dtype=torch.float32, device=dev)
            nbytes = capi.qlora_workspace_bytes(self.m, self.n, self.k, self.r,
                                                capi.QN_BWD)
            self.ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)

    def fwd(self):
        if self.dropout is not None:
            p, seed = self.dropout
            self.capi.qlora_linear_fwd_dropout(
                self.x, self.w, self.a, self.b, self.r, self.alpha, p, seed,
                y=self.y, y_dtype=self.ydt, t_save=self.t, ws=self.wsf)
            return
        self.capi.qlora_linear_fwd(self.x, self.w, self.a, self.b, self.r,
                                   self.alpha, y=self.y, y_dtype=self.ydt,
                                   t_save=self.t, ws=self.wsf)

    def bwd(self):
        if self.dropout is not None:
            p, seed = self.dropout
            self.capi.qlora_linear_bwd_dropout(
                self.dy, self.x, self.w, self.a, self.b, self.r, self.alpha,
                self.t, p, seed, dx=self.dx, dx_dtype=self.ydt, dA=self.da,
                dB=self.db, ws=self.ws)
            return
        self.capi.qlora_linear_bwd(self.dy, self.x, self.w, self.a, self.b,
                                   self.r, self.alpha, self.t, dx=self.dx,
                                   dx_dtype=self.ydt, dA=self.da, dB=self.db,
                                   ws=self.ws)


def kernel_times_ms(capi, name, fn, launches_per_call, reps):
    """Average duration (ms) of each launch of kernel `name` while calling
    fn() `reps` times, from HIP events the library records around it."""
    import torch
    cap = launches_per_call * reps
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(cap)]
    stops = [torch.cuda.Event(enable_timing=True) for _ in range(cap)]
    capi.qn_profile_kernel(name, starts, stops)
    for _ in range(reps):
        fn()
    n = capi.qn_profile_kernel(None)
    torch.cuda.synchronize()
    if n == 0:
        return None, 0
    return sum(s.elapsed_time(e) for s, e in zip(starts[:n], stops[:n])) / n, n


def timed(fn, reps, warmup=2):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / reps


def timed_graph(fn, reps, warmup=2):
    """Seconds per call of fn() replayed from a captured HIP graph, so that
    passes made of many short launches are not bound by host launch cost.
    The library's calls allocate nothing and issue no memset, so they can be
    captured; the first replays are checked against eager runs by the
    tests, here they are only timed."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / reps
    del g
    return sec


def bench_dequant_quant(reps, copies=3):
    """7B-class layer: dequant and quantize GB/s over all 7 projections.

    The dequant pass reads 104 MB of NF4 data, which the 256 MB MALL could
    keep between passes; the timed region cycles through `copies`
    independently quantized copies of the layer (3 x 104 MB > 256 MB), so
    each pass reads its input from HBM."""
    import torch
    from bit_nf4_quantized_14_amd import capi
    from bit_nf4_quantized_14_amd import workloads as wl
    wk = wl.workload("dequant7b")
    sets, outs, ws32 = [[] for _ in range(copies)], [], []
    params = 0
    for p in range(len(wk.projections)):
        w = torch.from_numpy(wl.weight(wk, p)).to("cuda")
        for c in range(copies):
            sets[c].append(capi.nf4_quantize(w))
        ws32.append(w)
        outs.append(torch.empty((w.shape[0], w.shape[1]), dtype=torch.bfloat16,
                                device="cuda"))
        params += w.numel()
    tens = sets[0]
    npk = sum(t.packed.numel() + t.qabs.numel() + 4 * t.gscale.numel() for t in tens)
    deq_bytes = npk + 2 * params
    q_bytes = 4 * params + npk

    def deq():                      # `copies` passes, one launch per copy
        for c in range(copies):
            capi.nf4_dequantize_batch(sets[c], outs)

    def deq_each():                 # the same, one call per projection
        for c in range(copies):
            for t, o in zip(sets[c], outs):
                capi.nf4_dequantize(t, o)

    def quant():
        for w, t in zip(ws32, tens):
            capi.nf4_quantize(w, t)

    res = {}
    for name, fn, kname, nbytes, passes, launches in (
            ("dequant7b", deq, "k_dequant", deq_bytes, copies, 1),
            ("quantize7b", quant, "k_quantize", q_bytes, 1, len(tens))):
        sec = timed_graph(fn, reps) / passes
        kt, _ = kernel_times_ms(capi, kname, fn, launches * passes, reps)
        ksum = kt * launches * 1e-3
        res[name] = {"params": params, "bytes_per_pass": nbytes,
                     "ms_per_pass": sec * 1e3,
                     "GB/s": nbytes / sec / 1e9,
                     "timing": "graph replay of the 7-projection pass",
                     "kernel": kname, "kernel_ms_per_pass": ksum * 1e3,
                     "kernel_GB/s": nbytes / ksum / 1e9,
                     "frac_hbm_peak": nbytes / ksum / 1e9 / HBM_PEAK_GBS}
        if name == "dequant7b":
            # HBM bytes of one whole-layer batched launch (counters)
            res[name]["traffic"] = measured_traffic("k_dequant<0>")
        else:
            t = measured_traffic("k_quantize<0>")
            res[name]["traffic_per_launch_avg"] = t
        log(f"{name}: {res[name]['GB/s']:.0f} GB/s graph, "
            f"{res[name]['kernel_GB/s']:.0f} GB/s kernel")
    # dequantize-and-merge of the same layer with an r = 16, alpha = 32
    # adapter per projection (one nf4_merge call per projection)
    mr, malpha = 16, 32.0
    ads = [(torch.from_numpy(wl.lora_a(wk, p, r=mr)).view(torch.bfloat16).to("cuda"),
            torch.from_numpy(wl.lora_b(wk, p, r=mr)).view(torch.bfloat16).to("cuda"))
           for p in range(len(wk.projections))]
    m_bytes = deq_bytes + sum(2 * mr * (t.rows + t.cols) for t in tens)

    def merge():
        for c in range(copies):
            for t, (a, b), o in zip(sets[c], ads, outs):
                capi.nf4_merge(t, a, b, mr, malpha, o)
    sec = timed_graph(merge, reps) / copies
    kt, _ = kernel_times_ms(capi, "k_merge", merge, len(tens) * copies, reps)
    ksum = kt * len(tens) * 1e-3
    res["merge7b"] = {"params": params, "r": mr, "alpha": malpha,
                      "bytes_per_pass": m_bytes, "ms_per_pass": sec * 1e3,
                      "GB/s": m_bytes / sec / 1e9,
                      "timing": "graph replay of the 7-projection pass (7 nf4_merge calls), "
                                f"cycling over {copies} weight copies (> MALL)",
                      "kernel": "k_merge", "kernel_ms_per_pass": ksum * 1e3,
                      "kernel_GB/s": m_bytes / ksum / 1e9,
                      "frac_hbm_peak": m_bytes / sec / 1e9 / HBM_PEAK_GBS,
                      "traffic_per_launch_avg": measured_traffic("k_merge<1>")}
    log(f"merge7b (r=16): {res['merge7b']['GB/s']:.0f} GB/s graph, "
        f"{res['merge7b']['kernel_GB/s']:.0f} GB/s kernel")
    # the same pass as seven separate calls (one launch per projection)
    sec = timed_graph(deq_each, reps) / copies
    res["dequant7b"]["per_call_GB/s"] = deq_bytes / sec / 1e9
    res["dequant7b"]["timing"] = ("graph replay of the 7-projection pass as one "
                                  "nf4_dequantize_batch launch, cycling over "
                                  f"{copies} weight copies (> MALL); per_call_GB/s: "
                                  "the same pass as 7 nf4_dequantize calls")
    log(f"dequant7b as 7 calls: {res['dequant7b']['per_call_GB/s']:.0f} GB/s graph")
    del sets, tens, outs, ws32, ads
    torch.cuda.empty_cache()
    return res


def bench_variants(reps, copies=3):
    """Codec variants over the 7B-class layer: for each 4-bit table (NF4,
    FP4, INT4) and block-constant storage (8-bit DQ, fp32, centered 8-bit):
    dequant GB/s (7 qn_dequantize calls per pass, cycling over `copies`
    quantized copies so the pass reads HBM) and the quantization error of
    the layer, sqrt(sum (w' - w)^2 / sum w^2), measured on the GPU."""
    import torch
    from bit_nf4_quantized_14_amd import capi
    from bit_nf4_quantized_14_amd import workloads as wl
    wk = wl.workload("dequant7b")
    ws32 = [torch.from_numpy(wl.weight(wk, p)).to("cuda")
            for p in range(len(wk.projections))]
    outs = [torch.empty(w.shape, dtype=torch.bfloat16, device="cuda") for w in ws32]
    params = sum(w.numel() for w in ws32)
    names = {capi.QN_CODE_NF4: "nf4", capi.QN_CODE_FP4: "fp4", capi.QN_CODE_INT4: "int4"}
    modes = {capi.QN_CONST_DQ8: "dq8", capi.QN_CONST_FP32: "fp32",
             capi.QN_CONST_CENTERED: "dq8c"}
    res = {}
    for code, cname in names.items():
        for mode, mname in modes.items():
            sets = [[capi.qn_quantize(w, code, mode) for w in ws32] for _ in range(copies)]
            tens = sets[0]
            nbytes = 2 * params + sum(
                t.packed.numel() + t.consts.numel() * t.consts.element_size()
                + 4 * (t.gscale.numel() + t.gmean.numel()) for t in tens)

            def deq():
                for c in range(copies):
                    for t, o in zip(sets[c], outs):
                        capi.qn_dequantize(t, o)
            sec = timed_graph(deq, reps) / copies
            num = den = 0.0
            for t, w, o in zip(tens, ws32, outs):
                capi.qn_dequantize(t, o)
                num += float(((o.float() - w) ** 2).sum(dtype=torch.float64))
                den += float((w.double() ** 2).sum())
            key = f"{cname}_{mname}"
            res[key] = {"bytes_per_pass": nbytes, "bits_per_weight":
                        8.0 * (nbytes - 2 * params) / params,
                        "ms_per_pass": sec * 1e3, "GB/s": nbytes / sec / 1e9,
                        "rel_rms_error": (num / den) ** 0.5}
            log(f"variant {key}: {res[key]['GB/s']:.0f} GB/s, "
                f"{res[key]['bits_per_weight']:.3f} bit/w, rel rms err "
                f"{res[key]['rel_rms_error']:.5f}")
            del sets, tens
    del ws32, outs
    torch.cuda.empty_cache()
    return {"variants7b": {"params": params, "timing": "graph replay of 7 "
                           "qn_dequantize calls per pass, cycling over "
                           f"{copies} copies (> MALL)", "variants": res}}


def bench_dropout(reps, p=0.05):
    """gate7b fwd+bwd with LoRA dropout p on the adapter input (the pages'
    lora_dropout), against the same step without dropout, both as graph
    replays of one fwd+bwd."""
    import torch
    from bit_nf4_quantized_14_amd import workloads as wl
    wk = wl.workload("gate7b")
    res = {}
    for name, drop in (("without", None), ("with", (p, 0x5EED))):
        pr = Problem(wk, 0, dropout=drop)

        def step():
            pr.fwd()
            pr.bwd()
        sec = timed_graph(step, reps)
        res[name] = {"ms_per_step": sec * 1e3,
                     "TFLOP/s": linear_flops(pr.m, pr.n, pr.k, pr.r) / sec / 1e12}
        del pr
        torch.cuda.empty_cache()
    res["p"] = p
    res["overhead"] = res["with"]["ms_per_step"] / res["without"]["ms_per_step"] - 1
    log(f"gate7b dropout p={p}: {res['with']['ms_per_step']:.3f} ms/step vs "
        f"{res['without']['ms_per_step']:.3f} without ({100 * res['overhead']:+.1f}%)")
    return {"gate7b_dropout": res}


def adapter_params_70b(r=16, layers=80):
    """Parameters of r-rank adapters on all 7 linear projections of every
    layer of a Llama-70B-class model (hidden 8192, GQA k/v 1024, MLP 28672)."""
    shapes = ((8192, 8192), (1024, 8192), (1024, 8192), (8192, 8192),
              (28672, 8192), (28672, 8192), (8192, 28672))
    return layers * sum(r * (n + k) for n, k in shapes)


def bench_adamw(reps, chunk=1 << 24):
    """8-bit AdamW over the adapters of a whole 70B-class model at r = 16
    (one flat buffer): the resident step (state in HBM) as GB/s of its
    algorithmic traffic, and the paged step (state in pinned host memory,
    pages of `chunk` elements through a double-buffered device staging
    area, copies on two streams of their own) as ms per step."""
    import torch
    from bit_nf4_quantized_14_amd import capi
    n = adapter_params_70b()
    gen = torch.Generator(device="cuda").manual_seed(1430)
    p = (torch.randn(n, generator=gen, device="cuda") * 0.01).to(torch.bfloat16)
    g = torch.randn(n, generator=gen, device="cuda") * 1e-3
    st = capi.AdamW8State.zeros(n)
    hp = dict(lr=2e-4, weight_decay=0.0)
    for t in range(1, 3):
        capi.qn_adamw8_step(p, g, st, t, **hp)
    nb = -(-n // capi.QN_ADAMW_BLOCK)
    nbytes = n * (2 + 4 + 1 + 1 + 2 + 1 + 1) + nb * 4 * 4

    def step():
        capi.qn_adamw8_step(p, g, st, 3, **hp)
    sec = timed_graph(step, reps)
    kt, _ = kernel_times_ms(capi, "k_adamw8", step, 1, reps)
    res = {"params": n, "bytes_per_step": nbytes, "ms_per_step": sec * 1e3,
           "GB/s": nbytes / sec / 1e9, "kernel": "k_adamw8",
           "kernel_ms": kt, "kernel_GB/s": nbytes / (kt * 1e-3) / 1e9,
           "frac_hbm_peak": nbytes / (kt * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "traffic": measured_traffic("k_adamw8"),
           "workload": "r=16 adapters on the 7 projections of 80 layers of "
                       "a 70B-class model, bf16 params, fp32 grads"}
    log(f"adamw8 resident: {sec*1e3:.3f} ms/step, {res['GB/s']:.0f} GB/s "
        f"(kernel {res['kernel_GB/s']:.0f} GB/s)")
    # paged: the same state in pinned host memory
    host = capi.AdamW8State(st.m_codes.cpu().pin_memory(), st.m_scale.cpu().pin_memory(),
                            st.r_codes.cpu().pin_memory(), st.r_scale.cpu().pin_memory())
    del st
    staging = torch.empty(capi.qn_adamw8_staging_bytes(chunk), dtype=torch.uint8,
                          device="cuda")
    h2d, d2h = torch.cuda.Stream(), torch.cuda.Stream()
    page_bytes = 2 * (2 * n + 8 * nb)     # state in and out

    def paged(t):
        capi.qn_adamw8_paged_step(p, g, host, staging, chunk, t,
                                  h2d_stream=h2d, d2h_stream=d2h, **hp)
    paged(3)
    torch.cuda.synchronize()
    prep = max(2, reps // 4)
    t0 = time.perf_counter()
    for i in range(prep):
        paged(4 + i)
    torch.cuda.synchronize()
    psec = (time.perf_counter() - t0) / prep
    res["paged"] = {"ms_per_step": psec * 1e3, "chunk": chunk,
                    "host_device_bytes_per_step": page_bytes,
                    "host_link_GB/s": page_bytes / psec / 1e9,
                    "timing": "wall clock over eager steps (pinned host state)"}
    log(f"adamw8 paged: {psec*1e3:.2f} ms/step, state traffic "
        f"{page_bytes / psec / 1e9:.1f} GB/s over the host link")
    del p, g, host, staging
    torch.cuda.empty_cache()
    return {"adamw8_70b_adapters": res}


def bench_70b(reps, do_train=True):
    import torch
    from bit_nf4_quantized_14_amd import capi
    from bit_nf4_quantized_14_amd import workloads as wl
    res = {}
    # skinny forward (M = 8)
    wk = wl.workload("skinny70b")
    probs = [Problem(wk, p, backward=False, y_dtype=capi.QN_F32)
             for p in range(len(wk.projections))]
    nbytes = 0
    for pr in probs:
        npk = pr.w.packed.numel() + pr.w.qabs.numel() + 4 * pr.w.gscale.numel()
        nbytes += npk + 2 * pr.r * (pr.n + pr.k) + 2 * pr.m * pr.k + 4 * pr.m * pr.n

    def skinny():
        for pr in probs:
            pr.fwd()
    # the same seven projections as one qlora_linear_fwd_batch call (one
    # partial and one reduce launch for the whole layer)
    batch = capi.FwdBatch([(pr.x, pr.w, pr.a, pr.b, pr.r, pr.alpha, pr.y,
                            capi.QN_F32, pr.t) for pr in probs])

    def skinny_batch():
        capi.qlora_linear_fwd_batch(batch)
    sec = timed_graph(skinny_batch, reps)
    sec_calls = timed_graph(skinny, reps)
    kp, _ = kernel_times_ms(capi, "k_skinny_partial", skinny_batch, 1, reps)
    kr, _ = kernel_times_ms(capi, "k_skinny_reduce", skinny_batch, 1, reps)
    kp1, _ = kernel_times_ms(capi, "k_skinny_partial", skinny, len(probs), reps)
    kr1, _ = kernel_times_ms(capi, "k_skinny_reduce", skinny, len(probs), reps)
    ksum = (kp + kr) * 1e-3
    per = {}
    for pr, (name, _, _) in zip(probs, wk.projections):
        npk = pr.w.packed.numel() + pr.w.qabs.numel() + 4 * pr.w.gscale.numel()
        b1 = npk + 2 * pr.r * (pr.n + pr.k) + 2 * pr.m * pr.k + 4 * pr.m * pr.n
        s1 = timed_graph(pr.fwd, reps)
        per[name] = {"bytes": b1, "ms": s1 * 1e3, "GB/s": b1 / s1 / 1e9}
    res["skinny70b"] = {"bytes_per_pass": nbytes, "ms_per_pass": sec * 1e3,
                        "GB/s": nbytes / sec / 1e9,
                        "timing": "graph replay of the 7-projection pass as one "
                                  "qlora_linear_fwd_batch call",
                        "frac_hbm_peak": nbytes / sec / 1e9 / HBM_PEAK_GBS,
                        "kernel_ms_per_pass": ksum * 1e3,
                        "k_skinny_partial_ms": kp, "k_skinny_reduce_ms": kr,
                        "kernel_GB/s": nbytes / ksum / 1e9,
                        "per_call_pass_ms": sec_calls * 1e3,
                        "per_call_pass_GB/s": nbytes / sec_calls / 1e9,
                        "per_call_partial_avg_ms": kp1,
                        "per_call_reduce_avg_ms": kr1,
                        "per_projection_single_call": per}
    log(f"skinny70b: {res['skinny70b']['GB/s']:.0f} GB/s batched (graph), "
        f"{res['skinny70b']['kernel_GB/s']:.0f} GB/s kernels "
        f"(partial {kp*1e3:.1f} us, reduce {kr*1e3:.1f} us); "
        f"7 single calls {res['skinny70b']['per_call_pass_GB/s']:.0f} GB/s")
    del batch
    del probs
    torch.cuda.empty_cache()
    if not do_train:
        return res
    wk = wl.workload("layer70b")
    flops = 0
    total = 0.0
    per = {}
    for p, (name, n, k) in enumerate(wk.projections):
        pr = Problem(wk, p)

        def step():
            pr.fwd()
            pr.bwd()
        sec = timed_graph(step, reps)
        f = linear_flops(pr.m, n, k, pr.r)
        per[name] = {"ms": sec * 1e3, "TFLOP/s": f / sec / 1e12}
        for kname, kf in (("k_fwd_gemm", 2 * pr.m * n * k + 2 * pr.m * n * pr.r),
                          ("k_bwd_dx_gemm", 2 * pr.m * n * k + 2 * pr.m * k * pr.r)):
            ms, _ = kernel_times_ms(capi, kname, step, 1, reps)
            if ms is not None:
                per[name][kname] = {"avg_ms": ms, "TFLOP/s": kf / (ms * 1e-3) / 1e12}
        flops += f
        total += sec
        del pr
        torch.cuda.empty_cache()
    res["layer70b"] = {"flops_per_pass": flops, "ms_per_pass": total * 1e3,
                       "TFLOP/s": flops / total / 1e12,
                       "timing": "graph replay of each projection's fwd+bwd; "
                                 "GEMM kernels by per-launch HIP events",
                       "frac_mfma_peak": flops / total / 1e12 / BF16_PEAK_TFLOPS,
                       "per_projection": per}
    log(f"layer70b: {res['layer70b']['TFLOP/s']:.1f} TFLOP/s")
    return res


def measured_traffic(kernel_key: str):
    """HBM bytes per launch of `kernel_key` from the committed rocprofv3
    counter summary (profiles/hbm_traffic.json, FETCH_SIZE/WRITE_SIZE scaled
    by a plain copy of known size), or None when the kernel's sources have
    changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        rec = json.load(open(path))
        k = rec["kernels"][kernel_key]
    except (OSError, ValueError, KeyError):
        return None
    from bit_nf4_quantized_14_amd.profiling import source_sha
    if k.get("source_sha256_16") != source_sha(kernel_key):
        return None
    return k["read_bytes"] + k["write_bytes"]


def cpu_baseline(m_sample: int, min_seconds: float = 10.0, max_reps: int = 30):
    """The CPU oracle (as it stands) on a bounded sample of the same step:
    the full weight is dequantized, forward+backward run on m_sample tokens;
    whole oracle steps are repeated until about min_seconds of CPU work."""
    import numpy as np

    import oracle
    from bit_nf4_quantized_14_amd import workloads as wl
    wk = wl.workload("gate7b")
    w = wl.weight(wk, 0)
    n, k = w.shape
    x = wl.activations(wk, 0, m=m_sample)
    a, b = wl.lora_a(wk, 0), wl.lora_b(wk, 0)
    dy = wl.grad_out(wk, 0, m=m_sample)
    packed, q, d = oracle.nf4_quantize(w)       # load-time, not timed
    reps, total = 0, 0.0
    while reps < max_reps and (reps == 0 or total < min_seconds):
        t0 = time.perf_counter()
        wbits = oracle.nf4_dequantize(packed, q, d, w.size).reshape(n, k)
        y, t = oracle.qlora_forward(x, wbits, a, b, wk.alpha, wk.r)
        oracle.qlora_backward(dy, x, wbits, a, b, wk.alpha, wk.r, t)
        total += time.perf_counter() - t0
        reps += 1
    sec = total / reps
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    try:       # threads the BLAS behind NumPy's float64 matmuls ran with
        from threadpoolctl import threadpool_info
        blas = [i["num_threads"] for i in threadpool_info()
                if i.get("user_api") == "blas"]
        if blas:
            cores = min(cores, max(blas))
    except Exception:
        pass
    flops = linear_flops(m_sample, n, k, wk.r)
    return {"value": flops / sec / 1e12, "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle", "seconds": total, "reps": reps,
            "sample": f"gate7b step on {m_sample} of {wk.m} tokens, repeated "
                      f"{reps} times ({total:.1f} s): oracle dequantization of "
                      f"the full 11008x4096 weight + float64 forward/backward; "
                      f"flops 4MNK+6Mr(K+N) at M={m_sample} per step"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--quick", action="store_true",
                    help="only the main step (no components, no CPU baseline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-70b", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=4096)
    ap.add_argument("--only", choices=("dequant", "variants", "adamw", "dropout",
                                       "skinny", "layer70b"),
                    help="run one component pass only (for profiling)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 256 MiB device-to-device copy, the "
                         "reference for scaling HBM byte counters")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}); the QLoRA linear layer is benchmarked on "
              f"one MI355X and multi-GPU runs are not part of this build.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from bit_nf4_quantized_14_amd import capi
    from bit_nf4_quantized_14_amd import workloads as wl

    # the profiling build: the same kernels, plus per-launch HIP events
    # around one named kernel (qn_profile_kernel) for the roofline figures
    capi.use_profiling_build()
    capi.lib()
    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.only:
        reps = max(3, args.steps)
        if args.only == "dequant":
            res = bench_dequant_quant(reps)
        elif args.only == "variants":
            res = bench_variants(reps)
        elif args.only == "adamw":
            res = bench_adamw(reps)
        elif args.only == "dropout":
            res = bench_dropout(reps)
        elif args.only == "skinny":
            res = bench_70b(reps, do_train=False)
        else:
            res = bench_70b(reps)
        print(json.dumps({"only": args.only, "components": res}), flush=True)
        return
    wk = wl.workload("gate7b")
    log("generating gate7b inputs")
    pr = Problem(wk, 0)
    m, n, k, r = pr.m, pr.n, pr.k, pr.r
    flops = linear_flops(m, n, k, r)

    def step():
        pr.fwd()
        pr.bwd()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # the dominant (slower) fused GEMM, from a short measurement of both
    gemm_flops = {"k_fwd_gemm": 2 * m * n * k + 2 * m * n * r,
                  "k_bwd_dx_gemm": 2 * m * n * k + 2 * m * k * r}
    pre = {kn: kernel_times_ms(capi, kn, step, 1, 3)[0] for kn in gemm_flops}
    dom = max(gemm_flops, key=lambda kn: pre[kn])

    # timed region: exactly K steps; the dominant kernel's launches are
    # bracketed by HIP events on the library's stream
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    stops = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    capi.qn_profile_kernel(dom, starts, stops)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / args.steps
    nrec = capi.qn_profile_kernel(None)
    dom_ms = sum(s.elapsed_time(e) for s, e in zip(starts[:nrec], stops[:nrec])) / nrec
    achieved = gemm_flops[dom] / (dom_ms * 1e-3) / 1e12
    value = flops / sec / 1e12
    log(f"gate7b fwd+bwd: {sec*1e3:.3f} ms/step, {value:.1f} TFLOP/s; "
        f"{dom} {dom_ms:.3f} ms = {achieved:.1f} TFLOP/s")

    # per-kernel breakdown, after the timed region (warm clocks); each
    # kernel's launches in 10 further steps, bracketed by HIP events
    kernels = {}
    for kname, per_step in (("k_fwd_gemm", 1), ("k_bwd_dx_gemm", 1),
                            ("k_rank_stream_t", 1), ("k_rank_stream_dy", 1),
                            ("k_rank_stream_da", 1), ("k_rank_finish", 3)):
        ms, cnt = kernel_times_ms(capi, kname, step, per_step, 10)
        if ms is not None:
            kernels[kname] = {"avg_ms": ms, "launches_per_step": per_step}
    for kname, f in gemm_flops.items():
        kernels[kname]["TFLOP/s"] = f / (kernels[kname]["avg_ms"] * 1e-3) / 1e12

    # the same step with fp32 Y and dX (the mode the 2e-3 parity gate is
    # stated on), timed the same way
    pr32 = Problem(wk, 0, y_dtype=capi.QN_F32)

    def step32():
        pr32.fwd()
        pr32.bwd()
    for _ in range(args.warmup):
        step32()
    sec32 = timed(step32, args.steps, warmup=0)
    fp32_mode = {"ms_per_step": sec32 * 1e3, "TFLOP/s": flops / sec32 / 1e12,
                 "frac_mfma_peak": flops / sec32 / 1e12 / BF16_PEAK_TFLOPS}
    log(f"gate7b fp32 outputs: {sec32*1e3:.3f} ms/step, "
        f"{fp32_mode['TFLOP/s']:.1f} TFLOP/s")
    del pr32
    # context: hipBLASLt (torch) bf16 GEMMs of the same shapes on the
    # dequantized weight, without the adapter terms
    wd = capi.nf4_dequantize(pr.w)
    import torch.nn.functional as F
    ref = {}
    for key, fn, f in (
            ("forward X W'^T", lambda: F.linear(pr.x, wd), 2 * m * n * k),
            ("backward dY W'", lambda: torch.matmul(pr.dy, wd), 2 * m * n * k)):
        sec_ref = timed(fn, args.steps, warmup=3)
        ref[key] = {"ms": sec_ref * 1e3, "TFLOP/s": f / sec_ref / 1e12}
    del wd
    log("hipBLASLt bf16: " + ", ".join(f"{k2} {v['TFLOP/s']:.0f} TFLOP/s"
                                      for k2, v in ref.items()))

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": sec * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,sigma^2) weights/activations of the "
                "Llama-7B gate projection shape; no checkpoint or dataset)",
        "config": {"workload": "gate7b: QLoRA linear fwd+bwd, W 11008x4096 "
                               "NF4+DQ, X 4096 tokens, r=16, alpha=32, bf16 "
                               "Y/dX",
                   "M": m, "N": n, "K": k, "r": r, "alpha": pr.alpha,
                   "flops_per_step": flops, "parallelism": "single-gpu"},
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": achieved,
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / BF16_PEAK_TFLOPS,
                     "traffic": measured_traffic(
                         "k_gemm<256, 256, true, false, false, false>"
                         if dom == "k_bwd_dx_gemm"
                         else "k_gemm<256, 256, false, false, false, false>"),
                     "traffic_unit": "HBM bytes per launch",
                     "avg_ms": dom_ms, "flops_per_launch": gemm_flops[dom]},
        "kernels": kernels,
        "fp32_mode": fp32_mode,
        "hipblaslt_bf16_reference": ref,
    }
    del pr
    torch.cuda.empty_cache()
    if not args.quick:
        comps = bench_dequant_quant(max(5, args.steps // 2))
        comps.update(bench_variants(max(3, args.steps // 4)))
        comps.update(bench_adamw(max(5, args.steps // 2)))
        comps.update(bench_dropout(max(5, args.steps // 2)))
        if not args.no_70b:
            comps.update(bench_70b(max(3, args.steps // 4)))
        out["components"] = comps
        if "dequant7b" in comps:
            # whole-pass throughput (graph replay over weight copies that do
            # not fit the MALL); the per-launch event figure is reported in
            # components and includes event overhead per launch
            out["dequant_GBps"] = comps["dequant7b"]["GB/s"]
    if not args.quick and not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(args.cpu_sample_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
