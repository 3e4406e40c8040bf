"""Seeded synthetic inputs for the QLoRA linear layer.

This module only draws random numbers and describes shapes; it holds none of
the quantization or matmul arithmetic.  It is the one piece of code shared by
the HIP-path tests/bench and the CPU oracle: both receive the very same bits.

Every tensor comes from its own NumPy ``default_rng`` stream keyed by
(1400 + workload index, projection index, tensor kind), so any tensor can be
regenerated alone and in any order.  Weights are fp32; activations, adapters
and upstream gradients are drawn in fp32 and converted to bf16 bit patterns
(uint16) by torch's CPU conversion.

Workloads (the pages train LoRA on every linear projection of a Llama-style
decoder layer, with r and alpha as in their LoraConfig snippets):

0 ``tiny``      one 256x512 projection, M=16 tokens, r=8, alpha=16
1 ``dequant7b`` the 7 frozen projections of a Llama-7B-class layer, weights
                N(0, 0.02^2) with 0.1% entries replaced by 0.1*Student-t(3)
2 ``gate7b``    the 7B gate projection 11008x4096, M=4096 tokens, r=16,
                alpha=32
3 ``layer70b``  the 7 projections of a Llama-70B-class layer (hidden 8192,
                GQA k/v 1024, MLP 28672), weights N(0, 0.015^2), M=2048
                tokens, r=64, alpha=16, forward and backward
4 ``skinny70b`` same shapes, M=8 tokens, r=16, alpha=32, forward only
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

SEED_BASE = 1400

# (name, out_features N, in_features K); W is [N, K] (Linear convention)
PROJ_7B = (("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096),
           ("o", 4096, 4096), ("gate", 11008, 4096), ("up", 11008, 4096),
           ("down", 4096, 11008))
PROJ_70B = (("q", 8192, 8192), ("k", 1024, 8192), ("v", 1024, 8192),
            ("o", 8192, 8192), ("gate", 28672, 8192), ("up", 28672, 8192),
            ("down", 8192, 28672))

_KIND = {"w": 0, "x": 1, "a": 2, "b": 3, "dy": 4, "mask": 5, "t": 6}


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    projections: tuple      # ((name, N, K), ...)
    w_sigma: float
    outliers: bool
    m: int                  # tokens (0: codec-only workload)
    r: int
    alpha: float
    backward: bool


WORKLOADS = (
    Workload(0, "tiny", (("tiny", 256, 512),), 0.02, False, 16, 8, 16.0, True),
    Workload(1, "dequant7b", PROJ_7B, 0.02, True, 0, 0, 0.0, False),
    Workload(2, "gate7b", (("gate", 11008, 4096),), 0.02, False, 4096, 16,
             32.0, True),
    Workload(3, "layer70b", PROJ_70B, 0.015, False, 2048, 64, 16.0, True),
    Workload(4, "skinny70b", PROJ_70B, 0.015, False, 8, 16, 32.0, False),
)


def workload(name_or_index) -> Workload:
    for wl in WORKLOADS:
        if wl.name == name_or_index or wl.index == name_or_index:
            return wl
    raise KeyError(name_or_index)


def _rng(wl_index: int, proj: int, kind: str) -> np.random.Generator:
    return np.random.default_rng([SEED_BASE + wl_index, proj, _KIND[kind]])


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), via torch's CPU cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def normal_f32(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    out = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        out *= np.float32(sigma)
    return out


def weight(wl: Workload, proj: int, rows: int | None = None,
           cols: int | None = None) -> np.ndarray:
    """fp32 frozen weight [N, K] of projection ``proj`` of workload ``wl``.

    ``rows``/``cols`` override the shape (edge-case tests draw ragged sizes
    from the same recipe)."""
    _, n, k = wl.projections[proj]
    n = n if rows is None else rows
    k = k if cols is None else cols
    rng = _rng(wl.index, proj, "w")
    w = normal_f32(rng, (n, k), wl.w_sigma)
    if wl.outliers:
        mrng = _rng(wl.index, proj, "mask")
        mask = mrng.random(size=(n, k), dtype=np.float32) < np.float32(1e-3)
        cnt = int(mask.sum())
        w[mask] = (0.1 * mrng.standard_t(3, size=cnt)).astype(np.float32)
    return w


def activations(wl: Workload, proj: int, m: int | None = None,
                k: int | None = None) -> np.ndarray:
    """bf16 bits of X [M, K] ~ N(0, 1)."""
    _, _, kk = wl.projections[proj]
    m = wl.m if m is None else m
    k = kk if k is None else k
    return to_bf16_bits(normal_f32(_rng(wl.index, proj, "x"), (m, k), 1.0))


def lora_a(wl: Workload, proj: int, r: int | None = None,
           k: int | None = None) -> np.ndarray:
    """bf16 bits of A [r, K] ~ N(0, 1/K)."""
    _, _, kk = wl.projections[proj]
    r = wl.r if r is None else r
    k = kk if k is None else k
    return to_bf16_bits(normal_f32(_rng(wl.index, proj, "a"), (r, k),
                                   float(1.0 / np.sqrt(k))))


def lora_b(wl: Workload, proj: int, r: int | None = None,
           n: int | None = None) -> np.ndarray:
    """bf16 bits of B [N, r] ~ N(0, 0.01^2) (nonzero so the adapter branch
    contributes)."""
    _, nn, _ = wl.projections[proj]
    r = wl.r if r is None else r
    n = nn if n is None else n
    return to_bf16_bits(normal_f32(_rng(wl.index, proj, "b"), (n, r), 0.01))


def grad_out(wl: Workload, proj: int, m: int | None = None,
             n: int | None = None) -> np.ndarray:
    """bf16 bits of dY [M, N] ~ N(0, 1)."""
    _, nn, _ = wl.projections[proj]
    m = wl.m if m is None else m
    n = nn if n is None else n
    return to_bf16_bits(normal_f32(_rng(wl.index, proj, "dy"), (m, n), 1.0))
