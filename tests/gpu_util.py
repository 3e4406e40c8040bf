"""Helpers shared by the GPU parity tests: upload seeded inputs, download
results as bit patterns, and the relative-error measure of the gate."""

import numpy as np
import torch

from bit_nf4_quantized_14_amd import capi

DEV = "cuda"
TOL = 2e-3                      # max|gpu - ref| / max|ref|, fp32 outputs
TOL_BF16 = 2.0 ** -8 + 2e-3     # outputs rounded to bf16


def bf16_dev(bits: np.ndarray):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(DEV)


def f32_dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def bits_host(t) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64_host(t) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        b = bits_host(t).astype(np.uint32) << 16
        return b.view(np.float32).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    den = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got - ref))) / (den if den > 0 else 1.0)


def quantize_dev(w_f32: np.ndarray):
    """GPU quantization of a host fp32 weight; returns (NF4Tensor, status)."""
    w = f32_dev(w_f32)
    rows, cols = (w_f32.shape if w_f32.ndim == 2 else (1, w_f32.size))
    out = capi.NF4Tensor.empty(rows, cols)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    capi.nf4_quantize(w.view(rows, cols), out, status)
    return out, status


def nf4_host(t: capi.NF4Tensor):
    return (t.packed.cpu().numpy(), t.qabs.cpu().numpy(),
            t.gscale.cpu().numpy())
