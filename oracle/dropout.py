"""Reference (oracle) LoRA dropout on the adapter branch.  TEST
INFRASTRUCTURE ONLY, like the rest of this package.

What the pages fix: LoraConfig carries lora_dropout (0.05 in "Qlora
Expert", Core Concept code and "QLoRA Guide", Example; 0.1 in "QLoRA
Implementation Details (2025 Edition)", Step 4), next to r, lora_alpha and
bias "none".

Readings taken here (the pages fix none of the following):

* Dropout acts on the input of the adapter branch only, as inverted
  dropout: X_d = X * mask / (1 - p) with mask[m, k] ~ Bernoulli(1 - p),
  so y = X W'^T + s (X_d A^T) B^T.  The backward uses the same mask:
  dA = s G^T X_d and dX = dY W' + s (G A) * mask / (1 - p) (the bf16
  rounding of X_d is passed through as the identity), with G = dY B and
  dB = s dY^T T, T = X_d A^T.
* The mask comes from the counter-based generator Philox4x32-10 (Salmon,
  Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3",
  SC 2011): for element (m, k) of X [M, K] the counter is (k, m // 4, 0, 0),
  the key is (seed mod 2^32, seed // 2^32), and the word is output number
  m % 4.  The element is dropped when word < floor(p * 2^32) (computed in
  double), so four consecutive rows of one column share one generator call.
* X_d = bf16_rne(fp32(x * c)) for kept elements, +0 for dropped ones, with
  c = fp32(1 / (1 - p)) computed in double.  The linear algebra on X_d is
  exact (float64), as for the layer without dropout.
"""

from __future__ import annotations

import numpy as np

from .nf4_oracle import bf16_bits_to_f64, bf16_rne_bits

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
MASK32 = 0xFFFFFFFF


def philox4x32_10(ctr, key):
    """Philox4x32 with 10 rounds.

    ctr: 4 uint32 arrays (or scalars) of the same shape; key: 2 uint32
    values.  Each round multiplies words 0 and 2 by M0 and M1 (64-bit
    products split into high and low halves), returns
    (hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0), and adds (W0, W1) to the key.
    """
    x = [np.asarray(c, dtype=np.uint64) & MASK32 for c in ctr]
    k0, k1 = int(key[0]) & MASK32, int(key[1]) & MASK32
    for _ in range(10):
        p0 = np.uint64(PHILOX_M0) * x[0]            # < 2^64, exact
        p1 = np.uint64(PHILOX_M1) * x[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(MASK32)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(MASK32)
        x = [hi1 ^ x[1] ^ np.uint64(k0), lo1, hi0 ^ x[3] ^ np.uint64(k1), lo0]
        k0 = (k0 + PHILOX_W0) & MASK32
        k1 = (k1 + PHILOX_W1) & MASK32
    return [v.astype(np.uint32) for v in x]


def threshold(p: float) -> int:
    """Words below this are dropped: floor(p * 2^32), p in [0, 1)."""
    if not 0.0 <= p < 1.0:
        raise ValueError("dropout probability must be in [0, 1)")
    return min(int(np.floor(p * 4294967296.0)), MASK32)


def keep_scale(p: float) -> np.float32:
    return np.float32(1.0 / (1.0 - p))


def keep_mask(M: int, K: int, p: float, seed: int) -> np.ndarray:
    """bool [M, K]: True where the element is kept."""
    m = np.arange(M, dtype=np.uint64)[:, None]
    k = np.arange(K, dtype=np.uint64)[None, :]
    zero = np.zeros((M, K), dtype=np.uint64)
    words = philox4x32_10((k + zero, (m >> np.uint64(2)) + zero, zero, zero),
                          (seed & MASK32, (seed >> 32) & MASK32))
    sel = (np.arange(M) % 4)[:, None]
    w = np.choose(sel + np.zeros((M, K), dtype=np.int64), words)
    return w >= np.uint32(threshold(p))


def dropout_x_bits(x_bits: np.ndarray, p: float, seed: int) -> np.ndarray:
    """bf16 bits of X_d: bf16_rne(fp32(x * c)) where kept, +0 elsewhere."""
    M, K = x_bits.shape
    keep = keep_mask(M, K, p, seed)
    x32 = bf16_bits_to_f64(x_bits).astype(np.float32)
    scaled = bf16_rne_bits((x32 * keep_scale(p)).astype(np.float32))
    return np.where(keep, scaled, np.uint16(0)).astype(np.uint16)


def forward_f64(x, xd, w, a, b, s: float):
    """Y = X W'^T + s (X_d A^T) B^T and T = X_d A^T (float64 inputs)."""
    t = xd @ a.T
    return x @ w.T + s * (t @ b.T), t


def backward_f64(dy, x, xd, w, a, b, s: float, mask_scale, t):
    """dX = dY W' + s (G A) * mask_scale; dA = s G^T X_d; dB = s dY^T T."""
    g = dy @ b
    dx = dy @ w + s * (g @ a) * mask_scale
    return dx, s * (g.T @ xd), s * (dy.T @ t)


def qlora_forward_dropout(x_bits, w_bits, a_bits, b_bits, alpha: float,
                          r: int, p: float, seed: int):
    """(Y, T) in float64 from bf16 bit patterns, with LoRA dropout."""
    xd = bf16_bits_to_f64(dropout_x_bits(x_bits, p, seed))
    return forward_f64(bf16_bits_to_f64(x_bits), xd, bf16_bits_to_f64(w_bits),
                       bf16_bits_to_f64(a_bits), bf16_bits_to_f64(b_bits),
                       alpha / r)


def qlora_backward_dropout(dy_bits, x_bits, w_bits, a_bits, b_bits,
                           alpha: float, r: int, p: float, seed: int, t):
    """(dX, dA, dB) in float64, with the forward's mask."""
    M, K = x_bits.shape
    keep = keep_mask(M, K, p, seed)
    ms = np.where(keep, float(keep_scale(p)), 0.0)
    xd = bf16_bits_to_f64(dropout_x_bits(x_bits, p, seed))
    return backward_f64(bf16_bits_to_f64(dy_bits), bf16_bits_to_f64(x_bits), xd,
                        bf16_bits_to_f64(w_bits), bf16_bits_to_f64(a_bits),
                        bf16_bits_to_f64(b_bits), alpha / r, ms, t)
