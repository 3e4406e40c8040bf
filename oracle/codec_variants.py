"""Reference (oracle) codec variants: other 4-bit tables and other ways of
storing the per-block constants.  TEST INFRASTRUCTURE ONLY, like the rest of
this package.

The pages name the alternatives without defining them:

* "Qlora Expert", Hyperparameter Guidance: the quant type "fp4" exists beside
  "nf4"; double quantization is switched on or off; Memory Math prices the
  block constants at 0.5 bit per weight without double quantization
  (4 bits + 0.5 bits).
* "QLoRA Guide", NF4 vs uniform INT4: uniform INT4 spreads its codes evenly,
  NF4 places them at normal quantiles.
* "QLoRA Implementation Details (2025 Edition)", Step 1 NF4 Math: the
  signed 4-bit integer range [-8, 7]; 4 Key Innovations table: NF4 against
  INT4.
* "QLORA: Efficient Finetuning of Quantized LLMs" (paper summary),
  Takeaways: NF4 beats FP4 and Int4 on pretrained weights.

Readings taken here (all stated because the pages fix none of them):

* Every variant keeps the NF4 scheme -- absmax per block of 64, n = fp32(w/c)
  by one IEEE division, the code is the number of fp32 midpoint thresholds
  strictly below n (nearest level, ties to the lower code), two codes per
  byte -- and swaps only the sorted 16-entry level table.  The stored code
  is the index into that sorted table.
* FP4 table: the 16 values of the 4-bit float E2M1 (1 sign, 2 exponent bits
  with bias 1, 1 mantissa bit; exponent field 0 is subnormal, 0.5 * m), i.e.
  +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}, divided by the largest (6) so the table
  spans [-1, 1] like NF4's.  Its two zeros (+0 and -0) both become the value
  +0 in the table (indices 7 and 8).
* INT4 table: the signed integers -8..7 of the [-8, 7] range, each divided
  by 7 (absmax maps to 7; -8/7 lies beyond -1 and is never chosen).
* Block constants without double quantization ("DQ off"): the fp32 absmax
  itself, c' = c.
* Centered double quantization (the cited paper's idea of subtracting the
  mean before a symmetric 8-bit code; its 8-bit float map is not on the
  pages, so a linear signed code is used): per group of 256 constants,
  mu = fp32(S / n) with S their fp32 pairwise sum (adjacent pairs, then
  adjacent pair sums, ..., over the group padded with zeros to 256) and n
  the number of constants in the group; dev_b = fp32(c_b - mu);
  d = fp32(max_b |dev_b| / 127); q_b = clip(rint_half_even(fp32(dev_b / d)),
  -127, 127) as int8; d = 0 and q = 0 when every dev_b is 0.  Decoding:
  c' = fp32(fp32(q * d) + mu), two roundings, no fused multiply-add.
"""

from __future__ import annotations

import numpy as np

from .nf4_oracle import (
    BLOCK,
    GROUP,
    _blocks,
    bf16_rne_bits,
    block_absmax,
    double_quantize,
    nf4_codes,
    nf4_levels,
    pack_nibbles,
    unpack_nibbles,
)

CODE_NF4, CODE_FP4, CODE_INT4 = 0, 1, 2
DQ_U8, DQ_NONE, DQ_CENTERED = 0, 1, 2


# ---------------------------------------------------------------------------
# Level tables
# ---------------------------------------------------------------------------

def e2m1_value(bits: int) -> float:
    """Value of a 4-bit E2M1 float (sign bit 3, exponent bits 2-1 with bias
    1, mantissa bit 0; exponent 0 is subnormal with value 0.5 * mantissa)."""
    sign = -1.0 if bits & 8 else 1.0
    e = (bits >> 1) & 3
    m = bits & 1
    mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return sign * mag


def fp4_levels() -> np.ndarray:
    """The 16 E2M1 values / 6, sorted ascending, both zeros as +0 (fp32)."""
    vals = sorted(e2m1_value(b) for b in range(16))
    top = max(vals)
    return np.array([abs(v) / top if v == 0 else v / top for v in vals],
                    dtype=np.float64).astype(np.float32)


def int4_levels() -> np.ndarray:
    """The integers -8..7 divided by 7, rounded once to fp32."""
    return np.array([(j - 8) / 7.0 for j in range(16)],
                    dtype=np.float64).astype(np.float32)


def levels(code: int) -> np.ndarray:
    if code == CODE_NF4:
        return nf4_levels()
    if code == CODE_FP4:
        return fp4_levels()
    if code == CODE_INT4:
        return int4_levels()
    raise ValueError(f"unknown code table {code}")


def thresholds(code: int) -> np.ndarray:
    """fp32 midpoints of adjacent levels, computed in float64."""
    lv = levels(code).astype(np.float64)
    return ((lv[:-1] + lv[1:]) / 2.0).astype(np.float32)


def zero_code(code: int) -> int:
    """The code a zero weight takes (also the odd-tail pad nibble)."""
    return int(np.count_nonzero(thresholds(code) < np.float32(0.0)))


# ---------------------------------------------------------------------------
# Block constants
# ---------------------------------------------------------------------------

def pairwise_sum_f32(x: np.ndarray) -> np.float32:
    """fp32 sum of up to 256 values by adjacent pairs, level by level, over
    the values padded with zeros to 256."""
    a = np.zeros(GROUP, dtype=np.float32)
    a[: x.shape[0]] = x
    while a.shape[0] > 1:
        a = (a[0::2] + a[1::2]).astype(np.float32)
    return a[0]


def centered_quantize(absmax: np.ndarray):
    """Centered signed 8-bit codes of the block constants.

    Returns (q int8[nb], d float32[ng], mu float32[ng]).
    """
    c = np.ascontiguousarray(absmax, dtype=np.float32)
    nb = c.shape[0]
    ng = -(-nb // GROUP)
    q = np.zeros(nb, dtype=np.int8)
    d = np.zeros(ng, dtype=np.float32)
    mu = np.zeros(ng, dtype=np.float32)
    for g, (s, e) in enumerate(_blocks(c, GROUP)):
        m = pairwise_sum_f32(c[s:e]) / np.float32(e - s)   # fp32 division
        mu[g] = m
        dev = (c[s:e] - m).astype(np.float32)
        dmax = np.abs(dev).max()
        if dmax == 0:
            continue
        dg = np.float32(dmax) / np.float32(127.0)
        d[g] = dg
        ratio = (dev / dg).astype(np.float32)
        q[s:e] = np.clip(np.rint(ratio), -127.0, 127.0).astype(np.int8)
    return q, d, mu


def block_constants(packed_consts, gscale, gmean, nb: int, dq: int) -> np.ndarray:
    """Decoded block constants c' (fp32[nb]) for each storage mode."""
    blk = np.arange(nb)
    if dq == DQ_NONE:
        return np.ascontiguousarray(packed_consts, dtype=np.float32)[:nb]
    if dq == DQ_U8:
        return (np.asarray(packed_consts, dtype=np.uint8).astype(np.float32)
                * gscale[blk // GROUP]).astype(np.float32)
    if dq == DQ_CENTERED:
        qd = (np.asarray(packed_consts, dtype=np.int8).astype(np.float32)
              * gscale[blk // GROUP]).astype(np.float32)
        return (qd + gmean[blk // GROUP]).astype(np.float32)
    raise ValueError(f"unknown constant mode {dq}")


# ---------------------------------------------------------------------------
# Quantize / dequantize
# ---------------------------------------------------------------------------

def quantize(w: np.ndarray, code: int, dq: int):
    """(packed, consts, gscale, gmean) of a weight for one variant.

    consts is uint8 (DQ_U8), float32 (DQ_NONE) or int8 (DQ_CENTERED) per
    block; gscale and gmean are float32 per group (empty where the mode has
    none).  Codes are always taken against the un-quantized block constant.
    """
    flat = np.ascontiguousarray(w, dtype=np.float32).reshape(-1)
    c = block_absmax(flat)
    codes = nf4_codes(flat, c, thresholds(code))
    packed = pack_nibbles(codes, pad=zero_code(code))
    empty = np.zeros(0, dtype=np.float32)
    if dq == DQ_NONE:
        return packed, c.copy(), empty, empty
    if dq == DQ_U8:
        q, d = double_quantize(c)
        return packed, q, d, empty
    if dq == DQ_CENTERED:
        q, d, mu = centered_quantize(c)
        return packed, q, d, mu
    raise ValueError(f"unknown constant mode {dq}")


def dequantize(packed, consts, gscale, gmean, numel: int, code: int,
               dq: int) -> np.ndarray:
    """bf16 bit patterns of w' = bf16_rne(fp32(L[code] * c'))."""
    nb = -(-numel // BLOCK)
    cp = block_constants(consts, gscale, gmean, nb, dq)
    codes = unpack_nibbles(packed, numel)
    vals = (levels(code)[codes] * cp[np.arange(numel) // BLOCK]).astype(np.float32)
    return bf16_rne_bits(vals)


def bits_per_weight(dq: int) -> float:
    """Storage per weight: 4-bit code plus the block constants' share."""
    per_block = {DQ_NONE: 32.0, DQ_U8: 8.0 + 32.0 / GROUP,
                 DQ_CENTERED: 8.0 + 64.0 / GROUP}[dq]
    return 4.0 + per_block / BLOCK
