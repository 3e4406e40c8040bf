"""Reference (oracle) implementation of the QLoRA linear layer, on the CPU.

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Plain NumPy, float32
wherever a rounding is part of the definition of the codec, float64 for the
linear algebra.  Slow on purpose: no blocking, fusion or reordering beyond
what the definitions state.

Sources (the pages, cited by title and section):

* "Qlora Expert" (skillsdirectory.com), section "Core Concept": NF4 places its
  16 levels at quantiles of N(0,1); double quantization quantizes the
  per-block fp32 constants to 8 bit; the frozen base is dequantized to bf16
  on the fly and never receives a gradient.
* "QLoRA: The 4-bit Revolution" (shshell.com), sections "1. 4-bit NormalFloat
  (NF4)" and "2. Double Quantization": 4 bits per weight, one scaling factor
  per block, scaling factors compressed from 32 to 8 bit.
* "QLoRA Implementation Details (2025 Edition)" (spritualkrishna.cloud),
  "Step 1 ... NF4 Math": blocks of 64 values; "Step 4": LoRA scale alpha/r.
* "QLoRA Guide" (dataaihub.co), "How QLoRA Works / Forward pass" diagram:
  output = W_bf16 x + B(A(x)); only A and B receive gradients, the
  dequantized W is a constant.  "NF4 vs uniform INT4": block-wise scaling.
* "QLORA: Efficient Finetuning of Quantized LLMs" (paper summary), "Notes":
  every pass loads 4-bit weights, dequantizes to BF16, multiplies, and
  computes gradients for the adapters only.

Readings taken where the pages are silent:

* Level construction: the pages fix only "16 levels at N(0,1) quantiles"
  containing an exact zero and +-1.  Read: 8 positive levels at the
  quantiles of equally spaced probabilities from 1/2 (exclusive) to delta,
  7 negative levels likewise, plus 0, normalised by the largest, with
  delta = 1 - (1/32 + 1/30)/2.
* Block scale = absmax of the 64 weights; a weight maps to the nearest level
  through fp32 midpoint thresholds, ties to the lower code.
* w / absmax is one IEEE fp32 division (round to nearest even).
* Double quantization: per group of 256 block constants, d = fp32(max/255),
  q = min(255, rint_half_even(fp32(c / d))); unsigned, no offset.  NF4 codes
  are taken against the un-quantized block constant.
* Dequantization: c' = fp32(fp32(q) * d); w' = bf16_rne(fp32(L[code] * c')).
* Packing: element 2i in bits 0-3 of byte i, element 2i+1 in bits 4-7;
  blocks and groups run over the row-major flattened weight; short tail
  block/group; an odd tail nibble is 7 (the zero level).
"""

from __future__ import annotations

import statistics

import numpy as np

BLOCK = 64     # weights per absmax block ("NF4 Math": 64 values/block)
GROUP = 256    # block constants per double-quantization group

_DELTA = 1.0 - 0.5 * (1.0 / 32.0 + 1.0 / 30.0)


# ---------------------------------------------------------------------------
# Codebook
# ---------------------------------------------------------------------------

def nf4_levels() -> np.ndarray:
    """The 16 NF4 levels as fp32, sorted ascending.

    "Qlora Expert", Core Concept: the 16 levels sit at quantiles of N(0,1).
    The level offset delta and the 7/8 split of negative/positive levels are
    a reading (module docstring): positive levels at probabilities
    delta, ..., spaced by (delta - 1/2)/8 toward 1/2 (1/2 itself excluded);
    negative levels mirror 7 probabilities spaced by (delta - 1/2)/7; plus an
    exact 0.  All values are divided by the largest so the set spans [-1, 1].
    Computed in float64 (statistics.NormalDist().inv_cdf), rounded once to
    fp32.
    """
    inv = statistics.NormalDist().inv_cdf
    pos = [inv(_DELTA + (0.5 - _DELTA) * i / 8.0) for i in range(8)]
    neg = [-inv(_DELTA + (0.5 - _DELTA) * i / 7.0) for i in range(7)]
    vals = sorted(pos + neg + [0.0])
    top = max(vals)
    return np.array([v / top for v in vals], dtype=np.float64).astype(np.float32)


def nf4_thresholds(levels: np.ndarray | None = None) -> np.ndarray:
    """15 fp32 decision thresholds: midpoints of adjacent levels.

    Nearest-level rounding ("minimizing quantization error", "Qlora Expert",
    Core Concept) through midpoints t_j = fp32((L_j + L_{j+1}) / 2), computed
    in float64 from the fp32 levels.
    """
    lv = nf4_levels() if levels is None else levels
    l64 = lv.astype(np.float64)
    return ((l64[:-1] + l64[1:]) / 2.0).astype(np.float32)


# ---------------------------------------------------------------------------
# bf16 helpers
# ---------------------------------------------------------------------------

def bf16_rne_bits(x) -> np.ndarray:
    """fp32 -> bf16 bit pattern (uint16) by round-to-nearest-even on the bits.

    "QLORA ... paper summary", Notes: weights are dequantized to BF16.  Finite
    inputs only: the upper 16 bits after adding 0x7FFF plus the lowest kept
    bit.
    """
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of a bf16 bit pattern, as float64."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_rne_from_f64(v) -> np.ndarray:
    """float64 -> bf16 bit pattern, rounded once to the nearest bf16 value,
    ties to even (no intermediate fp32 rounding).  Finite inputs only.

    A bf16 value has 8 significant bits: with |v| = f * 2**e, f in [0.5, 1)
    (frexp, exact), the representable neighbours are integer multiples of
    2**(e - 8) (of 2**-133 below the normal range), so the rounding is
    rint(|v| / 2**(e - 8)) -- an exact power-of-two scaling followed by
    NumPy's round-half-to-even.
    """
    a = np.ascontiguousarray(v, dtype=np.float64)
    _, e = np.frexp(np.abs(a))
    ulp_exp = np.maximum(e.astype(np.int64) - 8, -133)
    q = np.rint(np.ldexp(np.abs(a), -ulp_exp))          # exact scaling
    mag = np.ldexp(q, ulp_exp).astype(np.float32)        # exact in bf16
    out = np.where(np.signbit(a), -mag, mag).astype(np.float32)
    return (out.view(np.uint32) >> 16).astype(np.uint16)


# ---------------------------------------------------------------------------
# NF4 block quantization
# ---------------------------------------------------------------------------

def _blocks(flat: np.ndarray, size: int):
    """Yield (start, stop) of consecutive blocks of ``size``; short tail."""
    n = flat.shape[0]
    for s in range(0, n, size):
        yield s, min(s + size, n)


def block_absmax(w: np.ndarray) -> np.ndarray:
    """Per-block fp32 constant c_b = max |w| over each block of 64.

    "QLoRA Implementation Details", NF4 Math: block-wise quantization, 64
    values per block; "QLoRA Guide", NF4 vs uniform INT4: block-wise scaling
    limits how far an outlier spreads.  Blocks run over the row-major
    flattened tensor; the last block may be short.
    """
    flat = np.ascontiguousarray(w, dtype=np.float32).reshape(-1)
    if not np.all(np.isfinite(flat)):
        raise ValueError("non-finite weight")
    nb = -(-flat.shape[0] // BLOCK)
    c = np.zeros(nb, dtype=np.float32)
    full = (flat.shape[0] // BLOCK) * BLOCK
    if full:
        c[: full // BLOCK] = np.abs(flat[:full]).reshape(-1, BLOCK).max(axis=1)
    if full < flat.shape[0]:
        c[-1] = np.abs(flat[full:]).max()
    return c


def nf4_codes(w: np.ndarray, absmax: np.ndarray,
              thresholds: np.ndarray | None = None) -> np.ndarray:
    """4-bit code per weight (uint8 in 0..15).

    n = fp32(w / c_b) by one IEEE fp32 division (n = 0 when c_b = 0); the
    code is the number of thresholds strictly below n, i.e. the index of the
    nearest level with ties going to the lower code.  ``thresholds`` defaults
    to the NF4 midpoints; another sorted 16-level table's midpoints give the
    same rule for that table.
    """
    flat = np.ascontiguousarray(w, dtype=np.float32).reshape(-1)
    t = nf4_thresholds() if thresholds is None else thresholds
    codes = np.empty(flat.shape[0], dtype=np.uint8)
    chunk = 1 << 22
    for s in range(0, flat.shape[0], chunk):
        e = min(s + chunk, flat.shape[0])
        idx = np.arange(s, e) // BLOCK
        c = absmax[idx]
        n = np.zeros(e - s, dtype=np.float32)
        nz = c != 0
        n[nz] = flat[s:e][nz] / c[nz]          # float32 / float32 -> IEEE RNE
        count = np.zeros(e - s, dtype=np.uint8)
        for j in range(t.shape[0]):
            count += (n > t[j]).astype(np.uint8)
        codes[s:e] = count
    return codes


def pack_nibbles(codes: np.ndarray, pad: int = 7) -> np.ndarray:
    """Two codes per byte: element 2i in bits 0-3, element 2i+1 in bits 4-7.

    "QLoRA: The 4-bit Revolution", section 1: 4 bits per number.  The nibble
    order is a reading; an odd tail is padded with ``pad``, the code a zero
    weight takes (7, the NF4 zero level, by default).
    """
    c = np.ascontiguousarray(codes, dtype=np.uint8).reshape(-1)
    if c.shape[0] % 2:
        c = np.concatenate([c, np.array([pad], dtype=np.uint8)])
    return (c[0::2] | (c[1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray, numel: int) -> np.ndarray:
    """Inverse of pack_nibbles, trimmed to ``numel`` codes."""
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[0] * 2, dtype=np.uint8)
    out[0::2] = p & 0x0F
    out[1::2] = p >> 4
    return out[:numel]


# ---------------------------------------------------------------------------
# Double quantization of the block constants
# ---------------------------------------------------------------------------

def double_quantize(absmax: np.ndarray):
    """8-bit codes for the block constants, one fp32 scale per 256 of them.

    "Qlora Expert", Core Concept: the per-block fp32 quantization constants
    are themselves quantized to 8 bit; "QLoRA: The 4-bit Revolution",
    section 2: scaling factors go from 32-bit to 8-bit.  Group size 256 and
    the unsigned linear code are a reading: per group, s = max c_b,
    d = fp32(s / 255); q_b = min(255, rint_half_even(fp32(c_b / d))); a zero
    group gets d = 0 and q = 0.

    Returns (q uint8[nb], d float32[ng]).
    """
    c = np.ascontiguousarray(absmax, dtype=np.float32)
    nb = c.shape[0]
    ng = -(-nb // GROUP)
    q = np.zeros(nb, dtype=np.uint8)
    d = np.zeros(ng, dtype=np.float32)
    for g, (s, e) in enumerate(_blocks(c, GROUP)):
        smax = c[s:e].max()
        if smax == 0:
            continue
        dg = np.float32(smax) / np.float32(255.0)
        d[g] = dg
        ratio = c[s:e] / dg                      # float32 / float32
        q[s:e] = np.minimum(np.rint(ratio), 255.0).astype(np.uint8)
    return q, d


def nf4_quantize(w: np.ndarray):
    """Full quantization of a frozen weight: (packed, q, d).

    Composition of block_absmax, nf4_codes (against the un-quantized block
    constant), pack_nibbles and double_quantize.  Raises ValueError on a
    non-finite weight.
    """
    flat = np.ascontiguousarray(w, dtype=np.float32).reshape(-1)
    c = block_absmax(flat)
    codes = nf4_codes(flat, c)
    q, d = double_quantize(c)
    return pack_nibbles(codes), q, d


# ---------------------------------------------------------------------------
# Dequantization
# ---------------------------------------------------------------------------

def nf4_dequantize(packed: np.ndarray, q: np.ndarray, d: np.ndarray,
                   numel: int) -> np.ndarray:
    """bf16 bit patterns (uint16[numel]) of the dequantized weight.

    "QLORA ... paper summary", Notes: load the 4-bit weights, dequantize to
    BF16.  Per block: c' = fp32(fp32(q_b) * d_g); per weight:
    w' = bf16_rne(fp32(L[code] * c')).
    """
    lv = nf4_levels()
    codes = unpack_nibbles(packed, numel)
    blk = np.arange(numel) // BLOCK
    cprime = q.astype(np.float32)[blk] * d[blk // GROUP]     # float32 product
    vals = lv[codes] * cprime                               # float32 product
    return bf16_rne_bits(vals)


# ---------------------------------------------------------------------------
# Fused QLoRA linear: forward and backward (float64, exact inputs)
# ---------------------------------------------------------------------------

def forward_f64(x, w, a, b, s: float):
    """Y = X W^T + s (X A^T) B^T and T = X A^T on float64 values.

    "QLoRA Guide", Forward pass diagram: the dequantized W times x is summed
    with B(A(x)); "QLoRA Implementation Details", Step 4: the adapter branch
    is scaled by alpha/r.  Shapes follow the Linear convention: W [N,K],
    X [M,K], A [r,K], B [N,r].  Returns (Y [M,N], T [M,r]).
    """
    t = x @ a.T
    y = x @ w.T + s * (t @ b.T)
    return y, t


def backward_f64(dy, x, w, a, b, s: float, t=None):
    """(dX, dA, dB) of the fused linear on float64 values; no gradient to W.

    "QLoRA Guide", Forward pass: only A and B receive gradients, the
    dequantized W is treated as a constant; "QLORA ... paper summary", Notes:
    gradients only for the LoRA adapters.  With G = dY B:
      dX = dY W + s G A,  dA = s G^T X,  dB = s dY^T T,  T = X A^T.
    """
    if t is None:
        t = x @ a.T
    g = dy @ b
    dx = dy @ w + s * (g @ a)
    da = s * (g.T @ x)
    db = s * (dy.T @ t)
    return dx, da, db


def qlora_forward(x_bits, w_bits, a_bits, b_bits, alpha: float, r: int):
    """Forward of the QLoRA linear on bf16 bit-pattern inputs.

    X, the dequantized W' (from nf4_dequantize), A and B are used at their
    exact bf16 values; s = alpha / r; float64 arithmetic (forward_f64).
    Returns (Y [M,N], T [M,r]) as float64.
    """
    s = float(alpha) / float(r)
    return forward_f64(bf16_bits_to_f64(x_bits), bf16_bits_to_f64(w_bits),
                       bf16_bits_to_f64(a_bits), bf16_bits_to_f64(b_bits), s)


def qlora_backward(dy_bits, x_bits, w_bits, a_bits, b_bits, alpha: float,
                   r: int, t=None):
    """Backward of the QLoRA linear on bf16 bit-pattern inputs: (dX, dA, dB).

    s = alpha / r; float64 arithmetic (backward_f64); ``t`` is the forward's
    T = X A^T, recomputed when omitted.
    """
    s = float(alpha) / float(r)
    return backward_f64(bf16_bits_to_f64(dy_bits), bf16_bits_to_f64(x_bits),
                        bf16_bits_to_f64(w_bits), bf16_bits_to_f64(a_bits),
                        bf16_bits_to_f64(b_bits), s, t)


# ---------------------------------------------------------------------------
# Dequantize-and-merge
# ---------------------------------------------------------------------------

def merge_f64(w_bits, a_bits, b_bits, s: float):
    """Merged dense weight bf16(W' + s B A) and its exact value.

    "Qlora Expert", When to Use and Common Pitfalls: the adapter can be
    merged into a dense model only after dequantizing the base, which
    materialises the full bf16 weight; "QLoRA Implementation Details (2025
    Edition)", Step 7 (Merge & Save).  Reading: the merged weight is the
    dequantized base W' [N,K] plus the scaled low-rank update s B A
    (B [N,r], A [r,K]), computed exactly (float64 on the exact bf16 inputs)
    and rounded once to bf16.  Returns (bits uint16 [N,K], value float64).
    """
    w = bf16_bits_to_f64(w_bits)
    a = bf16_bits_to_f64(a_bits)
    b = bf16_bits_to_f64(b_bits)
    v = w + float(s) * (b @ a)
    return bf16_rne_from_f64(v), v
