"""Reference (oracle) 8-bit AdamW step on the LoRA adapters.  TEST
INFRASTRUCTURE ONLY, like the rest of this package.

What the pages fix:

* "Qlora Expert", Core Concept item 3 and Hyperparameter Guidance: paged
  optimizers keep the Adam moments in memory that pages between GPU and CPU
  RAM; the optimizer is "paged_adamw_8bit", 8-bit Adam states; learning rate
  2e-4 (7B-13B).
* "QLoRA Implementation Details (2025 Edition)", Step 5 Paged Optimizer:
  states in CPU RAM, paged in and out as needed; max_grad_norm 0.3.
* "QLORA ... paper summary", Notes: the adapters are stored and trained in
  BF16.

Readings taken here (the pages fix none of the following):

* AdamW = Adam with decoupled weight decay (Loshchilov and Hutter), the
  update torch.optim.AdamW performs: p <- p (1 - lr wd);
  m <- b1 m + (1 - b1) g; v <- b2 v + (1 - b2) g^2;
  p <- p - lr * (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps).
* Every step runs in fp32 in one fixed order, with no fused multiply-add,
  so the 8-bit codes and the bf16 parameter are decided by the same fp32
  values on every implementation.  The host constants are rounded once to
  fp32 from double: c1 = 1 - b1, c2 = 1 - b2, bc1 = 1 / (1 - b1^t),
  bc2 = 1 / (1 - b2^t), decay = 1 - lr wd.  Per element, with g already
  multiplied by the caller's gradient factor gs (fp32 product; gs carries
  gradient clipping):
      m  = b1 m' + c1 g                 (each product and the sum in fp32)
      v  = b2 v' + c2 (g g)
      u  = (m bc1) / (sqrt(v bc2) + eps)   (IEEE sqrt and division)
      p  = bf16_rne(p decay - lr u)
  where m', v' are the decoded stored moments.  The parameter update uses
  the fresh fp32 m, v; only the stored state is quantized.
* The 8-bit state: blocks of 256 consecutive elements; m is stored as the
  FP8 E4M3 code of m / s_m with s_m = fp32(max|m| / 448), and the second
  moment as the E4M3 code of r / s_r with r = sqrt(v) (fp32) and
  s_r = fp32(max r / 448), i.e. in the square-root domain, which halves
  the exponent range the code has to cover.  A block of zeros has scale 0
  and codes 0.  Decoding: m' = fp32(E4M3(code) s_m); r' = fp32(E4M3 s_r),
  v' = fp32(r' r').  A fresh state is all zero.
* E4M3 is the OCP 8-bit float (1 sign, 4 exponent bits with bias 7, 3
  mantissa bits, subnormals below 2^-6, largest finite 448, no infinity).
  Encoding rounds to nearest, ties to even, after clamping the magnitude to
  448; a value that rounds to zero is stored as code 0 (no -0).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .nf4_oracle import bf16_bits_to_f64, bf16_rne_bits

STATE_BLOCK = 256
E4M3_MAX = 448.0


# ---------------------------------------------------------------------------
# FP8 E4M3
# ---------------------------------------------------------------------------

def e4m3_value(code: np.ndarray) -> np.ndarray:
    """Exact value (float64) of E4M3 codes (uint8); NaN codes excluded."""
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    return sign * mag


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """E4M3 codes of fp32 values: clamp |x| to 448, round to nearest even."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)   # exact
    a = np.minimum(np.abs(x), E4M3_MAX)
    codes = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # subnormal range: multiples of 2^-9 (q = 8 is the smallest normal,
    # whose code is 8 as well)
    codes[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)
    nrm = ~sub
    if np.any(nrm):
        f, e = np.frexp(a[nrm])           # a = f 2^e, f in [0.5, 1)
        e = e.astype(np.int64) - 1        # a = (2f) 2^e, 2f in [1, 2)
        q = np.rint((2.0 * f - 1.0) * 8.0).astype(np.int64)
        carry = q == 8
        e = e + carry
        q = np.where(carry, 0, q)
        codes[nrm] = ((e + 7) << 3) | q
    neg = (x < 0) & (codes != 0)
    codes = codes | np.where(neg, 0x80, 0)
    return codes.astype(np.uint8)


# ---------------------------------------------------------------------------
# Blockwise 8-bit state
# ---------------------------------------------------------------------------

def quantize_state(x: np.ndarray):
    """(codes uint8[n], scales float32[ceil(n/256)]) of an fp32 vector."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    n = x.size
    nb = -(-n // STATE_BLOCK)
    codes = np.zeros(n, dtype=np.uint8)
    scales = np.zeros(nb, dtype=np.float32)
    for b in range(nb):
        s, e = b * STATE_BLOCK, min(b * STATE_BLOCK + STATE_BLOCK, n)
        amax = np.abs(x[s:e]).max()
        if amax == 0:
            continue
        sc = np.float32(amax) / np.float32(E4M3_MAX)           # fp32 division
        scales[b] = sc
        codes[s:e] = e4m3_encode((x[s:e] / sc).astype(np.float32))
    return codes, scales


def dequantize_state(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """fp32 values fp32(E4M3(code) * scale)."""
    n = codes.size
    blk = np.arange(n) // STATE_BLOCK
    v = e4m3_value(codes).astype(np.float32)                   # exact
    return (v * scales[blk]).astype(np.float32)


# ---------------------------------------------------------------------------
# The step
# ---------------------------------------------------------------------------

@dataclass
class HParams:
    lr: float = 2e-4
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0
    grad_scale: float = 1.0

    def constants(self, step: int):
        """fp32 constants of step `step` (1-based), each rounded once from
        double."""
        f = np.float32
        return dict(
            b1=f(self.beta1), b2=f(self.beta2), c1=f(1.0 - self.beta1),
            c2=f(1.0 - self.beta2), bc1=f(1.0 / (1.0 - self.beta1 ** step)),
            bc2=f(1.0 / (1.0 - self.beta2 ** step)), eps=f(self.eps),
            lr=f(self.lr), decay=f(1.0 - self.lr * self.weight_decay),
            gs=f(self.grad_scale))


@dataclass
class State8:
    m_codes: np.ndarray
    m_scales: np.ndarray
    r_codes: np.ndarray
    r_scales: np.ndarray

    @staticmethod
    def zeros(n: int) -> "State8":
        nb = -(-n // STATE_BLOCK)
        return State8(np.zeros(n, np.uint8), np.zeros(nb, np.float32),
                      np.zeros(n, np.uint8), np.zeros(nb, np.float32))


def moments_f32(m_old, v_old, g, k):
    """New fp32 moments from fp32 old moments and the fp32 gradient."""
    g = (np.asarray(g, np.float32) * k["gs"]).astype(np.float32)
    m = ((k["b1"] * m_old).astype(np.float32)
         + (k["c1"] * g).astype(np.float32)).astype(np.float32)
    gg = (g * g).astype(np.float32)
    v = ((k["b2"] * v_old).astype(np.float32)
         + (k["c2"] * gg).astype(np.float32)).astype(np.float32)
    return m, v


def param_update_f32(p32, m, v, k):
    """fp32 parameter after one step from the fresh fp32 moments."""
    den = (np.sqrt((v * k["bc2"]).astype(np.float32)) + k["eps"]).astype(np.float32)
    u = ((m * k["bc1"]).astype(np.float32) / den).astype(np.float32)
    return ((p32 * k["decay"]).astype(np.float32)
            - (k["lr"] * u).astype(np.float32)).astype(np.float32)


def adamw8_step(p_bits: np.ndarray, g: np.ndarray, st: State8, hp: HParams,
                step: int):
    """One 8-bit AdamW step.  Returns (new bf16 bits, new State8)."""
    k = hp.constants(step)
    m_old = dequantize_state(st.m_codes, st.m_scales)
    r_old = dequantize_state(st.r_codes, st.r_scales)
    v_old = (r_old * r_old).astype(np.float32)
    m, v = moments_f32(m_old, v_old, g, k)
    p32 = bf16_bits_to_f64(p_bits).astype(np.float32)
    p_new = bf16_rne_bits(param_update_f32(p32, m, v, k))
    mc, ms = quantize_state(m)
    rc, rs = quantize_state(np.sqrt(v).astype(np.float32))
    return p_new, State8(mc, ms, rc, rs)


def adamw_step_f32(p32: np.ndarray, g: np.ndarray, m: np.ndarray,
                   v: np.ndarray, hp: HParams, step: int):
    """The same step with fp32 parameters and unquantized fp32 moments
    (the 32-bit optimizer the 8-bit one approximates)."""
    k = hp.constants(step)
    m, v = moments_f32(m, v, g, k)
    return param_update_f32(np.asarray(p32, np.float32), m, v, k), m, v
