// HIP kernels (gfx950 / CDNA4) and C-ABI entry points of the QLoRA NF4
// linear-layer library.  Declarations and the contract of every entry point
// are in include/qlora_nf4.h.
//
// What is computed follows the pages "Qlora Expert" (Core Concept: NF4 at
// N(0,1) quantiles, double quantization of the block constants, bf16
// compute), "QLoRA Implementation Details (2025 Edition)" (Step 1 NF4 Math:
// 64-value blocks; Step 4: scale alpha/r), "QLoRA Guide" (Forward pass
// diagram: W_bf16 x + B(A(x)); only A and B get gradients) and the "QLORA ...
// paper summary" (Notes: load 4-bit, dequantize to BF16, multiply, adapter
// gradients only).
//
// Kernels
//   k_quantize     one workgroup per double-quant group (256 blocks)
//   k_dequant      packed-nibble stream, 32 weights per thread
//   k_fwd_gemm     Y = X W'^T (+ s T B^T as extra reduction steps), W'
//                  dequantized into LDS tile by tile, bf16 MFMA 32x32x16
//   k_bwd_dx_gemm  dX = dY W' (+ s G A), W' tile dequantized into LDS and
//                  read transposed
//   k_rank_stream  one pass over X or dY for the rank-r products: row sums
//                  (T = X A^T, G = dY B) and column sums (dB = dY^T s T,
//                  dA = (s G)^T X) as per-block partials
//   k_rank_finish  fixed-order reduction of those partials (no atomics) and
//                  the small layout conversions of A, B and T
//   k_skinny_*     forward for M <= 16 tokens (GEMV over the NF4 weight)
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>

#include "qlora_nf4.h"
#include "qn_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Codebook passed by value as a kernel argument (lands in SGPRs).
struct Codebook {
  float L[16];
  float T[15];
};

// ---------------------------------------------------------------------------
// bf16 helpers
// ---------------------------------------------------------------------------

// Two fp32 -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

__device__ __forceinline__ uint32_t perm(uint32_t s0, uint32_t s1,
                                         uint32_t sel) {
  return __builtin_amdgcn_perm(s0, s1, sel);
}

// (mask & a) | (~mask & b), a single v_bfi_b32.
__device__ __forceinline__ uint32_t bfi(uint32_t mask, uint32_t a,
                                        uint32_t b) {
  return (mask & a) | (~mask & b);
}

// ---------------------------------------------------------------------------
// NF4 decode: per-block 16-entry bf16 table, byte-sliced for v_perm_b32.
//
// For one block with constant c' = float(q) * d, entry j is
// bf16_rne(L[j] * c') (both products fp32).  The 16 bf16 entries are kept as
// four 8-byte tables: low bytes of entries 0-7 (ll) and 8-15 (lh), high
// bytes of entries 0-7 (hl) and 8-15 (hh).  A code's low 3 bits select a
// byte with v_perm_b32; its bit 3 chooses between the two halves.
// ---------------------------------------------------------------------------
struct Lut {
  uint32_t ll0, ll1, lh0, lh1, hl0, hl1, hh0, hh1;
};

__device__ __forceinline__ float block_cprime(const uint8_t* __restrict__ qabs,
                                              const float* __restrict__ gscale,
                                              int64_t block) {
  return static_cast<float>(qabs[block]) * gscale[block >> 8];
}

__device__ __forceinline__ Lut make_lut(const Codebook& cb, float cp) {
  uint32_t P[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
    P[k] = pack_bf16x2(cb.L[2 * k] * cp, cb.L[2 * k + 1] * cp);
  Lut t;
  // P[k] bytes: [lo e2k, hi e2k, lo e2k+1, hi e2k+1]
  t.ll0 = perm(P[1], P[0], 0x06040200u);
  t.hl0 = perm(P[1], P[0], 0x07050301u);
  t.ll1 = perm(P[3], P[2], 0x06040200u);
  t.hl1 = perm(P[3], P[2], 0x07050301u);
  t.lh0 = perm(P[5], P[4], 0x06040200u);
  t.hh0 = perm(P[5], P[4], 0x07050301u);
  t.lh1 = perm(P[7], P[6], 0x06040200u);
  t.hh1 = perm(P[7], P[6], 0x07050301u);
  return t;
}

// 8 codes (one packed dword, element i in bits 4i..4i+3) -> 8 bf16 in
// natural order (out[i] holds elements 2i, 2i+1, low half first).
__device__ __forceinline__ u32x4 decode8(uint32_t p, const Lut& t) {
  const uint32_t se = p & 0x07070707u;          // codes 0,2,4,6 (low 3 bits)
  const uint32_t so = (p >> 4) & 0x07070707u;   // codes 1,3,5,7
  // 0xFF per byte where bit 3 of the code is set (v_perm sign replication)
  const uint32_t me = perm(p << 4, p << 12, 0x0B090A08u);
  const uint32_t mo = perm(p, p << 8, 0x0B090A08u);
  const uint32_t le = bfi(me, perm(t.lh1, t.lh0, se), perm(t.ll1, t.ll0, se));
  const uint32_t he = bfi(me, perm(t.hh1, t.hh0, se), perm(t.hl1, t.hl0, se));
  const uint32_t lo = bfi(mo, perm(t.lh1, t.lh0, so), perm(t.ll1, t.ll0, so));
  const uint32_t ho = bfi(mo, perm(t.hh1, t.hh0, so), perm(t.hl1, t.hl0, so));
  // low bytes of elements 0..3 and 4..7, then high bytes
  const uint32_t l03 = perm(lo, le, 0x05010400u);
  const uint32_t l47 = perm(lo, le, 0x07030602u);
  const uint32_t h03 = perm(ho, he, 0x05010400u);
  const uint32_t h47 = perm(ho, he, 0x07030602u);
  u32x4 r;
  r.x = perm(h03, l03, 0x05010400u);
  r.y = perm(h03, l03, 0x07030602u);
  r.z = perm(h47, l47, 0x05010400u);
  r.w = perm(h47, l47, 0x07030602u);
  return r;
}

// Same lookup as decode8, with the 8 outputs in the order
// (0,2) (4,6) (1,3) (5,7): four v_perm_b32 fewer.  Only usable where the
// other MFMA operand is permuted the same way (permute8 below), because the
// order of a dot product's terms is free.
__device__ __forceinline__ u32x4 decode8p(uint32_t p, const Lut& t) {
  const uint32_t se = p & 0x07070707u;
  const uint32_t so = (p >> 4) & 0x07070707u;
  const uint32_t me = perm(p << 4, p << 12, 0x0B090A08u);
  const uint32_t mo = perm(p, p << 8, 0x0B090A08u);
  const uint32_t le = bfi(me, perm(t.lh1, t.lh0, se), perm(t.ll1, t.ll0, se));
  const uint32_t he = bfi(me, perm(t.hh1, t.hh0, se), perm(t.hl1, t.hl0, se));
  const uint32_t lo = bfi(mo, perm(t.lh1, t.lh0, so), perm(t.ll1, t.ll0, so));
  const uint32_t ho = bfi(mo, perm(t.hh1, t.hh0, so), perm(t.hl1, t.hl0, so));
  u32x4 r;
  r.x = perm(he, le, 0x05010400u);   // elements 0, 2
  r.y = perm(he, le, 0x07030602u);   // elements 4, 6
  r.z = perm(ho, lo, 0x05010400u);   // elements 1, 3
  r.w = perm(ho, lo, 0x07030602u);   // elements 5, 7
  return r;
}

// 8 consecutive bf16 (natural order) -> the order of decode8p.
__device__ __forceinline__ u32x4 permute8(const u32x4& v) {
  u32x4 r;
  r.x = perm(v.y, v.x, 0x05040100u);
  r.y = perm(v.w, v.z, 0x05040100u);
  r.z = perm(v.y, v.x, 0x07060302u);
  r.w = perm(v.w, v.z, 0x07060302u);
  return r;
}

// One element, used for ragged tails.
__device__ __forceinline__ uint16_t decode1(const Codebook& cb, uint32_t code,
                                            float cp) {
  return static_cast<uint16_t>(pack_bf16x2(cb.L[code] * cp, 0.0f) & 0xFFFFu);
}

// ---------------------------------------------------------------------------
// K1: quantization + double quantization.  One workgroup per group of 256
// blocks (16384 weights); each thread owns 8 consecutive weights in each of
// 8 passes (8 lanes per 64-weight block).
// ---------------------------------------------------------------------------
constexpr int QZ_THREADS = 256;
constexpr int QZ_PASSES = 8;  // 8 * 256 * 8 = 16384 weights

__global__ __launch_bounds__(QZ_THREADS) void k_quantize(
    const float* __restrict__ w, int64_t numel, uint8_t* __restrict__ packed,
    uint8_t* __restrict__ qabs, float* __restrict__ gscale,
    int32_t* __restrict__ status, Codebook cb) {
  __shared__ float s_c[256];
  __shared__ float s_wmax[QZ_THREADS / 64];
  const int tid = threadIdx.x;
  const int64_t g = blockIdx.x;
  const int64_t gbase = g * (int64_t)(QN_BLOCK * QN_GROUP);
  const int64_t nb_total = (numel + QN_BLOCK - 1) / QN_BLOCK;

  float v[QZ_PASSES][8];
  float cmine[QZ_PASSES];
  bool finite = true;
#pragma unroll
  for (int it = 0; it < QZ_PASSES; ++it) {
    const int64_t e0 = gbase + it * (QZ_THREADS * 8) + tid * 8;
    if (e0 + 8 <= numel) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(w + e0);
      const f32x4 b = *reinterpret_cast<const f32x4*>(w + e0 + 4);
      v[it][0] = a.x; v[it][1] = a.y; v[it][2] = a.z; v[it][3] = a.w;
      v[it][4] = b.x; v[it][5] = b.y; v[it][6] = b.z; v[it][7] = b.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[it][i] = (e0 + i < numel) ? w[e0 + i] : 0.0f;
    }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      finite = finite && __builtin_isfinite(v[it][i]);
      m = fmaxf(m, fabsf(v[it][i]));
    }
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    m = fmaxf(m, __shfl_xor(m, 4));
    cmine[it] = m;
    if ((tid & 7) == 0) s_c[it * (QZ_THREADS / 8) + (tid >> 3)] = m;
  }
  if (!finite && status != nullptr) *status = QN_ENONFINITE;
  __syncthreads();

  // group absmax
  const float cb_t = s_c[tid];
  float gm = cb_t;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) gm = fmaxf(gm, __shfl_xor(gm, off));
  if ((tid & 63) == 0) s_wmax[tid >> 6] = gm;
  __syncthreads();
  float smax = s_wmax[0];
#pragma unroll
  for (int i = 1; i < QZ_THREADS / 64; ++i) smax = fmaxf(smax, s_wmax[i]);
  const float d = (smax == 0.0f) ? 0.0f : smax / 255.0f;
  const int64_t b_this = g * QN_GROUP + tid;
  if (b_this < nb_total) {
    float qv = 0.0f;
    if (smax != 0.0f) qv = fminf(rintf(cb_t / d), 255.0f);
    qabs[b_this] = static_cast<uint8_t>(qv);
  }
  if (tid == 0) gscale[g] = d;

  // NF4 codes against the un-quantized block constant
  const int64_t nbytes = (numel + 1) / 2;
#pragma unroll
  for (int it = 0; it < QZ_PASSES; ++it) {
    const int64_t e0 = gbase + it * (QZ_THREADS * 8) + tid * 8;
    if (e0 >= numel) break;
    const float c = cmine[it];
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float n = (c == 0.0f) ? 0.0f : v[it][i] / c;
      uint32_t code = 0;
#pragma unroll
      for (int j = 0; j < 15; ++j) code += (n > cb.T[j]) ? 1u : 0u;
      word |= code << (4 * i);
    }
    const int64_t byte0 = e0 >> 1;
    if (byte0 + 4 <= nbytes) {
      *reinterpret_cast<uint32_t*>(packed + byte0) = word;
    } else {
      for (int i = 0; i < 4; ++i)
        if (byte0 + i < nbytes) packed[byte0 + i] = (word >> (8 * i)) & 0xFFu;
    }
  }
}

// ---------------------------------------------------------------------------
// K2: dequantization stream.  A wave handles spans of 2048 weights (1 KB of
// packed codes -> 4 KB of bf16, 32 blocks, inside one double-quant group).
// Lane l takes packed dword l + 64 j (j = 0..3) of the span, so every load
// instruction reads 256 contiguous bytes and every store instruction writes
// 1 KB contiguous (non-temporal); each dword (8 weights) lies in one block
// and gets that block's 16-entry LUT.  Spans are dealt round-robin to the
// waves; the next span's loads are issued before the current one is
// decoded.  Weights past the last whole span are done by k_dequant_tail.
// ---------------------------------------------------------------------------
constexpr int DQ_THREADS = 256;
constexpr int DQ_SPAN = 2048;                 // weights per span
#ifndef QN_DQ_GRID_CAP
#define QN_DQ_GRID_CAP 16384
#endif

struct DqRegs {
  uint32_t p[4];
  uint32_t q[4];
  float d;
};

// One launch dequantizes up to DQ_BATCH_MAX tensors: their whole spans are
// numbered consecutively (tensor i owns global spans [span0_i, span0_{i+1})).
constexpr int DQ_BATCH_MAX = QN_DEQUANT_BATCH_MAX;
struct DqTensor {
  const uint8_t* packed;
  const uint8_t* qabs;
  const float* gscale;
  uint16_t* out;
  int64_t span0;
};
struct DqBatch {
  DqTensor t[DQ_BATCH_MAX];
  int64_t nspans;       // total whole spans
  int count;
};

__global__ __launch_bounds__(DQ_THREADS) void k_dequant(DqBatch b, Codebook cb) {
  const int lane = threadIdx.x & 63;
  const int64_t wave0 = __builtin_amdgcn_readfirstlane(
      (int)(((int64_t)blockIdx.x * DQ_THREADS + threadIdx.x) >> 6));
  const int64_t nwaves = ((int64_t)gridDim.x * DQ_THREADS) >> 6;
  // tensor owning global span s (wave-uniform scan over <= 16 entries)
  auto owner = [&](int64_t s) {
    int i = 0;
    while (i + 1 < b.count && s >= b.t[i + 1].span0) ++i;
    return i;
  };
  auto load = [&](DqRegs& R, int64_t span) {
    const bool ok = span < b.nspans;
    const int ti = ok ? owner(span) : 0;
    const int64_t sp = ok ? span - b.t[ti].span0 : 0;
    const uint32_t* pw = reinterpret_cast<const uint32_t*>(b.t[ti].packed) + sp * (DQ_SPAN / 8);
    const uint8_t* qb = b.t[ti].qabs + sp * (DQ_SPAN / 64);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      R.p[j] = pw[lane + 64 * j];
      R.q[j] = qb[(lane >> 3) + 8 * j];
    }
    R.d = ok ? b.t[ti].gscale[(sp * (DQ_SPAN / 64)) >> 8] : 0.0f;
  };
  DqRegs cur;
  int64_t span = wave0;
  load(cur, span);
  for (; span < b.nspans; span += nwaves) {
    DqRegs nxt;
    load(nxt, span + nwaves);
    const int ti = owner(span);
    u32x4* o = reinterpret_cast<u32x4*>(b.t[ti].out + (span - b.t[ti].span0) * DQ_SPAN);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const Lut t = make_lut(cb, static_cast<float>(cur.q[j]) * cur.d);
      // streaming store: the output is not re-read here, and keeping it out
      // of L2 avoids a large write-back when the kernel retires
      __builtin_nontemporal_store(decode8(cur.p[j], t), &o[lane + 64 * j]);
    }
    cur = nxt;
  }
}

__global__ __launch_bounds__(DQ_THREADS) void k_dequant_tail(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ qabs,
    const float* __restrict__ gscale, int64_t e0, int64_t numel,
    uint16_t* __restrict__ out, Codebook cb) {
  const int64_t e = e0 + (int64_t)blockIdx.x * DQ_THREADS + threadIdx.x;
  if (e >= numel) return;
  const uint32_t byte = packed[e >> 1];
  const uint32_t code = (e & 1) ? (byte >> 4) : (byte & 0xFu);
  out[e] = decode1(cb, code, block_cprime(qabs, gscale, e >> 6));
}

// ---------------------------------------------------------------------------
// MFMA helpers.  v_mfma_f32_32x32x16_bf16: lane l supplies row (l % 32) of A
// and column (l % 32) of B, each with 8 consecutive reduction elements
// starting at 8 * (l / 32).  Accumulator register v of lane l holds
// C[8 * (v / 4) + 4 * (l / 32) + (v % 4)][l % 32].
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b,
                                         const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
      __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0,
      0);
}

// v_mfma_f32_16x16x32_bf16: lane l supplies row (l % 16) of A and column
// (l % 16) of B with 8 reduction elements from 8 * (l / 16); accumulator v
// of lane l holds C[4 * (l / 16) + v][l % 16].
__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b,
                                        const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
      __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0,
      0);
}

__device__ __forceinline__ void split_bf16(float x, uint16_t& hi,
                                           uint16_t& lo) {
  const uint32_t h = pack_bf16x2(x, 0.0f) & 0xFFFFu;
  const float rest = x - bf16_to_f32(h);
  hi = static_cast<uint16_t>(h);
  lo = static_cast<uint16_t>(pack_bf16x2(rest, 0.0f) & 0xFFFFu);
}

__device__ __forceinline__ void store_out(void* out, int out_bf16,
                                          int64_t idx, float v) {
  if (out_bf16)
    reinterpret_cast<uint16_t*>(out)[idx] =
        static_cast<uint16_t>(pack_bf16x2(v, 0.0f) & 0xFFFFu);
  else
    reinterpret_cast<float*>(out)[idx] = v;
}

// ---------------------------------------------------------------------------
// K3/K4: fused dequant + MFMA GEMM, one template for both directions.
//
//   forward  (BWD = false): Y[M,N]  = X[M,K]  W'^T  + (s T) B^T
//   backward (BWD = true) : dX[M,K] = dY[M,N] W'    + (s G) A
//
// Output tile BM x BN, reduction step 64.  The 256 x 256 tile runs 8 waves
// (2 x 4, two waves per SIMD, 128 x 64 of the output each), the 128 x 128
// tile 4 waves (2 x 2, 64 x 64 each), as tiles of v_mfma_f32_32x32x16_bf16
// with fp32 accumulators.  With two waves on a SIMD, one wave's LDS writes,
// buffer loads and dequantization issue while the other's MFMAs run; a
// single wave has to issue all of them between its own MFMAs.
//
// Per reduction step:
//  * the A tile (X or dY rows, bf16) is loaded into registers (16 bytes per
//    thread per chunk) and written to LDS after the step's MFMAs: 128-byte
//    rows with the 16-byte chunk index XOR-swizzled by (row / 2) & 7, so the
//    16 lanes of one ds_read_b128 phase (16 rows) cover all 64 LDS banks;
//  * the weight tile arrives as packed nibbles (16 bytes = 32 weights per
//    thread) + the 8-bit block code + the group scale in registers; each
//    thread builds its block's 16-entry bf16 LUT (v_perm) and dequantizes
//    into LDS.  Forward: W' [BN rows n][64 k], 128-byte rows, swizzled like
//    A, read as MFMA B operands with ds_read_b128.  Backward: W' [64 rows
//    n][BN k], chunks XOR-swizzled by bwd_swz, read column-wise with
//    ds_read_b64_tr_b16.
// LDS is double-buffered.  While the MFMAs consume step i, the A tile of
// step i+1 streams into the other buffer and the weight tile of step i+1
// (loaded one step earlier) is dequantized into it; the dequantization is
// woven between the MFMAs in fenced groups (one MFMA, then up to six VALU
// ops).  Global loads go through buffer resources whose range check returns
// zeros, which covers ragged M, N and K tiles without branches.
// The adapter term is 2r extra reduction steps with the A side s*T (or s*G)
// split into bf16 hi + lo parts, so the fp32 intermediate keeps ~16
// mantissa bits.
// ---------------------------------------------------------------------------
constexpr int G_BK = 64;
constexpr uint32_t G_OOB = 0x80000000u;   // buffer offset past every range
constexpr int G_RSRC_FLAGS = 0x00020000;

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)bytes, G_RSRC_FLAGS);
}

template <int BM, int BN, bool BWD>
struct GemmCfg {
  static constexpr int WAVES_M = 2, WAVES_N = BN == 256 ? 4 : 2;
  static constexpr int WAVES = WAVES_M * WAVES_N, NT = 64 * WAVES;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;  // per-wave tile
  static constexpr int TM = WM / 32, TN = WN / 32;             // MFMA tiles
  static constexpr int A_BYTES = BM * 128;                     // swizzled
  static constexpr int A_CHUNKS = BM * 8 / NT;                 // 16 B per thread
  static constexpr int EPT = 64 * BN / NT;                     // weights/thread
  static constexpr int WDW = EPT / 8;                          // packed dwords
  // threads per weight row: forward rows are 64 weights, backward rows BN
  static constexpr int TPR = BWD ? BN / EPT : 64 / EPT;
  static constexpr int PW = BWD ? BN : G_BK;                   // row pitch
  static constexpr int W_BYTES = 64 * BN * 2;
  static constexpr int MFMAS = 4 * TM * TN;                    // per step
  static_assert(EPT == 32 && WDW == 4, "one 16-byte load per thread");
  static_assert(A_CHUNKS * NT == BM * 8, "A tile loads");
  static_assert(NT == (BN == 256 ? 512 : 256), "k_gemm launch bounds");
};

// XOR for the 16-byte chunk index c of row r of the backward weight tile
// [64][BN]: the 16 lanes of a ds_write_b128 phase and the 32 lanes of a
// ds_read_b64_tr_b16 phase each cover all 64 LDS banks.
template <int BN>
__device__ __forceinline__ int bwd_swz(int r, int c) {
  return BN == 256 ? 4 * (r & 3) + 2 * (r & 1) + ((c >> 4) & 1) : 5 * (r & 3);
}

// Packed weight bytes of one step for one thread (32 weights), plus its
// block code and group scale (raw; c' = q * d is formed when the tile is
// dequantized).
struct WRegs {
  u32x4 w;
  uint32_t q;
  float d;
};

// Where a thread's dequantized weights go: its 16-byte chunk d (8 weights)
// is stored at base + 8 * (d ^ x).
struct WDst {
  uint16_t* base;
  int x;
};

template <int BM, int BN, bool BWD>
__device__ __forceinline__ WDst gemm_wdst(uint16_t* sW, int tid) {
  using C = GemmCfg<BM, BN, BWD>;
  const int row = tid / C::TPR, c0 = (tid % C::TPR) * (C::EPT / 8);
  const int x = BWD ? bwd_swz<BN>(row, c0) : ((row >> 1) & 7);
  // c0 is a multiple of 4 and d < 4: (c0 + d) ^ x = (c0 ^ (x & ~3)) + (d ^ (x & 3))
  return {sW + row * C::PW + 8 * (c0 ^ (x & ~3)), x & 3};
}

template <int BM, int BN, bool BWD>
__device__ __forceinline__ void gemm_load_w(WRegs& R, rsrc_t rp, rsrc_t rq,
                                            rsrc_t rd, int N, int K, int c0,
                                            int red0, int tid) {
  using C = GemmCfg<BM, BN, BWD>;
  int n, k;
  if (!BWD) {
    n = c0 + tid / C::TPR;           // output column = weight row
    k = red0 + (tid % C::TPR) * C::EPT;
  } else {
    n = red0 + tid / C::TPR;         // reduction index = weight row
    k = c0 + (tid % C::TPR) * C::EPT;
  }
  const bool ok = n < N && k < K;
  const int64_t e = (int64_t)n * K + k;
  const uint32_t op = ok ? (uint32_t)(e >> 1) : G_OOB;
  const uint32_t ob = ok ? (uint32_t)(e >> 6) : G_OOB;
  const uint32_t og = ok ? (uint32_t)((e >> 14) << 2) : G_OOB;
  R.w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, op, 0, 0));
  R.q = __builtin_amdgcn_raw_buffer_load_b8(rq, ob, 0, 0);
  R.d = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, og, 0, 0));
}

template <int BM, int BN, bool BWD>
__device__ __forceinline__ void gemm_dequant_w(const WRegs& R, uint16_t* sW,
                                               const Codebook& cb, int tid) {
  const WDst dst = gemm_wdst<BM, BN, BWD>(sW, tid);
  const Lut t = make_lut(cb, static_cast<float>(R.q) * R.d);
  const uint32_t wd[4] = {R.w.x, R.w.y, R.w.z, R.w.w};
#pragma unroll
  for (int d = 0; d < 4; ++d)
    *reinterpret_cast<u32x4*>(dst.base + 8 * (d ^ dst.x)) = decode8(wd[d], t);
}

// A tile of one step: 16-byte global loads into registers (thread t takes
// chunks q = t + NT i; chunk q is row q / 8, 16-byte column q % 8, so eight
// consecutive lanes read one 128-byte row segment), written to LDS after the
// step's MFMAs at the row's swizzled slot (q % 8) ^ ((row / 2) & 7).
// (A buffer_load ... lds per 1 KB costs the issuing SIMD far more than a
// load plus a ds_write_b128.)
template <int BM, int BN, bool BWD>
struct ARegs {
  u32x4 v[GemmCfg<BM, BN, BWD>::A_CHUNKS];
};

template <int BM, int BN, bool BWD>
__device__ __forceinline__ void gemm_load_a(ARegs<BM, BN, BWD>& R, rsrc_t ra,
                                            int M, int KRED, int m0, int red0,
                                            int tid) {
  using C = GemmCfg<BM, BN, BWD>;
#pragma unroll
  for (int i = 0; i < C::A_CHUNKS; ++i) {
    const int q = tid + C::NT * i, row = q >> 3;
    const int col = red0 + 8 * (q & 7);
    const bool ok = m0 + row < M && col < KRED;
    const uint32_t off =
        ok ? (uint32_t)(((int64_t)(m0 + row) * KRED + col) * 2) : G_OOB;
    R.v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0));
  }
}

template <int BM, int BN, bool BWD>
__device__ __forceinline__ void gemm_store_a(const ARegs<BM, BN, BWD>& R,
                                             char* sA, int tid) {
  using C = GemmCfg<BM, BN, BWD>;
#pragma unroll
  for (int i = 0; i < C::A_CHUNKS; ++i) {
    const int q = tid + C::NT * i, row = q >> 3;
    *reinterpret_cast<u32x4*>(sA + row * 128 + (((q & 7) ^ ((row >> 1) & 7)) << 4)) = R.v[i];
  }
}

// Transposed B operand for the backward: lane l needs 8 consecutive
// reduction rows (8 * (l / 32) ...) of output column (col0 + l % 32).  Each
// ds_read_b64_tr_b16 serves 4 rows: in every group of 16 lanes, lane
// q = 4j + p addresses row j, columns 4p..4p+3 of the group's 16 columns,
// and lane q receives column q of the 4 rows.
template <int BN>
__device__ __forceinline__ u32x4 lds_read_bT(const uint16_t* sW, int row0,
                                             int col0, int lane) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const int grp = lane >> 4, q = lane & 15;
  const int row = row0 + 8 * (grp >> 1) + (q >> 2);
  const int col = col0 + 16 * (grp & 1) + 4 * (q & 3);
  // rows row and row + 4 have the same swizzle (it depends on row & 3)
  const int pc = (((col >> 3) ^ bwd_swz<BN>(row, col >> 3)) << 3) | (col & 7);
  const uint16_t* p0 = sW + row * BN + pc;
  const uint16_t* p1 = p0 + 4 * BN;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(const_cast<uint16_t*>(p0)));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(const_cast<uint16_t*>(p1)));
  u32x4 r;
  r.x = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
  r.y = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
  r.z = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
  r.w = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
  return r;
}

// 16 bytes of row r, logical chunk c of a 128-byte-row tile swizzled by
// (r / 2) & 7 (the A tile, and the forward weight tile).
__device__ __forceinline__ u32x4 lds_read_row128(const void* t, int r, int c) {
  return *reinterpret_cast<const u32x4*>(static_cast<const char*>(t) + r * 128 +
                                         ((c ^ ((r >> 1) & 7)) << 4));
}

// Fragments of one k16 slice: A rows and B columns.
template <int BM, int BN, bool BWD>
__device__ __forceinline__ void gemm_frags(const char* sA, const uint16_t* sW,
                                           int wm, int wn, int lane, int kk,
                                           u32x4 (&a)[GemmCfg<BM, BN, BWD>::TM],
                                           u32x4 (&b)[GemmCfg<BM, BN, BWD>::TN]) {
  using C = GemmCfg<BM, BN, BWD>;
  const int chunk = 2 * kk + (lane >> 5);
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
    a[i] = lds_read_row128(sA, wm * C::WM + i * 32 + (lane & 31), chunk);
#pragma unroll
  for (int j = 0; j < C::TN; ++j) {
    if (!BWD)
      b[j] = lds_read_row128(sW, wn * C::WN + j * 32 + (lane & 31), chunk);
    else
      b[j] = lds_read_bT<BN>(sW, kk * 16, wn * C::WN + j * 32, lane);
  }
}

// VALU instructions placed after each MFMA by the interleaving below.
constexpr int G_VALU_PER_MFMA = 6;

// The four k16 slices of one step with the dequantization of the next weight
// tile woven in: one decode8 (28 VALU ops and a 16-byte LDS write) after
// every MPD MFMAs, each group fenced and ordered MFMA / VALU so the VALU
// work issues in the shadow of the MFMAs instead of after them.
template <int BM, int BN, bool BWD>
__device__ __forceinline__ void gemm_mma_deq(
    const char* sA, const uint16_t* sW, uint16_t* sWn, const WRegs& R,
    const Codebook& cb, int wm, int wn, int tid, int lane,
    f32x16 (&acc)[GemmCfg<BM, BN, BWD>::TM][GemmCfg<BM, BN, BWD>::TN]) {
  using C = GemmCfg<BM, BN, BWD>;
  constexpr int MPK = C::TM * C::TN;     // MFMAs per k16 slice
  constexpr int DPK = C::WDW / 4;        // decode8 per k16 slice
  constexpr int MPD = MPK / DPK;         // MFMAs per decode8
  static_assert(C::WDW % 4 == 0 && MPK % DPK == 0, "decode split");
  const WDst dst = gemm_wdst<BM, BN, BWD>(sWn, tid);
  const Lut t = make_lut(cb, static_cast<float>(R.q) * R.d);
  const uint32_t wd[4] = {R.w.x, R.w.y, R.w.z, R.w.w};
  u32x4 a[2][C::TM], b[2][C::TN];
  gemm_frags<BM, BN, BWD>(sA, sW, wm, wn, lane, 0, a[0], b[0]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    if (kk < 3)
      gemm_frags<BM, BN, BWD>(sA, sW, wm, wn, lane, kk + 1, a[(kk + 1) & 1],
                              b[(kk + 1) & 1]);
#pragma unroll
    for (int g = 0; g < MPK; ++g) {
      const int i = g / C::TN, j = g % C::TN;
      acc[i][j] = mfma32(a[kk & 1][i], b[kk & 1][j], acc[i][j]);
      if (g % MPD == MPD - 1) {
        const int d = kk * DPK + g / MPD;
        *reinterpret_cast<u32x4*>(dst.base + 8 * (d ^ dst.x)) = decode8(wd[d], t);
#pragma unroll
        for (int h = 0; h < MPD; ++h) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, G_VALU_PER_MFMA, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

// Maps the linear workgroup index to an output tile so that each XCD (the
// hardware deals workgroups round-robin over 8 XCDs) works on a contiguous
// run of tiles, and runs walk the N direction first: a run shares A rows in
// that XCD's L2.
__device__ __forceinline__ void gemm_tile_of(int tiles_m, int tiles_n,
                                             int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  int pid = blockIdx.x;
  if ((total & 7) == 0) pid = (pid & 7) * (total >> 3) + (pid >> 3);
  tm = pid / tiles_n;
  tn = pid % tiles_n;
}

// One reduction step: MFMAs on (sAc, sWc) while the next A tile streams into
// sAn and the weight tile held in Wc is dequantized into sWn.
template <int BM, int BN, bool BWD>
__device__ __forceinline__ void gemm_step(
    int st, char* sAc, uint16_t* sWc, char* sAn, uint16_t* sWn, WRegs& Wc,
    rsrc_t ra, rsrc_t rp, rsrc_t rq, rsrc_t rd, int M, int N, int K, int KRED,
    int m0, int c0, int wave, int wm, int wn, int tid, int lane,
    const Codebook& cb,
    f32x16 (&acc)[GemmCfg<BM, BN, BWD>::TM][GemmCfg<BM, BN, BWD>::TN]) {
  WRegs Wn;
  ARegs<BM, BN, BWD> An;
  gemm_load_a<BM, BN, BWD>(An, ra, M, KRED, m0, (st + 1) * G_BK, tid);
  gemm_load_w<BM, BN, BWD>(Wn, rp, rq, rd, N, K, c0, (st + 2) * G_BK, tid);
  gemm_mma_deq<BM, BN, BWD>(sAc, sWc, sWn, Wc, cb, wm, wn, tid, lane, acc);
  gemm_store_a<BM, BN, BWD>(An, sAn, tid);
  __builtin_amdgcn_s_waitcnt(0);   // all counters: loads and LDS writes done
  __syncthreads();
  Wc = Wn;
}

template <int BM, int BN, bool BWD>
__global__ __launch_bounds__((BN == 256 ? 512 : 256), 1) void k_gemm(
    const uint16_t* __restrict__ Aop, const uint8_t* __restrict__ packed,
    const uint8_t* __restrict__ qabs, const float* __restrict__ gscale,
    const uint16_t* __restrict__ La_hi, const uint16_t* __restrict__ La_lo,
    const uint16_t* __restrict__ Lb, int M, int N, int K, int rpad,
    void* __restrict__ out, int out_bf16, Codebook cb) {
  using C = GemmCfg<BM, BN, BWD>;
  // Four distinct LDS buffers so that the compiler can see that the tiles
  // being filled never alias the tiles being read.
  __shared__ __attribute__((aligned(16))) char sA0[C::A_BYTES];
  __shared__ __attribute__((aligned(16))) char sA1[C::A_BYTES];
  __shared__ __attribute__((aligned(16))) uint16_t sW0[C::W_BYTES / 2];
  __shared__ __attribute__((aligned(16))) uint16_t sW1[C::W_BYTES / 2];
  const int NOUT = BWD ? K : N;        // output columns
  const int KRED = BWD ? N : K;        // reduction length
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  int tm, tn;
  gemm_tile_of((M + BM - 1) / BM, (NOUT + BN - 1) / BN, tm, tn);
  const int m0 = tm * BM, c0 = tn * BN;

  const int64_t numel = (int64_t)N * K;
  const rsrc_t ra = make_rsrc(Aop, (uint32_t)((int64_t)M * KRED * 2));
  const rsrc_t rp = make_rsrc(packed, (uint32_t)((numel + 1) >> 1));
  const rsrc_t rq = make_rsrc(qabs, (uint32_t)((numel + 63) >> 6));
  const rsrc_t rd = make_rsrc(gscale, (uint32_t)(((numel + 16383) >> 14) << 2));

  f32x16 acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // Steps past the end read out of range: their tiles are zeros (a zero
  // block constant dequantizes every code to zero), so the loop runs whole
  // pairs of steps without branches.
  const int nsteps = (KRED + G_BK - 1) / G_BK;
  WRegs Wc;
  {
    ARegs<BM, BN, BWD> A0;
    gemm_load_a<BM, BN, BWD>(A0, ra, M, KRED, m0, 0, tid);
    gemm_store_a<BM, BN, BWD>(A0, sA0, tid);
  }
  gemm_load_w<BM, BN, BWD>(Wc, rp, rq, rd, N, K, c0, 0, tid);
  gemm_dequant_w<BM, BN, BWD>(Wc, sW0, cb, tid);
  gemm_load_w<BM, BN, BWD>(Wc, rp, rq, rd, N, K, c0, G_BK, tid);
  __builtin_amdgcn_s_waitcnt(0);   // all counters: loads landed in LDS/regs
  __syncthreads();
  for (int st = 0; st < nsteps; st += 2) {
    gemm_step<BM, BN, BWD>(st, sA0, sW0, sA1, sW1, Wc, ra, rp, rq, rd, M, N, K,
                           KRED, m0, c0, wave, wm, wn, tid, lane, cb, acc);
    gemm_step<BM, BN, BWD>(st + 1, sA1, sW1, sA0, sW0, Wc, ra, rp, rq, rd, M, N,
                           K, KRED, m0, c0, wave, wm, wn, tid, lane, cb, acc);
  }

  // Adapter term, 2 * rpad more reduction steps straight from global memory
  // (small, L2-resident arrays): A side the bf16 hi and lo parts of s*T
  // (forward) or s*G (backward), [M][rpad]; B side [NOUT][rpad], B (forward)
  // or A^T (backward), zero-padded to rpad columns.
  {
    const rsrc_t rh = make_rsrc(La_hi, (uint32_t)((int64_t)M * rpad * 2));
    const rsrc_t rl = make_rsrc(La_lo, (uint32_t)((int64_t)M * rpad * 2));
    const rsrc_t rb = make_rsrc(Lb, (uint32_t)((int64_t)NOUT * rpad * 2));
    for (int j0 = 0; j0 < rpad; j0 += 16) {
      const int jc = j0 + 8 * (lane >> 5);
      u32x4 ah[C::TM], al[C::TM], b[C::TN];
#pragma unroll
      for (int i = 0; i < C::TM; ++i) {
        const uint32_t off =
            (uint32_t)(((int64_t)(m0 + wm * C::WM + i * 32 + (lane & 31)) * rpad + jc) * 2);
        ah[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rh, off, 0, 0));
        al[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rl, off, 0, 0));
      }
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        const uint32_t off =
            (uint32_t)(((int64_t)(c0 + wn * C::WN + j * 32 + (lane & 31)) * rpad + jc) * 2);
        b[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0));
      }
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
          acc[i][j] = mfma32(ah[i], b[j], acc[i][j]);
          acc[i][j] = mfma32(al[i], b[j], acc[i][j]);
        }
    }
  }

#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * C::WM + i * 32 + 8 * (v >> 2) +
                        4 * (lane >> 5) + (v & 3);
        const int col = c0 + wn * C::WN + j * 32 + (lane & 31);
        if (row < M && col < NOUT)
          store_out(out, out_bf16, (int64_t)row * NOUT + col, acc[i][j][v]);
      }
}

// ---------------------------------------------------------------------------
// K5: rank-r side products, streamed over one large bf16 operand S [M][C]
// (X or dY, row-major) in stages of 64 SUB columns:
//   rows part  prow: P[m][j] = sum_c S[m][c] R[j][c]   (T = X A^T, G = dY B)
//   cols part  pcol: Q[c][j] = sum_m S[m][c] U[m][j]   (dB = dY^T (s T),
//                                                       dA^T = X^T (s G))
// Workgroup (bx, by) owns rows [RM by, RM by + RM) and stages
// [cpb bx, cpb bx + cpb); its row sums over those stages go to
// prow[bx][m][j] and its column sums over its rows to pcol[by][c][j]
// (fp32, rpad = 16 JT columns).  k_rank_finish adds the partials in a fixed
// order, so results do not depend on scheduling.  The backward's dY is read
// once for both G and dB.
//
// Each stage of S (RM rows) and of R (rpad rows, given [r][C]) goes global
// -> LDS with buffer_load ... lds into double-buffered tiles of 128-byte
// rows whose 16-byte chunks are XOR-swizzled by rs_swz(row): the 16 lanes
// of a ds_read_b128 phase (16 rows) and the 32 lanes of a
// ds_read_b64_tr_b16 phase (8 rows x 2 chunks) each cover all 64 banks.
// U (the bf16 hi and lo parts of s T or s G, given transposed [r][ldu]) is
// staged once per workgroup.  Both parts use v_mfma_f32_16x16x32_bf16: the
// rows part pairs S rows with R rows, the cols part pairs S columns (read
// transposed) with U rows; hi and lo are two MFMAs into one accumulator.
// Buffer loads return zeros outside S, R and U, which covers ragged M, C
// and r.
// ---------------------------------------------------------------------------
enum { RS_ROWS = 1, RS_COLS = 2 };

// RM rows per workgroup, stages of 64 SUB columns, NBUF LDS buffers (NBUF - 1
// stages in flight): about 32 KB of S per stage for r <= 32, less for the
// wider adapters whose R and U tiles take more LDS.
__host__ __device__ constexpr int rs_rm(int mode, int jt) {
  return mode == RS_ROWS ? 64 : (jt <= 2 ? 256 : 64);
}
__host__ __device__ constexpr int rs_sub(int mode, int jt) {
  return jt >= 8 ? 1 : (jt == 4 ? 2 : (mode == RS_ROWS ? 4 : 1));
}
__host__ __device__ constexpr int rs_nbuf(int jt) { return jt >= 16 ? 2 : 3; }

__device__ __forceinline__ int rs_swz(int row) {
  return (((row >> 3) & 1) << 2) | (((row >> 1) & 1) << 1) | ((row >> 2) & 1);
}

// NR rows x 64 columns (columns col0.. of rows 0..nvalid-1 of the
// resource, row pitch ld elements) into a swizzled LDS tile.  Instruction q
// fills rows 8q..8q+7: lane l writes 16 bytes at tile + 1024 q + 16 l, that
// is row 8q + l/8, slot l%8, which holds logical chunk (l%8) ^ rs_swz(row).
template <int NR>
__device__ __forceinline__ void rs_dma(rsrc_t rs, char* tile, int64_t ld,
                                       int nvalid, int col0, int C, int wave,
                                       int lane) {
  static_assert(NR % 8 == 0, "tile rows");
#pragma unroll
  for (int q0 = 0; q0 < NR / 8; q0 += 4) {
    const int q = q0 + wave;
    if (q < NR / 8) {
      const int row = 8 * q + (lane >> 3);
      const int col = col0 + 8 * ((lane & 7) ^ rs_swz(row));
      const uint32_t off = (row < nvalid && col < C)
                               ? (uint32_t)(((int64_t)row * ld + col) * 2)
                               : G_OOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(tile + q * 1024),
                                               16, off, 0, 0, 0);
    }
  }
}

// Same layout, 4 bytes per lane: instruction q fills rows 2q, 2q+1 (lane l
// writes tile + 256 q + 4 l: row 2q + l/32, dword l%32).  Used for 16-row
// tiles so that every wave issues the same number of loads.
template <int NR>
__device__ __forceinline__ void rs_dma4(rsrc_t rs, char* tile, int64_t ld,
                                        int nvalid, int col0, int C, int wave,
                                        int lane) {
  static_assert(NR % 8 == 0, "tile rows");
#pragma unroll
  for (int i = 0; i < NR / 8; ++i) {
    const int q = wave + 4 * i;
    const int row = 2 * q + (lane >> 5), d = lane & 31;
    const int col = col0 + 8 * ((d >> 2) ^ rs_swz(row)) + 2 * (d & 3);
    const uint32_t off = (row < nvalid && col < C)
                             ? (uint32_t)(((int64_t)row * ld + col) * 2)
                             : G_OOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(tile + q * 256),
                                             4, off, 0, 0, 0);
  }
}

// 16 bytes of row `row`, logical chunk lc, of a swizzled tile.
__device__ __forceinline__ u32x4 rs_read_row(const char* tile, int row, int lc) {
  return *reinterpret_cast<const u32x4*>(tile + row * 128 +
                                         ((lc ^ rs_swz(row)) << 4));
}

// Transposed operand of v_mfma_f32_16x16x32_bf16 from a swizzled tile:
// lane l gets column col0 + l % 16, rows row0 + 8 (l / 16) .. + 7 (two
// ds_read_b64_tr_b16; within each 16-lane group, lane q addresses row
// q / 4 (+ 4), columns 4 (q % 4) .. + 3).
__device__ __forceinline__ u32x4 rs_read_colT(const char* tile, int row0,
                                              int col0, int lane) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const int g = lane >> 4, q = lane & 15;
  const int row = row0 + 8 * g + (q >> 2);
  const int col = col0 + 4 * (q & 3);
  const char* p0 = tile + row * 128 +
                   ((((col >> 3) ^ rs_swz(row)) << 4) | ((col & 7) * 2));
  const char* p1 = tile + (row + 4) * 128 +
                   ((((col >> 3) ^ rs_swz(row + 4)) << 4) | ((col & 7) * 2));
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(const_cast<char*>(p0)));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(const_cast<char*>(p1)));
  u32x4 v;
  v.x = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
  v.y = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
  v.z = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
  v.w = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
  return v;
}

template <int MODE, int JT>
struct RsCfg {
  static constexpr bool ROWS = (MODE & RS_ROWS) != 0;
  static constexpr bool COLS = (MODE & RS_COLS) != 0;
  static constexpr int RM = rs_rm(MODE, JT), SUB = rs_sub(MODE, JT);
  static constexpr int NBUF = rs_nbuf(JT);
  static constexpr int RP = 16 * JT, PU = RM + 8, TR = RM / 64;
  static constexpr int S_BYTES = SUB * RM * 128;
  static constexpr int R_BYTES = ROWS ? SUB * RP * 128 : 16;
  static constexpr int U_ELEMS = COLS ? RP * PU : 8;
  // vector-memory instructions per wave for one stage (the same in every
  // wave, so a vmcnt immediate can wait for all but the newest stage)
  static constexpr int DMA = SUB * (RM / 32 + (ROWS ? (RP == 16 ? 2 : RP / 32) : 0));
  static_assert(DMA < 64, "vmcnt range");
};

// Workgroup barrier without the release/acquire fences of __syncthreads:
// with global stores in flight those fences make every wave wait for its
// stores (vmcnt(0)) at each barrier.  Callers wait for the LDS traffic that
// must be visible (RS_WAIT_VM includes lgkmcnt(0)); the signal fences keep
// the compiler from moving memory operations across the barrier.
__device__ __forceinline__ void wg_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// s_waitcnt vmcnt(n) expcnt(7) lgkmcnt(0) (gfx9 encoding)
#define RS_WAIT_VM(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (((n) >> 4) << 14))

template <int MODE, int JT>
__device__ __forceinline__ void rs_stage_dma(rsrc_t rs, rsrc_t rr, char* dS,
                                             char* dR, int64_t C, int nvalid,
                                             int r, int stage, int wave,
                                             int lane) {
  using G = RsCfg<MODE, JT>;
#pragma unroll
  for (int u = 0; u < G::SUB; ++u) {
    const int col0 = (stage * G::SUB + u) * 64;
    rs_dma<G::RM>(rs, dS + u * G::RM * 128, C, nvalid, col0, (int)C, wave, lane);
    if (G::ROWS) {
      if (G::RP == 16)
        rs_dma4<G::RP>(rr, dR + u * G::RP * 128, C, r, col0, (int)C, wave, lane);
      else
        rs_dma<G::RP>(rr, dR + u * G::RP * 128, C, r, col0, (int)C, wave, lane);
    }
  }
}

template <int MODE, int JT>
__device__ __forceinline__ void rs_stage_compute(
    const char* sS, const char* sR, const uint16_t* sUh, const uint16_t* sUl,
    int wave, int lane, f32x4 (&accR)[RsCfg<MODE, JT>::TR][JT],
    f32x4 (&accC)[RsCfg<MODE, JT>::SUB][JT]) {
  using G = RsCfg<MODE, JT>;
#pragma unroll
  for (int u = 0; u < G::SUB; ++u) {
    const char* tS = sS + u * G::RM * 128;
    if (G::ROWS) {
      const char* tR = sR + u * G::RP * 128;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        u32x4 b[JT];
#pragma unroll
        for (int t = 0; t < JT; ++t)
          b[t] = rs_read_row(tR, 16 * t + (lane & 15), 4 * s + (lane >> 4));
#pragma unroll
        for (int tr = 0; tr < G::TR; ++tr) {
          const u32x4 a = rs_read_row(
              tS, wave * (G::RM / 4) + 16 * tr + (lane & 15), 4 * s + (lane >> 4));
#pragma unroll
          for (int t = 0; t < JT; ++t) accR[tr][t] = mfma16(a, b[t], accR[tr][t]);
        }
      }
    }
    if (G::COLS) {
#pragma unroll
      for (int t = 0; t < JT; ++t) accC[u][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
      for (int s2 = 0; s2 < G::RM / 32; ++s2) {
        const u32x4 a = rs_read_colT(tS, 32 * s2, 16 * wave, lane);
#pragma unroll
        for (int t = 0; t < JT; ++t) {
          const int uo = (16 * t + (lane & 15)) * G::PU + 32 * s2 + 8 * (lane >> 4);
          accC[u][t] = mfma16(a, *reinterpret_cast<const u32x4*>(sUh + uo), accC[u][t]);
          accC[u][t] = mfma16(a, *reinterpret_cast<const u32x4*>(sUl + uo), accC[u][t]);
        }
      }
    }
  }
}

// Column sums of one stage: accC[u][t][v] = Q[c][j] with
// c = 64 (SUB stage + u) + 16 wave + 4 (l / 16) + v, j = 16 t + l % 16.
// Buffer stores: columns past C fall outside the range and are dropped, so
// every wave issues the same stores.
template <int MODE, int JT>
__device__ __forceinline__ void rs_store_cols(
    rsrc_t rc, int stage, int C, int wave, int lane,
    const f32x4 (&accC)[RsCfg<MODE, JT>::SUB][JT]) {
  using G = RsCfg<MODE, JT>;
#pragma unroll
  for (int u = 0; u < G::SUB; ++u) {
    const int cb = (stage * G::SUB + u) * 64 + 16 * wave + 4 * (lane >> 4);
#pragma unroll
    for (int t = 0; t < JT; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int c = cb + v;
        const uint32_t off =
            c < C ? (uint32_t)((c * G::RP + 16 * t + (lane & 15)) * 4) : G_OOB;
        const float x = accC[u][t][v];   // element copy, then reinterpret
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), rc, off, 0, 0);
      }
  }
}

template <int MODE, int JT>
__global__ __launch_bounds__(256) void k_rank_stream(
    const uint16_t* __restrict__ S, int M, int C,
    const uint16_t* __restrict__ R, int r, const uint16_t* __restrict__ Uh,
    const uint16_t* __restrict__ Ul, int ldu, int cpb,
    float* __restrict__ prow, float* __restrict__ pcol) {
  using G = RsCfg<MODE, JT>;
  // distinct buffers, so the compiler can tell the tile being filled from
  // the tiles being read
  __shared__ __attribute__((aligned(16))) char sS0[G::S_BYTES];
  __shared__ __attribute__((aligned(16))) char sS1[G::S_BYTES];
  __shared__ __attribute__((aligned(16))) char sS2[G::NBUF > 2 ? G::S_BYTES : 16];
  __shared__ __attribute__((aligned(16))) char sR0[G::R_BYTES];
  __shared__ __attribute__((aligned(16))) char sR1[G::R_BYTES];
  __shared__ __attribute__((aligned(16))) char sR2[G::NBUF > 2 ? G::R_BYTES : 16];
  __shared__ __attribute__((aligned(16))) uint16_t sUh[G::U_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t sUl[G::U_ELEMS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m0 = blockIdx.y * G::RM;
  const int nvalid = min(G::RM, M - m0);
  const int nst = (C + 64 * G::SUB - 1) / (64 * G::SUB);
  const int sb = blockIdx.x * cpb, se = min(nst, sb + cpb);
  const rsrc_t rs = make_rsrc(S + (int64_t)m0 * C, (uint32_t)((int64_t)nvalid * C * 2));
  const rsrc_t rr = make_rsrc(R, G::ROWS ? (uint32_t)((int64_t)r * C * 2) : 0u);
  const rsrc_t rc = make_rsrc(G::COLS ? pcol + (int64_t)blockIdx.y * C * G::RP : nullptr,
                              G::COLS ? (uint32_t)((int64_t)C * G::RP * 4) : 0u);

  f32x4 accR[G::TR][JT];
#pragma unroll
  for (int tr = 0; tr < G::TR; ++tr)
#pragma unroll
    for (int t = 0; t < JT; ++t) accR[tr][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 accC[G::SUB][JT];

  // U block of this workgroup's rows: [rpad][RM] of the transposed [r][ldu]
  constexpr int MC = G::RM / 8, UCH = G::RP * MC;
  constexpr int UL = G::COLS ? UCH / 256 : 0;
  static_assert(!G::COLS || UCH % 256 == 0, "U staging");
  u32x4 uh[UL > 0 ? UL : 1], ul[UL > 0 ? UL : 1];
  if constexpr (G::COLS) {
    const rsrc_t ruh = make_rsrc(Uh, (uint32_t)((int64_t)r * ldu * 2));
    const rsrc_t rul = make_rsrc(Ul, (uint32_t)((int64_t)r * ldu * 2));
#pragma unroll
    for (int k = 0; k < UL; ++k) {
      const int i = 256 * k + tid, j = i / MC, m = m0 + 8 * (i % MC);
      const uint32_t off = (j < r && m < ldu)
                               ? (uint32_t)(((int64_t)j * ldu + m) * 2) : G_OOB;
      uh[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ruh, off, 0, 0));
      ul[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rul, off, 0, 0));
    }
  }
  rs_stage_dma<MODE, JT>(rs, rr, sS0, sR0, C, nvalid, r, sb, wave, lane);
  const bool two = G::NBUF == 3 && sb + 1 < se;
  if (two)
    rs_stage_dma<MODE, JT>(rs, rr, sS1, sR1, C, nvalid, r, sb + 1, wave, lane);
  if constexpr (G::COLS) {
#pragma unroll
    for (int k = 0; k < UL; ++k) {
      const int i = 256 * k + tid, j = i / MC, mc = i % MC;
      *reinterpret_cast<u32x4*>(sUh + j * G::PU + 8 * mc) = uh[k];
      *reinterpret_cast<u32x4*>(sUl + j * G::PU + 8 * mc) = ul[k];
    }
  }
  if (two) RS_WAIT_VM(G::DMA);
  else RS_WAIT_VM(0);
  wg_barrier();

  // One stage: store the previous stage's column sums, compute on buffer
  // `cur`, start the stage NBUF - 1 ahead into buffer `far`, then wait until
  // the next stage has landed (with three buffers the newest one stays in
  // flight; its loads are the last ones issued, and loads complete in order).
#define RS_BODY(I, CS, CR, FS, FR)                                            \
  do {                                                                        \
    if (G::COLS && (I) > sb)                                                  \
      rs_store_cols<MODE, JT>(rc, (I) - 1, C, wave, lane, accC);              \
    rs_stage_compute<MODE, JT>(CS, CR, sUh, sUl, wave, lane, accR, accC);     \
    if ((I) + G::NBUF - 1 < se) {                                             \
      rs_stage_dma<MODE, JT>(rs, rr, FS, FR, C, nvalid, r, (I) + G::NBUF - 1, \
                             wave, lane);                                     \
      if (G::NBUF == 3) RS_WAIT_VM(G::DMA);                                   \
      else RS_WAIT_VM(0);                                                     \
    } else {                                                                  \
      RS_WAIT_VM(0);                                                          \
    }                                                                         \
    wg_barrier();                                                          \
  } while (0)

  if constexpr (G::NBUF == 3) {
    for (int st = sb; st < se; st += 3) {
      RS_BODY(st, sS0, sR0, sS2, sR2);
      if (st + 1 < se) RS_BODY(st + 1, sS1, sR1, sS0, sR0);
      if (st + 2 < se) RS_BODY(st + 2, sS2, sR2, sS1, sR1);
    }
  } else {
    for (int st = sb; st < se; st += 2) {
      RS_BODY(st, sS0, sR0, sS1, sR1);
      if (st + 1 < se) RS_BODY(st + 1, sS1, sR1, sS0, sR0);
    }
  }
#undef RS_BODY
  if (G::COLS) rs_store_cols<MODE, JT>(rc, se - 1, C, wave, lane, accC);
  if (G::ROWS) {
    // accR[tr][t][v] = P[m = wave RM/4 + 16 tr + 4 (l / 16) + v][j = 16 t + l % 16]
    float* dst = prow + ((int64_t)blockIdx.x * M + m0) * G::RP;
#pragma unroll
    for (int tr = 0; tr < G::TR; ++tr)
#pragma unroll
      for (int t = 0; t < JT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = wave * (G::RM / 4) + 16 * tr + 4 * (lane >> 4) + v;
          if (m < nvalid) dst[(int64_t)m * G::RP + 16 * t + (lane & 15)] = accR[tr][t][v];
        }
  }
}

// ---------------------------------------------------------------------------
// k_rank_finish: up to four small jobs in one launch, one thread per output
// element, blocks [0, nbR) rows job, then cols, pad1, pad2.
//  rows: v[m][j] = sum_b src[b bstride + m ld + j] (b in order; 0 for
//        j >= jvalid and for M <= m < Mp) -> out[m][jvalid] = v,
//        hi/lo[m][rpad] and hiT/loT[jvalid][Mp] = bf16 hi/lo of scale v;
//  cols: out[c sc + j sj] = sum_b src[(b C + c) rpad + j]  (j < r);
//  pad:  dst[row dw + col] = col < valid ? src[row rs + col cs] : 0.
// ---------------------------------------------------------------------------
struct FinishRows {
  const float* src;
  int64_t bstride;
  int ld, nb, M, Mp, jvalid, rpad;
  float scale;
  float* out;
  uint16_t *hi, *lo, *hiT, *loT;
};
struct FinishCols {
  const float* src;
  int nb, C, r, rpad;
  float* out;
  int64_t sc, sj;
};
struct FinishPad {
  const uint16_t* src;
  uint16_t* dst;
  int rows, dw, valid;
  int64_t rs, cs;
};
struct FinishArgs {
  FinishRows R;
  FinishCols Cc;
  FinishPad P1, P2;
  int nbR, nbC, nbP1, nbP2;
};

__device__ __forceinline__ void finish_pad(const FinishPad& p, int64_t idx) {
  if (idx >= (int64_t)p.rows * p.dw) return;
  const int64_t row = idx / p.dw, col = idx % p.dw;
  p.dst[idx] = col < p.valid ? p.src[row * p.rs + col * p.cs] : (uint16_t)0;
}

__global__ __launch_bounds__(256) void k_rank_finish(FinishArgs a) {
  int b = blockIdx.x;
  const int tid = threadIdx.x;
  if (b < a.nbR) {
    const FinishRows& p = a.R;
    const int64_t idx = (int64_t)b * 256 + tid;
    if (idx >= (int64_t)p.Mp * p.rpad) return;
    const int m = (int)(idx / p.rpad), j = (int)(idx % p.rpad);
    float v = 0.0f;
    if (m < p.M && j < p.jvalid)
      for (int k = 0; k < p.nb; ++k)
        v += p.src[k * p.bstride + (int64_t)m * p.ld + j];
    uint16_t h, l;
    split_bf16(p.scale * v, h, l);
    if (m < p.M) {
      if (p.out != nullptr && j < p.jvalid) p.out[(int64_t)m * p.jvalid + j] = v;
      if (p.hi != nullptr) {
        p.hi[(int64_t)m * p.rpad + j] = h;
        p.lo[(int64_t)m * p.rpad + j] = l;
      }
    }
    if (p.hiT != nullptr && j < p.jvalid) {
      p.hiT[(int64_t)j * p.Mp + m] = h;
      p.loT[(int64_t)j * p.Mp + m] = l;
    }
    return;
  }
  b -= a.nbR;
  if (b < a.nbC) {
    const FinishCols& p = a.Cc;
    const int64_t idx = (int64_t)b * 256 + tid;
    if (idx >= (int64_t)p.C * p.r) return;
    const int64_t c = idx / p.r, j = idx % p.r;
    float v = 0.0f;
    for (int k = 0; k < p.nb; ++k)
      v += p.src[((int64_t)k * p.C + c) * p.rpad + j];
    p.out[c * p.sc + j * p.sj] = v;
    return;
  }
  b -= a.nbC;
  if (b < a.nbP1) {
    finish_pad(a.P1, (int64_t)b * 256 + tid);
    return;
  }
  b -= a.nbP1;
  if (b < a.nbP2) finish_pad(a.P2, (int64_t)b * 256 + tid);
}

// ---------------------------------------------------------------------------
// K6: skinny forward (M <= 16 tokens): HBM-bound GEMV over the NF4 weight.
//
// Workgroup = 8 waves; wave w owns 16 consecutive "rows" of the weight-like
// operand: rows [0, N) are the NF4 weight W, rows [N, N + rpad) are the
// adapter's A (bf16), so T = X A^T comes out of the same pass.  Grid.y
// splits K into slices of KS columns; the workgroup stages its X slice
// (M rows, zero above M) in LDS once.  Per 256-column chunk, lane
// (n = l % 16, g = l / 16) loads the 32 packed bytes of block g of row n,
// builds that block's 16-entry bf16 LUT and decodes 8 weights per
// v_mfma_f32_16x16x32_bf16 step (t = 0..7 takes weights 8t..8t+7 of the
// block); the matching A operand is X[m][64 g + 8 t ...] from LDS.  The
// next chunk's weight bytes are loaded before the current chunk is decoded.
// A persistent workgroup takes a contiguous run of work items ordered
// slice-major, so its X slice stays in LDS across the row blocks of one
// slice.  Partial sums go to part[slice][m][row] (fp32, m < M), combined by
// k_skinny_reduce.
// ---------------------------------------------------------------------------
constexpr int SK_WAVES = 8;
constexpr int SK_ROWS = 16 * SK_WAVES;       // rows per workgroup
constexpr int SK_KS_MAX = 4096;              // longest K slice

struct SkRegs {
  u32x4 w0, w1;
  uint32_t q;
  float d;
};

__global__ __launch_bounds__(512) void k_skinny_partial(
    const uint16_t* __restrict__ X, int M, const uint8_t* __restrict__ packed,
    const uint8_t* __restrict__ qabs, const float* __restrict__ gscale,
    const uint16_t* __restrict__ A, int N, int K, int r, int rpad, int KS,
    int wg_rows, int nitems, float* __restrict__ part, Codebook cb) {
  // rows [0, N) weight, [N, Np16) zero padding, [Np16, Np16 + rpad) adapter
  const int Np16 = (N + 15) & ~15;
  const int rows_total = Np16 + rpad;
  const int XP = KS + 8;                       // sX pitch (bf16)
  extern __shared__ __attribute__((aligned(16))) uint16_t sX[];   // (M+1) x XP
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int64_t numel = (int64_t)N * K;
  const rsrc_t rp = make_rsrc(packed, (uint32_t)((numel + 1) >> 1));
  const rsrc_t rq = make_rsrc(qabs, (uint32_t)((numel + 63) >> 6));
  const rsrc_t rd = make_rsrc(gscale, (uint32_t)(((numel + 16383) >> 14) << 2));
  const rsrc_t ra = make_rsrc(A, (uint32_t)((int64_t)r * K * 2));
  const rsrc_t rx = make_rsrc(X, (uint32_t)((int64_t)M * K * 2));

  // work items (block of SK_ROWS rows, K slice), item = slice * wg_rows +
  // row block; this workgroup takes items [ib, ie)
  const int ipw = (nitems + gridDim.x - 1) / gridDim.x;
  const int ib = blockIdx.x * ipw, ie = min(nitems, ib + ipw);
  for (int c = tid; c < KS / 8; c += 512)
    *reinterpret_cast<u32x4*>(sX + M * XP + 8 * c) = u32x4{0u, 0u, 0u, 0u};
  int staged = -1;                               // slice held in sX
  for (int item = ib; item < ie; ++item) {
    const int rb = item % wg_rows, slice = item / wg_rows;
    const int k0 = slice * KS;
    const int klen = min(KS, K - k0);
    const int row0 = rb * SK_ROWS + wave * 16;   // first row of the wave
    const int row = row0 + n;

    // X slice -> LDS (M rows, columns >= klen zero), each 8-element group
    // permuted into the order decode8p produces; loads issued before use.
    if (slice != staged) {
      if (staged >= 0) __syncthreads();          // sX still being read
      staged = slice;
      const int groups = M * (KS / 8);
      // batches of 4 loads per thread, all issued before their LDS writes
      for (int i0 = 0; i0 < groups; i0 += 4 * 512) {
        u32x4 xv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int idx = i0 + tid + 512 * i;
          const int m = idx / (KS / 8), c = 8 * (idx % (KS / 8));
          const bool ok = idx < groups && c < klen;
          xv[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
              rx, ok ? (uint32_t)(((int64_t)m * K + k0 + c) * 2) : G_OOB, 0, 0));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int idx = i0 + tid + 512 * i;
          if (idx < groups) {
            const int m = idx / (KS / 8), c = 8 * (idx % (KS / 8));
            *reinterpret_cast<u32x4*>(sX + m * XP + c) = permute8(xv[i]);
          }
        }
      }
      __syncthreads();
    }

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (row0 < rows_total) {
      const bool is_w = row0 < Np16;             // wave-uniform
      // lanes whose A-operand row is >= M read the all-zero row M of sX
      const uint16_t* xrow = sX + (n < M ? n : M) * XP + 64 * g;
      auto load = [&](SkRegs& R, int kc) {
        const int k = k0 + kc + 64 * g;
        const int64_t e = (int64_t)row * K + k;
        const bool okw = is_w && kc + 64 * g < klen && row < N;
        const uint32_t op = okw ? (uint32_t)(e >> 1) : G_OOB;
        R.w0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, op, 0, 0));
        R.w1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, op + 16, 0, 0));
        R.q = __builtin_amdgcn_raw_buffer_load_b8(rq, okw ? (uint32_t)(e >> 6) : G_OOB, 0, 0);
        R.d = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
            rd, okw ? (uint32_t)((e >> 14) << 2) : G_OOB, 0, 0));
      };
      auto chunk = [&](const SkRegs& R, int kc) {
        u32x4 a[8];
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8)
          a[s8] = *reinterpret_cast<const u32x4*>(xrow + kc + 8 * s8);
        if (is_w) {
          const Lut t = make_lut(cb, static_cast<float>(R.q) * R.d);
          const uint32_t wd[8] = {R.w0.x, R.w0.y, R.w0.z, R.w0.w,
                                  R.w1.x, R.w1.y, R.w1.z, R.w1.w};
#pragma unroll
          for (int s8 = 0; s8 < 8; ++s8) acc = mfma16(a[s8], decode8p(wd[s8], t), acc);
        } else {
          const int j = row - Np16;
          const int k = k0 + kc + 64 * g;
          const bool ok = kc + 64 * g < klen && j < r;
#pragma unroll
          for (int s8 = 0; s8 < 8; ++s8) {
            const u32x4 b = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                ra, ok ? (uint32_t)(((int64_t)j * K + k + 8 * s8) * 2) : G_OOB, 0, 0));
            acc = mfma16(a[s8], permute8(b), acc);
          }
        }
      };
      // two register sets, loaded one chunk ahead, no copies between them
      SkRegs ra0, ra1;
      load(ra0, 0);
      for (int kc = 0; kc < klen; kc += 512) {
        load(ra1, kc + 256);
        chunk(ra0, kc);
        if (kc + 256 >= klen) break;
        load(ra0, kc + 512);
        chunk(ra1, kc + 256);
      }
    }
    // acc[v] = C[m = 4 g + v][row n]
    if (row < rows_total) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = 4 * g + v;
        if (m < M) part[((int64_t)slice * M + m) * rows_total + row] = acc[v];
      }
    }
  }
}

// Y[m][n] = sum_slices part[.][m][n] + s * sum_j T[m][j] B[n][j], and
// T[m][j] = sum_slices part[.][m][Np16 + j] (written to t_save by block 0).
// One thread per (m, n) output for 64 columns x 16 rows per workgroup; the
// slices are summed as four interleaved running sums combined in a fixed
// order, so the loads of a thread overlap and the result is deterministic.
__global__ __launch_bounds__(256) void k_skinny_reduce(
    const float* __restrict__ part, int slices, int M, int N, int r, int rpad,
    const uint16_t* __restrict__ B, float s, float* __restrict__ t_save,
    void* __restrict__ Y, int y_bf16) {
  __shared__ float sT[16 * QN_MAX_RANK];
  const int Np16 = (N + 15) & ~15;
  const int64_t rows_total = Np16 + rpad;
  for (int idx = threadIdx.x; idx < M * r; idx += 256) {
    const int m = idx / r, j = idx % r;
    float t[4] = {0.f, 0.f, 0.f, 0.f};
    int sl = 0;
    for (; sl + 4 <= slices; sl += 4)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        t[u] += part[((int64_t)(sl + u) * M + m) * rows_total + Np16 + j];
    for (; sl < slices; ++sl) t[0] += part[((int64_t)sl * M + m) * rows_total + Np16 + j];
    const float v = (t[0] + t[1]) + (t[2] + t[3]);
    sT[idx] = v;
    if (blockIdx.x == 0) t_save[idx] = v;
  }
  __syncthreads();
  const int n = blockIdx.x * 64 + (threadIdx.x & 63);
  if (n >= N) return;
#pragma unroll
  for (int mm = 0; mm < 4; ++mm) {
    const int m = (threadIdx.x >> 6) + 4 * mm;
    if (m >= M) break;
    float y[4] = {0.f, 0.f, 0.f, 0.f};
    int sl = 0;
    for (; sl + 4 <= slices; sl += 4)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        y[u] += part[((int64_t)(sl + u) * M + m) * rows_total + n];
    for (; sl < slices; ++sl) y[0] += part[((int64_t)sl * M + m) * rows_total + n];
    float lora = 0.f;
    for (int j = 0; j < r; ++j)
      lora += sT[m * r + j] * bf16_to_f32(B[(int64_t)n * r + j]);
    store_out(Y, y_bf16, (int64_t)m * N + n,
              ((y[0] + y[1]) + (y[2] + y[3])) + s * lora);
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

const Codebook& codebook() {
  static const Codebook cb = [] {
    Codebook c;
    qn::derive_codebook(c.L, c.T);
    return c;
  }();
  return cb;
}

bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

int check_launch() {
  return hipGetLastError() == hipSuccess ? QN_OK : QN_EHIP;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool valid_tensor(const nf4_tensor* w) {
  return w != nullptr && w->packed != nullptr && w->qabs != nullptr &&
         w->gscale != nullptr && w->rows > 0 && w->cols > 0 &&
         aligned16(w->packed);
}

// Rank-tile dispatch: JT = number of 16-wide tiles of r, rounded up to a
// power of two (1, 2, 4, 8, 16 covers r <= 256); rpad = 16 JT.
int rank_tiles(int r) {
  int jt = 1;
  while (jt * 16 < r) jt *= 2;
  return jt;
}

bool valid_linear(int64_t M, const nf4_tensor* w, int32_t r) {
  if (!valid_tensor(w) || M <= 0) return false;
  if (r < 1 || r > QN_MAX_RANK) return false;
  const int64_t N = w->rows, K = w->cols;
  if (K % QN_BLOCK != 0 || N % 8 != 0) return false;
  // 32-bit index arithmetic inside the GEMM kernels
  if (M > (1LL << 30) || N > (1LL << 30) || K > (1LL << 30)) return false;
  // buffer-resource ranges are 32-bit byte counts (offsets past 2^31 mean
  // "out of range"): every operand read through one stays below 2 GiB
  const int64_t lim = 1LL << 31;
  if (M * K * 2 >= lim || M * N * 2 >= lim || N * K / 2 >= lim) return false;
  // fp32 rank-r partial rows [N or K][rpad] addressed through a resource
  if (std::max(N, K) * 4 * 16 * rank_tiles(r) >= lim) return false;
  return true;
}

// Per-launch event recording for one named kernel (qn_profile_kernel).
struct ProfileHook {
  char name[64] = {0};
  void** ev_start = nullptr;
  void** ev_stop = nullptr;
  int32_t capacity = 0;
  int32_t count = 0;
} g_prof;

struct ProfScope {
  hipStream_t st;
  int slot = -1;
  ProfScope(const char* kname, hipStream_t s) : st(s) {
    if (g_prof.capacity > 0 && g_prof.count < g_prof.capacity &&
        std::strcmp(g_prof.name, kname) == 0) {
      slot = g_prof.count++;
      (void)hipEventRecord((hipEvent_t)g_prof.ev_start[slot], st);
    }
  }
  ~ProfScope() {
    if (slot >= 0) (void)hipEventRecord((hipEvent_t)g_prof.ev_stop[slot], st);
  }
};

#define QN_LAUNCH_SHM(kname, kernel, grid, block, shm, st, ...)       \
  do {                                                                \
    ProfScope qn_prof_scope_(kname, st);                              \
    hipLaunchKernelGGL(kernel, grid, block, shm, st, __VA_ARGS__);    \
  } while (0)
#define QN_LAUNCH(kname, kernel, grid, block, st, ...) \
  QN_LAUNCH_SHM(kname, kernel, grid, block, 0, st, __VA_ARGS__)

// Fused GEMM launch: 256 x 256 tiles when they give at least ~one
// workgroup per CU, otherwise 128 x 128.
template <int BM, int BN, bool BWD>
void launch_gemm_t(hipStream_t st, const uint16_t* Aop, const nf4_tensor* w,
                   const uint16_t* La_hi, const uint16_t* La_lo,
                   const uint16_t* Lb, int M, int rpad, void* out,
                   int out_bf16) {
  const int N = (int)w->rows, K = (int)w->cols;
  const int nout = BWD ? K : N;
  const unsigned tiles = (unsigned)(cdiv(M, BM) * cdiv(nout, BN));
  QN_LAUNCH(BWD ? "k_bwd_dx_gemm" : "k_fwd_gemm", (k_gemm<BM, BN, BWD>),
            dim3(tiles), dim3(GemmCfg<BM, BN, BWD>::NT), st, Aop, w->packed, w->qabs, w->gscale,
            La_hi, La_lo, Lb, M, N, K, rpad, out, out_bf16, codebook());
}

template <bool BWD>
void launch_gemm(hipStream_t st, const uint16_t* Aop, const nf4_tensor* w,
                 const uint16_t* La_hi, const uint16_t* La_lo,
                 const uint16_t* Lb, int M, int rpad, void* out,
                 int out_bf16) {
  const int64_t nout = BWD ? w->cols : w->rows;
  if (cdiv(M, 256) * cdiv(nout, 256) >= 192)
    launch_gemm_t<256, 256, BWD>(st, Aop, w, La_hi, La_lo, Lb, M, rpad, out,
                                 out_bf16);
  else
    launch_gemm_t<128, 128, BWD>(st, Aop, w, La_hi, La_lo, Lb, M, rpad, out,
                                 out_bf16);
}


#define QN_RANK_DISPATCH(r, CALL)                \
  switch (rank_tiles(r)) {                       \
    case 1: { constexpr int JT = 1; CALL; break; }   \
    case 2: { constexpr int JT = 2; CALL; break; }   \
    case 4: { constexpr int JT = 4; CALL; break; }   \
    case 8: { constexpr int JT = 8; CALL; break; }   \
    default: { constexpr int JT = 16; CALL; break; } \
  }

// Rank-stream geometry: RM rows per workgroup, stages of 64 SUB columns,
// and enough column blocks for one long-lived workgroup per CU (each keeps
// two stages in flight).
struct StreamPlan {
  int rm, sub, mb, nb, cpb;
};

StreamPlan stream_plan(int mode, int64_t M, int64_t C, int jt) {
  StreamPlan P;
  P.rm = rs_rm(mode, jt);
  P.sub = rs_sub(mode, jt);
  P.mb = (int)cdiv(M, P.rm);
  const int64_t nst = cdiv(C, 64 * P.sub);
  const int64_t want = std::max<int64_t>(1, cdiv(256, P.mb));
  const int64_t nb = std::min(nst, want);
  P.cpb = (int)cdiv(nst, nb);
  P.nb = (int)cdiv(nst, P.cpb);
  return P;
}

template <int MODE>
void launch_rank_stream(hipStream_t st, const char* kname, const StreamPlan& P,
                        const uint16_t* S, int M, int C, const uint16_t* R,
                        int r, const uint16_t* Uh, const uint16_t* Ul, int ldu,
                        float* prow, float* pcol) {
  const dim3 grid((unsigned)P.nb, (unsigned)P.mb);
  QN_RANK_DISPATCH(r, QN_LAUNCH(kname, (k_rank_stream<MODE, JT>), grid,
                                dim3(256), st, S, M, C, R, r, Uh, Ul, ldu,
                                P.cpb, prow, pcol));
}

FinishArgs finish_args() {
  FinishArgs a;
  std::memset(&a, 0, sizeof(a));
  return a;
}

void launch_finish(hipStream_t st, FinishArgs& a) {
  a.nbR = a.R.src != nullptr ? (int)cdiv((int64_t)a.R.Mp * a.R.rpad, 256) : 0;
  a.nbC = a.Cc.src != nullptr ? (int)cdiv((int64_t)a.Cc.C * a.Cc.r, 256) : 0;
  a.nbP1 = a.P1.src != nullptr ? (int)cdiv((int64_t)a.P1.rows * a.P1.dw, 256) : 0;
  a.nbP2 = a.P2.src != nullptr ? (int)cdiv((int64_t)a.P2.rows * a.P2.dw, 256) : 0;
  const int nblk = a.nbR + a.nbC + a.nbP1 + a.nbP2;
  if (nblk > 0)
    QN_LAUNCH("k_rank_finish", k_rank_finish, dim3((unsigned)nblk), dim3(256),
              st, a);
}

// Skinny path plan: K slices of ks columns (multiple of 256, <= 2048),
// enough slices for ~2 workgroups per CU.
struct SkinnyPlan {
  int slices, ks, rows_total, wg_rows;
};

constexpr int SK_WGS_PER_CU = 2;     // resident skinny workgroups per CU
constexpr int64_t SK_LDS_PER_WG = 64 * 1024;   // X tile budget (bytes)

SkinnyPlan skinny_plan(int64_t M, int64_t N, int64_t K, int r) {
  SkinnyPlan P;
  P.rows_total = (int)(((N + 15) & ~15LL) + 16 * rank_tiles(r));
  P.wg_rows = (int)cdiv(P.rows_total, SK_ROWS);
  const int64_t kchunks = cdiv(K, 256);
  // longest slice whose X tile ((M + 1) rows, zero row included) leaves room
  // for two workgroups per CU, and enough slices for ~2 items per workgroup
  int64_t ks_max = (SK_LDS_PER_WG / (2 * (M + 1)) - 8) / 256 * 256;
  ks_max = std::max<int64_t>(256, std::min<int64_t>(ks_max, SK_KS_MAX));
  int64_t slices = std::max<int64_t>(cdiv(K, ks_max),
                                     cdiv(256 * SK_WGS_PER_CU * 2, P.wg_rows));
  slices = std::min<int64_t>(slices, kchunks);
  const int64_t ks = cdiv(kchunks, slices) * 256;
  P.ks = (int)ks;
  P.slices = (int)cdiv(K, ks);
  return P;
}

template <typename T>
T* ws_at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

}  // namespace

namespace qn {

FwdWorkspace fwd_workspace_layout(int64_t M, int64_t N, int64_t K,
                                  int32_t r) {
  FwdWorkspace L{};
  L.rpad = 16 * rank_tiles(r);
  if (M <= qn::QN_SKINNY_M) {
    const SkinnyPlan P = skinny_plan(M, N, K, r);
    L.slices = P.slices;
    L.ks = P.ks;
    L.part = 0;
    L.total = align256(size_t(P.slices) * M * P.rows_total * 4);
    return L;
  }
  const StreamPlan P = stream_plan(RS_ROWS, M, K, rank_tiles(r));
  size_t off = 0;
  L.th = off;
  off += align256(size_t(M) * L.rpad * 2);
  L.tl = off;
  off += align256(size_t(M) * L.rpad * 2);
  L.bp = off;
  off += align256(size_t(N) * L.rpad * 2);
  L.prow = off;
  off += align256(size_t(P.nb) * M * L.rpad * 4);
  L.total = off;
  return L;
}

BwdWorkspace bwd_workspace_layout(int64_t M, int64_t N, int64_t K,
                                  int32_t r) {
  BwdWorkspace L{};
  const int jt = rank_tiles(r);
  L.rpad = 16 * jt;
  L.mp = cdiv(M, 8) * 8;
  const StreamPlan Pg = stream_plan(RS_ROWS | RS_COLS, M, N, jt);
  const StreamPlan Pa = stream_plan(RS_COLS, M, K, jt);
  const size_t pcol = std::max(size_t(Pg.mb) * N, size_t(Pa.mb) * K);
  size_t off = 0;
  L.bt = off;
  off += align256(size_t(r) * N * 2);
  L.uth = off;
  off += align256(size_t(r) * L.mp * 2);
  L.utl = off;
  off += align256(size_t(r) * L.mp * 2);
  L.atp = off;
  off += align256(size_t(K) * L.rpad * 2);
  L.gh = off;
  off += align256(size_t(M) * L.rpad * 2);
  L.gl = off;
  off += align256(size_t(M) * L.rpad * 2);
  L.ugh = off;
  off += align256(size_t(r) * L.mp * 2);
  L.ugl = off;
  off += align256(size_t(r) * L.mp * 2);
  L.prow = off;
  off += align256(size_t(Pg.nb) * M * L.rpad * 4);
  L.pcol = off;
  off += align256(pcol * L.rpad * 4);
  L.total = off;
  return L;
}

}  // namespace qn

extern "C" {

int qn_profile_kernel(const char* name, void** ev_start, void** ev_stop,
                      int32_t capacity) {
  const int32_t recorded = g_prof.count;
  if (name == nullptr) {
    g_prof = ProfileHook();
    return recorded;
  }
  if (ev_start == nullptr || ev_stop == nullptr || capacity < 0 ||
      std::strlen(name) >= sizeof(g_prof.name))
    return QN_EINVAL;
  g_prof = ProfileHook();
  std::strcpy(g_prof.name, name);
  g_prof.ev_start = ev_start;
  g_prof.ev_stop = ev_stop;
  g_prof.capacity = capacity;
  return recorded;
}

const char* qn_strerror(int code) {
  switch (code) {
    case QN_OK: return "success";
    case QN_EINVAL: return "invalid argument";
    case QN_EWORKSPACE: return "workspace too small";
    case QN_EHIP: return "HIP launch error";
    case QN_ENONFINITE: return "non-finite weight";
    default: return "unknown error";
  }
}

int nf4_quantize(const float* w, const nf4_tensor* out, int32_t* status_dev,
                 void* stream) {
  if (w == nullptr || !valid_tensor(out) || !aligned16(w)) return QN_EINVAL;
  const int64_t numel = out->rows * out->cols;
  const int64_t nb = cdiv(numel, QN_BLOCK);
  const int64_t ng = cdiv(nb, QN_GROUP);
  if (ng > 0x7FFFFFFFLL) return QN_EINVAL;
  QN_LAUNCH("k_quantize", k_quantize, dim3((unsigned)ng), dim3(QZ_THREADS),
            (hipStream_t)stream, w, numel, out->packed, out->qabs,
            out->gscale, status_dev, codebook());
  return check_launch();
}

int nf4_dequantize_batch(const nf4_tensor* w, uint16_t* const* w_bf16,
                         int32_t count, void* stream) {
  if (w == nullptr || w_bf16 == nullptr || count < 1 || count > DQ_BATCH_MAX)
    return QN_EINVAL;
  DqBatch b;
  std::memset(&b, 0, sizeof(b));
  int64_t spans = 0;
  for (int i = 0; i < count; ++i) {
    if (!valid_tensor(&w[i]) || w_bf16[i] == nullptr || !aligned16(w_bf16[i]))
      return QN_EINVAL;
    b.t[i] = DqTensor{w[i].packed, w[i].qabs, w[i].gscale, w_bf16[i], spans};
    spans += w[i].rows * w[i].cols / DQ_SPAN;
  }
  b.nspans = spans;
  b.count = count;
  hipStream_t st = (hipStream_t)stream;
  if (spans > 0) {
    // up to 64 waves per CU; larger passes walk several spans per wave
    const int64_t grid = std::min<int64_t>(cdiv(spans, DQ_THREADS / 64), QN_DQ_GRID_CAP);
    QN_LAUNCH("k_dequant", k_dequant, dim3((unsigned)grid), dim3(DQ_THREADS),
              st, b, codebook());
  }
  for (int i = 0; i < count; ++i) {
    const int64_t numel = w[i].rows * w[i].cols;
    const int64_t e0 = numel / DQ_SPAN * DQ_SPAN;
    if (e0 < numel)
      QN_LAUNCH("k_dequant_tail", k_dequant_tail,
                dim3((unsigned)cdiv(numel - e0, DQ_THREADS)), dim3(DQ_THREADS),
                st, w[i].packed, w[i].qabs, w[i].gscale, e0, numel, w_bf16[i],
                codebook());
  }
  return check_launch();
}

int nf4_dequantize(const nf4_tensor* w, uint16_t* w_bf16, void* stream) {
  return nf4_dequantize_batch(w, &w_bf16, 1, stream);
}

size_t qlora_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t r,
                             int32_t which) {
  if (M <= 0 || N <= 0 || K <= 0 || r < 1 || r > QN_MAX_RANK) return 0;
  if (which == QN_FWD) return qn::fwd_workspace_layout(M, N, K, r).total;
  if (which == QN_BWD) return qn::bwd_workspace_layout(M, N, K, r).total;
  return 0;
}

int qlora_linear_fwd(const uint16_t* x, int64_t M, const nf4_tensor* w,
                     const uint16_t* A, const uint16_t* B, int32_t r,
                     float alpha, void* y, int32_t y_dtype, float* t_save,
                     void* ws, size_t ws_bytes, void* stream) {
  if (x == nullptr || A == nullptr || B == nullptr || y == nullptr ||
      t_save == nullptr)
    return QN_EINVAL;
  if (!valid_linear(M, w, r)) return QN_EINVAL;
  if (y_dtype != QN_F32 && y_dtype != QN_BF16) return QN_EINVAL;
  if (!aligned16(x) || !aligned16(A) || !aligned16(y) || !aligned16(t_save))
    return QN_EINVAL;
  const int64_t N = w->rows, K = w->cols;
  const qn::FwdWorkspace L = qn::fwd_workspace_layout(M, N, K, r);
  if (ws == nullptr || ws_bytes < L.total || !aligned16(ws))
    return QN_EWORKSPACE;
  const float s = alpha / (float)r;
  const int Mi = (int)M, Ni = (int)N, Ki = (int)K;
  hipStream_t st = (hipStream_t)stream;
  if (M <= qn::QN_SKINNY_M) {
    const SkinnyPlan P = skinny_plan(M, N, K, r);
    float* part = ws_at<float>(ws, L.part);
    const int nitems = P.wg_rows * P.slices;
    const size_t shm = size_t(M + 1) * (P.ks + 8) * 2;
    QN_LAUNCH_SHM("k_skinny_partial", k_skinny_partial,
                  dim3((unsigned)std::min(nitems, 256 * SK_WGS_PER_CU)),
                  dim3(512), shm, st, x, Mi, w->packed, w->qabs, w->gscale, A,
                  Ni, Ki, (int)r, L.rpad, P.ks, P.wg_rows, nitems, part,
                  codebook());
    QN_LAUNCH("k_skinny_reduce", k_skinny_reduce,
              dim3((unsigned)cdiv(N, 64)), dim3(256), st, part, P.slices, Mi,
              Ni, (int)r, L.rpad, B, s, t_save, y, (int)(y_dtype == QN_BF16));
    return check_launch();
  }
  uint16_t* Th = ws_at<uint16_t>(ws, L.th);
  uint16_t* Tl = ws_at<uint16_t>(ws, L.tl);
  uint16_t* Bp = ws_at<uint16_t>(ws, L.bp);
  float* prow = ws_at<float>(ws, L.prow);
  const int jt = rank_tiles(r);
  // T = X A^T: partials over column blocks of X
  const StreamPlan P = stream_plan(RS_ROWS, M, K, jt);
  launch_rank_stream<RS_ROWS>(st, "k_rank_stream_t", P, x, Mi, Ki, A, (int)r,
                              nullptr, nullptr, 0, prow, nullptr);
  // T (fp32, saved), hi/lo parts of s T, B zero-padded to [N][rpad]
  FinishArgs fa = finish_args();
  fa.R = FinishRows{prow, (int64_t)M * L.rpad, L.rpad, P.nb, Mi, Mi, (int)r,
                    L.rpad, s, t_save, Th, Tl, nullptr, nullptr};
  fa.P1 = FinishPad{B, Bp, Ni, L.rpad, (int)r, (int64_t)r, (int64_t)1};
  launch_finish(st, fa);
  launch_gemm<false>(st, x, w, Th, Tl, Bp, Mi, L.rpad, y,
                     (int)(y_dtype == QN_BF16));
  return check_launch();
}

int qlora_linear_bwd(const uint16_t* dy, const uint16_t* x, int64_t M,
                     const nf4_tensor* w, const uint16_t* A,
                     const uint16_t* B, int32_t r, float alpha,
                     const float* t_saved, void* dx, int32_t dx_dtype,
                     float* dA, float* dB, void* ws, size_t ws_bytes,
                     void* stream) {
  if (dy == nullptr || x == nullptr || A == nullptr || B == nullptr ||
      t_saved == nullptr || dx == nullptr || dA == nullptr || dB == nullptr)
    return QN_EINVAL;
  if (!valid_linear(M, w, r)) return QN_EINVAL;
  if (dx_dtype != QN_F32 && dx_dtype != QN_BF16) return QN_EINVAL;
  if (!aligned16(dy) || !aligned16(x) || !aligned16(A) || !aligned16(dx))
    return QN_EINVAL;
  const int64_t N = w->rows, K = w->cols;
  const qn::BwdWorkspace L = qn::bwd_workspace_layout(M, N, K, r);
  if (ws == nullptr || ws_bytes < L.total || !aligned16(ws))
    return QN_EWORKSPACE;
  uint16_t* Bt = ws_at<uint16_t>(ws, L.bt);
  uint16_t* UTh = ws_at<uint16_t>(ws, L.uth);
  uint16_t* UTl = ws_at<uint16_t>(ws, L.utl);
  uint16_t* Atp = ws_at<uint16_t>(ws, L.atp);
  uint16_t* Gh = ws_at<uint16_t>(ws, L.gh);
  uint16_t* Gl = ws_at<uint16_t>(ws, L.gl);
  uint16_t* UGh = ws_at<uint16_t>(ws, L.ugh);
  uint16_t* UGl = ws_at<uint16_t>(ws, L.ugl);
  float* prow = ws_at<float>(ws, L.prow);
  float* pcol = ws_at<float>(ws, L.pcol);
  const float s = alpha / (float)r;
  const int Mi = (int)M, Ni = (int)N, Ki = (int)K, Mp = (int)L.mp;
  const int jt = rank_tiles(r);
  hipStream_t st = (hipStream_t)stream;

  // s T transposed (hi/lo), A^T padded to [K][rpad], B^T
  FinishArgs f0 = finish_args();
  f0.R = FinishRows{t_saved, 0, (int)r, 1, Mi, Mp, (int)r, L.rpad, s,
                    nullptr, nullptr, nullptr, UTh, UTl};
  f0.P1 = FinishPad{A, Atp, Ki, L.rpad, (int)r, (int64_t)1, K};
  f0.P2 = FinishPad{B, Bt, (int)r, Ni, Ni, (int)1, (int64_t)r};
  launch_finish(st, f0);
  // one pass over dY: G = dY B (column-block partials), dB = dY^T (s T)
  // (row-block partials)
  const StreamPlan Pg = stream_plan(RS_ROWS | RS_COLS, M, N, jt);
  launch_rank_stream<RS_ROWS | RS_COLS>(st, "k_rank_stream_dy", Pg, dy, Mi, Ni,
                                        Bt, (int)r, UTh, UTl, Mp, prow, pcol);
  // hi/lo parts of s G (row-major and transposed), dB
  FinishArgs f1 = finish_args();
  f1.R = FinishRows{prow, (int64_t)M * L.rpad, L.rpad, Pg.nb, Mi, Mp, (int)r,
                    L.rpad, s, nullptr, Gh, Gl, UGh, UGl};
  f1.Cc = FinishCols{pcol, Pg.mb, Ni, (int)r, L.rpad, dB, (int64_t)r, 1};
  launch_finish(st, f1);
  // dX = dY W' + (s G) A
  launch_gemm<true>(st, dy, w, Gh, Gl, Atp, Mi, L.rpad, dx,
                    (int)(dx_dtype == QN_BF16));
  // dA = (s G)^T X: row-block partials of out[k][j] -> dA[j][k]
  const StreamPlan Pa = stream_plan(RS_COLS, M, K, jt);
  launch_rank_stream<RS_COLS>(st, "k_rank_stream_da", Pa, x, Mi, Ki, nullptr,
                              (int)r, UGh, UGl, Mp, nullptr, pcol);
  FinishArgs f2 = finish_args();
  f2.Cc = FinishCols{pcol, Pa.mb, Ki, (int)r, L.rpad, dA, (int64_t)1, K};
  launch_finish(st, f2);
  return check_launch();
}

}  // extern "C"
