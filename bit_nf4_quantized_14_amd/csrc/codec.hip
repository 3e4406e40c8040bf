// NF4 codec kernels of the QLoRA NF4 library: quantization with double
// quantization (K1) and dequantization to bf16 (K2), and their C entry
// points.  What is computed follows "Qlora Expert" (Core Concept: NF4 at
// N(0,1) quantiles, double quantization of the block constants),
// "QLoRA Implementation Details (2025 Edition)" (Step 1 NF4 Math: 64-value
// blocks) and the "QLORA ... paper summary" (Notes: load 4-bit, dequantize
// to BF16).
#include "qn_host.h"

namespace {

using namespace qn;

// Storage of the per-block constants (QN_CONST_*): 8-bit codes with one
// fp32 scale per group (double quantization), the fp32 absmax itself, or
// centered signed 8-bit codes with a scale and a mean per group.
enum ConstMode { CM_DQ8 = QN_CONST_DQ8, CM_FP32 = QN_CONST_FP32,
                 CM_CENTERED = QN_CONST_CENTERED };

// Centered decode c' = fp32(fp32(q d) + mu): two roundings, never fused.
__device__ __forceinline__ float centered_cprime(int32_t q, float d,
                                                 float mu) {
#pragma clang fp contract(off)
  const float p = static_cast<float>(q) * d;
  return p + mu;
}

// Decoded block constant from the raw per-block entry (zero-extended u8,
// fp32 bits, or sign-extended i8) and the group's scale and mean.
template <int CM>
__device__ __forceinline__ float cprime_of(uint32_t raw, float d, float mu) {
  if constexpr (CM == CM_DQ8) return static_cast<float>(raw) * d;
  else if constexpr (CM == CM_FP32) return __uint_as_float(raw);
  else return centered_cprime(static_cast<int32_t>(raw), d, mu);
}

template <int CM>
__device__ __forceinline__ uint32_t const_raw(const void* consts, int64_t b) {
  if constexpr (CM == CM_DQ8)
    return static_cast<const uint8_t*>(consts)[b];
  else if constexpr (CM == CM_FP32)
    return static_cast<const uint32_t*>(consts)[b];
  else
    return static_cast<uint32_t>(
        static_cast<int32_t>(static_cast<const int8_t*>(consts)[b]));
}

// ---------------------------------------------------------------------------
// K1: quantization + double quantization.  One workgroup per group of 256
// blocks (16384 weights); each thread owns 8 consecutive weights in each of
// 8 passes (8 lanes per 64-weight block).
// ---------------------------------------------------------------------------
constexpr int QZ_THREADS = 256;
constexpr int QZ_PASSES = 8;  // 8 * 256 * 8 = 16384 weights

// Threshold search by buckets.  n = w / absmax lies in [-1, 1]; bucket
// b = floor(64 n) + 64 (an exact scaling and floor) covers
// [(b - 64) / 64, (b - 63) / 64).  Every table's thresholds are more than
// 1/64 apart, so a bucket holds at most one of them: the code (the number
// of thresholds strictly below n) is base[b], the number below the bucket,
// plus (n > thr[b]) for the bucket's own threshold (thr = 2, above every n,
// where there is none).  Built on the host from the fp32 thresholds.
constexpr int QZ_BUCKETS = 129;
struct QuantLut {
  float thr[QZ_BUCKETS];
  uint8_t base[QZ_BUCKETS];
};

bool make_quant_lut(const Codebook& cb, QuantLut* out) {
  for (int b = 0; b < QZ_BUCKETS; ++b) {
    const double lo = (b - 64) / 64.0, hi = (b - 63) / 64.0;
    int below = 0, inside = 0;
    float thr = 2.0f;
    for (int j = 0; j < 15; ++j) {
      if (double(cb.T[j]) < lo) ++below;
      else if (double(cb.T[j]) < hi) { ++inside; thr = cb.T[j]; }
    }
    if (inside > 1) return false;
    out->thr[b] = thr;
    out->base[b] = static_cast<uint8_t>(below);
  }
  return true;
}

template <int CM>
__global__ __launch_bounds__(QZ_THREADS) void k_quantize(
    const float* __restrict__ w, int64_t numel, uint8_t* __restrict__ packed,
    void* __restrict__ consts, float* __restrict__ gscale,
    float* __restrict__ gmean, int32_t* __restrict__ status, QuantLut lut) {
  __shared__ float s_c[256];
  __shared__ uint2 s_lut[QZ_BUCKETS];     // (threshold bits, base code)
  for (int i = threadIdx.x; i < QZ_BUCKETS; i += QZ_THREADS)
    s_lut[i] = make_uint2(__float_as_uint(lut.thr[i]), lut.base[i]);
  __shared__ float s_wmax[QZ_THREADS / 64];
  __shared__ float s_wsum[QZ_THREADS / 64];
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

  // block constant of block `tid` of this group (0 past the last block)
  const float cb_t = s_c[tid];
  const int64_t b_this = g * QN_GROUP + tid;
  if constexpr (CM == CM_DQ8) {
    // group absmax -> d = max / 255, q = min(255, rint(c / d))
    float gm = cb_t;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) gm = fmaxf(gm, __shfl_xor(gm, off));
    if ((tid & 63) == 0) s_wmax[tid >> 6] = gm;
    __syncthreads();
    float smax = s_wmax[0];
#pragma unroll
    for (int i = 1; i < QZ_THREADS / 64; ++i) smax = fmaxf(smax, s_wmax[i]);
    const float d = (smax == 0.0f) ? 0.0f : smax / 255.0f;
    if (b_this < nb_total) {
      float qv = 0.0f;
      if (smax != 0.0f) qv = fminf(rintf(cb_t / d), 255.0f);
      static_cast<uint8_t*>(consts)[b_this] = static_cast<uint8_t>(qv);
    }
    if (tid == 0) gscale[g] = d;
  } else if constexpr (CM == CM_FP32) {
    if (b_this < nb_total) static_cast<float*>(consts)[b_this] = cb_t;
  } else {
    // pairwise sum over the 256 (zero-padded) constants: the xor butterfly
    // with offsets 1, 2, ..., 32 adds adjacent pairs level by level inside
    // a wave (a + b == b + a, so both partners hold the same sum); the four
    // wave sums finish the last two levels
    float sum = cb_t;
#pragma unroll
    for (int off = 1; off <= 32; off <<= 1) sum = sum + __shfl_xor(sum, off);
    if ((tid & 63) == 0) s_wsum[tid >> 6] = sum;
    __syncthreads();
    const float total = (s_wsum[0] + s_wsum[1]) + (s_wsum[2] + s_wsum[3]);
    const int64_t left = nb_total - g * QN_GROUP;
    const int nvalid = left < QN_GROUP ? static_cast<int>(left) : QN_GROUP;
    const float mu = total / static_cast<float>(nvalid);
    const bool valid = b_this < nb_total;
    const float dev = cb_t - mu;
    float am = valid ? fabsf(dev) : 0.0f;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) am = fmaxf(am, __shfl_xor(am, off));
    if ((tid & 63) == 0) s_wmax[tid >> 6] = am;
    __syncthreads();
    float dmax = s_wmax[0];
#pragma unroll
    for (int i = 1; i < QZ_THREADS / 64; ++i) dmax = fmaxf(dmax, s_wmax[i]);
    const float d = (dmax == 0.0f) ? 0.0f : dmax / 127.0f;
    if (valid) {
      float qv = 0.0f;
      if (dmax != 0.0f) qv = fminf(fmaxf(rintf(dev / d), -127.0f), 127.0f);
      static_cast<int8_t*>(consts)[b_this] =
          static_cast<int8_t>(static_cast<int32_t>(qv));
    }
    if (tid == 0) {
      gscale[g] = d;
      gmean[g] = mu;
    }
  }

  // NF4 codes against the un-quantized block constant
  const int64_t nbytes = (numel + 1) / 2;
#pragma unroll
  for (int it = 0; it < QZ_PASSES; ++it) {
    const int64_t e0 = gbase + it * (QZ_THREADS * 8) + tid * 8;
    if (e0 >= numel) break;
    // an all-zero block (c = 0) holds only +-0, and +-0 / 1 = +-0 gets the
    // code of n = 0: dividing by 1 there keeps the divides branch-free
    const float c = cmine[it] == 0.0f ? 1.0f : cmine[it];
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float n = v[it][i] / c;
      // floor(64 n) in [-64, 64]; the clamp (NaN -> -64) only matters for
      // non-finite weights, which set the status flag
      const float fb = fminf(fmaxf(floorf(n * 64.0f), -64.0f), 64.0f);
      const uint2 e = s_lut[static_cast<int>(fb) + 64];
      const uint32_t code = e.y + (n > __uint_as_float(e.x) ? 1u : 0u);
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
  float mu;
};

// One launch dequantizes up to DQ_BATCH_MAX tensors: their whole spans are
// numbered consecutively (tensor i owns global spans [span0_i, span0_{i+1})).
constexpr int DQ_BATCH_MAX = QN_DEQUANT_BATCH_MAX;
struct DqTensor {
  const uint8_t* packed;
  const void* consts;
  const float* gscale;
  const float* gmean;
  uint16_t* out;
  int64_t span0;
};
struct DqBatch {
  DqTensor t[DQ_BATCH_MAX];
  int64_t nspans;       // total whole spans
  int count;
};

template <int CM>
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
    const int64_t blk0 = sp * (DQ_SPAN / 64);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      R.p[j] = pw[lane + 64 * j];
      R.q[j] = const_raw<CM>(b.t[ti].consts, blk0 + (lane >> 3) + 8 * j);
    }
    R.d = (CM != CM_FP32 && ok) ? b.t[ti].gscale[blk0 >> 8] : 0.0f;
    R.mu = (CM == CM_CENTERED && ok) ? b.t[ti].gmean[blk0 >> 8] : 0.0f;
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
      const Lut t = make_lut(cb, cprime_of<CM>(cur.q[j], cur.d, cur.mu));
      // streaming store: the output is not re-read here, and keeping it out
      // of L2 avoids a large write-back when the kernel retires
      __builtin_nontemporal_store(decode8(cur.p[j], t), &o[lane + 64 * j]);
    }
    cur = nxt;
  }
}

template <int CM>
__global__ __launch_bounds__(DQ_THREADS) void k_dequant_tail(
    DqTensor t, int64_t e0, int64_t numel, Codebook cb) {
  const int64_t e = e0 + (int64_t)blockIdx.x * DQ_THREADS + threadIdx.x;
  if (e >= numel) return;
  const uint32_t byte = t.packed[e >> 1];
  const uint32_t code = (e & 1) ? (byte >> 4) : (byte & 0xFu);
  const int64_t blk = e >> 6;
  const float d = CM != CM_FP32 ? t.gscale[blk >> 8] : 0.0f;
  const float mu = CM == CM_CENTERED ? t.gmean[blk >> 8] : 0.0f;
  t.out[e] = decode1(cb, code, cprime_of<CM>(const_raw<CM>(t.consts, blk), d, mu));
}

// Host side: launch quantization / dequantization for one constant mode.
template <int CM>
int launch_quantize(const float* w, int64_t numel, uint8_t* packed,
                    void* consts, float* gscale, float* gmean,
                    int32_t* status, const Codebook& cb, hipStream_t st) {
  const int64_t nb = cdiv(numel, QN_BLOCK);
  const int64_t ng = cdiv(nb, QN_GROUP);
  if (ng > 0x7FFFFFFFLL) return QN_EINVAL;
  QuantLut lut;
  if (!make_quant_lut(cb, &lut)) return QN_EINVAL;   // not for these tables
  QN_LAUNCH("k_quantize", k_quantize<CM>, dim3((unsigned)ng), dim3(QZ_THREADS),
            st, w, numel, packed, consts, gscale, gmean, status, lut);
  return check_launch();
}

template <int CM>
int launch_dequant(const DqTensor* t, const int64_t* numel, int count,
                   const Codebook& cb, hipStream_t st) {
  DqBatch b;
  std::memset(&b, 0, sizeof(b));
  int64_t spans = 0;
  for (int i = 0; i < count; ++i) {
    b.t[i] = t[i];
    b.t[i].span0 = spans;
    spans += numel[i] / DQ_SPAN;
  }
  b.nspans = spans;
  b.count = count;
  if (spans > 0) {
    // up to 64 waves per CU; larger passes walk several spans per wave
    const int64_t grid = std::min<int64_t>(cdiv(spans, DQ_THREADS / 64), QN_DQ_GRID_CAP);
    QN_LAUNCH("k_dequant", k_dequant<CM>, dim3((unsigned)grid), dim3(DQ_THREADS),
              st, b, cb);
  }
  for (int i = 0; i < count; ++i) {
    const int64_t e0 = numel[i] / DQ_SPAN * DQ_SPAN;
    if (e0 < numel[i])
      QN_LAUNCH("k_dequant_tail", k_dequant_tail<CM>,
                dim3((unsigned)cdiv(numel[i] - e0, DQ_THREADS)), dim3(DQ_THREADS),
                st, t[i], e0, numel[i], cb);
  }
  return check_launch();
}

// Codebook kernel arguments of the QN_CODE_* tables (host-derived once).
const Codebook* variant_codebook(int code) {
  struct Tabs {
    Codebook c[3];
  };
  static const Tabs tabs = [] {
    Tabs t;
    for (int i = 0; i < 3; ++i) derive_variant_codebook(i, t.c[i].L, t.c[i].T);
    return t;
  }();
  return (code >= 0 && code < 3) ? &tabs.c[code] : nullptr;
}

bool valid_qtensor(const qn_qtensor* t) {
  if (t == nullptr || t->packed == nullptr || t->consts == nullptr ||
      t->rows <= 0 || t->cols <= 0 || !aligned16(t->packed))
    return false;
  if (t->code < QN_CODE_NF4 || t->code > QN_CODE_INT4) return false;
  switch (t->consts_mode) {
    case QN_CONST_DQ8: return t->gscale != nullptr;
    case QN_CONST_FP32: return (reinterpret_cast<uintptr_t>(t->consts) & 3u) == 0;
    case QN_CONST_CENTERED: return t->gscale != nullptr && t->gmean != nullptr;
    default: return false;
  }
}

}  // namespace

extern "C" {

int nf4_quantize(const float* w, const nf4_tensor* out, int32_t* status_dev,
                 void* stream) {
  if (w == nullptr || !valid_tensor(out) || !aligned16(w)) return QN_EINVAL;
  return launch_quantize<CM_DQ8>(w, out->rows * out->cols, out->packed,
                                 out->qabs, out->gscale, nullptr, status_dev,
                                 qn::codebook(), (hipStream_t)stream);
}

int nf4_dequantize_batch(const nf4_tensor* w, uint16_t* const* w_bf16,
                         int32_t count, void* stream) {
  if (w == nullptr || w_bf16 == nullptr || count < 1 || count > DQ_BATCH_MAX)
    return QN_EINVAL;
  DqTensor t[DQ_BATCH_MAX];
  int64_t numel[DQ_BATCH_MAX];
  for (int i = 0; i < count; ++i) {
    if (!valid_tensor(&w[i]) || w_bf16[i] == nullptr || !aligned16(w_bf16[i]))
      return QN_EINVAL;
    t[i] = DqTensor{w[i].packed, w[i].qabs, w[i].gscale, nullptr, w_bf16[i], 0};
    numel[i] = w[i].rows * w[i].cols;
  }
  return launch_dequant<CM_DQ8>(t, numel, count, qn::codebook(),
                                (hipStream_t)stream);
}

int nf4_dequantize(const nf4_tensor* w, uint16_t* w_bf16, void* stream) {
  return nf4_dequantize_batch(w, &w_bf16, 1, stream);
}

int qn_quantize(const float* w, const qn_qtensor* out, int32_t* status_dev,
                void* stream) {
  if (w == nullptr || !valid_qtensor(out) || !aligned16(w)) return QN_EINVAL;
  const Codebook& cb = *variant_codebook(out->code);
  const int64_t numel = out->rows * out->cols;
  hipStream_t st = (hipStream_t)stream;
  switch (out->consts_mode) {
    case QN_CONST_DQ8:
      return launch_quantize<CM_DQ8>(w, numel, out->packed, out->consts,
                                     out->gscale, nullptr, status_dev, cb, st);
    case QN_CONST_FP32:
      return launch_quantize<CM_FP32>(w, numel, out->packed, out->consts,
                                      nullptr, nullptr, status_dev, cb, st);
    default:
      return launch_quantize<CM_CENTERED>(w, numel, out->packed, out->consts,
                                          out->gscale, out->gmean, status_dev,
                                          cb, st);
  }
}

int qn_dequantize(const qn_qtensor* w, uint16_t* w_bf16, void* stream) {
  if (!valid_qtensor(w) || w_bf16 == nullptr || !aligned16(w_bf16))
    return QN_EINVAL;
  const Codebook& cb = *variant_codebook(w->code);
  const int64_t numel = w->rows * w->cols;
  const DqTensor t{w->packed, w->consts, w->gscale, w->gmean, w_bf16, 0};
  hipStream_t st = (hipStream_t)stream;
  switch (w->consts_mode) {
    case QN_CONST_DQ8: return launch_dequant<CM_DQ8>(&t, &numel, 1, cb, st);
    case QN_CONST_FP32: return launch_dequant<CM_FP32>(&t, &numel, 1, cb, st);
    default: return launch_dequant<CM_CENTERED>(&t, &numel, 1, cb, st);
  }
}

}  // extern "C"
