// 8-bit AdamW step on the LoRA adapters, resident or paged through host
// memory.  "Qlora Expert" (Core Concept item 3: paged optimizers page the
// Adam moments between GPU and CPU memory; Hyperparameter Guidance:
// paged_adamw_8bit, 8-bit Adam states), "QLoRA Implementation Details (2025
// Edition)" (Step 5 Paged Optimizer: states in CPU RAM, paged in and out as
// needed), "QLORA ... paper summary" (Notes: adapters stored and trained in
// BF16).
//
// Per element, in this fp32 order and never fused (host constants rounded
// once from double: c1 = 1-b1, c2 = 1-b2, bc1 = 1/(1-b1^t),
// bc2 = 1/(1-b2^t), decay = 1-lr*wd):
//   g = g * gs;  m = b1 m' + c1 g;  v = b2 v' + c2 (g g)
//   p = bf16_rne(p decay - lr ((m bc1) / (sqrt(v bc2) + eps)))
// m' and v' = r'^2 are decoded from the stored state: per block of 256
// elements, E4M3 codes of m / s_m and of r / s_r with r = sqrt(v),
// s = fp32(block absmax / 448).
#include <cmath>
#include <vector>

#include "qn_host.h"

namespace {

using namespace qn;

constexpr int AW_BLOCK = QN_ADAMW_BLOCK;     // elements per state block
constexpr int AW_THREADS = 256;              // 4 waves, 4 blocks per wave step
constexpr float AW_E4M3_MAX = 448.0f;

struct AdamConsts {
  float b1, b2, c1, c2, bc1, bc2, eps, lr, decay, gs;
};

// OCP E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
// subnormals m * 2^-9, largest finite 448) through gfx950's conversion
// instructions: v_cvt_f32_fp8 decodes one byte of a dword exactly;
// v_cvt_pk_fp8_f32 rounds two fp32 values to nearest even into two bytes.
// The encoder clamps the magnitude to 448 first and stores a value that
// rounds to zero as code 0 (the instruction keeps the sign: 0x80).
template <int BYTE>
__device__ __forceinline__ float e4m3_value(uint32_t word) {
  return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(word), BYTE);
}

__device__ __forceinline__ uint32_t e4m3_encode4(float x0, float x1, float x2,
                                                 float x3) {
  auto c = [](float x) { return fminf(fmaxf(x, -AW_E4M3_MAX), AW_E4M3_MAX); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(c(x0), c(x1), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c(x2), c(x3), w, true);
  const uint32_t u = static_cast<uint32_t>(w);
  // 0x80 in each byte whose magnitude bits are nonzero
  const uint32_t nz = ((u & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) & 0x80808080u;
  return (u & 0x7F7F7F7Fu) | (u & nz);
}

struct Elem {
  float m, v, p;
};

// One element's step: new moments and the new fp32 parameter.
__device__ __forceinline__ Elem adam_elem(float g, float mo, float ro,
                                          float p, const AdamConsts& k) {
#pragma clang fp contract(off)
  Elem r;
  const float gg = g * k.gs;
  const float vo = ro * ro;
  r.m = k.b1 * mo + k.c1 * gg;
  const float g2 = gg * gg;
  r.v = k.b2 * vo + k.c2 * g2;
  const float den = sqrtf(r.v * k.bc2) + k.eps;
  const float u = (r.m * k.bc1) / den;
  r.p = p * k.decay - k.lr * u;
  return r;
}

// Maximum over the 16 lanes that hold one block (lanes 16 j .. 16 j + 15).
__device__ __forceinline__ float group_max16(float x) {
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

// x_i / s for the 16 values of a block whose absolute maximum is amax, as
// the correctly rounded fp32 quotient wherever it can decide an E4M3 code.
// The block is scaled by 2^k, k = 64 - exponent(amax) (clamped to the
// normal exponents): power-of-two scalings are exact, and then every value
// whose quotient reaches 2^-10 (the smallest magnitude with a nonzero code)
// is large enough that the fma residuals below stay normal.  With y the
// correctly rounded reciprocal of the scaled divisor, q = x y refined twice
// by r = x - q s (one fma, exact) and q + r y is RN(x / s) (Markstein's
// correction, which holds without underflow).  Smaller quotients may differ
// from RN in their last bit; all of them encode to code 0.  A block maximum
// that is not finite takes the IEEE division.
__device__ __forceinline__ void block_quot16(const float (&x)[16], float amax,
                                             float s, float (&q)[16]) {
#pragma clang fp contract(off)
  if (!__builtin_isfinite(amax)) {
#pragma unroll
    for (int i = 0; i < 16; ++i) q[i] = x[i] / s;
    return;
  }
  int k = 64 - __builtin_amdgcn_frexp_expf(amax);
  k = k > 127 ? 127 : (k < -126 ? -126 : k);
  const float sc = __builtin_ldexpf(1.0f, k);
  const float s2 = s * sc;
  const float y = 1.0f / s2;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float a = x[i] * sc;
    const float q0 = a * y;
    const float q1 = __builtin_fmaf(__builtin_fmaf(-q0, s2, a), y, q0);
    q[i] = __builtin_fmaf(__builtin_fmaf(-q1, s2, a), y, q1);
  }
}

__device__ __forceinline__ void e4m3_decode4(uint32_t w, float s, float* out) {
  out[0] = e4m3_value<0>(w) * s;
  out[1] = e4m3_value<1>(w) * s;
  out[2] = e4m3_value<2>(w) * s;
  out[3] = e4m3_value<3>(w) * s;
}

// Operands of one lane: 16 consecutive elements of one block (gradients,
// bf16 parameters as 8 words, the codes of each moment as 4 words) and the
// block's two scales.
struct AwLoads {
  f32x4 g[4];
  u32x4 p[2];
  u32x4 mc, rc;
  float sm, sr;
};

struct AwOut {
  u32x4 p[2];
  u32x4 mc, rc;
  float sm, sr;
};

// One block's step for the 16 lanes that hold it (16 elements per lane).
__device__ __forceinline__ AwOut adam_block(const AwLoads& L,
                                            const AdamConsts& k) {
  const float g[16] = {L.g[0].x, L.g[0].y, L.g[0].z, L.g[0].w,
                       L.g[1].x, L.g[1].y, L.g[1].z, L.g[1].w,
                       L.g[2].x, L.g[2].y, L.g[2].z, L.g[2].w,
                       L.g[3].x, L.g[3].y, L.g[3].z, L.g[3].w};
  const uint32_t pw[8] = {L.p[0].x, L.p[0].y, L.p[0].z, L.p[0].w,
                          L.p[1].x, L.p[1].y, L.p[1].z, L.p[1].w};
  const uint32_t mw[4] = {L.mc.x, L.mc.y, L.mc.z, L.mc.w};
  const uint32_t rw[4] = {L.rc.x, L.rc.y, L.rc.z, L.rc.w};
  float mo[16], ro[16];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    e4m3_decode4(mw[j], L.sm, mo + 4 * j);
    e4m3_decode4(rw[j], L.sr, ro + 4 * j);
  }
  float m[16], r[16], pn[16];
  float am = 0.0f, ar = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float pv = bf16_to_f32(i & 1 ? pw[i >> 1] >> 16 : pw[i >> 1] & 0xFFFFu);
    const Elem el = adam_elem(g[i], mo[i], ro[i], pv, k);
    m[i] = el.m;
    r[i] = sqrtf(el.v);            // r = sqrt(v), the stored quantity
    pn[i] = el.p;
    am = fmaxf(am, fabsf(m[i]));
    ar = fmaxf(ar, r[i]);
  }
  am = group_max16(am);
  ar = group_max16(ar);
  const float sm = am / AW_E4M3_MAX;
  const float sr = ar / AW_E4M3_MAX;
  float qm[16], qr[16];
  block_quot16(m, am, sm, qm);
  block_quot16(r, ar, sr, qr);
  AwOut o;
  uint32_t mcw[4], rcw[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    mcw[j] = am == 0.0f ? 0u
                        : e4m3_encode4(qm[4 * j], qm[4 * j + 1], qm[4 * j + 2],
                                       qm[4 * j + 3]);
    rcw[j] = ar == 0.0f ? 0u
                        : e4m3_encode4(qr[4 * j], qr[4 * j + 1], qr[4 * j + 2],
                                       qr[4 * j + 3]);
  }
  o.mc = u32x4{mcw[0], mcw[1], mcw[2], mcw[3]};
  o.rc = u32x4{rcw[0], rcw[1], rcw[2], rcw[3]};
  uint32_t po[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) po[j] = pack_bf16x2(pn[2 * j], pn[2 * j + 1]);
  o.p[0] = u32x4{po[0], po[1], po[2], po[3]};
  o.p[1] = u32x4{po[4], po[5], po[6], po[7]};
  o.sm = am == 0.0f ? 0.0f : sm;
  o.sr = ar == 0.0f ? 0.0f : sr;
  return o;
}

// A wave steps 4 whole blocks (1024 consecutive elements, lane l holding
// elements 16 l .. 16 l + 15 of them) per iteration, the loads of its next
// 4 blocks in flight; two register sets alternate, every iteration issues
// the same loads and stores (out of range for blocks past the whole ones),
// so the compiler's waits leave the next loads in flight.  A short last
// block is done afterwards by lanes 0..15 of one wave with per-element
// guards (its missing elements count as zero for the block maxima and are
// not stored).
__global__ __launch_bounds__(AW_THREADS) void k_adamw8(
    uint16_t* __restrict__ p, const float* __restrict__ g, int64_t n,
    uint8_t* __restrict__ mc, float* __restrict__ ms,
    uint8_t* __restrict__ rc, float* __restrict__ rs, AdamConsts k) {
  const int lane = threadIdx.x & 63;
  const int64_t nwhole = n / AW_BLOCK;
  const int64_t nquad = (nwhole + 3) / 4;          // groups of 4 blocks
  const int64_t wave0 = __builtin_amdgcn_readfirstlane(
      (int)(((int64_t)blockIdx.x * AW_THREADS + threadIdx.x) >> 6));
  const int64_t nwaves = ((int64_t)gridDim.x * AW_THREADS) >> 6;
  const int blk = lane >> 4;                       // block of the quad
  // per-quad buffer resources: offsets stay small whatever n is
  auto loadq = [&](AwLoads& L, int64_t qd) {
    const int64_t b = 4 * qd + blk;
    const bool ok = qd < nquad && b < nwhole;
    const int64_t e0 = qd < nquad ? 4 * qd * AW_BLOCK : 0;
    const rsrc_t rg = make_rsrc(g + e0, 4 * AW_BLOCK * 4);
    const rsrc_t rp = make_rsrc(p + e0, 4 * AW_BLOCK * 2);
    const rsrc_t rm = make_rsrc(mc + e0, 4 * AW_BLOCK);
    const rsrc_t rr = make_rsrc(rc + e0, 4 * AW_BLOCK);
    const rsrc_t rsm = make_rsrc(ms + (qd < nquad ? 4 * qd : 0), 16);
    const rsrc_t rsr = make_rsrc(rs + (qd < nquad ? 4 * qd : 0), 16);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      L.g[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
          rg, ok ? (uint32_t)(64 * lane + 16 * j) : G_OOB, 0, 0));
#pragma unroll
    for (int j = 0; j < 2; ++j)
      L.p[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
          rp, ok ? (uint32_t)(32 * lane + 16 * j) : G_OOB, 0, 0));
    L.mc = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
        rm, ok ? (uint32_t)(16 * lane) : G_OOB, 0, 0));
    L.rc = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
        rr, ok ? (uint32_t)(16 * lane) : G_OOB, 0, 0));
    L.sm = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
        rsm, ok ? (uint32_t)(4 * blk) : G_OOB, 0, 0));
    L.sr = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
        rsr, ok ? (uint32_t)(4 * blk) : G_OOB, 0, 0));
  };
  auto stepq = [&](const AwLoads& L, int64_t qd) {
    const AwOut o = adam_block(L, k);
    const int64_t b = 4 * qd + blk;
    const bool ok = b < nwhole;
    const int64_t e0 = 4 * qd * AW_BLOCK;
    const rsrc_t rp = make_rsrc(p + e0, 4 * AW_BLOCK * 2);
    const rsrc_t rm = make_rsrc(mc + e0, 4 * AW_BLOCK);
    const rsrc_t rr = make_rsrc(rc + e0, 4 * AW_BLOCK);
    const rsrc_t rsm = make_rsrc(ms + 4 * qd, 16);
    const rsrc_t rsr = make_rsrc(rs + 4 * qd, 16);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      __builtin_amdgcn_raw_buffer_store_b128(
          o.p[j], rp, ok ? (uint32_t)(32 * lane + 16 * j) : G_OOB, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(o.mc, rm, ok ? (uint32_t)(16 * lane) : G_OOB,
                                           0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(o.rc, rr, ok ? (uint32_t)(16 * lane) : G_OOB,
                                           0, 0);
    const bool lead = ok && (lane & 15) == 0;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o.sm), rsm,
                                          lead ? (uint32_t)(4 * blk) : G_OOB, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o.sr), rsr,
                                          lead ? (uint32_t)(4 * blk) : G_OOB, 0, 0);
  };
  if (nquad > 0) {
    AwLoads A, B;
    int64_t qd = wave0;
    loadq(A, qd);
    for (; qd + nwaves < nquad; qd += 2 * nwaves) {
      loadq(B, qd + nwaves);
      stepq(A, qd);
      loadq(A, qd + 2 * nwaves);
      stepq(B, qd + nwaves);
    }
    if (qd < nquad) stepq(A, qd);
  }
  if (n % AW_BLOCK != 0 && wave0 == 0) {
    // the short last block: lanes 0..15, guarded per element
    const int64_t b = nwhole;
    const int64_t e0 = b * AW_BLOCK + 16 * (lane & 15);
    AwLoads L;
    float gv[16];
    uint32_t pb[16], mb[16], rb[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bool in = lane < 16 && e0 + i < n;
      gv[i] = in ? g[e0 + i] : 0.0f;
      pb[i] = in ? static_cast<uint32_t>(p[e0 + i]) : 0u;
      mb[i] = in ? static_cast<uint32_t>(mc[e0 + i]) : 0u;
      rb[i] = in ? static_cast<uint32_t>(rc[e0 + i]) : 0u;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      L.g[j] = f32x4{gv[4 * j], gv[4 * j + 1], gv[4 * j + 2], gv[4 * j + 3]};
      const uint32_t m4 = mb[4 * j] | (mb[4 * j + 1] << 8) | (mb[4 * j + 2] << 16) |
                          (mb[4 * j + 3] << 24);
      const uint32_t r4 = rb[4 * j] | (rb[4 * j + 1] << 8) | (rb[4 * j + 2] << 16) |
                          (rb[4 * j + 3] << 24);
      if (j == 0) { L.mc.x = m4; L.rc.x = r4; }
      if (j == 1) { L.mc.y = m4; L.rc.y = r4; }
      if (j == 2) { L.mc.z = m4; L.rc.z = r4; }
      if (j == 3) { L.mc.w = m4; L.rc.w = r4; }
    }
    uint32_t pw[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) pw[j] = pb[2 * j] | (pb[2 * j + 1] << 16);
    L.p[0] = u32x4{pw[0], pw[1], pw[2], pw[3]};
    L.p[1] = u32x4{pw[4], pw[5], pw[6], pw[7]};
    L.sm = ms[b];
    L.sr = rs[b];
    const AwOut o = adam_block(L, k);
    const uint32_t po[8] = {o.p[0].x, o.p[0].y, o.p[0].z, o.p[0].w,
                            o.p[1].x, o.p[1].y, o.p[1].z, o.p[1].w};
    const uint32_t mo[4] = {o.mc.x, o.mc.y, o.mc.z, o.mc.w};
    const uint32_t ro[4] = {o.rc.x, o.rc.y, o.rc.z, o.rc.w};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (lane < 16 && e0 + i < n) {
        p[e0 + i] = static_cast<uint16_t>(i & 1 ? po[i >> 1] >> 16 : po[i >> 1] & 0xFFFFu);
        mc[e0 + i] = static_cast<uint8_t>(mo[i >> 2] >> (8 * (i & 3)));
        rc[e0 + i] = static_cast<uint8_t>(ro[i >> 2] >> (8 * (i & 3)));
      }
    }
    if (lane == 0) {
      ms[b] = o.sm;
      rs[b] = o.sr;
    }
  }
}

AdamConsts adam_consts(const qn_adamw_hparams* hp, int64_t step) {
  AdamConsts k;
  k.b1 = static_cast<float>(hp->beta1);
  k.b2 = static_cast<float>(hp->beta2);
  k.c1 = static_cast<float>(1.0 - hp->beta1);
  k.c2 = static_cast<float>(1.0 - hp->beta2);
  k.bc1 = static_cast<float>(1.0 / (1.0 - std::pow(hp->beta1, double(step))));
  k.bc2 = static_cast<float>(1.0 / (1.0 - std::pow(hp->beta2, double(step))));
  k.eps = static_cast<float>(hp->eps);
  k.lr = static_cast<float>(hp->lr);
  k.decay = static_cast<float>(1.0 - hp->lr * hp->weight_decay);
  k.gs = static_cast<float>(hp->grad_scale);
  return k;
}

bool valid_hparams(const qn_adamw_hparams* hp, int64_t step) {
  return hp != nullptr && step >= 1 && hp->beta1 >= 0.0 && hp->beta1 < 1.0 &&
         hp->beta2 >= 0.0 && hp->beta2 < 1.0 && hp->eps > 0.0 &&
         std::isfinite(hp->lr) && std::isfinite(hp->weight_decay) &&
         std::isfinite(hp->grad_scale);
}

bool valid_state(const qn_adamw8_state* st) {
  return st != nullptr && st->m_codes != nullptr && st->m_scale != nullptr &&
         st->r_codes != nullptr && st->r_scale != nullptr &&
         (reinterpret_cast<uintptr_t>(st->m_codes) & 3u) == 0 &&
         (reinterpret_cast<uintptr_t>(st->r_codes) & 3u) == 0;
}

int launch_adamw8(uint16_t* p, const float* g, int64_t n, uint8_t* mc,
                  float* ms, uint8_t* rc, float* rs, const AdamConsts& k,
                  hipStream_t st) {
  const int64_t nquad = cdiv(n / AW_BLOCK, 4);     // 4 blocks per wave step
  const int64_t grid = std::max<int64_t>(
      1, std::min<int64_t>(cdiv(nquad, AW_THREADS / 64), 8192));
  QN_LAUNCH("k_adamw8", k_adamw8, dim3((unsigned)grid), dim3(AW_THREADS), st,
            p, g, n, mc, ms, rc, rs, k);
  return check_launch();
}

// Byte layout of one staging slot for `chunk` elements.
struct Slot {
  size_t mc, ms, rc, rs, bytes;
};
Slot slot_layout(int64_t chunk) {
  const size_t nb = static_cast<size_t>(cdiv(chunk, AW_BLOCK));
  Slot s;
  s.mc = 0;
  s.rc = align256(s.mc + chunk);
  s.ms = align256(s.rc + chunk);
  s.rs = align256(s.ms + 4 * nb);
  s.bytes = align256(s.rs + 4 * nb);
  return s;
}

}  // namespace

extern "C" {

int qn_adamw8_step(uint16_t* p, const float* g, int64_t n,
                   const qn_adamw8_state* st, const qn_adamw_hparams* hp,
                   int64_t step, void* stream) {
  if (p == nullptr || g == nullptr || n <= 0 || !valid_state(st) ||
      !valid_hparams(hp, step) || !aligned16(g) ||
      (reinterpret_cast<uintptr_t>(p) & 7u) != 0)
    return QN_EINVAL;
  return launch_adamw8(p, g, n, st->m_codes, st->m_scale, st->r_codes,
                       st->r_scale, adam_consts(hp, step), (hipStream_t)stream);
}

size_t qn_adamw8_staging_bytes(int64_t chunk) {
  if (chunk < AW_BLOCK || chunk % AW_BLOCK != 0) return 0;
  return 2 * slot_layout(chunk).bytes;
}

int qn_adamw8_paged_step(uint16_t* p, const float* g, int64_t n,
                         const qn_adamw8_state* host_st, void* staging,
                         size_t staging_bytes, int64_t chunk,
                         const qn_adamw_hparams* hp, int64_t step,
                         void* stream, void* h2d_stream, void* d2h_stream) {
  if (p == nullptr || g == nullptr || n <= 0 || !valid_state(host_st) ||
      !valid_hparams(hp, step) || !aligned16(g) || staging == nullptr ||
      !aligned16(staging) || (reinterpret_cast<uintptr_t>(p) & 7u) != 0)
    return QN_EINVAL;
  const size_t need = qn_adamw8_staging_bytes(chunk);
  if (need == 0) return QN_EINVAL;
  if (staging_bytes < need) return QN_EWORKSPACE;
  const Slot L = slot_layout(chunk);
  const AdamConsts k = adam_consts(hp, step);
  hipStream_t cs = (hipStream_t)stream;
  hipStream_t hs = h2d_stream ? (hipStream_t)h2d_stream : cs;
  hipStream_t ds = d2h_stream ? (hipStream_t)d2h_stream : cs;
  const int64_t nch = cdiv(n, chunk);

  // events: per chunk H2D done, step done, D2H done; then the start (on the
  // compute stream) and the two copy streams' tails for an error exit;
  // destroyed at the end (released once they complete)
  std::vector<hipEvent_t> ev(3 * nch + 3, nullptr);
  int rc_all = QN_OK;
  auto mk = [&](hipEvent_t* e) {
    if (hipEventCreateWithFlags(e, hipEventDisableTiming) != hipSuccess)
      rc_all = QN_EHIP;
  };
  for (auto& e : ev) mk(&e);
  auto ok = [&](hipError_t r) {
    if (r != hipSuccess) rc_all = QN_EHIP;
  };
  bool queued = false;           // copies may be in flight on hs / ds
  if (rc_all == QN_OK) {
    hipEvent_t start = ev[3 * nch];
    // nothing earlier on the compute stream (a previous step's write-back
    // included) may still touch the host state when the first copy starts
    ok(hipEventRecord(start, cs));
    ok(hipStreamWaitEvent(hs, start, 0));
    ok(hipStreamWaitEvent(ds, start, 0));
    char* base = static_cast<char*>(staging);
    queued = true;
    for (int64_t i = 0; i < nch && rc_all == QN_OK; ++i) {
      const int64_t e0 = i * chunk;
      const int64_t len = std::min<int64_t>(chunk, n - e0);
      const int64_t b0 = e0 / AW_BLOCK;
      const size_t nbl = static_cast<size_t>(cdiv(len, AW_BLOCK));
      char* s = base + (i & 1) * L.bytes;
      hipEvent_t eh = ev[3 * i], ek = ev[3 * i + 1], ed = ev[3 * i + 2];
      if (i >= 2) ok(hipStreamWaitEvent(hs, ev[3 * (i - 2) + 2], 0));
      ok(hipMemcpyAsync(s + L.mc, host_st->m_codes + e0, len, hipMemcpyHostToDevice, hs));
      ok(hipMemcpyAsync(s + L.rc, host_st->r_codes + e0, len, hipMemcpyHostToDevice, hs));
      ok(hipMemcpyAsync(s + L.ms, host_st->m_scale + b0, 4 * nbl, hipMemcpyHostToDevice, hs));
      ok(hipMemcpyAsync(s + L.rs, host_st->r_scale + b0, 4 * nbl, hipMemcpyHostToDevice, hs));
      ok(hipEventRecord(eh, hs));
      ok(hipStreamWaitEvent(cs, eh, 0));
      if (rc_all != QN_OK) break;
      const int r = launch_adamw8(p + e0, g + e0, len,
                                  reinterpret_cast<uint8_t*>(s + L.mc),
                                  reinterpret_cast<float*>(s + L.ms),
                                  reinterpret_cast<uint8_t*>(s + L.rc),
                                  reinterpret_cast<float*>(s + L.rs), k, cs);
      if (r != QN_OK) rc_all = r;
      ok(hipEventRecord(ek, cs));
      ok(hipStreamWaitEvent(ds, ek, 0));
      ok(hipMemcpyAsync(host_st->m_codes + e0, s + L.mc, len, hipMemcpyDeviceToHost, ds));
      ok(hipMemcpyAsync(host_st->r_codes + e0, s + L.rc, len, hipMemcpyDeviceToHost, ds));
      ok(hipMemcpyAsync(host_st->m_scale + b0, s + L.ms, 4 * nbl, hipMemcpyDeviceToHost, ds));
      ok(hipMemcpyAsync(host_st->r_scale + b0, s + L.rs, 4 * nbl, hipMemcpyDeviceToHost, ds));
      ok(hipEventRecord(ed, ds));
    }
    // the compute stream reaches the end of the call only after the last
    // write-back (the copy streams run in order)
    if (rc_all == QN_OK) ok(hipStreamWaitEvent(cs, ev[3 * (nch - 1) + 2], 0));
  }
  if (rc_all != QN_OK && queued) {
    // An error after copies were queued: the compute stream still waits for
    // everything queued on the copy streams, so the host state and the
    // staging area are not in use once the stream reaches this point; if
    // that cannot be arranged, the copy streams are drained before return.
    hipEvent_t th = ev[3 * nch + 1], td = ev[3 * nch + 2];
    const bool waited =
        th != nullptr && td != nullptr && hipEventRecord(th, hs) == hipSuccess &&
        hipEventRecord(td, ds) == hipSuccess &&
        hipStreamWaitEvent(cs, th, 0) == hipSuccess &&
        hipStreamWaitEvent(cs, td, 0) == hipSuccess;
    if (!waited) {
      (void)hipStreamSynchronize(hs);
      (void)hipStreamSynchronize(ds);
    }
  }
  for (auto& e : ev)
    if (e != nullptr) hipEventDestroy(e);
  return rc_all;
}

}  // extern "C"
