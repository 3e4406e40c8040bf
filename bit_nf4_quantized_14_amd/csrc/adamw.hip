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
constexpr int AW_THREADS = 256;              // 4 waves, one block per wave
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

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

// Operands of one lane for one block: 4 gradients, 4 bf16 parameters, 4
// codes of each moment, the block's two scales.
struct AwLoads {
  float g[4];
  uint32_t p01, p23, mc, rc;
  float sm, sr;
};

// One block's step for one lane; `n_here` elements of the lane's four are
// real (4 for whole blocks).  Returns the outputs packed for storing.
struct AwOut {
  uint32_t p01, p23, mc, rc;
  float sm, sr;
};

__device__ __forceinline__ AwOut adam_block(const AwLoads& L,
                                            const AdamConsts& k) {
  const float pv[4] = {bf16_to_f32(L.p01 & 0xFFFFu), bf16_to_f32(L.p01 >> 16),
                       bf16_to_f32(L.p23 & 0xFFFFu), bf16_to_f32(L.p23 >> 16)};
  const float mo[4] = {e4m3_value<0>(L.mc) * L.sm, e4m3_value<1>(L.mc) * L.sm,
                       e4m3_value<2>(L.mc) * L.sm, e4m3_value<3>(L.mc) * L.sm};
  const float ro[4] = {e4m3_value<0>(L.rc) * L.sr, e4m3_value<1>(L.rc) * L.sr,
                       e4m3_value<2>(L.rc) * L.sr, e4m3_value<3>(L.rc) * L.sr};
  Elem el[4];
  float am = 0.0f, ar = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    el[i] = adam_elem(L.g[i], mo[i], ro[i], pv[i], k);
    el[i].v = sqrtf(el[i].v);      // r = sqrt(v), the stored quantity
    am = fmaxf(am, fabsf(el[i].m));
    ar = fmaxf(ar, el[i].v);
  }
  am = wave_max(am);
  ar = wave_max(ar);
  const float sm = am / AW_E4M3_MAX;
  const float sr = ar / AW_E4M3_MAX;
  AwOut o;
  o.mc = am == 0.0f ? 0u
                    : e4m3_encode4(el[0].m / sm, el[1].m / sm, el[2].m / sm,
                                   el[3].m / sm);
  o.rc = ar == 0.0f ? 0u
                    : e4m3_encode4(el[0].v / sr, el[1].v / sr, el[2].v / sr,
                                   el[3].v / sr);
  o.p01 = pack_bf16x2(el[0].p, el[1].p);
  o.p23 = pack_bf16x2(el[2].p, el[3].p);
  o.sm = am == 0.0f ? 0.0f : sm;
  o.sr = ar == 0.0f ? 0.0f : sr;
  return o;
}

// A wave owns one 256-element block per iteration (lane l: elements
// 4l .. 4l+3) and issues the loads of its next block before stepping the
// current one.  The whole blocks run in the loop; a short last block is
// done afterwards by one wave with per-element guards (its missing
// elements count as zero for the block maxima and are not stored).
__global__ __launch_bounds__(AW_THREADS) void k_adamw8(
    uint16_t* __restrict__ p, const float* __restrict__ g, int64_t n,
    uint8_t* __restrict__ mc, float* __restrict__ ms,
    uint8_t* __restrict__ rc, float* __restrict__ rs, AdamConsts k) {
  const int lane = threadIdx.x & 63;
  const int64_t nwhole = n / AW_BLOCK;
  const int64_t wave0 = ((int64_t)blockIdx.x * AW_THREADS + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * AW_THREADS) >> 6;
  auto load = [&](AwLoads& L, int64_t b) {
    const int64_t bb = b < nwhole ? b : 0;     // keep loads in range
    const int64_t e0 = bb * AW_BLOCK + 4 * lane;
    const f32x4 g4 = *reinterpret_cast<const f32x4*>(g + e0);
    const uint2 p4 = *reinterpret_cast<const uint2*>(p + e0);
    L.g[0] = g4.x; L.g[1] = g4.y; L.g[2] = g4.z; L.g[3] = g4.w;
    L.p01 = p4.x;
    L.p23 = p4.y;
    L.mc = *reinterpret_cast<const uint32_t*>(mc + e0);
    L.rc = *reinterpret_cast<const uint32_t*>(rc + e0);
    L.sm = ms[bb];
    L.sr = rs[bb];
  };
  if (nwhole > 0) {
    AwLoads cur;
    int64_t b = wave0;
    if (b < nwhole) load(cur, b);
    for (; b < nwhole; b += nwaves) {
      AwLoads nxt;
      if (b + nwaves < nwhole) load(nxt, b + nwaves);
      const AwOut o = adam_block(cur, k);
      const int64_t e0 = b * AW_BLOCK + 4 * lane;
      *reinterpret_cast<uint2*>(p + e0) = make_uint2(o.p01, o.p23);
      *reinterpret_cast<uint32_t*>(mc + e0) = o.mc;
      *reinterpret_cast<uint32_t*>(rc + e0) = o.rc;
      if (lane == 0) {
        ms[b] = o.sm;
        rs[b] = o.sr;
      }
      cur = nxt;
    }
  }
  if (n % AW_BLOCK != 0 && wave0 == 0) {
    const int64_t b = nwhole;
    const int64_t e0 = b * AW_BLOCK + 4 * lane;
    AwLoads L;
    L.mc = L.rc = 0;
    uint32_t pb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool in = e0 + i < n;
      L.g[i] = in ? g[e0 + i] : 0.0f;
      pb[i] = in ? static_cast<uint32_t>(p[e0 + i]) : 0u;
      L.mc |= (in ? static_cast<uint32_t>(mc[e0 + i]) : 0u) << (8 * i);
      L.rc |= (in ? static_cast<uint32_t>(rc[e0 + i]) : 0u) << (8 * i);
    }
    L.p01 = pb[0] | (pb[1] << 16);
    L.p23 = pb[2] | (pb[3] << 16);
    L.sm = ms[b];
    L.sr = rs[b];
    const AwOut o = adam_block(L, k);
    const uint32_t po[4] = {o.p01 & 0xFFFFu, o.p01 >> 16, o.p23 & 0xFFFFu,
                            o.p23 >> 16};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (e0 + i < n) {
        p[e0 + i] = static_cast<uint16_t>(po[i]);
        mc[e0 + i] = static_cast<uint8_t>(o.mc >> (8 * i));
        rc[e0 + i] = static_cast<uint8_t>(o.rc >> (8 * i));
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
  const int64_t nb = cdiv(n, AW_BLOCK);
  const int64_t grid = std::min<int64_t>(cdiv(nb, AW_THREADS / 64), 8192);
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

  // events: start (on the compute stream), and per chunk H2D done, step
  // done, D2H done; destroyed at the end (released once they complete)
  std::vector<hipEvent_t> ev(3 * nch + 1, nullptr);
  int rc_all = QN_OK;
  auto mk = [&](hipEvent_t* e) {
    if (hipEventCreateWithFlags(e, hipEventDisableTiming) != hipSuccess)
      rc_all = QN_EHIP;
  };
  for (auto& e : ev) mk(&e);
  auto ok = [&](hipError_t r) {
    if (r != hipSuccess) rc_all = QN_EHIP;
  };
  if (rc_all == QN_OK) {
    hipEvent_t start = ev[3 * nch];
    // nothing earlier on the compute stream (a previous step's write-back
    // included) may still touch the host state when the first copy starts
    ok(hipEventRecord(start, cs));
    ok(hipStreamWaitEvent(hs, start, 0));
    ok(hipStreamWaitEvent(ds, start, 0));
    char* base = static_cast<char*>(staging);
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
  for (auto& e : ev)
    if (e != nullptr) hipEventDestroy(e);
  return rc_all;
}

}  // extern "C"
