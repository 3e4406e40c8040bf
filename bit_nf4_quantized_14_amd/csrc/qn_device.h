// Device-side pieces shared by the kernels of the QLoRA NF4 library: vector
// types, the codebook kernel argument, bf16 helpers, the per-block bf16
// lookup table and nibble decoders, MFMA wrappers and buffer resources.
// Every function is inline; each translation unit keeps its kernels in an
// anonymous namespace.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace qn {

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

// The same table built by two adjacent lanes (2i, 2i+1) that decode the same
// block: each lane forms the products of one half of the levels (entries
// 0-7 on the even lane, 8-15 on the odd one) and takes the other half from
// its neighbour with a DPP swap, so each lane does half the multiplies,
// conversions and byte splits.  The odd lane ends up with the two halves in
// swapped slots; it decodes codes whose bit 3 is flipped (`flip`, XORed
// into each packed dword), which selects the right slot.  The entries are
// the same fp32 products as make_lut's, so the decoded weights are
// bit-identical.
struct LutHalf {
  float L[8];      // levels 8 (lane & 1) .. + 7
  uint32_t flip;   // 0 on the even lane, 0x88888888 on the odd lane
};

__device__ __forceinline__ LutHalf lut_half(const Codebook& cb, int lane) {
  LutHalf h;
  const bool odd = (lane & 1) != 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) h.L[i] = odd ? cb.L[8 + i] : cb.L[i];
  h.flip = odd ? 0x88888888u : 0u;
  return h;
}

// v_mov_b32 with DPP quad_perm [1, 0, 3, 2]: the value of the other lane of
// the pair.
__device__ __forceinline__ uint32_t pair_swap(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}

__device__ __forceinline__ Lut make_lut_pair(const LutHalf& h, float cp) {
  uint32_t P[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    P[k] = pack_bf16x2(h.L[2 * k] * cp, h.L[2 * k + 1] * cp);
  // low and high bytes of this lane's entries 0-3 and 4-7 of its half
  const uint32_t l0 = perm(P[1], P[0], 0x06040200u);
  const uint32_t h0 = perm(P[1], P[0], 0x07050301u);
  const uint32_t l1 = perm(P[3], P[2], 0x06040200u);
  const uint32_t h1 = perm(P[3], P[2], 0x07050301u);
  Lut t;
  t.ll0 = l0;
  t.hl0 = h0;
  t.ll1 = l1;
  t.hl1 = h1;
  t.lh0 = pair_swap(l0);
  t.hh0 = pair_swap(h0);
  t.lh1 = pair_swap(l1);
  t.hh1 = pair_swap(h1);
  return t;
}

// The same table built by lanes l and l + 32 of a wave that decode the same
// block: the lower lane forms the byte planes of entries 0-7, the upper
// lane those of entries 8-15, and v_permlane32_swap of each plane with
// itself hands every lane both (its first result is the lower lane's value,
// its second the upper lane's), so no lane needs a flip.
__device__ __forceinline__ LutHalf lut_half32(const Codebook& cb, int lane) {
  LutHalf h;
  const bool up = lane >= 32;
#pragma unroll
  for (int i = 0; i < 8; ++i) h.L[i] = up ? cb.L[8 + i] : cb.L[i];
  h.flip = 0u;
  return h;
}

__device__ __forceinline__ Lut make_lut_swap32(const LutHalf& h, float cp) {
  uint32_t P[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    P[k] = pack_bf16x2(h.L[2 * k] * cp, h.L[2 * k + 1] * cp);
  const uint32_t l0 = perm(P[1], P[0], 0x06040200u);
  const uint32_t h0 = perm(P[1], P[0], 0x07050301u);
  const uint32_t l1 = perm(P[3], P[2], 0x06040200u);
  const uint32_t h1 = perm(P[3], P[2], 0x07050301u);
  const auto s0 = __builtin_amdgcn_permlane32_swap(l0, l0, false, false);
  const auto s1 = __builtin_amdgcn_permlane32_swap(h0, h0, false, false);
  const auto s2 = __builtin_amdgcn_permlane32_swap(l1, l1, false, false);
  const auto s3 = __builtin_amdgcn_permlane32_swap(h1, h1, false, false);
  Lut t;
  t.ll0 = s0[0];
  t.lh0 = s0[1];
  t.hl0 = s1[0];
  t.hh0 = s1[1];
  t.ll1 = s2[0];
  t.lh1 = s2[1];
  t.hl1 = s3[0];
  t.hh1 = s3[1];
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
// LoRA dropout mask (inverted dropout on the adapter branch input).
// Element (m, k) of X is kept when word m % 4 of Philox4x32-10 at counter
// (k, m / 4, 0, 0) under key (key0, key1) is >= thresh; a kept element
// becomes bf16_rne(fp32(x) * scale), a dropped one 0.
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC 2011): ten rounds of two
// 32x32 -> 64-bit products of words 0 and 2 with M0, M1, the output
// (hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0), and the key advanced by
// (W0, W1) after each round.
// ---------------------------------------------------------------------------
struct DropArgs {
  uint32_t key0, key1;
  uint32_t thresh;
  float scale;
};

__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1,
                                               uint32_t k0, uint32_t k1) {
  constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  constexpr uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
  uint32_t x0 = c0, x1 = c1, x2 = 0, x3 = 0;
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    // one 32 x 32 -> 64-bit product each (v_mad_u64_u32), rather than
    // separate high and low multiplies
    const uint64_t p0 = static_cast<uint64_t>(M0) * x0;
    const uint64_t p1 = static_cast<uint64_t>(M1) * x2;
    const uint32_t hi0 = static_cast<uint32_t>(p0 >> 32), lo0 = static_cast<uint32_t>(p0);
    const uint32_t hi1 = static_cast<uint32_t>(p1 >> 32), lo1 = static_cast<uint32_t>(p1);
    x0 = hi1 ^ x1 ^ k0;
    x1 = lo1;
    x2 = hi0 ^ x3 ^ k1;
    x3 = lo0;
    k0 += W0;
    k1 += W1;
  }
  u32x4 r;
  r.x = x0;
  r.y = x1;
  r.z = x2;
  r.w = x3;
  return r;
}

// The value of lane (lane ^ dd) of this lane's quad, dd = 1..3: a DPP
// quad_perm move, no LDS round trip.
__device__ __forceinline__ uint32_t quad_xor(uint32_t v, int dd) {
  return static_cast<uint32_t>(
      dd == 1 ? __builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1, 0xF, 0xF, false)
      : dd == 2 ? __builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x4E, 0xF, 0xF, false)
                : __builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x1B, 0xF, 0xF, false));
}

__device__ __forceinline__ uint32_t pick4(const u32x4& w, int sel) {
  const uint32_t a = w.x, b = w.y, c = w.z, d = w.w;
  return sel == 0 ? a : (sel == 1 ? b : (sel == 2 ? c : d));
}

// One bf16 element (low 16 bits of x16) after dropout with Philox word w.
__device__ __forceinline__ uint32_t drop_bf16(uint32_t x16, uint32_t w,
                                              const DropArgs& d) {
  return w >= d.thresh
             ? (pack_bf16x2(bf16_to_f32(x16 & 0xFFFFu) * d.scale, 0.0f) & 0xFFFFu)
             : 0u;
}

// 8 consecutive columns k0 .. k0 + 7 of row m (natural order, two per
// dword), where the four lanes of this lane's quad hold rows
// m - m % 4 .. + 3 of the same columns (m % 4 == lane % 4).  The quad
// shares the 8 generator calls: lane j = m % 4 computes columns
// k0 + 2j + t (t = 0, 1), and source lane s sends word s ^ dd of each to
// lane s ^ dd, so lane j receives word j of column 2 (j ^ dd) + t.
__device__ __forceinline__ u32x4 drop_row8(const u32x4& a, int m, int k0,
                                           const DropArgs& d) {
  const uint32_t q = static_cast<uint32_t>(m) >> 2;
  const int j = m & 3;
  const u32x4 p0 = philox4x32_10(k0 + 2 * j, q, d.key0, d.key1);
  const u32x4 p1 = philox4x32_10(k0 + 2 * j + 1, q, d.key0, d.key1);
  uint32_t recv0[4], recv1[4];   // [dd]: word j of columns 2 (j ^ dd) + 0 / 1
#pragma unroll
  for (int dd = 0; dd < 4; ++dd) {
    const uint32_t s0 = pick4(p0, j ^ dd), s1 = pick4(p1, j ^ dd);
    recv0[dd] = dd == 0 ? s0 : quad_xor(s0, dd);
    recv1[dd] = dd == 0 ? s1 : quad_xor(s1, dd);
  }
  u32x4 v0, v1;
  v0.x = recv0[0]; v0.y = recv0[1]; v0.z = recv0[2]; v0.w = recv0[3];
  v1.x = recv1[0]; v1.y = recv1[1]; v1.z = recv1[2]; v1.w = recv1[3];
  const uint32_t in[4] = {a.x, a.y, a.z, a.w};
  uint32_t out[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    // columns 2h and 2h + 1 arrived with dd = h ^ j
    const uint32_t wl = pick4(v0, h ^ j), wh = pick4(v1, h ^ j);
    out[h] = drop_bf16(in[h], wl, d) | (drop_bf16(in[h] >> 16, wh, d) << 16);
  }
  u32x4 r;
  r.x = out[0];
  r.y = out[1];
  r.z = out[2];
  r.w = out[3];
  return r;
}

// 8 consecutive rows m0 .. m0 + 7 (m0 % 4 == 0) of column k (natural
// order, two per dword): two generator calls.
__device__ __forceinline__ u32x4 drop_col8(const u32x4& a, int m0, int k,
                                           const DropArgs& d) {
  const uint32_t q = static_cast<uint32_t>(m0) >> 2;
  const u32x4 w0 = philox4x32_10(k, q, d.key0, d.key1);
  const u32x4 w1 = philox4x32_10(k, q + 1, d.key0, d.key1);
  u32x4 r;
  r.x = drop_bf16(a.x, w0.x, d) | (drop_bf16(a.x >> 16, w0.y, d) << 16);
  r.y = drop_bf16(a.y, w0.z, d) | (drop_bf16(a.y >> 16, w0.w, d) << 16);
  r.z = drop_bf16(a.z, w1.x, d) | (drop_bf16(a.z >> 16, w1.y, d) << 16);
  r.w = drop_bf16(a.w, w1.z, d) | (drop_bf16(a.w >> 16, w1.w, d) << 16);
  return r;
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
// Buffer resources: global loads and stores go through a resource whose
// range check returns zeros (drops stores) past the end, which covers ragged
// tiles without branches.
// ---------------------------------------------------------------------------
constexpr uint32_t G_OOB = 0x80000000u;   // buffer offset past every range
constexpr int G_RSRC_FLAGS = 0x00020000;

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)bytes, G_RSRC_FLAGS);
}

}  // namespace qn
