// Fused dequant + MFMA GEMM of the QLoRA NF4 library (the forward and
// backward base products).  "QLoRA Guide" (Forward pass diagram: dequantize
// W to bf16, multiply, add the adapter path) and the "QLORA ... paper
// summary" (Notes: dequantize to BF16, then matmul; gradients for the
// adapters only, through the dequantized weight for dX).
#include "qn_host.h"

namespace {

using namespace qn;

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
//    thread per chunk) and written to LDS behind the last slice's MFMAs:
//    128-byte rows with the 16-byte chunk index XOR-swizzled by (row / 2) & 7, so the
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
// woven between the MFMAs in fenced groups (one MFMA, the next slice's
// fragment read, then up to four VALU ops).  Global loads go through buffer resources whose range check returns
// zeros, which covers ragged M, N and K tiles without branches.
// The adapter term is 2r extra reduction steps with the A side s*T (or s*G)
// split into bf16 hi + lo parts, so the fp32 intermediate keeps ~16
// mantissa bits.
// ---------------------------------------------------------------------------

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

// Eight weights as stored in the LDS tile.  Forward rows run along the
// reduction, so the order must match the A operand: natural order.  The
// backward tile's rows run along the output columns, so its 16-byte chunks
// hold their eight columns in decode8p order (0 2 4 6 1 3 5 7), four
// v_perm_b32 cheaper; gemm_col maps an MFMA output column back.
template <bool BWD>
__device__ __forceinline__ u32x4 gemm_decode(uint32_t p, const Lut& t) {
  return BWD ? decode8p(p, t) : decode8(p, t);
}

// Output column of accumulator column (lane % 32) of MFMA tile j.  In the
// backward, position q of each group of eight holds column
// 2 (q % 4) + q / 4.
template <int BM, int BN, bool BWD>
__device__ __forceinline__ int gemm_col(int c0, int wn, int j, int lane) {
  const int q = lane & 31;
  const int base = c0 + wn * GemmCfg<BM, BN, BWD>::WN + j * 32;
  return BWD ? base + (q & ~7) + ((q & 3) << 1) + ((q >> 2) & 1) : base + q;
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
                                               const LutHalf& lh, int tid) {
  const WDst dst = gemm_wdst<BM, BN, BWD>(sW, tid);
  const Lut t = make_lut_pair(lh, static_cast<float>(R.q) * R.d);
  const uint32_t wd[4] = {R.w.x ^ lh.flip, R.w.y ^ lh.flip, R.w.z ^ lh.flip,
                          R.w.w ^ lh.flip};
#pragma unroll
  for (int d = 0; d < 4; ++d)
    *reinterpret_cast<u32x4*>(dst.base + 8 * (d ^ dst.x)) = gemm_decode<BWD>(wd[d], t);
}

// A tile of one step: 16-byte global loads into registers (thread t takes
// chunks q = t + NT i; chunk q is row q / 8, 16-byte column q % 8, so eight
// consecutive lanes read one 128-byte row segment), written to LDS behind
// the MFMAs of the step's last slice at the row's swizzled slot
// (q % 8) ^ ((row / 2) & 7).
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

// Global loads of one reduction step, for a thread of a tile.
//
// Fast addressing (CHK = false): every bound a load depends on is either a
// per-thread constant (rows of A past M, weight rows or columns past the
// tile's edge) or the same for the whole workgroup (steps past the end of
// the reduction), because the reduction length is a multiple of the 64-wide
// step.  Each thread's offsets of step 0 are formed once, with G_OOB baked
// in where its element lies outside the operand; a step adds its advance as
// the scalar offset, and a step past the end loads through a zero-sized
// range.  The only per-step vector work is the group-scale offset, whose
// 16384-weight groups do not follow the 64-wide steps.  The scalar offset
// is outside the range check, so it is only ever added to offsets that
// stay inside the operand.
// Checked addressing (CHK = true, the backward when N % 64 != 0, whose last
// step is partial): every offset and bound is formed per step.
template <int BM, int BN, bool BWD, bool CHK>
struct GemmLoader {
  using C = GemmCfg<BM, BN, BWD>;
  const uint16_t* Aop;
  const uint8_t* packed;
  const uint8_t* qabs;
  const float* gscale;
  uint32_t a_bytes, p_bytes, q_bytes, d_bytes;
  int M, N, K, KRED, m0, c0, tid;
  uint32_t a_vo[C::A_CHUNKS];   // A chunk offsets at step 0 (fast)
  uint32_t w_vo, q_vo, e0;      // packed / code offsets and element index
                                // at step 0 (fast)

  __device__ __forceinline__ void init() {
    if constexpr (!CHK) {
#pragma unroll
      for (int i = 0; i < C::A_CHUNKS; ++i) {
        const int q = tid + C::NT * i, row = q >> 3;
        a_vo[i] = m0 + row < M
                      ? (uint32_t)(((int64_t)(m0 + row) * KRED + 8 * (q & 7)) * 2)
                      : G_OOB;
      }
      int n, k;
      if (!BWD) {
        n = c0 + tid / C::TPR;
        k = (tid % C::TPR) * C::EPT;
      } else {
        n = tid / C::TPR;
        k = c0 + (tid % C::TPR) * C::EPT;
      }
      const bool ok = BWD ? k < K : n < N;
      e0 = (uint32_t)((int64_t)n * K + k);
      w_vo = ok ? e0 >> 1 : G_OOB;
      q_vo = ok ? e0 >> 6 : G_OOB;
    }
  }

  __device__ __forceinline__ void load_a(ARegs<BM, BN, BWD>& R, int red0) const {
    if constexpr (CHK) {
      gemm_load_a<BM, BN, BWD>(R, make_rsrc(Aop, a_bytes), M, KRED, m0, red0, tid);
    } else {
      const rsrc_t ra = make_rsrc(Aop, red0 < KRED ? a_bytes : 0u);
#pragma unroll
      for (int i = 0; i < C::A_CHUNKS; ++i)
        R.v[i] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, a_vo[i], red0 * 2, 0));
    }
  }

  __device__ __forceinline__ void load_w(WRegs& R, int red0) const {
    if constexpr (CHK) {
      gemm_load_w<BM, BN, BWD>(R, make_rsrc(packed, p_bytes),
                               make_rsrc(qabs, q_bytes), make_rsrc(gscale, d_bytes),
                               N, K, c0, red0, tid);
    } else {
      const bool live = red0 < KRED;
      const rsrc_t rp = make_rsrc(packed, live ? p_bytes : 0u);
      const rsrc_t rq = make_rsrc(qabs, live ? q_bytes : 0u);
      const rsrc_t rd = make_rsrc(gscale, live ? d_bytes : 0u);
      // element advance of the step: along the row (forward) or red0 rows
      // down (backward)
      const uint32_t adv = BWD ? (uint32_t)red0 * (uint32_t)K : (uint32_t)red0;
      R.w = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, w_vo, (int)(adv >> 1), 0));
      R.q = __builtin_amdgcn_raw_buffer_load_b8(rq, q_vo, (int)(adv >> 6), 0);
      R.d = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                          rd, ((e0 + adv) >> 14) << 2, 0, 0));
    }
  }
};

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
constexpr int G_VALU_PER_MFMA = 4;

// The four k16 slices of one step with the dequantization of the next weight
// tile woven in: one decode8 (28 VALU ops and a 16-byte LDS write) after
// every MPD MFMAs, each group fenced and ordered MFMA / VALU so the VALU
// work issues in the shadow of the MFMAs instead of after them.  The next
// slice's fragment reads are pinned one behind each of the first MFMAs, so
// they issue early instead of just before the MFMAs that consume them
// (forward -1.5% per launch; the register allocator otherwise sinks them
// to reuse the current fragments' registers), and the next step's A tile
// (loaded at the start of the step) is written to LDS behind the MFMAs of
// the last slice instead of after them (forward -3%, backward -2%).
template <int BM, int BN, bool BWD>
__device__ __forceinline__ void gemm_mma_deq(
    const char* sA, const uint16_t* sW, uint16_t* sWn, const WRegs& R,
    const ARegs<BM, BN, BWD>& An, char* sAn,
    const LutHalf& lh, int wm, int wn, int tid, int lane,
    f32x16 (&acc)[GemmCfg<BM, BN, BWD>::TM][GemmCfg<BM, BN, BWD>::TN]) {
  using C = GemmCfg<BM, BN, BWD>;
  constexpr int MPK = C::TM * C::TN;     // MFMAs per k16 slice
  constexpr int DPK = C::WDW / 4;        // decode8 per k16 slice
  constexpr int MPD = MPK / DPK;         // MFMAs per decode8
  static_assert(C::WDW % 4 == 0 && MPK % DPK == 0, "decode split");
  const WDst dst = gemm_wdst<BM, BN, BWD>(sWn, tid);
  const Lut t = make_lut_pair(lh, static_cast<float>(R.q) * R.d);
  const uint32_t wd[4] = {R.w.x ^ lh.flip, R.w.y ^ lh.flip, R.w.z ^ lh.flip,
                          R.w.w ^ lh.flip};
  u32x4 a[2][C::TM], b[2][C::TN];
  gemm_frags<BM, BN, BWD>(sA, sW, wm, wn, lane, 0, a[0], b[0]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    if (kk < 3)
      gemm_frags<BM, BN, BWD>(sA, sW, wm, wn, lane, kk + 1, a[(kk + 1) & 1],
                              b[(kk + 1) & 1]);
    if (kk == 3) gemm_store_a<BM, BN, BWD>(An, sAn, tid);
#pragma unroll
    for (int g = 0; g < MPK; ++g) {
      const int i = g / C::TN, j = g % C::TN;
      acc[i][j] = mfma32(a[kk & 1][i], b[kk & 1][j], acc[i][j]);
      if (g % MPD == MPD - 1) {
        const int d = kk * DPK + g / MPD;
        *reinterpret_cast<u32x4*>(dst.base + 8 * (d ^ dst.x)) = gemm_decode<BWD>(wd[d], t);
#pragma unroll
        for (int h = 0; h < MPD; ++h) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
          if (kk < 3 && h < (BWD ? C::TM + 2 * C::TN : C::TM + C::TN))
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); // DS read
          if (kk == 3 && h < C::A_CHUNKS)
            __builtin_amdgcn_sched_group_barrier(0x200, 1, 0); // DS write
          __builtin_amdgcn_sched_group_barrier(0x002, G_VALU_PER_MFMA, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

// Output tile of tile index i in grouped order: groups of G_GROUP_M tile
// rows, walked column by column inside a group, so that any 32 consecutive
// indices cover 4 tile rows x 8 tile columns.  A bijection of
// [0, tiles_m * tiles_n).
constexpr int G_GROUP_M = 4;

__device__ __forceinline__ void gemm_tile_at(int i, int tiles_m, int tiles_n,
                                             int& tm, int& tn) {
  const int group = i / (G_GROUP_M * tiles_n);
  const int first = group * G_GROUP_M;
  const int rows = min(G_GROUP_M, tiles_m - first);
  const int in = i - group * G_GROUP_M * tiles_n;
  tm = first + in % rows;
  tn = in / rows;
}

// The hardware deals workgroups round-robin over the 8 XCDs; workgroup pid
// of the first `nwhole` takes tile index (pid % 8) * (nwhole / 8) + pid / 8,
// so each XCD works through a contiguous run of indices: at any moment its
// 32 CUs hold a 4 x 8 block of tiles, whose A row tiles and weight column
// tiles its L2 shares.
__device__ __forceinline__ int gemm_xcd_index(int pid, int nwhole) {
  return (nwhole & 7) == 0 ? (pid & 7) * (nwhole >> 3) + (pid >> 3) : pid;
}

// Kernel-side view of a GemmSplit: workgroups [0, whole) take whole tiles;
// workgroup whole + i rem + t is piece i (0 or 1) of split tile t, over
// reduction steps [0, h) or [h, nsteps), h = nsteps / 2 rounded down to
// even (the pieces of a tile lie on one XCD when rem is a multiple of 8).
struct SplitArgs {
  int whole, rem;
  float* part;       // [rem][TM TN 4][NT] float4: one partial tile each
  uint32_t* cnt;     // [rem][2]: arrivals, partial-ready flag
  int32_t* status;   // QN_ESYNC when a partial never became ready
};

// Exchange of a split tile's partial (AMDGPU memory model, agent scope, so
// the two pieces may run on different XCDs): the piece that arrives first
// stores its partial with ordinary stores, meets its workgroup barrier and
// sets the ready flag with a release store (L2 write-back before the flag);
// the second piece polls the flag with relaxed loads, then an acquire fence
// (L2 and L1 invalidate) orders its ordinary loads of the partial after it.
// The poll is bounded: if the flag never rises the tile is written as NaN
// and the status word reports QN_ESYNC instead of adding an unready partial.
constexpr int G_SPLIT_SPIN = 1 << 22;    // polls of ~2 x 64 cycles each

template <int BM, int BN, bool BWD>
__device__ __forceinline__ void gemm_put_partial(
    rsrc_t rp, int tid,
    const f32x16 (&acc)[GemmCfg<BM, BN, BWD>::TM][GemmCfg<BM, BN, BWD>::TN]) {
  using C = GemmCfg<BM, BN, BWD>;
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int u = (i * C::TN + j) * 4 + q;
        const f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1],
                         acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rp,
                                               (uint32_t)((u * C::NT + tid) * 16), 0,
                                               0);
      }
}

template <int BM, int BN, bool BWD>
__device__ __forceinline__ void gemm_add_partial(
    rsrc_t rp, int tid,
    f32x16 (&acc)[GemmCfg<BM, BN, BWD>::TM][GemmCfg<BM, BN, BWD>::TN]) {
  using C = GemmCfg<BM, BN, BWD>;
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int u = (i * C::TN + j) * 4 + q;
        const f32x4 v = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                       rp, (uint32_t)((u * C::NT + tid) * 16), 0, 0));
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][4 * q + e] += v[e];
        if (q == 3) {
          // the sums are formed here, one accumulator tile at a time, not
          // sunk into the epilogue's conditional stores (where the loaded
          // values would stay live and spill)
          asm volatile("" : "+v"(acc[i][j]));
          __builtin_amdgcn_sched_barrier(0);
        }
      }
}

// One reduction step: MFMAs on (sAc, sWc) while the next A tile streams into
// sAn and the weight tile held in Wc is dequantized into sWn.
template <int BM, int BN, bool BWD, bool CHK>
__device__ __forceinline__ void gemm_step(
    int st, char* sAc, uint16_t* sWc, char* sAn, uint16_t* sWn, WRegs& Wc,
    const GemmLoader<BM, BN, BWD, CHK>& ld, int wm, int wn, int tid, int lane,
    const LutHalf& lh,
    f32x16 (&acc)[GemmCfg<BM, BN, BWD>::TM][GemmCfg<BM, BN, BWD>::TN]) {
  WRegs Wn;
  ARegs<BM, BN, BWD> An;
  ld.load_a(An, (st + 1) * G_BK);
  ld.load_w(Wn, (st + 2) * G_BK);
  gemm_mma_deq<BM, BN, BWD>(sAc, sWc, sWn, Wc, An, sAn, lh, wm, wn, tid, lane, acc);
  __builtin_amdgcn_s_waitcnt(0);   // all counters: loads and LDS writes done
  __syncthreads();
  Wc = Wn;
}

// Adapter term, 2 * rpad more reduction steps straight from global memory
// (small, L2-resident arrays): A side the bf16 hi and lo parts of s*T
// (forward) or s*G (backward), [M][rpad]; B side [NOUT][rpad], B (forward)
// or A^T (backward), zero-padded to rpad columns.
template <int BM, int BN, bool BWD>
__device__ __forceinline__ void gemm_adapter(
    const uint16_t* La_hi, const uint16_t* La_lo, const uint16_t* Lb, int M,
    int NOUT, int rpad, int m0, int c0, int wm, int wn, int lane,
    f32x16 (&acc)[GemmCfg<BM, BN, BWD>::TM][GemmCfg<BM, BN, BWD>::TN]) {
  using C = GemmCfg<BM, BN, BWD>;
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
          (uint32_t)(((int64_t)gemm_col<BM, BN, BWD>(c0, wn, j, lane) * rpad + jc) * 2);
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

// LoRA dropout on the adapter term of dX: accumulator element (row, col)
// times mask(row, col) / (1 - p).  Accumulator v of lane l holds row
// 8 (v / 4) + 4 (l / 32) + v % 4 of its 32 x 32 tile, so each group of four
// (rows r0 .. r0 + 3, r0 % 4 == 0, one column) is one generator call.
template <int BM, int BN, bool BWD>
__device__ __forceinline__ void gemm_drop_acc(
    int m0, int c0, int wm, int wn, int lane, const DropArgs& dp,
    f32x16 (&acc)[GemmCfg<BM, BN, BWD>::TM][GemmCfg<BM, BN, BWD>::TN]) {
  using C = GemmCfg<BM, BN, BWD>;
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
      const int col = gemm_col<BM, BN, BWD>(c0, wn, j, lane);
#pragma unroll
      for (int vg = 0; vg < 4; ++vg) {
        const int r0 = m0 + wm * C::WM + i * 32 + 8 * vg + 4 * (lane >> 5);
        const u32x4 w = philox4x32_10(static_cast<uint32_t>(col),
                                      static_cast<uint32_t>(r0) >> 2, dp.key0,
                                      dp.key1);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float x = acc[i][j][4 * vg + t];
          acc[i][j][4 * vg + t] = ws[t] >= dp.thresh ? x * dp.scale : 0.0f;
        }
      }
    }
}

// The exchange of split tile t.  Returns false for the piece that arrives
// first (its partial is stored and the flag raised: the workgroup exits);
// true for the second, with rpart set to the partial to add (a zero-sized
// range, and acc NaN, if the partial never became ready).
template <int BM, int BN, bool BWD>
__device__ __forceinline__ bool gemm_split_exchange(
    const SplitArgs& sp, int t, int tid,
    f32x16 (&acc)[GemmCfg<BM, BN, BWD>::TM][GemmCfg<BM, BN, BWD>::TN],
    rsrc_t& rpart) {
  using C = GemmCfg<BM, BN, BWD>;
  __shared__ uint32_t s_arrived, s_ready;
  uint32_t* cnt = sp.cnt + 2 * t;
  rpart = make_rsrc(sp.part + (int64_t)t * BM * BN, (uint32_t)(BM * BN * 4));
  if (tid == 0)
    s_arrived = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (s_arrived == 0) {
    gemm_put_partial<BM, BN, BWD>(rpart, tid, acc);
    __syncthreads();   // every wave's stores precede the release below
    if (tid == 0)
      __hip_atomic_store(cnt + 1, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    return false;
  }
  // The other piece is past its arrival and only has stores left, so this
  // wait is short; the bound only guards against a hang.
  if (tid == 0) {
    int it = 0;
    while (__hip_atomic_load(cnt + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               0u &&
           ++it < G_SPLIT_SPIN)
      __builtin_amdgcn_s_sleep(2);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    s_ready = it < G_SPLIT_SPIN;
    if (it >= G_SPLIT_SPIN)
      __hip_atomic_store(sp.status, (int32_t)QN_ESYNC, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    // back to zero for the next launch (a kernel boundary orders these
    // stores before it)
    __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(cnt + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (s_ready == 0) {
    // an unready partial is never added: the tile becomes NaN
    rpart = make_rsrc(sp.part, 0u);
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = __builtin_nanf("");
  }
  return true;
}

// SPLIT: the grid holds split pieces (SplitArgs); without it the kernel
// has none of their code.
template <int BM, int BN, bool BWD, bool DROP, bool SPLIT, bool CHK>
__global__ __launch_bounds__((BN == 256 ? 512 : 256), 1) void k_gemm(
    const uint16_t* __restrict__ Aop, const uint8_t* __restrict__ packed,
    const uint8_t* __restrict__ qabs, const float* __restrict__ gscale,
    const uint16_t* __restrict__ La_hi, const uint16_t* __restrict__ La_lo,
    const uint16_t* __restrict__ Lb, int M, int N, int K, int rpad,
    void* __restrict__ out, int out_bf16, Codebook cb, DropArgs dp,
    SplitArgs sp) {
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
  const int tiles_n = (NOUT + BN - 1) / BN;
  const int nsteps = (KRED + G_BK - 1) / G_BK;
  const int tiles_m = (M + BM - 1) / BM;
  int tm, tn, s0 = 0, s1 = nsteps, split = -1;
  if (!SPLIT || (int)blockIdx.x < sp.whole) {
    gemm_tile_at(gemm_xcd_index(blockIdx.x, SPLIT ? sp.whole : tiles_m * tiles_n),
                 tiles_m, tiles_n, tm, tn);
  } else {
    const int q = blockIdx.x - sp.whole;
    const bool second = q >= sp.rem;
    split = second ? q - sp.rem : q;
    gemm_tile_at(sp.whole + split, tiles_m, tiles_n, tm, tn);
    const int h = (nsteps / 2) & ~1;
    s0 = second ? h : 0;
    s1 = second ? nsteps : h;
  }
  const int m0 = tm * BM, c0 = tn * BN;

  const int64_t numel = (int64_t)N * K;
  GemmLoader<BM, BN, BWD, CHK> ld;
  ld.Aop = Aop;
  ld.packed = packed;
  ld.qabs = qabs;
  ld.gscale = gscale;
  ld.a_bytes = (uint32_t)((int64_t)M * KRED * 2);
  ld.p_bytes = (uint32_t)((numel + 1) >> 1);
  ld.q_bytes = (uint32_t)((numel + 63) >> 6);
  ld.d_bytes = (uint32_t)(((numel + 16383) >> 14) << 2);
  ld.M = M;
  ld.N = N;
  ld.K = K;
  ld.KRED = KRED;
  ld.m0 = m0;
  ld.c0 = c0;
  ld.tid = tid;
  ld.init();

  // lanes 2i and 2i+1 hold weights of the same 64-weight block (32 each)
  // and build its table together
  const LutHalf lh = lut_half(cb, lane);

  f32x16 acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // with dropout the (masked) adapter term goes first; dY W' is then added
  // on top by the main loop
  if constexpr (DROP) {
    gemm_adapter<BM, BN, BWD>(La_hi, La_lo, Lb, M, NOUT, rpad, m0, c0, wm, wn,
                              lane, acc);
    gemm_drop_acc<BM, BN, BWD>(m0, c0, wm, wn, lane, dp, acc);
  }

  // Steps past the end read out of range: their tiles are zeros (a zero
  // block constant dequantizes every code to zero), so the loop runs whole
  // pairs of steps without branches.  A small piece covers an even number
  // of steps, so only a range that ends at the last step can run over.
  // reduction steps [R0, R1) into acc
#define GEMM_MAINLOOP(R0, R1)                                                  \
  do {                                                                         \
    const int r0_ = (R0), r1_ = (R1);                                          \
    WRegs Wc;                                                                  \
    {                                                                          \
      ARegs<BM, BN, BWD> A0;                                                   \
      ld.load_a(A0, r0_ * G_BK);                                               \
      gemm_store_a<BM, BN, BWD>(A0, sA0, tid);                                 \
    }                                                                          \
    ld.load_w(Wc, r0_ * G_BK);                                                 \
    gemm_dequant_w<BM, BN, BWD>(Wc, sW0, lh, tid);                             \
    ld.load_w(Wc, (r0_ + 1) * G_BK);                                           \
    __builtin_amdgcn_s_waitcnt(0); /* loads landed in LDS and registers */     \
    __syncthreads();                                                           \
    for (int st = r0_; st < r1_; st += 2) {                                    \
      gemm_step<BM, BN, BWD, CHK>(st, sA0, sW0, sA1, sW1, Wc, ld, wm, wn, tid, \
                                  lane, lh, acc);                              \
      gemm_step<BM, BN, BWD, CHK>(st + 1, sA1, sW1, sA0, sW0, Wc, ld, wm, wn,  \
                                  tid, lane, lh, acc);                         \
    }                                                                          \
  } while (0)
  GEMM_MAINLOOP(s0, s1);
#undef GEMM_MAINLOOP

  // The adapter term goes with the piece that starts at step 0; in a split
  // launch every tile runs its code, with a zero-sized buffer range (reads
  // return zeros, no memory traffic) where it does not apply, so that acc has
  // one path and stays in registers.
  if constexpr (!DROP)
    gemm_adapter<BM, BN, BWD>(La_hi, La_lo, Lb,
                              (!SPLIT || split < 0 || s0 == 0) ? M : 0, NOUT,
                              rpad, m0, c0, wm, wn, lane, acc);

  if constexpr (SPLIT) {
    // Every tile runs the add (a zero-sized range where there is no partial)
    // so that acc has one path and stays in registers.
    rsrc_t rpart = make_rsrc(sp.part, 0u);
    if (split >= 0 && !gemm_split_exchange<BM, BN, BWD>(sp, split, tid, acc, rpart))
      return;
    gemm_add_partial<BM, BN, BWD>(rpart, tid, acc);
    // Keep those loads out of the stores below: a wait for a load would also
    // wait for every store issued before it (one counter, in order).
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_sched_barrier(0);
  }

  // One 32-bit offset per accumulator tile (out of range for a column past
  // the edge), so each element is one store (and one convert for bf16).
  // Used while every offset of the tile stays below 2^31.  A tile whose
  // rows all lie below M puts the row step in the scalar offset; the range
  // check covers only the vector offset (plus the instruction offset), so
  // the last row tile of a ragged M adds the row step to the vector offset
  // instead and its rows past M land beyond the buffer's range.
  const int es = out_bf16 ? 2 : 4;
  if (((int64_t)m0 + BM) * NOUT * es < (int64_t(1) << 31)) {
    const rsrc_t ro = make_rsrc(out, (uint32_t)((int64_t)M * NOUT * es));
    const bool rows_full = m0 + BM <= M;
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        const int row0 = m0 + wm * C::WM + i * 32 + 4 * (lane >> 5);
        const int col = gemm_col<BM, BN, BWD>(c0, wn, j, lane);
        const uint32_t vo =
            col < NOUT ? (uint32_t)(row0 * NOUT + col) * (uint32_t)es : G_OOB;
        if (rows_full) {
          if (out_bf16) {
#pragma unroll
            for (int v = 0; v < 16; ++v)
              __builtin_amdgcn_raw_buffer_store_b16(
                  static_cast<uint16_t>(pack_bf16x2(acc[i][j][v], 0.0f) & 0xFFFFu),
                  ro, vo, (8 * (v >> 2) + (v & 3)) * NOUT * 2, 0);
          } else {
#pragma unroll
            for (int v = 0; v < 16; ++v)
              __builtin_amdgcn_raw_buffer_store_b32(
                  __float_as_uint(acc[i][j][v]), ro, vo,
                  (8 * (v >> 2) + (v & 3)) * NOUT * 4, 0);
          }
        } else {
          // vo + step stays below 2^32: step < (m0 + BM) * NOUT * es < 2^31
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const uint32_t o = vo + (uint32_t)((8 * (v >> 2) + (v & 3)) * NOUT * es);
            if (out_bf16)
              __builtin_amdgcn_raw_buffer_store_b16(
                  static_cast<uint16_t>(pack_bf16x2(acc[i][j][v], 0.0f) & 0xFFFFu),
                  ro, o, 0, 0);
            else
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][v]),
                                                    ro, o, 0, 0);
          }
        }
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * C::WM + i * 32 + 8 * (v >> 2) +
                        4 * (lane >> 5) + (v & 3);
        const int col = gemm_col<BM, BN, BWD>(c0, wn, j, lane);
        if (row < M && col < NOUT)
          store_out(out, out_bf16, (int64_t)row * NOUT + col, acc[i][j][v]);
      }
}

}  // namespace

namespace qn {

template <int BM, int BN, bool BWD, bool CHK>
void launch_gemm_t(hipStream_t st, const uint16_t* Aop, const nf4_tensor* w,
                   const uint16_t* La_hi, const uint16_t* La_lo,
                   const uint16_t* Lb, int M, int rpad, void* out,
                   int out_bf16, const DropArgs* drop, const SplitArgs& sp) {
  const int N = (int)w->rows, K = (int)w->cols;
  const int nout = BWD ? K : N;
  const unsigned tiles = (unsigned)(cdiv(M, BM) * cdiv(nout, BN));
  const unsigned grid = sp.rem == 0 ? tiles : (unsigned)(sp.whole + 2 * sp.rem);
  if constexpr (BWD) {
    if (drop != nullptr) {
      QN_LAUNCH("k_bwd_dx_gemm", (k_gemm<BM, BN, BWD, true, false, CHK>),
                dim3(grid), dim3(GemmCfg<BM, BN, BWD>::NT), st, Aop, w->packed,
                w->qabs, w->gscale, La_hi, La_lo, Lb, M, N, K, rpad, out,
                out_bf16, qn::codebook(), *drop, sp);
      return;
    }
  }
  const DropArgs none{};
  if (sp.rem > 0) {
    QN_LAUNCH(BWD ? "k_bwd_dx_gemm" : "k_fwd_gemm",
              (k_gemm<BM, BN, BWD, false, true, CHK>), dim3(grid),
              dim3(GemmCfg<BM, BN, BWD>::NT), st, Aop, w->packed, w->qabs,
              w->gscale, La_hi, La_lo, Lb, M, N, K, rpad, out, out_bf16,
              qn::codebook(), none, sp);
    return;
  }
  QN_LAUNCH(BWD ? "k_bwd_dx_gemm" : "k_fwd_gemm",
            (k_gemm<BM, BN, BWD, false, false, CHK>), dim3(grid),
            dim3(GemmCfg<BM, BN, BWD>::NT), st, Aop, w->packed, w->qabs,
            w->gscale, La_hi, La_lo, Lb, M, N, K, rpad, out, out_bf16,
            qn::codebook(), none, sp);
}

// Checked per-step addressing only where the reduction can end in a partial
// step: the backward (reduction over N) when N % 64 != 0.
template <int BM, int BN, bool BWD>
void launch_gemm_c(hipStream_t st, const uint16_t* Aop, const nf4_tensor* w,
                   const uint16_t* La_hi, const uint16_t* La_lo,
                   const uint16_t* Lb, int M, int rpad, void* out,
                   int out_bf16, const DropArgs* drop, const SplitArgs& sp) {
  if (BWD && w->rows % G_BK != 0)
    launch_gemm_t<BM, BN, BWD, true>(st, Aop, w, La_hi, La_lo, Lb, M, rpad, out,
                                     out_bf16, drop, sp);
  else
    launch_gemm_t<BM, BN, BWD, false>(st, Aop, w, La_hi, La_lo, Lb, M, rpad,
                                      out, out_bf16, drop, sp);
}

template <bool BWD>
void launch_gemm(hipStream_t st, const uint16_t* Aop, const nf4_tensor* w,
                 const uint16_t* La_hi, const uint16_t* La_lo,
                 const uint16_t* Lb, int M, int rpad, void* out,
                 int out_bf16, const DropArgs* drop, void* split_ws) {
  const int64_t nout = BWD ? w->cols : w->rows;
  const int64_t kred = BWD ? w->rows : w->cols;
  SplitArgs sa{0, 0, nullptr, nullptr, nullptr};
  if (split_ws != nullptr) {
    const GemmSplit sp = gemm_split_plan(M, nout, kred, drop != nullptr);
    char* base = static_cast<char*>(split_ws);
    // (the plan's tile edge is the one chosen below: gemm_big_tiles decides both)
    if (sp.rem > 0)
      sa = SplitArgs{sp.whole, sp.rem,
                     reinterpret_cast<float*>(base + gemm_split_part_offset(sp)),
                     reinterpret_cast<uint32_t*>(base + G_SPLIT_HDR),
                     reinterpret_cast<int32_t*>(base)};
  }
  if (gemm_big_tiles(M, nout))
    launch_gemm_c<256, 256, BWD>(st, Aop, w, La_hi, La_lo, Lb, M, rpad, out,
                                 out_bf16, drop, sa);
  else
    launch_gemm_c<128, 128, BWD>(st, Aop, w, La_hi, La_lo, Lb, M, rpad, out,
                                 out_bf16, drop, sa);
}

template void launch_gemm<false>(hipStream_t, const uint16_t*, const nf4_tensor*,
                                 const uint16_t*, const uint16_t*,
                                 const uint16_t*, int, int, void*, int,
                                 const DropArgs*, void*);
template void launch_gemm<true>(hipStream_t, const uint16_t*, const nf4_tensor*,
                                const uint16_t*, const uint16_t*,
                                const uint16_t*, int, int, void*, int,
                                const DropArgs*, void*);

}  // namespace qn
