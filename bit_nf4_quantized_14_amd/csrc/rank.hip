// Rank-r side products of the QLoRA linear layer: T = X A^T, G = dY B,
// dB = s dY^T T and dA = s G^T X ("QLoRA Guide", Forward pass diagram:
// B(A(x)); "QLoRA Implementation Details (2025 Edition)", Step 4: scale
// alpha / r; only A and B get gradients).
#include "qn_host.h"

namespace {

using namespace qn;


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

template <int MODE, int JT, bool DROP>
struct RsCfg {
  static constexpr bool ROWS = (MODE & RS_ROWS) != 0;
  static constexpr bool COLS = (MODE & RS_COLS) != 0;
  static constexpr int RM = rs_rm(MODE, JT, DROP), SUB = rs_sub(MODE, JT, DROP);
  static constexpr int NBUF = rs_nbuf(MODE, JT);
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

template <int MODE, int JT, bool DROP>
__device__ __forceinline__ void rs_stage_dma(rsrc_t rs, rsrc_t rr, char* dS,
                                             char* dR, int64_t C, int nvalid,
                                             int r, int stage, int wave,
                                             int lane) {
  using G = RsCfg<MODE, JT, DROP>;
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

// With DROP, S is X and each operand read from the S tile is replaced by
// its LoRA-dropout version (qn_device.h) at its absolute (row, column):
// rows m0 + local row, columns 64 (SUB stage + u) + local column.
template <int MODE, int JT, bool DROP>
__device__ __forceinline__ void rs_stage_compute(
    const char* sS, const char* sR, const uint16_t* sUh, const uint16_t* sUl,
    int wave, int lane, f32x4 (&accR)[RsCfg<MODE, JT, DROP>::TR][JT],
    f32x4 (&accC)[RsCfg<MODE, JT, DROP>::SUB][JT], int stage, int m0,
    const DropArgs& dp) {
  using G = RsCfg<MODE, JT, DROP>;
#pragma unroll
  for (int u = 0; u < G::SUB; ++u) {
    const char* tS = sS + u * G::RM * 128;
    const int col0 = (stage * G::SUB + u) * 64;
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
          const int lrow = wave * (G::RM / 4) + 16 * tr + (lane & 15);
          u32x4 a = rs_read_row(tS, lrow, 4 * s + (lane >> 4));
          if constexpr (DROP)
            a = drop_row8(a, m0 + lrow, col0 + 8 * (4 * s + (lane >> 4)), dp);
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
        u32x4 a = rs_read_colT(tS, 32 * s2, 16 * wave, lane);
        if constexpr (DROP)
          a = drop_col8(a, m0 + 32 * s2 + 8 * (lane >> 4),
                        col0 + 16 * wave + (lane & 15), dp);
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
template <int MODE, int JT, bool DROP>
__device__ __forceinline__ void rs_store_cols(
    rsrc_t rc, int stage, int C, int wave, int lane,
    const f32x4 (&accC)[RsCfg<MODE, JT, DROP>::SUB][JT]) {
  using G = RsCfg<MODE, JT, DROP>;
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

template <int MODE, int JT, bool DROP>
__global__ __launch_bounds__(256) void k_rank_stream(
    const uint16_t* __restrict__ S, int M, int C,
    const uint16_t* __restrict__ R, int r, const uint16_t* __restrict__ Uh,
    const uint16_t* __restrict__ Ul, int ldu, int cpb,
    float* __restrict__ prow, float* __restrict__ pcol, DropArgs dp) {
  using G = RsCfg<MODE, JT, DROP>;
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
  rs_stage_dma<MODE, JT, DROP>(rs, rr, sS0, sR0, C, nvalid, r, sb, wave, lane);
  const bool two = G::NBUF == 3 && sb + 1 < se;
  if (two)
    rs_stage_dma<MODE, JT, DROP>(rs, rr, sS1, sR1, C, nvalid, r, sb + 1, wave, lane);
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
  // `cur` while the stage NBUF - 1 ahead streams into buffer `far` (the
  // buffer of the stage before, which every wave has left at the last
  // barrier), then wait until the next stage has landed.  With three buffers
  // the loads start after the compute and the newest stage stays in flight
  // across the barrier (its loads are the last ones issued, and loads
  // complete in order); with two, they start before the compute, so that
  // their latency runs under it.
#define RS_BODY(I, CS, CR, FS, FR)                                            \
  do {                                                                        \
    if (G::COLS && (I) > sb)                                                  \
      rs_store_cols<MODE, JT, DROP>(rc, (I) - 1, C, wave, lane, accC);              \
    const bool ahead_ = (I) + G::NBUF - 1 < se;                               \
    if (G::NBUF == 2 && ahead_)                                               \
      rs_stage_dma<MODE, JT, DROP>(rs, rr, FS, FR, C, nvalid, r, (I) + 1, wave,     \
                             lane);                                           \
    rs_stage_compute<MODE, JT, DROP>(CS, CR, sUh, sUl, wave, lane, accR,      \
                                     accC, (I), m0, dp);                      \
    if (G::NBUF == 3 && ahead_) {                                             \
      rs_stage_dma<MODE, JT, DROP>(rs, rr, FS, FR, C, nvalid, r, (I) + 2, wave,     \
                             lane);                                           \
      RS_WAIT_VM(G::DMA);                                                     \
    } else {                                                                  \
      RS_WAIT_VM(0);                                                          \
    }                                                                         \
    wg_barrier();                                                             \
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
  if (G::COLS) rs_store_cols<MODE, JT, DROP>(rc, se - 1, C, wave, lane, accC);
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

// sum_{k < nb} src[k stride], added in k order, eight loads in flight
// before they are added.
__device__ __forceinline__ float finish_sum(const float* __restrict__ src,
                                            int64_t stride, int nb) {
  float v = 0.0f;
  for (int k0 = 0; k0 < nb; k0 += 8) {
    float t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) t[u] = k0 + u < nb ? src[(k0 + u) * stride] : 0.0f;
#pragma unroll
    for (int u = 0; u < 8; ++u) v += t[u];
  }
  return v;
}

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
      v = finish_sum(p.src + (int64_t)m * p.ld + j, p.bstride, p.nb);
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
    const float v = finish_sum(p.src + c * p.rpad + j, (int64_t)p.C * p.rpad, p.nb);
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

}  // namespace

namespace qn {

// Rank-stream geometry: RM rows per workgroup, stages of 64 SUB columns,
// and enough column blocks for one long-lived workgroup per CU (each keeps
// two stages in flight).
template <int MODE>
void launch_rank_stream(hipStream_t st, const char* kname, const StreamPlan& P,
                        const uint16_t* S, int M, int C, const uint16_t* R,
                        int r, const uint16_t* Uh, const uint16_t* Ul, int ldu,
                        float* prow, float* pcol, const DropArgs* drop) {
  const dim3 grid((unsigned)P.nb, (unsigned)P.mb);
  // the dY pass (rows and columns at once) never carries dropout
  if constexpr (MODE != (RS_ROWS | RS_COLS)) {
    if (drop != nullptr) {
      const DropArgs dp = *drop;
      QN_RANK_DISPATCH(r, QN_LAUNCH(kname, (k_rank_stream<MODE, JT, true>), grid,
                                    dim3(256), st, S, M, C, R, r, Uh, Ul, ldu,
                                    P.cpb, prow, pcol, dp));
      return;
    }
  }
  const DropArgs none{};
  QN_RANK_DISPATCH(r, QN_LAUNCH(kname, (k_rank_stream<MODE, JT, false>), grid,
                                dim3(256), st, S, M, C, R, r, Uh, Ul, ldu,
                                P.cpb, prow, pcol, none));
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

template void launch_rank_stream<RS_ROWS>(hipStream_t, const char*, const StreamPlan&,
                                          const uint16_t*, int, int, const uint16_t*,
                                          int, const uint16_t*, const uint16_t*, int,
                                          float*, float*, const DropArgs*);
template void launch_rank_stream<RS_COLS>(hipStream_t, const char*, const StreamPlan&,
                                          const uint16_t*, int, int, const uint16_t*,
                                          int, const uint16_t*, const uint16_t*, int,
                                          float*, float*, const DropArgs*);
template void launch_rank_stream<RS_ROWS | RS_COLS>(
    hipStream_t, const char*, const StreamPlan&, const uint16_t*, int, int,
    const uint16_t*, int, const uint16_t*, const uint16_t*, int, float*, float*,
    const DropArgs*);

}  // namespace qn
