// Skinny forward of the QLoRA linear layer (M <= 16 tokens): an HBM-bound
// GEMV over the NF4 weight with the adapter's T = X A^T in the same pass
// ("QLoRA Guide", Forward pass diagram; "QLORA ... paper summary", Notes:
// dequantize to BF16, multiply).  One launch pair serves a batch of up to
// QN_FWD_BATCH_MAX projections (qlora_linear_fwd_batch; a single
// qlora_linear_fwd with M <= 16 is a batch of one).
#include "qn_host.h"

namespace {

using namespace qn;

// ---------------------------------------------------------------------------
// K6: skinny forward, partial sums.
//
// Tiles: 16 rows of one projection x one K slice of KS columns, numbered
// projection by projection and, inside a projection, slice-major, one list
// for the whole batch.  Rows [0, N) of a projection are its NF4 weight W;
// its adapter A (bf16) takes rows [Nw, Nw + rpad), Nw = N rounded up to 16,
// so T comes out of the same pass; a tile holds weight rows or adapter rows,
// never both, and a slice's adapter tiles follow its weight tiles.
//
// The grid is SK_WGS_PER_CU = 2 workgroups of SK_WAVES = 8 waves per CU.
// The host cuts the list into 2 G_CUS runs whose costs (in 256-column
// chunks) are within one tile of an equal share.  Workgroups c and
// c + G_CUS take runs 2c and 2c + 1: adjacent tiles, and the same XCD (the
// hardware deals workgroups to the XCDs by index mod 8), so the two share
// L2 lines of X and of the adapter rows.  Inside a workgroup's run wave w
// takes every eighth tile, starting with tile w.  (Cutting G_CUS runs in
// halves by tile count instead left one workgroup with 3x the work of
// another where the cheap tiles of a short last slice met full ones.)
// Wherever the run changes projection or slice, the workgroup stages that
// slice of X in LDS (M rows, then an all-zero row M), each 8-element group
// permuted into the order decode8p produces.
//
// A wave's weight tiles of one slice are one stream, chunk by chunk (256
// columns): lane (n = l % 16, g = l / 16) loads the 32 packed bytes of
// block g of row n, builds that block's 16-entry bf16 table and decodes 8
// weights per v_mfma_f32_16x16x32_bf16 (t = 0..7 takes weights 8t..8t+7 of
// the block); the matching A operand is X[m][64 g + 8 t ...] from LDS.  The
// loads run two chunks ahead of the decode through three register sets,
// also across tile boundaries, and a chunk's eight MFMAs alternate between
// two accumulators.  Partial sums go to part[slice][m][row] (fp32, m < M).
// ---------------------------------------------------------------------------

static_assert(SK_WGS_PER_CU == 2, "two workgroups per CU");

struct SkProj {
  const uint16_t* X;
  const uint8_t* packed;
  const uint8_t* qabs;
  const float* gscale;
  const uint16_t* A;
  float* part;
  int M, N, K, r, KS, wtiles, tps, tile0;
};

// bound[j]: first tile of run j (skinny_bounds over 2 G_CUS runs); run 2c
// belongs to workgroup c, run 2c + 1 to workgroup c + G_CUS.
// wave_steps: the batch's chunk steps per wave of the grid (total cost /
// waves), the yardstick of a wave's progress.
struct SkArgs {
  SkProj p[QN_FWD_BATCH_MAX];
  int nproj, wave_steps;
  int bound[SK_WGS_PER_CU * G_CUS + 1];
};

// Issue priority by progress.  A SIMD's waves share its VALU, and at equal
// priority the oldest wave issues first; left alone, the older workgroup's
// waves run ahead and the younger ones finish the kernel by themselves,
// with too few waves to cover the memory latency.  Each wave therefore
// starts at priority 3 and steps down at 1/4, 1/2 and 3/4 of wave_steps
// chunk steps, so that the waves behind issue first and the waves of a
// SIMD stay within about a quarter of their work of each other.
struct SkPrio {
  int done = 0, band = 0, next = 0, quarter = 1;
  __device__ void start(int wave_steps) {
    quarter = max(1, wave_steps / 4);
    next = quarter;
    __builtin_amdgcn_s_setprio(3);
  }
  __device__ void advance(int steps) {
    done += steps;
    if (done >= next && band < 3) {
      ++band;
      next += quarter;
      if (band == 1)
        __builtin_amdgcn_s_setprio(2);
      else if (band == 2)
        __builtin_amdgcn_s_setprio(1);
      else
        __builtin_amdgcn_s_setprio(0);
    }
  }
};

struct SkRegs {
  u32x4 w0, w1;
  uint32_t q;
  float d;
};

// The projection and K slice that a segment of tiles shares (uniform values,
// copied from the kernel arguments once per segment).
struct SkRun {
  int M, N, K, KS, r, Nw, rows_total, k0, klen, slice;
  const uint16_t* X;
  const uint16_t* A;
  float* part;
  rsrc_t rp, rq, rd;
};

__device__ __forceinline__ void sk_run_of(const SkArgs& a, int p, int slice,
                                          SkRun& R) {
  const SkProj& P = a.p[p];
  R.M = P.M;
  R.N = P.N;
  R.K = P.K;
  R.KS = P.KS;
  R.r = P.r;
  R.Nw = 16 * P.wtiles;
  R.rows_total = 16 * P.tps;
  R.slice = slice;
  R.k0 = slice * P.KS;
  R.klen = min(P.KS, P.K - R.k0);
  R.X = P.X;
  R.A = P.A;
  R.part = P.part;
  const int64_t numel = (int64_t)P.N * P.K;
  R.rp = make_rsrc(P.packed, (uint32_t)((numel + 1) >> 1));
  R.rq = make_rsrc(P.qabs, (uint32_t)((numel + 63) >> 6));
  R.rd = make_rsrc(P.gscale, (uint32_t)(((numel + 16383) >> 14) << 2));
}

// X slice of the run -> LDS (M rows, columns >= klen zero, then the
// all-zero row M), each 8-element group permuted into the order decode8p
// produces.
__device__ __forceinline__ void sk_stage_x(const SkRun& R, uint16_t* sX,
                                           int tid) {
  const int M = R.M, K = R.K, KS = R.KS, XP = KS + 8;
  const rsrc_t rx = make_rsrc(R.X, (uint32_t)((int64_t)M * K * 2));
  for (int c = tid; c < KS / 8; c += 512)
    *reinterpret_cast<u32x4*>(sX + M * XP + 8 * c) = u32x4{0u, 0u, 0u, 0u};
  const int groups = M * (KS / 8);
  // batches of 4 loads per thread, all issued before their LDS writes
  for (int i0 = 0; i0 < groups; i0 += 4 * 512) {
    u32x4 xv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = i0 + tid + 512 * i;
      const int m = idx / (KS / 8), c = 8 * (idx % (KS / 8));
      const bool ok = idx < groups && c < R.klen;
      xv[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
          rx, ok ? (uint32_t)(((int64_t)m * K + R.k0 + c) * 2) : G_OOB, 0, 0));
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
}

// The eight A operands (X[m][64 g + 8 t ...], t = 0..7) of a chunk; lanes
// whose row is >= M read the all-zero row M.
__device__ __forceinline__ void sk_read_x(const SkRun& R, const uint16_t* sX,
                                          int n, int g, int kc, u32x4 (&xa)[8]) {
  const uint16_t* xrow = sX + (n < R.M ? n : R.M) * (R.KS + 8) + 64 * g + kc;
#pragma unroll
  for (int s8 = 0; s8 < 8; ++s8)
    xa[s8] = *reinterpret_cast<const u32x4*>(xrow + 8 * s8);
}

// acc[v] = C[m = 4 g + v][row] -> part[slice][m][row] for the lanes whose
// token m is < M (the others address past the range and are dropped).
__device__ __forceinline__ void sk_store(const SkRun& R, int row, int g,
                                         const f32x4& acc) {
  const rsrc_t rpt = make_rsrc(
      R.part, (uint32_t)((int64_t)(R.slice + 1) * R.M * R.rows_total * 4));
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int m = 4 * g + v;
    const uint32_t off =
        m < R.M ? (uint32_t)((((int64_t)R.slice * R.M + m) * R.rows_total + row) * 4)
                : G_OOB;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[v]), rpt, off, 0, 0);
  }
}

// Weight bytes, block code and group scale of the lane's block whose first
// element is 64 qb (qb = element index / 64, so the packed bytes start at
// 32 qb, the code at qb and the group scale at 4 (qb / 256)).  `skip`
// (qb = ~0) addresses past every range: the block's constant loads as 0,
// which makes all 64 weights +-0.  `oob` (0 or G_OOB) drops the packed
// loads of positions past the run.  Rows past N address past the ranges by
// themselves.  Every step of the stream issues these same four loads, so
// the wait before a chunk's decode leaves the next two chunks in flight.
__device__ __forceinline__ void sk_load(const SkRun& R, uint32_t qb, bool skip,
                                        uint32_t oob, SkRegs& W) {
  const uint32_t qm = skip ? ~0u : qb;
  const uint32_t op = (qb << 5) | oob;
  W.w0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(R.rp, op, 0, 0));
  W.w1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(R.rp, op, 16, 0));
  W.q = __builtin_amdgcn_raw_buffer_load_b8(R.rq, qm, 0, 0);
  W.d = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
      R.rd, (qm >> 6) & ~3u, 0, 0));
}

__device__ __forceinline__ void sk_decode_chunk(const u32x4 (&xa)[8],
                                                const SkRegs& W,
                                                const Codebook& cb, f32x4& acc0,
                                                f32x4& acc1) {
  const Lut t = make_lut(cb, static_cast<float>(W.q) * W.d);
  const uint32_t wd[8] = {W.w0.x, W.w0.y, W.w0.z, W.w0.w,
                          W.w1.x, W.w1.y, W.w1.z, W.w1.w};
#pragma unroll
  for (int s8 = 0; s8 < 8; s8 += 2) {
    acc0 = mfma16(xa[s8], decode8p(wd[s8], t), acc0);
    acc1 = mfma16(xa[s8 + 1], decode8p(wd[s8 + 1], t), acc1);
  }
}

__global__ __launch_bounds__(512) void k_skinny_partial(SkArgs args,
                                                        Codebook cb) {
  extern __shared__ __attribute__((aligned(16))) uint16_t sX[];   // (M+1) x (KS+8)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;

  // this workgroup's run of tiles
  const int run = SK_WGS_PER_CU * (blockIdx.x % G_CUS) + blockIdx.x / G_CUS;
  const int ib = args.bound[run], ie = args.bound[run + 1];

  SkPrio prio;
  prio.start(args.wave_steps);
  int p = 0, staged_p = -1, staged_slice = -1;
  int tile = ib;
  while (tile < ie) {
    // segment: the tiles of one projection and slice, [tile, seg_end)
    while (p + 1 < args.nproj && tile >= args.p[p + 1].tile0) ++p;
    const int tps = args.p[p].tps, wtiles = args.p[p].wtiles;
    const int local = tile - args.p[p].tile0;
    const int slice = local / tps, t_seg = local % tps;
    const int seg_end = min(ie, tile + (tps - t_seg));
    SkRun R;
    sk_run_of(args, p, slice, R);
    const bool restage = p != staged_p || slice != staged_slice;
    // this wave's first tile of the segment (slice-local index): every
    // eighth tile of the run, counted from ib
    const int first = t_seg + ((wave - (tile - ib)) % SK_WAVES + SK_WAVES) % SK_WAVES;
    const int t_end = t_seg + (seg_end - tile);          // slice-local end
    const int w_end = min(t_end, wtiles);                // end of weight tiles
    const int nw = first < w_end ? (w_end - first + SK_WAVES - 1) / SK_WAVES : 0;

    // Weight tiles first, tile first + 8 i for i < nw: one stream of
    // nw * nch chunk steps.  The lane's load address is one running block
    // index qb, moved by a uniform step: 4 blocks to the next chunk, 128
    // rows down and back to the slice's first chunk at a tile boundary.
    const int nch = (R.klen + 255) / 256;          // chunks per tile
    const int steps = nw * nch;
    const uint32_t K64 = (uint32_t)R.K / 64;
    const uint32_t wrap = (uint32_t)(16 * SK_WAVES) * K64 - 4u * (uint32_t)(nch - 1);
    // On a tile's last chunk, lanes whose 64 columns lie past the slice
    // load a zero block constant (only when the slice is not a whole number
    // of chunks).
    const bool tail_dead = 64 * g >= R.klen - 256 * (nch - 1);
    uint32_t qb = (uint32_t)(first * 16 + n) * K64 + (uint32_t)(R.k0 / 64 + g);
    int pc = 0;                                    // chunk being loaded
    int cc = 0, ctile = first;                     // chunk being decoded
    auto load_next = [&](int s_load, SkRegs& W) {
      sk_load(R, qb, pc == nch - 1 && tail_dead, s_load < steps ? 0u : G_OOB, W);
      const bool wrapped = pc == nch - 1;
      qb += wrapped ? wrap : 4u;
      pc = wrapped ? 0 : pc + 1;
    };
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    f32x4 acc0 = zero4, acc1 = zero4;
    const uint16_t* xb = sX + (n < R.M ? n : R.M) * (R.KS + 8) + 64 * g;
    auto decode_step = [&](const SkRegs& W) {
      u32x4 xa[8];
      const uint16_t* xr = xb + 256 * cc;
#pragma unroll
      for (int s8 = 0; s8 < 8; ++s8)
        xa[s8] = *reinterpret_cast<const u32x4*>(xr + 8 * s8);
      sk_decode_chunk(xa, W, cb, acc0, acc1);
      const bool tile_end = cc == nch - 1;
      if (tile_end) {
        sk_store(R, ctile * 16 + n, g, acc0 + acc1);
        acc0 = zero4;
        acc1 = zero4;
      }
      ctile += tile_end ? SK_WAVES : 0;
      cc = tile_end ? 0 : cc + 1;
    };
    // Three steps per iteration, the register sets rotating; the number of
    // vector memory instructions between a chunk's loads and its decode is
    // the same on every path through the loop, so the waits keep two chunks
    // in flight.  The last one or two steps follow the loop.
    SkRegs W0, W1, W2;
    // (the scheduler must not interleave the two chunks' loads: the waits in
    // the loop count on W0's loads being issued before W1's)
    load_next(0, W0);
    __builtin_amdgcn_sched_barrier(0);
    load_next(1, W1);
    __builtin_amdgcn_sched_barrier(0);
    // the first two chunks are in flight while the X slice is staged
    if (restage) {
      if (staged_p >= 0) __syncthreads();        // sX still being read
      staged_p = p;
      staged_slice = slice;
      sk_stage_x(R, sX, tid);
      __syncthreads();
    }
    int s0 = 0;
    for (; s0 + 3 <= steps; s0 += 3) {
      prio.advance(3);
      load_next(s0 + 2, W2);
      decode_step(W0);
      load_next(s0 + 3, W0);
      decode_step(W1);
      load_next(s0 + 4, W1);
      decode_step(W2);
    }
    if (s0 < steps) decode_step(W0);
    if (s0 + 1 < steps) decode_step(W1);

    // Adapter tiles (T = X A^T, A bf16): the wave's tiles at or past
    // wtiles, plain loads of A, chunk by chunk.
    const rsrc_t ra = make_rsrc(R.A, (uint32_t)((int64_t)R.r * R.K * 2));
    for (int t = first + nw * SK_WAVES; t < t_end; t += SK_WAVES) {
      const int j = (t - wtiles) * 16 + n;
      f32x4 a0 = zero4, a1 = zero4;
      for (int kc = 0; kc < R.klen; kc += 256) {
        u32x4 xa[8];
        sk_read_x(R, sX, n, g, kc, xa);
        const int k = R.k0 + kc + 64 * g;
        const bool ok = kc + 64 * g < R.klen && j < R.r;
        const uint32_t o = ok ? (uint32_t)(((int64_t)j * R.K + k) * 2) : G_OOB;
        u32x4 b[8];
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8)
          b[s8] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
              ra, o, 16 * s8, 0));
#pragma unroll
        for (int s8 = 0; s8 < 8; s8 += 2) {
          a0 = mfma16(xa[s8], permute8(b[s8]), a0);
          a1 = mfma16(xa[s8 + 1], permute8(b[s8 + 1]), a1);
        }
      }
      sk_store(R, R.Nw + j, g, a0 + a1);
    }
    tile = seg_end;
  }
}

// Sum over the K slices of one partial-sum element, slice order fixed; the
// loads of eight slices are issued before they are added.
__device__ __forceinline__ float sum_slices(const float* __restrict__ p,
                                            int64_t stride, int slices) {
  float acc = 0.f;
  for (int sl = 0; sl < slices; sl += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = sl + u < slices ? p[(int64_t)(sl + u) * stride] : 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u];
  }
  return acc;
}

// ---------------------------------------------------------------------------
// Reduce: Y[m][n] = sum_slices part[.][m][n] + s * sum_j T[m][j] B[n][j],
// and T[m][j] = sum_slices part[.][m][Nw + j] (written to t_save by the
// blocks of the first column block).  The blocks of all projections form one
// grid; block b of projection p covers columns [256 bx, 256 bx + 256) of
// tokens [4 by, 4 by + 4), four adjacent outputs per thread (16-byte partial
// loads; N % 8 == 0, so a thread's four columns are all in range or all
// out).  Every load a thread needs goes out before the first is waited for:
// its rows of B (r <= 16), then SKR_SL slices of its outputs and of its T
// element (r <= 64) at a time.
// ---------------------------------------------------------------------------
struct SkRProj {
  const float* part;
  const uint16_t* B;
  float* t_save;
  void* Y;
  float s;
  int slices, M, N, r, rpad, y_bf16, blk0;
};

struct SkRArgs {
  SkRProj p[QN_FWD_BATCH_MAX];
  int nproj;
};

constexpr int SKR_SL = 16;    // slice loads in flight per summed element
constexpr int SKR_COLS = 256; // columns per block

// sum_j t[j] * B row j (16-byte rows of eight bf16), j in order
__device__ __forceinline__ float skr_dot8(const float* t, const u32x4& w, float acc) {
  const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    acc += t[2 * h] * __uint_as_float(ww[h] << 16);
    acc += t[2 * h + 1] * __uint_as_float(ww[h] & 0xFFFF0000u);
  }
  return acc;
}

__global__ __launch_bounds__(256) void k_skinny_reduce(SkRArgs args) {
  __shared__ float sT[4 * QN_MAX_RANK];
  int p = 0;
  while (p + 1 < args.nproj && (int)blockIdx.x >= args.p[p + 1].blk0) ++p;
  const SkRProj& P = args.p[p];
  const int M = P.M, N = P.N, r = P.r;
  const int Nw = (N + 15) / 16 * 16;
  const int64_t rows_total = Nw + P.rpad;
  const int64_t stride = (int64_t)M * rows_total;      // between slices
  const int nbx = (N + SKR_COLS - 1) / SKR_COLS;
  const int local = blockIdx.x - P.blk0;
  const int bx = local % nbx, by = local / nbx;
  const int mb = 4 * by;
  const int mrows = min(4, M - mb);
  const int n0 = bx * SKR_COLS + 4 * (threadIdx.x & 63);
  const int mi = threadIdx.x >> 6;
  const bool live = n0 < N && mi < mrows;
  const int m = mb + mi;
  const bool b16 = (r & 7) == 0 && (reinterpret_cast<uintptr_t>(P.B) & 15) == 0;
  // (lanes without outputs read valid addresses, row 0 and slice 0, and drop
  // what they read, so that no load sits behind a branch)
  const uint16_t* b = P.B + (live ? (int64_t)n0 * r : 0);
  u32x4 brow[4][2];
  if (b16 && r <= 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 2; ++q)
        brow[i][q] = 8 * q < r ? *reinterpret_cast<const u32x4*>(b + i * r + 8 * q)
                               : u32x4{0u, 0u, 0u, 0u};
  }
  const int tidx = threadIdx.x;
  const bool tl = r <= 64 && tidx < mrows * r;
  const int tm = mb + (tl ? tidx / r : 0), tj = tl ? tidx % r : 0;
  const float* py = P.part + (live ? (int64_t)m * rows_total + n0 : 0);
  const float* pt = P.part + (tl ? (int64_t)tm * rows_total + Nw + tj : 0);
  float y[4] = {0.f, 0.f, 0.f, 0.f}, tsum = 0.f;
  for (int sl = 0; sl < P.slices; sl += SKR_SL) {
    f32x4 yv[SKR_SL];
    float tv[SKR_SL];
#pragma unroll
    for (int u = 0; u < SKR_SL; ++u) {
      const bool in = sl + u < P.slices;
      const int64_t o = (int64_t)(in ? sl + u : 0) * stride;
      yv[u] = *reinterpret_cast<const f32x4*>(py + o);
      tv[u] = pt[o];
      if (!(live && in)) yv[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (!(tl && in)) tv[u] = 0.f;
    }
#pragma unroll
    for (int u = 0; u < SKR_SL; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] += yv[u][i];
#pragma unroll
    for (int u = 0; u < SKR_SL; ++u) tsum += tv[u];
  }
  if (tl) {
    sT[tidx] = tsum;
    if (bx == 0) P.t_save[(int64_t)tm * r + tj] = tsum;
  }
  if (r > 64) {
    for (int idx = threadIdx.x; idx < mrows * r; idx += 256) {
      const int mm = mb + idx / r, j = idx % r;
      const float v = sum_slices(P.part + (int64_t)mm * rows_total + Nw + j, stride,
                                 P.slices);
      sT[idx] = v;
      if (bx == 0) P.t_save[(int64_t)mm * r + j] = v;
    }
  }
  __syncthreads();
  if (!live) return;
  const float* t = sT + mi * r;
  float lora[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint16_t* bi = b + i * r;
    if (b16 && r <= 16) {
      lora[i] = skr_dot8(t, brow[i][0], lora[i]);
      if (r > 8) lora[i] = skr_dot8(t + 8, brow[i][1], lora[i]);
    } else if (b16) {
      for (int j0 = 0; j0 < r; j0 += 8)
        lora[i] = skr_dot8(t + j0, *reinterpret_cast<const u32x4*>(bi + j0), lora[i]);
    } else {
      for (int jj = 0; jj < r; ++jj) lora[i] += t[jj] * bf16_to_f32(bi[jj]);
    }
  }
  const int64_t o = (int64_t)m * N + n0;
  if (P.y_bf16) {
    uint2 v;
    v.x = pack_bf16x2(y[0] + P.s * lora[0], y[1] + P.s * lora[1]);
    v.y = pack_bf16x2(y[2] + P.s * lora[2], y[3] + P.s * lora[3]);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(P.Y) + o) = v;
  } else {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(P.Y) + o) =
        f32x4{y[0] + P.s * lora[0], y[1] + P.s * lora[1], y[2] + P.s * lora[2],
              y[3] + P.s * lora[3]};
  }
}

}  // namespace

namespace qn {

void launch_skinny(hipStream_t st, const SkinnyJob* jobs, int count,
                   const SkinnyPlan* plans, char* ws) {
  static_assert(sizeof(SkArgs) + sizeof(Codebook) <= 4096, "kernel arguments");
  SkArgs a{};
  SkRArgs ra{};
  a.nproj = ra.nproj = count;
  int64_t K[QN_FWD_BATCH_MAX];
  int tiles = 0, blocks = 0;
  size_t shm = 16, off = 0;                 // X tile bytes, partials offset
  for (int i = 0; i < count; ++i) {
    const SkinnyJob& J = jobs[i];
    const SkinnyPlan& P = plans[i];
    float* part = reinterpret_cast<float*>(ws + off);
    off += align256(skinny_part_bytes(J.M, P));
    a.p[i] = SkProj{J.x, J.w->packed, J.w->qabs, J.w->gscale, J.A, part,
                    J.M, (int)J.w->rows, (int)J.w->cols, J.r,
                    P.ks, P.wtiles, P.tps, tiles};
    tiles += P.tps * P.slices;
    K[i] = J.w->cols;
    shm = std::max(shm, size_t(J.M + 1) * (P.ks + 8) * 2);
    ra.p[i] = SkRProj{part, J.B, J.t_save, J.y, J.s, P.slices, J.M,
                      (int)J.w->rows, J.r, 16 * rank_tiles(J.r), J.y_bf16, blocks};
    blocks += (int)(cdiv(J.w->rows, SKR_COLS) * cdiv(J.M, 4));
  }
  skinny_bounds(plans, K, count, SK_WGS_PER_CU * G_CUS, a.bound);
  int64_t cost = 0;
  for (int i = 0; i < count; ++i) cost += int64_t(plans[i].tps) * cdiv(K[i], 256);
  a.wave_steps = (int)(cost / (G_CUS * SK_WGS_PER_CU * SK_WAVES));
  QN_LAUNCH_SHM("k_skinny_partial", k_skinny_partial,
                dim3((unsigned)(G_CUS * SK_WGS_PER_CU)), dim3(512), shm, st, a,
                qn::codebook());
  QN_LAUNCH("k_skinny_reduce", k_skinny_reduce, dim3((unsigned)blocks),
            dim3(256), st, ra);
}

}  // namespace qn
