// Internal declarations shared by the host-side translation units of the
// QLoRA NF4 library.  Not part of the public C ABI.
#pragma once

#include <cstddef>
#include <cstdint>

#include "qlora_nf4.h"

namespace qn {

// 16 NF4 levels and 15 midpoint thresholds, derived on the host in double
// precision (codebook.cpp).
void derive_codebook(float levels[16], float thresholds[15]);

// Levels and thresholds of a QN_CODE_* table; false for an unknown table.
bool derive_variant_codebook(int code, float levels[16], float thresholds[15]);

inline bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

inline bool valid_tensor(const nf4_tensor* w) {
  return w != nullptr && w->packed != nullptr && w->qabs != nullptr &&
         w->gscale != nullptr && w->rows > 0 && w->cols > 0 &&
         aligned16(w->packed);
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Rank-tile dispatch: JT = number of 16-wide tiles of r, rounded up to a
// power of two (1, 2, 4, 8, 16 covers r <= 256); rpad = 16 JT.
inline int rank_tiles(int r) {
  int jt = 1;
  while (jt * 16 < r) jt *= 2;
  return jt;
}

// Shape rules of the fused calls (plan.cpp).
bool valid_linear(int64_t M, const nf4_tensor* w, int32_t r);

// ---- fused GEMM (gemm.hip): 256 x 256 output tiles when they give at
// least ~one workgroup per CU, otherwise 128 x 128.
constexpr int G_CUS = 256;     // MI355X compute units
constexpr int G_BK = 64;       // reduction step
bool gemm_big_tiles(int64_t M, int64_t nout);

// Split reduction (GemmSplit; no split with dropout): a tile computed as
// two workgroups over the two halves of the reduction.  The piece that
// finishes first leaves its fp32 partial tile in the split area and exits,
// the second adds it (two fp32 terms, so the result does not depend on which
// finishes first) and stores the tile.  With 256 x 256 tiles, the tiles of
// a ragged last wave that fills at most half of the GPU; with 128 x 128
// tiles (a small grid), every tile of a grid of at most G_CUS tiles.  Split
// area (the first bytes of a general-path workspace): int32 status word
// (QN_OK, or QN_ESYNC if a partial never became ready), 4 bytes of padding,
// 2 counter words per split tile, then at gemm_split_part_offset one partial
// tile of tile * tile floats per split tile.  The status word and the
// counters must be zero at launch (the second piece of each tile sets its
// counters back to zero).
struct GemmSplit {
  int whole, rem;       // whole tiles, split tiles
  int tile;             // tile edge of the split tiles (256 or 128)
};
constexpr size_t G_SPLIT_HDR = 8;   // status word + padding before the counters
GemmSplit gemm_split_plan(int64_t M, int64_t nout, int64_t kred, bool drop);
size_t gemm_split_bytes(const GemmSplit& sp);        // whole split area
size_t gemm_split_part_offset(const GemmSplit& sp);  // offset of the partials

// ---- rank-r streams (rank.hip): one pass over X or dY forming row sums
// (T = X A^T, G = dY B) and/or column sums (dB, dA) as per-block partials.
enum { RS_ROWS = 1, RS_COLS = 2 };

// RM rows per workgroup, stages of 64 SUB columns, NBUF LDS buffers (NBUF - 1
// stages in flight): about 32 KB of S per stage for r <= 32, less for the
// wider adapters whose R and U tiles take more LDS.  The passes with column
// sums write one fp32 partial [C][rpad] per RM rows, so they keep RM = 256
// up to r = 64 (with two buffers at r = 64: 64 KB of S, 16 KB of R and
// 67.6 KB of U).
//
// The passes over X with LoRA dropout (RS_ROWS: T, RS_COLS: dA) spend most
// of their time in the generator's integer arithmetic, which one wave per
// SIMD cannot overlap with its own loads, so they run two workgroups per
// CU where the LDS allows: the T pass up to jt = 8 with half-width stages
// (at most 72 KB each), the dA pass up to jt = 4 with 128-row blocks (at
// most 67 KB each; twice the column-sum partials).
constexpr int rs_wgs_per_cu(int mode, int jt, bool drop) {
  return drop && ((mode == RS_ROWS && jt <= 8) || (mode == RS_COLS && jt <= 4)) ? 2 : 1;
}
constexpr int rs_rm(int mode, int jt, bool drop = false) {
  return mode == RS_ROWS ? 64
                         : (jt <= 4 ? (rs_wgs_per_cu(mode, jt, drop) == 2 ? 128 : 256) : 64);
}
constexpr int rs_sub(int mode, int jt, bool drop = false) {
  return (jt >= 8 ? 1
                  : (jt == 4 ? (mode == RS_ROWS ? 2 : 1) : (mode == RS_ROWS ? 4 : 1))) /
         (mode == RS_ROWS && rs_wgs_per_cu(mode, jt, drop) == 2 && jt < 8 ? 2 : 1);
}
constexpr int rs_nbuf(int mode, int jt) {
  return jt >= 16 || (jt == 4 && mode != RS_ROWS) ? 2 : 3;
}

struct StreamPlan {
  int rm, sub, mb, nb, cpb;   // rows per block, stage width (x64), row
                              // blocks, column blocks, stages per block
};
StreamPlan stream_plan(int mode, int64_t M, int64_t C, int jt, bool drop = false);

// ---- skinny forward (skinny.hip), M <= QN_SKINNY_M tokens.
constexpr int64_t QN_SKINNY_M = 16;
constexpr int SK_WAVES = 8;                  // waves per workgroup
constexpr int SK_KS_MAX = 4096;              // longest K slice
constexpr int SK_WGS_PER_CU = 2;             // resident workgroups per CU
// tiles (16 rows x one K slice, one wave's work item) a call aims for:
// about 4 per wave of the grid
constexpr int SK_TARGET_TILES = 4 * SK_WAVES * SK_WGS_PER_CU * G_CUS;
struct SkinnyPlan {
  int slices, ks;
  int wtiles;       // tiles of weight rows per slice, cdiv(N, 16)
  int tps;          // tiles per slice: wtiles, then rpad / 16 adapter tiles
  int rows_total;   // 16 tps: rows of the partial sums
};
// One projection of a skinny (batched) forward.
struct SkinnyJob {
  const uint16_t* x;
  int M;
  const nf4_tensor* w;
  const uint16_t* A;
  const uint16_t* B;
  int r;
  float s;
  float* t_save;
  void* y;
  int y_bf16;
};
// K slices of one projection: at least enough that the X slice ((M + 1)
// rows, the zero row included) leaves LDS room for SK_WGS_PER_CU
// workgroups per CU; more, up to about want_tiles tiles, as long as a slice
// keeps >= 128 M columns (the fp32 partial sums then add at most 1/8 of the
// packed weight bytes) or the projection has fewer tiles than the grid has
// waves.
SkinnyPlan skinny_plan(int64_t M, int64_t N, int64_t K, int r,
                       int64_t want_tiles = SK_TARGET_TILES);
// Plans of a batch: each projection asks for its share (by weight count) of
// SK_BATCH_TILES tiles.
constexpr int SK_BATCH_TILES = 2 * SK_TARGET_TILES;
void skinny_plan_batch(const SkinnyJob* jobs, int count, SkinnyPlan* out);
// fp32 partial sums [slices][M][rows_total] of one projection
inline size_t skinny_part_bytes(int64_t M, const SkinnyPlan& P) {
  return size_t(P.slices) * size_t(M) * size_t(P.rows_total) * 4;
}
// Tiles of a batch, numbered projection by projection, slice-major inside a
// projection; the cost of a tile is the number of 256-column chunks of its
// slice.  bound[c] (c = 0 .. nslots) is the first tile whose cost starts at
// or after floor(c T / nslots), T the batch's total cost, so slot c owns
// tiles [bound[c], bound[c + 1]) and every slot's cost is within one tile of
// T / nslots.  Returns the tile count.
int skinny_bounds(const SkinnyPlan* plans, const int64_t* K, int count,
                  int nslots, int32_t* bound);

// Workspace layouts of the fused calls (byte offsets, 256-byte aligned).
// rpad = r rounded up to 16, 32, 64, 128 or 256 (the adapter MFMA width).
// M <= QN_SKINNY_M takes the skinny (GEMV) forward.
struct FwdWorkspace {
  size_t split;     // status word, counters and partial tiles of the GEMM's
                    // split last wave (GEMM path; offset 0)
  size_t th, tl;    // bf16 [M, rpad]  hi/lo parts of s*T      (GEMM path)
  size_t bp;        // bf16 [N, rpad]  B zero-padded           (GEMM path)
  size_t prow;      // fp32 [nb, M, rpad] column-block partials of T
  size_t part;      // fp32 [slices, M, rows] K-slice partials (skinny path)
  int32_t slices, ks;
  size_t total;
  int32_t rpad;
};

struct BwdWorkspace {
  size_t split;     // status word, counters and partial tiles of the dX
                    // GEMM's split last wave (offset 0)
  size_t bt;        // bf16 [r, N]     B transposed
  size_t uth, utl;  // bf16 [r, Mp]    hi/lo parts of s*T, transposed
  size_t atp;       // bf16 [K, rpad]  A transposed, zero-padded
  size_t gh, gl;    // bf16 [M, rpad]  hi/lo parts of s*G, G = dY B
  size_t ugh, ugl;  // bf16 [r, Mp]    hi/lo parts of s*G, transposed
  size_t prow;      // fp32 [nb, M, rpad] column-block partials of G
  size_t pcol;      // fp32 [mb, max(N, K), rpad] row-block partials of dB, dA
  size_t total;
  int64_t mp;       // M rounded up to a multiple of 8
  int32_t rpad;
};

// general: the layout of the general path also for M <= QN_SKINNY_M (a
// forward with dropout never takes the skinny path).  split: room for the
// partial tiles of a split last wave (without it the GEMM never splits and
// the split area holds only the status word).
FwdWorkspace fwd_workspace_layout(int64_t M, int64_t N, int64_t K, int32_t r,
                                  bool general, bool split = true);
BwdWorkspace bwd_workspace_layout(int64_t M, int64_t N, int64_t K, int32_t r);

}  // namespace qn
