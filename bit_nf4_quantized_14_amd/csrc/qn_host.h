// Host-side pieces shared by the translation units of the QLoRA NF4 library:
// argument checks, the per-launch profiling hook, and the launchers each
// kernel file exports to the entry points.  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>

#include "qlora_nf4.h"
#include "qn_device.h"
#include "qn_internal.h"

namespace qn {

// Codebook kernel argument (host-derived once, codebook.cpp).
const Codebook& codebook();

inline bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

inline int check_launch() {
  return hipGetLastError() == hipSuccess ? QN_OK : QN_EHIP;
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline bool valid_tensor(const nf4_tensor* w) {
  return w != nullptr && w->packed != nullptr && w->qabs != nullptr &&
         w->gscale != nullptr && w->rows > 0 && w->cols > 0 &&
         aligned16(w->packed);
}

// Rank-tile dispatch: JT = number of 16-wide tiles of r, rounded up to a
// power of two (1, 2, 4, 8, 16 covers r <= 256); rpad = 16 JT.
inline int rank_tiles(int r) {
  int jt = 1;
  while (jt * 16 < r) jt *= 2;
  return jt;
}

bool valid_linear(int64_t M, const nf4_tensor* w, int32_t r);

// Per-launch event recording for one named kernel (qn_profile_kernel).
struct ProfileHook {
  char name[64] = {0};
  void** ev_start = nullptr;
  void** ev_stop = nullptr;
  int32_t capacity = 0;
  int32_t count = 0;
};
extern ProfileHook g_prof;

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


#define QN_RANK_DISPATCH(r, CALL)                \
  switch (qn::rank_tiles(r)) {                   \
    case 1: { constexpr int JT = 1; CALL; break; }   \
    case 2: { constexpr int JT = 2; CALL; break; }   \
    case 4: { constexpr int JT = 4; CALL; break; }   \
    case 8: { constexpr int JT = 8; CALL; break; }   \
    default: { constexpr int JT = 16; CALL; break; } \
  }

template <typename T>
T* ws_at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// ---- gemm.hip: fused dequant + MFMA GEMM (Y = X W'^T + s T B^T or
// dX = dY W' + s G A), 256 x 256 or 128 x 128 tiles by size.
// drop (backward only): the adapter term s G A is multiplied elementwise by
// the dropout mask / (1 - p) before dY W' is added; nullptr for none.
//
// Ragged last wave: when the 256 x 256 tiles leave a last wave that fills
// only part of the GPU, each of its tiles is computed as two pieces over
// disjoint reduction ranges, a big one and a small one, sized so that the
// pieces fill the CUs about evenly (GemmSplit; no split with dropout).  The
// first piece to finish leaves its fp32 partial tile in `split_part`, the
// second adds it and stores the tile.  split_part holds rem * 256 * 256
// floats, split_cnt 2 * rem words that must be zero at launch (the second
// piece of each tile sets them back to zero).
struct GemmSplit {
  int whole, rem, ks;   // whole tiles, split tiles, reduction steps of the
                        // small piece (the big one takes the rest)
};
GemmSplit gemm_split_plan(int64_t M, int64_t nout, int64_t kred, bool drop);
size_t gemm_split_bytes(const GemmSplit& sp);   // partials + counters
size_t gemm_split_counters(const GemmSplit& sp); // byte offset of the counters

template <bool BWD>
void launch_gemm(hipStream_t st, const uint16_t* Aop, const nf4_tensor* w,
                 const uint16_t* La_hi, const uint16_t* La_lo,
                 const uint16_t* Lb, int M, int rpad, void* out, int out_bf16,
                 const DropArgs* drop = nullptr, void* split_ws = nullptr);

// ---- rank.hip: rank-r side products and their reductions.
enum { RS_ROWS = 1, RS_COLS = 2 };

struct StreamPlan {
  int rm, sub, mb, nb, cpb;
};
StreamPlan stream_plan(int mode, int64_t M, int64_t C, int jt);

// drop: LoRA dropout applied to S (= X) in the RS_ROWS and RS_COLS passes,
// or nullptr.
template <int MODE>
void launch_rank_stream(hipStream_t st, const char* kname, const StreamPlan& P,
                        const uint16_t* S, int M, int C, const uint16_t* R,
                        int r, const uint16_t* Uh, const uint16_t* Ul, int ldu,
                        float* prow, float* pcol,
                        const DropArgs* drop = nullptr);

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

FinishArgs finish_args();
void launch_finish(hipStream_t st, FinishArgs& a);

// ---- skinny.hip: forward for M <= 16 tokens.
struct SkinnyPlan {
  int slices, ks, rows_total, wg_rows;
};
SkinnyPlan skinny_plan(int64_t M, int64_t N, int64_t K, int r);
void launch_skinny(hipStream_t st, const uint16_t* x, int M,
                   const nf4_tensor* w, const uint16_t* A, const uint16_t* B,
                   int r, int rpad, float s, float* t_save, void* y,
                   int y_bf16, float* part);

}  // namespace qn
