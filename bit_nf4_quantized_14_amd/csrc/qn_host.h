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


inline int check_launch() {
  return hipGetLastError() == hipSuccess ? QN_OK : QN_EHIP;
}


// Kernel launch.  The library built with QN_PROFILE_HOOK (the profiling
// variant, libqlora_nf4_prof.so) can record HIP events around the launches
// of one named kernel (qn_profile_kernel); the default build has no such
// state and launches directly.
#ifdef QN_PROFILE_HOOK
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
#else
#define QN_LAUNCH_SHM(kname, kernel, grid, block, shm, st, ...) \
  hipLaunchKernelGGL(kernel, grid, block, shm, st, __VA_ARGS__)
#endif
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
template <bool BWD>
void launch_gemm(hipStream_t st, const uint16_t* Aop, const nf4_tensor* w,
                 const uint16_t* La_hi, const uint16_t* La_lo,
                 const uint16_t* Lb, int M, int rpad, void* out, int out_bf16,
                 const DropArgs* drop = nullptr, void* split_ws = nullptr);

// ---- rank.hip: rank-r side products and their reductions.

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

// ---- skinny.hip: forward for M <= 16 tokens, a batch of up to
// QN_FWD_BATCH_MAX projections in one launch pair; ws holds each
// projection's partial sums (skinny_part_bytes, 256-byte aligned, in order).
void launch_skinny(hipStream_t st, const SkinnyJob* jobs, int count,
                   const SkinnyPlan* plans, char* ws);

}  // namespace qn
