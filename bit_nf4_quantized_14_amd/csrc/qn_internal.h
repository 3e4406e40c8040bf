// Internal declarations shared by the host-side translation units of the
// QLoRA NF4 library.  Not part of the public C ABI.
#pragma once

#include <cstddef>
#include <cstdint>

namespace qn {

// 16 NF4 levels and 15 midpoint thresholds, derived on the host in double
// precision (codebook.cpp).
void derive_codebook(float levels[16], float thresholds[15]);

// Levels and thresholds of a QN_CODE_* table; false for an unknown table.
bool derive_variant_codebook(int code, float levels[16], float thresholds[15]);

// Workspace layouts of the fused calls (byte offsets, 256-byte aligned).
// rpad = r rounded up to 16, 32, 64, 128 or 256 (the adapter MFMA width).
// M <= QN_SKINNY_M takes the skinny (GEMV) forward.
constexpr int64_t QN_SKINNY_M = 16;

struct FwdWorkspace {
  size_t th, tl;    // bf16 [M, rpad]  hi/lo parts of s*T      (GEMM path)
  size_t bp;        // bf16 [N, rpad]  B zero-padded           (GEMM path)
  size_t prow;      // fp32 [nb, M, rpad] column-block partials of T
  size_t part;      // fp32 [slices, 16, rows] K-slice partials (skinny path)
  size_t split;     // partial tiles + counters of the GEMM's split last wave
  int32_t slices, ks;
  size_t total;
  int32_t rpad;
};

struct BwdWorkspace {
  size_t bt;        // bf16 [r, N]     B transposed
  size_t uth, utl;  // bf16 [r, Mp]    hi/lo parts of s*T, transposed
  size_t atp;       // bf16 [K, rpad]  A transposed, zero-padded
  size_t gh, gl;    // bf16 [M, rpad]  hi/lo parts of s*G, G = dY B
  size_t ugh, ugl;  // bf16 [r, Mp]    hi/lo parts of s*G, transposed
  size_t prow;      // fp32 [nb, M, rpad] column-block partials of G
  size_t pcol;      // fp32 [mb, max(N, K), rpad] row-block partials of dB, dA
  size_t split;     // partial tiles + counters of the dX GEMM's split last wave
  size_t total;
  int64_t mp;       // M rounded up to a multiple of 8
  int32_t rpad;
};

// general: the layout of the general path also for M <= QN_SKINNY_M (a
// forward with dropout never takes the skinny path).
FwdWorkspace fwd_workspace_layout(int64_t M, int64_t N, int64_t K, int32_t r,
                                  bool general);
BwdWorkspace bwd_workspace_layout(int64_t M, int64_t N, int64_t K, int32_t r);

}  // namespace qn
