// Internal declarations shared by the host-side translation units of the
// QLoRA NF4 library.  Not part of the public C ABI.
#pragma once

#include <cstddef>
#include <cstdint>

namespace qn {

// 16 NF4 levels and 15 midpoint thresholds, derived on the host in double
// precision (codebook.cpp).
void derive_codebook(float levels[16], float thresholds[15]);

// Workspace layout of the backward pass (byte offsets, 256-byte aligned).
struct BwdWorkspace {
  size_t bt;        // bf16 [r, N]   B transposed
  size_t g;         // fp32 [M, r]   G = dY B
  size_t part_db;   // fp32 [chunks, N, r] split-M partials of dY^T T
  size_t part_da;   // fp32 [chunks, K, r] split-M partials of G^T X
  size_t total;
  int64_t chunks;   // number of M chunks
};

BwdWorkspace bwd_workspace_layout(int64_t M, int64_t N, int64_t K, int32_t r);

}  // namespace qn
