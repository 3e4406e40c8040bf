// Skinny forward of the QLoRA linear layer (M <= 16 tokens): an HBM-bound
// GEMV over the NF4 weight with the adapter's T = X A^T in the same pass
// ("QLoRA Guide", Forward pass diagram; "QLORA ... paper summary", Notes:
// dequantize to BF16, multiply).
#include "qn_host.h"

namespace {

using namespace qn;

// ---------------------------------------------------------------------------
// K6: skinny forward (M <= 16 tokens): HBM-bound GEMV over the NF4 weight.
//
// Workgroup = 8 waves; wave w owns 16 consecutive "rows" of the weight-like
// operand: rows [0, N) are the NF4 weight W, rows [N, N + rpad) are the
// adapter's A (bf16), so T = X A^T comes out of the same pass.  Grid.y
// splits K into slices of KS columns; the workgroup stages its X slice
// (M rows, zero above M) in LDS once.  Per 256-column chunk, lane
// (n = l % 16, g = l / 16) loads the 32 packed bytes of block g of row n,
// builds that block's 16-entry bf16 LUT and decodes 8 weights per
// v_mfma_f32_16x16x32_bf16 step (t = 0..7 takes weights 8t..8t+7 of the
// block); the matching A operand is X[m][64 g + 8 t ...] from LDS.  The
// next chunk's weight bytes are loaded before the current chunk is decoded.
// A persistent workgroup takes a contiguous run of work items ordered
// slice-major, so its X slice stays in LDS across the row blocks of one
// slice.  Partial sums go to part[slice][m][row] (fp32, m < M), combined by
// k_skinny_reduce.
// ---------------------------------------------------------------------------

// Items [ib, ie) of this workgroup.  The grid is two workgroups per CU;
// workgroups b and b + gridDim.x / 2 (the same XCD, typically the same CU)
// split one CU's share of the items, and the CU shares differ by at most
// one item.
__device__ __forceinline__ void skinny_items(int nitems, int& ib, int& ie) {
  const int per = gridDim.x / 2;                 // CU slots
  const int b = blockIdx.x;
  const int c = b % per, h = b / per;
  const int cb = (int)((int64_t)c * nitems / per);
  const int ce = (int)((int64_t)(c + 1) * nitems / per);
  const int mid = cb + (ce - cb + 1) / 2;
  ib = h == 0 ? cb : mid;
  ie = h == 0 ? mid : ce;
}

struct SkRegs {
  u32x4 w0, w1;
  uint32_t q;
  float d;
};

__global__ __launch_bounds__(512) void k_skinny_partial(
    const uint16_t* __restrict__ X, int M, const uint8_t* __restrict__ packed,
    const uint8_t* __restrict__ qabs, const float* __restrict__ gscale,
    const uint16_t* __restrict__ A, int N, int K, int r, int rpad, int KS,
    int wg_rows, int nitems, float* __restrict__ part, Codebook cb) {
  // rows [0, N) weight, [N, Np16) zero padding, [Np16, Np16 + rpad) adapter
  const int Np16 = (N + 15) & ~15;
  const int rows_total = Np16 + rpad;
  const int XP = KS + 8;                       // sX pitch (bf16)
  extern __shared__ __attribute__((aligned(16))) uint16_t sX[];   // (M+1) x XP
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int64_t numel = (int64_t)N * K;
  const rsrc_t rp = make_rsrc(packed, (uint32_t)((numel + 1) >> 1));
  const rsrc_t rq = make_rsrc(qabs, (uint32_t)((numel + 63) >> 6));
  const rsrc_t rd = make_rsrc(gscale, (uint32_t)(((numel + 16383) >> 14) << 2));
  const rsrc_t ra = make_rsrc(A, (uint32_t)((int64_t)r * K * 2));
  const rsrc_t rx = make_rsrc(X, (uint32_t)((int64_t)M * K * 2));

  // work items (block of SK_ROWS rows, K slice), item = slice * wg_rows +
  // row block; this workgroup takes items [ib, ie)
  int ib, ie;
  skinny_items(nitems, ib, ie);
  for (int c = tid; c < KS / 8; c += 512)
    *reinterpret_cast<u32x4*>(sX + M * XP + 8 * c) = u32x4{0u, 0u, 0u, 0u};
  int staged = -1;                               // slice held in sX
  for (int item = ib; item < ie; ++item) {
    const int rb = item % wg_rows, slice = item / wg_rows;
    const int k0 = slice * KS;
    const int klen = min(KS, K - k0);
    const int row0 = rb * SK_ROWS + wave * 16;   // first row of the wave
    const int row = row0 + n;

    // X slice -> LDS (M rows, columns >= klen zero), each 8-element group
    // permuted into the order decode8p produces; loads issued before use.
    if (slice != staged) {
      if (staged >= 0) __syncthreads();          // sX still being read
      staged = slice;
      const int groups = M * (KS / 8);
      // batches of 4 loads per thread, all issued before their LDS writes
      for (int i0 = 0; i0 < groups; i0 += 4 * 512) {
        u32x4 xv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int idx = i0 + tid + 512 * i;
          const int m = idx / (KS / 8), c = 8 * (idx % (KS / 8));
          const bool ok = idx < groups && c < klen;
          xv[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
              rx, ok ? (uint32_t)(((int64_t)m * K + k0 + c) * 2) : G_OOB, 0, 0));
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
      __syncthreads();
    }

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (row0 < rows_total) {
      const bool is_w = row0 < Np16;             // wave-uniform
      // lanes whose A-operand row is >= M read the all-zero row M of sX
      const uint16_t* xrow = sX + (n < M ? n : M) * XP + 64 * g;
      auto load = [&](SkRegs& R, int kc) {
        const int k = k0 + kc + 64 * g;
        const int64_t e = (int64_t)row * K + k;
        const bool okw = is_w && kc + 64 * g < klen && row < N;
        const uint32_t op = okw ? (uint32_t)(e >> 1) : G_OOB;
        R.w0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, op, 0, 0));
        R.w1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, op + 16, 0, 0));
        R.q = __builtin_amdgcn_raw_buffer_load_b8(rq, okw ? (uint32_t)(e >> 6) : G_OOB, 0, 0);
        R.d = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
            rd, okw ? (uint32_t)((e >> 14) << 2) : G_OOB, 0, 0));
      };
      auto chunk = [&](const SkRegs& R, int kc) {
        u32x4 a[8];
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8)
          a[s8] = *reinterpret_cast<const u32x4*>(xrow + kc + 8 * s8);
        if (is_w) {
          const Lut t = make_lut(cb, static_cast<float>(R.q) * R.d);
          const uint32_t wd[8] = {R.w0.x, R.w0.y, R.w0.z, R.w0.w,
                                  R.w1.x, R.w1.y, R.w1.z, R.w1.w};
#pragma unroll
          for (int s8 = 0; s8 < 8; ++s8) acc = mfma16(a[s8], decode8p(wd[s8], t), acc);
        } else {
          const int j = row - Np16;
          const int k = k0 + kc + 64 * g;
          const bool ok = kc + 64 * g < klen && j < r;
#pragma unroll
          for (int s8 = 0; s8 < 8; ++s8) {
            const u32x4 b = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                ra, ok ? (uint32_t)(((int64_t)j * K + k + 8 * s8) * 2) : G_OOB, 0, 0));
            acc = mfma16(a[s8], permute8(b), acc);
          }
        }
      };
      // two register sets, loaded one chunk ahead, no copies between them
      // (the loop is VALU-bound on the decode; deeper prefetch measured no
      // faster)
      SkRegs ra0, ra1;
      load(ra0, 0);
      for (int kc = 0; kc < klen; kc += 512) {
        load(ra1, kc + 256);
        chunk(ra0, kc);
        if (kc + 256 >= klen) break;
        load(ra0, kc + 512);
        chunk(ra1, kc + 256);
      }
    }
    // acc[v] = C[m = 4 g + v][row n]
    if (row < rows_total) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = 4 * g + v;
        if (m < M) part[((int64_t)slice * M + m) * rows_total + row] = acc[v];
      }
    }
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

// Y[m][n] = sum_slices part[.][m][n] + s * sum_j T[m][j] B[n][j], and
// T[m][j] = sum_slices part[.][m][Np16 + j] (written to t_save by the
// blocks with blockIdx.x == 0).  Workgroup (bx, by) covers columns
// [64 bx, 64 bx + 64) of tokens [4 by, 4 by + 4), one output per thread.
__global__ __launch_bounds__(256) void k_skinny_reduce(
    const float* __restrict__ part, int slices, int M, int N, int r, int rpad,
    const uint16_t* __restrict__ B, float s, float* __restrict__ t_save,
    void* __restrict__ Y, int y_bf16) {
  __shared__ float sT[4 * QN_MAX_RANK];
  const int Np16 = (N + 15) & ~15;
  const int64_t rows_total = Np16 + rpad;
  const int64_t stride = (int64_t)M * rows_total;      // between slices
  const int mb = 4 * blockIdx.y;
  const int mrows = min(4, M - mb);
  for (int idx = threadIdx.x; idx < mrows * r; idx += 256) {
    const int m = mb + idx / r, j = idx % r;
    const float v = sum_slices(part + (int64_t)m * rows_total + Np16 + j, stride, slices);
    sT[idx] = v;
    if (blockIdx.x == 0) t_save[(int64_t)m * r + j] = v;
  }
  __syncthreads();
  const int n = blockIdx.x * 64 + (threadIdx.x & 63);
  const int mi = threadIdx.x >> 6;
  if (n >= N || mi >= mrows) return;
  const int m = mb + mi;
  const float y = sum_slices(part + (int64_t)m * rows_total + n, stride, slices);
  const float* t = sT + mi * r;
  const uint16_t* b = B + (int64_t)n * r;
  float lora = 0.f;
  if ((r & 7) == 0 && (reinterpret_cast<uintptr_t>(B) & 15) == 0) {
    // 16-byte aligned rows of B: 8 weights per load
    for (int j0 = 0; j0 < r; j0 += 8) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(b + j0);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        lora += t[j0 + 2 * h] * __uint_as_float(ww[h] << 16);
        lora += t[j0 + 2 * h + 1] * __uint_as_float(ww[h] & 0xFFFF0000u);
      }
    }
  } else {
    for (int jj = 0; jj < r; ++jj) lora += t[jj] * bf16_to_f32(b[jj]);
  }
  store_out(Y, y_bf16, (int64_t)m * N + n, y + s * lora);
}

}  // namespace

namespace qn {

void launch_skinny(hipStream_t st, const uint16_t* x, int M,
                   const nf4_tensor* w, const uint16_t* A, const uint16_t* B,
                   int r, int rpad, float s, float* t_save, void* y,
                   int y_bf16, float* part) {
  const int64_t N = w->rows, K = w->cols;
  const SkinnyPlan P = skinny_plan(M, N, K, r);
  const int nitems = P.wg_rows * P.slices;
  const size_t shm = size_t(M + 1) * (P.ks + 8) * 2;
  QN_LAUNCH_SHM("k_skinny_partial", k_skinny_partial,
                dim3((unsigned)(G_CUS * SK_WGS_PER_CU)),
                dim3(512), shm, st, x, M, w->packed, w->qabs, w->gscale, A,
                (int)N, (int)K, r, rpad, P.ks, P.wg_rows, nitems, part,
                qn::codebook());
  QN_LAUNCH("k_skinny_reduce", k_skinny_reduce,
            dim3((unsigned)cdiv(N, 64), (unsigned)cdiv(M, 4)), dim3(256), st,
            part, P.slices, M,
            (int)N, r, rpad, B, s, t_save, y, y_bf16);
}

}  // namespace qn
