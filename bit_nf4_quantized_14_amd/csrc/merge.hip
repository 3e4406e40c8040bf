// Dequantize-and-merge of the QLoRA NF4 library: W_merged = bf16(W' + s B A),
// the dense bf16 weight with the adapter folded in.  "Qlora Expert", When to
// Use and Common Pitfalls: merging the adapter into a dense model requires
// dequantizing the base, which materialises the full bf16 weight; "QLoRA
// Implementation Details (2025 Edition)", Step 7 (Merge & Save).  s = alpha/r
// as in the linear layer ("QLoRA Implementation Details", Step 4).
//
// One workgroup per 64 x 64 tile of W (256 threads; about 30 KB of LDS, so
// five workgroups share a CU and their phases overlap):
//  * each thread owns 16 consecutive weights of one row (a quarter of a
//    64-weight block): one 8-byte load of packed codes, its block code and
//    group scale, the block's bf16 LUT and two decode8;
//  * the rank-r product P = B_tile A_tile runs on v_mfma_f32_32x32x16_bf16:
//    the A tile (r x 128, zero past r) and the B tile (64 x r) are staged in
//    LDS, A read column-wise with ds_read_b64_tr_b16 (rows 16 banks apart);
//  * P goes through LDS into row order, and each thread forms
//    fma(s, P, W') in fp32 and rounds to bf16 (RNE) into an LDS output
//    tile, which is written out so that every store instruction covers
//    whole 128-byte row runs (non-temporal stores).
// HBM-bound: per weight 0.5 + 1/64 + 4/16384 bytes in and 2 bytes out, plus
// A (L2-resident, shared by every row tile) and B.
#include "qn_host.h"

namespace {

using namespace qn;

constexpr int MG_ROWS = 64, MG_COLS = 64, MG_THREADS = 256;
constexpr int MG_EPT = MG_ROWS * MG_COLS / MG_THREADS;   // weights per thread
static_assert(MG_EPT == 16, "two packed dwords per thread");

template <int JT>
struct MgCfg {
  static constexpr int RP = 16 * JT;          // r rounded up to the MFMA k
  static constexpr int AP = MG_COLS + 32;     // A tile pitch (bf16)
  static constexpr int BP = RP + 8;           // B tile pitch (bf16)
  static constexpr int PP = MG_COLS + 4;      // P tile pitch (fp32)
  static constexpr int OP = MG_COLS + 8;      // output tile pitch (bf16)
};

// Transposed B operand of v_mfma_f32_32x32x16_bf16 from a row-major LDS
// tile: lane l gets column col0 + l % 32 of rows row0 + 8 (l / 32) .. + 7.
// Each ds_read_b64_tr_b16 serves 4 rows: in every group of 16 lanes, lane
// q = 4j + p addresses row j, columns 4p .. 4p+3 of the group's 16 columns,
// and lane q receives column q of the 4 rows.
__device__ __forceinline__ u32x4 mg_read_colT(const uint16_t* t, int pitch,
                                              int row0, int col0, int lane) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const int grp = lane >> 4, q = lane & 15;
  const int row = row0 + 8 * (grp >> 1) + (q >> 2);
  const int col = col0 + 16 * (grp & 1) + 4 * (q & 3);
  const uint16_t* p0 = t + row * pitch + col;
  const uint16_t* p1 = p0 + 4 * pitch;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(const_cast<uint16_t*>(p0)));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(const_cast<uint16_t*>(p1)));
  u32x4 v;
  v.x = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
  v.y = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
  v.z = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
  v.w = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
  return v;
}

template <int JT>
__global__ __launch_bounds__(MG_THREADS) void k_merge(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ qabs,
    const float* __restrict__ gscale, const uint16_t* __restrict__ A,
    const uint16_t* __restrict__ B, int N, int K, int r, float s,
    uint16_t* __restrict__ out, Codebook cb) {
  using G = MgCfg<JT>;
  // the output tile reuses the A tile's storage: A is last read by the
  // MFMAs, which every wave has finished at the barrier after the P writes
  constexpr int AO = G::RP * G::AP > MG_ROWS * G::OP ? G::RP * G::AP
                                                      : MG_ROWS * G::OP;
  __shared__ __attribute__((aligned(16))) uint16_t sAO[AO];
  __shared__ __attribute__((aligned(16))) uint16_t sB[MG_ROWS * G::BP];
  __shared__ __attribute__((aligned(16))) float sP[MG_ROWS * G::PP];
  uint16_t* const sA = sAO;
  uint16_t* const sO = sAO;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave >> 1, wk = wave & 1;
  const int n0 = blockIdx.x * MG_ROWS, k0 = blockIdx.y * MG_COLS;
  const int64_t numel = (int64_t)N * K;

  // this thread's 16 weights: row n0 + rn, columns k0 + rc .. + 15
  const int rn = tid >> 2, rc = MG_EPT * (tid & 3);
  const bool mine = n0 + rn < N && k0 + rc < K;
  const int64_t e = (int64_t)(n0 + rn) * K + k0 + rc;
  const rsrc_t rp = make_rsrc(packed, (uint32_t)((numel + 1) >> 1));
  const rsrc_t rq = make_rsrc(qabs, (uint32_t)((numel + 63) >> 6));
  const rsrc_t rd = make_rsrc(gscale, (uint32_t)(((numel + 16383) >> 14) << 2));
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 wv = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
      rp, mine ? (uint32_t)(e >> 1) : G_OOB, 0, 0));
  const uint32_t qv = __builtin_amdgcn_raw_buffer_load_b8(
      rq, mine ? (uint32_t)(e >> 6) : G_OOB, 0, 0);
  const float dv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
      rd, mine ? (uint32_t)((e >> 14) << 2) : G_OOB, 0, 0));

  // A tile [RP][MG_COLS]: rows j < r of A [r][K], zero past r and past K
  const rsrc_t ra = make_rsrc(A, (uint32_t)((int64_t)r * K * 2));
  constexpr int ACH = MG_COLS / 8;                  // 16-byte chunks per row
  static_assert((G::RP * ACH) % MG_THREADS == 0 || G::RP * ACH < MG_THREADS,
                "A tile loads");
#pragma unroll
  for (int i0 = 0; i0 < G::RP * ACH; i0 += MG_THREADS) {
    const int i = i0 + tid, j = i / ACH, c = 8 * (i % ACH);
    if (j >= G::RP) break;
    const uint32_t off = (j < r && k0 + c < K)
                             ? (uint32_t)(((int64_t)j * K + k0 + c) * 2) : G_OOB;
    *reinterpret_cast<u32x4*>(sA + j * G::AP + c) = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0));
  }
  // B tile [64][RP]: rows n0.. of B [N][r], zero past r and past N
#pragma unroll
  for (int i0 = 0; i0 < MG_ROWS * G::RP; i0 += MG_THREADS) {
    const int i = i0 + tid, n = i / G::RP, j = i % G::RP;
    sB[n * G::BP + j] = (n0 + n < N && j < r) ? B[(int64_t)(n0 + n) * r + j]
                                              : (uint16_t)0;
  }
  __syncthreads();

  // P = B_tile A_tile: wave (wn, wk) owns rows 32 wn .., columns 32 wk ..
  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
#pragma unroll
  for (int sj = 0; sj < JT; ++sj) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(
        sB + (32 * wn + (lane & 31)) * G::BP + 16 * sj + 8 * (lane >> 5));
    acc = mfma32(a, mg_read_colT(sA, G::AP, 16 * sj, 32 * wk, lane), acc);
  }
  // acc[v] = P[row 32 wn + 8 (v / 4) + 4 (l / 32) + v % 4][col 32 wk + l % 32]
#pragma unroll
  for (int v = 0; v < 16; ++v)
    sP[(32 * wn + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3)) * G::PP +
       32 * wk + (lane & 31)] = acc[v];
  __syncthreads();

  if (mine) {
    const Lut lut = make_lut(cb, static_cast<float>(qv) * dv);
    const uint32_t wd[2] = {wv.x, wv.y};
    const float* prow = sP + rn * G::PP + rc;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const u32x4 wb = decode8(wd[g], lut);    // 8 dequantized bf16 weights
      const uint32_t wp[4] = {wb.x, wb.y, wb.z, wb.w};
      u32x4 res;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float p0 = prow[8 * g + 2 * h], p1 = prow[8 * g + 2 * h + 1];
        const float v0 = fmaf(s, p0, bf16_to_f32(wp[h] & 0xFFFFu));
        const float v1 = fmaf(s, p1, bf16_to_f32(wp[h] >> 16));
        res[h] = pack_bf16x2(v0, v1);
      }
      *reinterpret_cast<u32x4*>(sO + rn * G::OP + rc + 8 * g) = res;
    }
  }
  __syncthreads();
  // write-out in store order: each wave instruction covers 8 rows x 128
  // contiguous bytes (16-byte chunk q of the tile is row q / ACH, column
  // chunk q % ACH), non-temporal
#pragma unroll
  for (int i = 0; i < MG_ROWS * ACH / MG_THREADS; ++i) {
    const int q = tid + MG_THREADS * i, row = q / ACH, c = 8 * (q % ACH);
    if (n0 + row < N && k0 + c < K)
      __builtin_nontemporal_store(
          *reinterpret_cast<const u32x4*>(sO + row * G::OP + c),
          reinterpret_cast<u32x4*>(out + (int64_t)(n0 + row) * K + k0 + c));
  }
}

}  // namespace

extern "C" {

int nf4_merge(const nf4_tensor* w, const uint16_t* A, const uint16_t* B,
              int32_t r, float alpha, uint16_t* w_merged, void* stream) {
  if (!valid_tensor(w) || A == nullptr || B == nullptr ||
      w_merged == nullptr || !aligned16(A) || !aligned16(w_merged))
    return QN_EINVAL;
  if (r < 1 || r > QN_MAX_RANK) return QN_EINVAL;
  const int64_t N = w->rows, K = w->cols;
  if (K % QN_BLOCK != 0) return QN_EINVAL;
  const int64_t lim = 1LL << 31;
  if (N > (1LL << 30) || K > (1LL << 30) || N * K / 2 >= lim ||
      (int64_t)r * K * 2 >= lim)
    return QN_EINVAL;
  const float s = alpha / (float)r;
  hipStream_t st = (hipStream_t)stream;
  if (cdiv(K, MG_COLS) > 65535) return QN_EINVAL;      // grid.y limit
  const dim3 grid((unsigned)cdiv(N, MG_ROWS), (unsigned)cdiv(K, MG_COLS));
  QN_RANK_DISPATCH(r, QN_LAUNCH("k_merge", k_merge<JT>, grid, dim3(MG_THREADS),
                                st, w->packed, w->qabs, w->gscale, A, B, (int)N,
                                (int)K, (int)r, s, w_merged, codebook()));
  return check_launch();
}

}  // extern "C"
