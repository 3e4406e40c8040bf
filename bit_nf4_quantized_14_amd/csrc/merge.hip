// Dequantize-and-merge of the QLoRA NF4 library: W_merged = bf16(W' + s B A),
// the dense bf16 weight with the adapter folded in.  "Qlora Expert", When to
// Use and Common Pitfalls: merging the adapter into a dense model requires
// dequantizing the base, which materialises the full bf16 weight; "QLoRA
// Implementation Details (2025 Edition)", Step 7 (Merge & Save).  s = alpha/r
// as in the linear layer ("QLoRA Implementation Details", Step 4).
//
// Tiles of 64 x 64 weights, numbered row block by row block; each of a
// fixed grid of workgroups (256 threads, four per CU) takes a contiguous
// run of them and loads the codes, constants and A tile of the tile two
// ahead into registers while it works on the current one.  Per tile:
//  * the rank-r product runs on v_mfma_f32_32x32x16_bf16 as P^T = A^T B^T,
//    the A tile (r x 64, zero past r) read column-wise from LDS with
//    ds_read_b64_tr_b16, the B tile (64 x r, reloaded only when the row
//    block changes) row-wise; lane l of wave (wn, wk) ends up with P at row
//    32 wn + l % 32, columns 32 wk + 8 m + 4 h + 0..3 (m = 0..3, h = l / 32);
//  * the thread dequantizes exactly those 16 weights (half of each packed
//    dword of its row's 32-weight run, one block LUT, two decode8), forms
//    fma(s, P, W') in fp32 and rounds to bf16 (RNE) into an LDS output
//    tile, which is written out so that every store instruction covers
//    whole 128-byte row runs (non-temporal stores).
// HBM-bound: per weight 0.5 + 1/64 + 4/16384 bytes in and 2 bytes out, plus
// A (L2-resident, shared by every row tile) and B.
#include "qn_host.h"

namespace {

using namespace qn;

constexpr int MG_ROWS = 64, MG_COLS = 64, MG_THREADS = 256;
constexpr int MG_WGS_PER_CU = 4;     // grid: this many workgroups per CU
constexpr int MG_NT = 2;             // cache policy of the output stores: non-temporal
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

// 8 codes (one packed dword, element i in bits 4i..4i+3) -> the fp32 values
// of their 8 bf16 table entries, in natural order.  The same table lookups
// as decode8; each fp32 word is then one v_perm of the entry's two bytes
// over two zero bytes, instead of interleaving bf16 pairs and widening them.
__device__ __forceinline__ void decode8_f32(uint32_t p, const Lut& t, float (&f)[8]) {
  const uint32_t se = p & 0x07070707u;
  const uint32_t so = (p >> 4) & 0x07070707u;
  const uint32_t me = perm(p << 4, p << 12, 0x0B090A08u);
  const uint32_t mo = perm(p, p << 8, 0x0B090A08u);
  // byte k: low / high byte of element 2k (e) or 2k + 1 (o)
  const uint32_t le = bfi(me, perm(t.lh1, t.lh0, se), perm(t.ll1, t.ll0, se));
  const uint32_t he = bfi(me, perm(t.hh1, t.hh0, se), perm(t.hl1, t.hl0, se));
  const uint32_t lo = bfi(mo, perm(t.lh1, t.lh0, so), perm(t.ll1, t.ll0, so));
  const uint32_t ho = bfi(mo, perm(t.hh1, t.hh0, so), perm(t.hl1, t.hl0, so));
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    // bytes: zero, zero, low byte k of src1, high byte k of src0 (4 + k)
    const uint32_t sel = 0x0C0Cu | ((uint32_t)k << 16) | ((uint32_t)(4 + k) << 24);
    f[2 * k] = __uint_as_float(perm(he, le, sel));
    f[2 * k + 1] = __uint_as_float(perm(ho, lo, sel));
  }
}

// Global loads of one tile that do not depend on the previous one: the 16
// packed bytes of this thread's row half-block (it decodes half of them),
// its block code and group scale, and its chunks of the A tile [RP][MG_COLS]
// (rows j < r of A [r][K], zero past r).
template <int JT>
struct MgLoads {
  static constexpr int ACH = MG_COLS / 8;                 // 16-byte chunks per row
  static constexpr int NA = (16 * JT * ACH + MG_THREADS - 1) / MG_THREADS;
  u32x4 w;
  uint32_t q;
  float d;
  u32x4 a[NA];
};

template <int JT>
__global__ __launch_bounds__(MG_THREADS) void k_merge(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ qabs,
    const float* __restrict__ gscale, const uint16_t* __restrict__ A,
    const uint16_t* __restrict__ B, int N, int K, int r, float s, int tiles_k,
    int ntiles, uint16_t* __restrict__ out, Codebook cb) {
  using G = MgCfg<JT>;
  using L = MgLoads<JT>;
  __shared__ __attribute__((aligned(16))) uint16_t sA[G::RP * G::AP];
  __shared__ __attribute__((aligned(16))) uint16_t sB[MG_ROWS * G::BP];
  __shared__ __attribute__((aligned(16))) uint16_t sO[MG_ROWS * G::OP];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave >> 1, wk = wave & 1;
  const int64_t numel = (int64_t)N * K;
  const rsrc_t rd = make_rsrc(gscale, (uint32_t)(((numel + 16383) >> 14) << 2));
  const rsrc_t rb = make_rsrc(B, (uint32_t)((int64_t)N * r * 2));
  // The MFMA gives lane l the products of row 32 wn + l % 32 of the tile at
  // columns 32 wk + 8 m + 4 h + t (m, t = 0..3, h = l / 32): this thread
  // dequantizes and writes exactly those 16 weights.
  const int rn = 32 * wn + (lane & 31), h = lane >> 5;
  constexpr int ACH = L::ACH;

  // this workgroup's run of tiles
  const int tb = (int)((int64_t)blockIdx.x * ntiles / gridDim.x);
  const int te = (int)((int64_t)(blockIdx.x + 1) * ntiles / gridDim.x);

  // Offsets inside a tile, the same for every tile: each tile's loads go
  // through resources based at the tile's first row and column whose range
  // ends after its last row below N (rows past N read zeros), and past the
  // run through zero-sized ones, so a lane's offsets are constants.
  const uint32_t ow = (uint32_t)rn * (uint32_t)(K / 2) + 16u * (uint32_t)wk;
  const uint32_t oq = (uint32_t)rn * (uint32_t)(K / 64);
  const uint32_t oe = (uint32_t)rn * (uint32_t)K;    // element index of the row
  uint32_t oa[L::NA];
#pragma unroll
  for (int u = 0; u < L::NA; ++u) {
    const int i = tid + MG_THREADS * u, j = i / ACH, c = 8 * (i % ACH);
    oa[u] = (j < r && i < G::RP * ACH) ? (uint32_t)((j * K + c) * 2) : G_OOB;
  }
  // lanes l and l + 32 dequantize the same block and build its table together
  const LutHalf lh = lut_half32(cb, lane);

  // Loads of tile t (every tile issues the same vector memory instructions).
  auto load = [&](L& ld, int t) {
    const bool live = t < te;
    const int n0 = (t / tiles_k) * MG_ROWS, k0 = (t % tiles_k) * MG_COLS;
    const int rows = min(MG_ROWS, N - n0);
    const uint32_t e0 = (uint32_t)n0 * (uint32_t)K + (uint32_t)k0;
    const rsrc_t tp = make_rsrc(packed + e0 / 2,
                                live ? ((uint32_t)(rows - 1) * (uint32_t)K + 64u) / 2 : 0u);
    const rsrc_t tq = make_rsrc(qabs + e0 / 64,
                                live ? (uint32_t)(rows - 1) * (uint32_t)(K / 64) + 1u : 0u);
    const rsrc_t ta = make_rsrc(A + k0, live ? (uint32_t)(((r - 1) * K + MG_COLS) * 2) : 0u);
    ld.w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(tp, ow, 0, 0));
    ld.q = __builtin_amdgcn_raw_buffer_load_b8(tq, oq, 0, 0);
    // group scale: the groups of 16384 weights do not follow the tiles
    ld.d = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
        live ? rd : make_rsrc(gscale, 0u), ((oe + e0) >> 14) << 2, 0, 0));
#pragma unroll
    for (int u = 0; u < L::NA; ++u)
      ld.a[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
          ta, oa[u], 0, 0));
  };

  int b_n0 = -1;                                  // row block of the B tile in LDS
  // Tile t from the loads in `cur`; the loads of tile t + 2 go into `ahead`.
  auto step = [&](int t, const L& cur, L& ahead) {
    const int n0 = (t / tiles_k) * MG_ROWS, k0 = (t % tiles_k) * MG_COLS;
    if (n0 != b_n0) {
      // B tile [64][RP]: rows n0.. of B [N][r], zero past r and past N
      // (once per row block of the run)
      b_n0 = n0;
      constexpr int NB = MG_ROWS * G::RP / MG_THREADS;
      uint16_t bv[NB];
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int i = tid + MG_THREADS * u, n = i / G::RP, j = i % G::RP;
        bv[u] = __builtin_amdgcn_raw_buffer_load_b16(
            rb, (n0 + n < N && j < r) ? (uint32_t)(((int64_t)(n0 + n) * r + j) * 2)
                                      : G_OOB, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int i = tid + MG_THREADS * u, n = i / G::RP, j = i % G::RP;
        sB[n * G::BP + j] = bv[u];
      }
    }
#pragma unroll
    for (int u = 0; u < L::NA; ++u) {
      const int i = tid + MG_THREADS * u, j = i / ACH, c = 8 * (i % ACH);
      if (i < G::RP * ACH) *reinterpret_cast<u32x4*>(sA + j * G::AP + c) = cur.a[u];
    }
    __syncthreads();   // A and B tiles written; the last tile's sO read out
    load(ahead, t + 2);

    // P^T = A_tile^T B_tile^T: acc[v] = P[row rn][col 32 wk + 8 (v / 4) +
    // 4 h + v % 4]
    f32x16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
#pragma unroll
    for (int sj = 0; sj < JT; ++sj) {
      const u32x4 b = *reinterpret_cast<const u32x4*>(
          sB + (32 * wn + (lane & 31)) * G::BP + 16 * sj + 8 * h);
      acc = mfma32(mg_read_colT(sA, G::AP, 16 * sj, 32 * wk, lane), b, acc);
    }

    // codes of columns 32 wk + 8 m + 4 h .. + 3: half h of packed dword m
    const uint32_t sel = h ? 0x07060302u : 0x05040100u;
    const uint32_t wd[2] = {__builtin_amdgcn_perm(cur.w.y, cur.w.x, sel),
                            __builtin_amdgcn_perm(cur.w.w, cur.w.z, sel)};
    const Lut lut = make_lut_swap32(lh, static_cast<float>(cur.q) * cur.d);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      // 8 dequantized weights: columns 8 (2 g) + 4 h + 0..3, then 8 (2 g + 1) + ...
      float wf[8];
      decode8_f32(wd[g], lut, wf);
      uint32_t res[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int v = 8 * g + 2 * i;             // acc index of the pair
        const float v0 = fmaf(s, acc[v], wf[2 * i]);
        const float v1 = fmaf(s, acc[v + 1], wf[2 * i + 1]);
        res[i] = pack_bf16x2(v0, v1);
      }
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      uint16_t* o = sO + rn * G::OP + 32 * wk + 16 * g + 4 * h;
      *reinterpret_cast<u32x2*>(o) = u32x2{res[0], res[1]};
      *reinterpret_cast<u32x2*>(o + 8) = u32x2{res[2], res[3]};
    }
    __syncthreads();   // the output tile is complete
    // write-out in store order: each wave instruction covers 8 rows x 128
    // contiguous bytes (16-byte chunk q of the tile is row q / ACH, column
    // chunk q % ACH), non-temporal; the resource ends after the tile's last
    // row below N, so rows past N fall out of range
    const int rows = min(MG_ROWS, N - n0);
    const rsrc_t ro = make_rsrc(out + (int64_t)n0 * K + k0,
                                (uint32_t)(((rows - 1) * K + MG_COLS) * 2));
#pragma unroll
    for (int i = 0; i < MG_ROWS * ACH / MG_THREADS; ++i) {
      const int q = tid + MG_THREADS * i, row = q / ACH, c = 8 * (q % ACH);
      __builtin_amdgcn_raw_buffer_store_b128(
          *reinterpret_cast<const u32x4*>(sO + row * G::OP + c), ro,
          (uint32_t)((row * K + c) * 2), 0, MG_NT);
    }
  };

  // Three register sets in rotation (no copies between them, so the waits
  // before a tile's first use of its loads leave the next tile's in flight).
  L L0, L1, L2;
  load(L0, tb);
  load(L1, tb + 1);
  int t = tb;
  for (; t + 3 <= te; t += 3) {
    step(t, L0, L2);
    step(t + 1, L1, L0);
    step(t + 2, L2, L1);
  }
  if (t < te) step(t, L0, L2);
  if (t + 1 < te) step(t + 1, L1, L0);
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
  const int64_t tiles_k = K / MG_COLS, ntiles = cdiv(N, MG_ROWS) * tiles_k;
  if (ntiles > 0x7FFFFFFFLL) return QN_EINVAL;
  const unsigned grid = (unsigned)std::min<int64_t>(ntiles, MG_WGS_PER_CU * G_CUS);
  QN_RANK_DISPATCH(r, QN_LAUNCH("k_merge", k_merge<JT>, dim3(grid), dim3(MG_THREADS),
                                st, w->packed, w->qabs, w->gscale, A, B, (int)N,
                                (int)K, (int)r, s, (int)tiles_k, (int)ntiles,
                                w_merged, codebook()));
  return check_launch();
}

}  // extern "C"
