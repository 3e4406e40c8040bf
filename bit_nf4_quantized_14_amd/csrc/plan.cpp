// Host-side planning of the QLoRA NF4 library's fused calls: shape rules,
// GEMM tile choice and the split of a ragged last wave, the rank-r stream
// blocking, the skinny path's K slices, and the workspace layouts.  Plain
// C++ with no HIP dependency, so the plans can be checked on the host.
#include <algorithm>

#include "qn_internal.h"

namespace qn {

bool valid_linear(int64_t M, const nf4_tensor* w, int32_t r) {
  if (!valid_tensor(w) || M <= 0) return false;
  if (r < 1 || r > QN_MAX_RANK) return false;
  const int64_t N = w->rows, K = w->cols;
  if (K % QN_BLOCK != 0 || N % 8 != 0) return false;
  // 32-bit index arithmetic inside the GEMM kernels
  if (M > (1LL << 30) || N > (1LL << 30) || K > (1LL << 30)) return false;
  // buffer-resource ranges are 32-bit byte counts (offsets past 2^31 mean
  // "out of range"): every operand read through one stays below 2 GiB
  const int64_t lim = 1LL << 31;
  if (M * K * 2 >= lim || M * N * 2 >= lim || N * K / 2 >= lim) return false;
  // fp32 rank-r partial rows [N or K][rpad] addressed through a resource
  if (std::max(N, K) * 4 * 16 * rank_tiles(r) >= lim) return false;
  return true;
}

// Fused GEMM launch: 256 x 256 tiles when they give at least ~one
// workgroup per CU, otherwise 128 x 128.
bool gemm_big_tiles(int64_t M, int64_t nout) {
  return cdiv(M, 256) * cdiv(nout, 256) >= 192;
}

// Split of the ragged last wave: with R <= G_CUS / 2 tiles left, each of
// them becomes two pieces over half the reduction each, 2 R workgroups that
// all run at once.  With more tiles left the split does not pay: a wave
// that leaves CUs idle runs its tiles at a higher clock (the package is
// power-limited), and splitting 174-176 of 256 into a 3/4 and a 1/4 piece
// measured 3-5% slower than leaving them whole, against 6-13% faster for
// halves of 2-90 tiles.  No split with dropout either (its adapter term is
// masked before the main loop).
GemmSplit gemm_split_plan(int64_t M, int64_t nout, int64_t kred, bool drop) {
  GemmSplit sp{0, 0, 0};
  if (drop || !gemm_big_tiles(M, nout)) return sp;
  const int64_t tiles = cdiv(M, 256) * cdiv(nout, 256);
  const int64_t rem = tiles % G_CUS;
  if (rem == 0 || 2 * rem > G_CUS) return sp;
  const int64_t nsteps = cdiv(kred, G_BK);
  const int64_t ks = (nsteps / 2) & ~int64_t(1);
  if (ks < 2 || nsteps - ks < 2) return sp;
  sp.whole = (int)(tiles - rem);
  sp.rem = (int)rem;
  sp.ks = (int)ks;
  return sp;
}

size_t gemm_split_part_offset(const GemmSplit& sp) {
  return align256(G_SPLIT_HDR + size_t(sp.rem) * 8);
}

size_t gemm_split_bytes(const GemmSplit& sp) {
  return gemm_split_part_offset(sp) + size_t(sp.rem) * 256 * 256 * 4;
}

StreamPlan stream_plan(int mode, int64_t M, int64_t C, int jt) {
  StreamPlan P;
  P.rm = rs_rm(mode, jt);
  P.sub = rs_sub(mode, jt);
  P.mb = (int)cdiv(M, P.rm);
  const int64_t nst = cdiv(C, 64 * P.sub);
  const int64_t want = std::max<int64_t>(1, cdiv(256, P.mb));
  const int64_t nb = std::min(nst, want);
  P.cpb = (int)cdiv(nst, nb);
  P.nb = (int)cdiv(nst, P.cpb);
  return P;
}


// Skinny path plan: K slices of ks columns (multiple of 256, short enough
// that the X slice leaves LDS room for two workgroups per CU), and enough
// slices for ~2 items per workgroup.  The grid is two workgroups per CU
// whatever the item count; the items are split so that the CUs' shares
// differ by at most one item (skinny_items).
constexpr int64_t SK_LDS_PER_WG = 64 * 1024;   // X tile budget (bytes)

SkinnyPlan skinny_plan(int64_t M, int64_t N, int64_t K, int r) {
  SkinnyPlan P;
  P.rows_total = (int)(((N + 15) & ~15LL) + 16 * rank_tiles(r));
  P.wg_rows = (int)cdiv(P.rows_total, SK_ROWS);
  const int64_t kchunks = cdiv(K, 256);
  // longest slice whose X tile ((M + 1) rows, zero row included) leaves room
  // for two workgroups per CU, and enough slices for ~2 items per workgroup
  int64_t ks_max = (SK_LDS_PER_WG / (2 * (M + 1)) - 8) / 256 * 256;
  ks_max = std::max<int64_t>(256, std::min<int64_t>(ks_max, SK_KS_MAX));
  int64_t slices = std::max<int64_t>(cdiv(K, ks_max),
                                     cdiv((int64_t)G_CUS * SK_WGS_PER_CU * 2, P.wg_rows));
  slices = std::min<int64_t>(slices, kchunks);
  const int64_t ks = cdiv(kchunks, slices) * 256;
  P.ks = (int)ks;
  P.slices = (int)cdiv(K, ks);
  return P;
}

FwdWorkspace fwd_workspace_layout(int64_t M, int64_t N, int64_t K,
                                  int32_t r, bool general, bool split) {
  FwdWorkspace L{};
  L.rpad = 16 * rank_tiles(r);
  if (M <= qn::QN_SKINNY_M && !general) {
    const SkinnyPlan P = skinny_plan(M, N, K, r);
    L.slices = P.slices;
    L.ks = P.ks;
    L.part = 0;
    L.total = align256(size_t(P.slices) * M * P.rows_total * 4);
    return L;
  }
  const StreamPlan P = stream_plan(RS_ROWS, M, K, rank_tiles(r));
  size_t off = 0;
  L.split = off;   // status word first
  off += align256(gemm_split_bytes(split ? gemm_split_plan(M, N, K, false)
                                         : GemmSplit{0, 0, 0}));
  L.th = off;
  off += align256(size_t(M) * L.rpad * 2);
  L.tl = off;
  off += align256(size_t(M) * L.rpad * 2);
  L.bp = off;
  off += align256(size_t(N) * L.rpad * 2);
  L.prow = off;
  off += align256(size_t(P.nb) * M * L.rpad * 4);
  L.total = off;
  return L;
}

BwdWorkspace bwd_workspace_layout(int64_t M, int64_t N, int64_t K,
                                  int32_t r) {
  BwdWorkspace L{};
  const int jt = rank_tiles(r);
  L.rpad = 16 * jt;
  L.mp = cdiv(M, 8) * 8;
  const StreamPlan Pg = stream_plan(RS_ROWS | RS_COLS, M, N, jt);
  const StreamPlan Pa = stream_plan(RS_COLS, M, K, jt);
  const size_t pcol = std::max(size_t(Pg.mb) * N, size_t(Pa.mb) * K);
  size_t off = 0;
  L.split = off;   // status word first
  off += align256(gemm_split_bytes(gemm_split_plan(M, K, N, false)));
  L.bt = off;
  off += align256(size_t(r) * N * 2);
  L.uth = off;
  off += align256(size_t(r) * L.mp * 2);
  L.utl = off;
  off += align256(size_t(r) * L.mp * 2);
  L.atp = off;
  off += align256(size_t(K) * L.rpad * 2);
  L.gh = off;
  off += align256(size_t(M) * L.rpad * 2);
  L.gl = off;
  off += align256(size_t(M) * L.rpad * 2);
  L.ugh = off;
  off += align256(size_t(r) * L.mp * 2);
  L.ugl = off;
  off += align256(size_t(r) * L.mp * 2);
  L.prow = off;
  off += align256(size_t(Pg.nb) * M * L.rpad * 4);
  L.pcol = off;
  off += align256(pcol * L.rpad * 4);
  L.total = off;
  return L;
}

}  // namespace qn
