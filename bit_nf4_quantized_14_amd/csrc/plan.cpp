// Host-side planning of the QLoRA NF4 library's fused calls: shape rules,
// GEMM tile choice and the split of a ragged last wave, the rank-r stream
// blocking, the skinny path's K slices, and the workspace layouts.  Plain
// C++ with no HIP dependency, so the plans can be checked on the host.
#include <algorithm>
#include <vector>

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
// halves of 2-90 tiles.  A grid of 128 x 128 tiles (fewer than 192 big
// tiles) with at most G_CUS tiles has every tile split, two such
// workgroups fitting on a CU (the 70B k/v forward, 128 tiles: 104 -> 71 us;
// four pieces per tile, a tree of exchanges, measured 75-78 us).  No split
// with dropout (its adapter term is masked before the main loop), and none
// for a reduction shorter than 8 steps.
GemmSplit gemm_split_plan(int64_t M, int64_t nout, int64_t kred, bool drop) {
  GemmSplit sp{0, 0, 0};
  if (drop || cdiv(kred, G_BK) < 8) return sp;
  if (gemm_big_tiles(M, nout)) {
    const int64_t tiles = cdiv(M, 256) * cdiv(nout, 256);
    const int64_t rem = tiles % G_CUS;
    if (rem == 0 || 2 * rem > G_CUS) return sp;
    return GemmSplit{(int)(tiles - rem), (int)rem, 256};
  }
  const int64_t tiles = cdiv(M, 128) * cdiv(nout, 128);
  if (tiles > G_CUS) return sp;
  return GemmSplit{0, (int)tiles, 128};
}

size_t gemm_split_part_offset(const GemmSplit& sp) {
  return align256(G_SPLIT_HDR + size_t(sp.rem) * 8);
}

size_t gemm_split_bytes(const GemmSplit& sp) {
  return gemm_split_part_offset(sp) + size_t(sp.rem) * sp.tile * sp.tile * 4;
}

StreamPlan stream_plan(int mode, int64_t M, int64_t C, int jt, bool drop) {
  StreamPlan P;
  P.rm = rs_rm(mode, jt, drop);
  P.sub = rs_sub(mode, jt, drop);
  P.mb = (int)cdiv(M, P.rm);
  const int64_t nst = cdiv(C, 64 * P.sub);
  const int64_t want =
      std::max<int64_t>(1, cdiv(int64_t(G_CUS) * rs_wgs_per_cu(mode, jt, drop), P.mb));
  const int64_t nb = std::min(nst, want);
  P.cpb = (int)cdiv(nst, nb);
  P.nb = (int)cdiv(nst, P.cpb);
  return P;
}


// Skinny path plan (the rule is stated where SkinnyPlan is declared).
// X tile budget (bytes); with two workgroups per CU the X tiles take at most
// 128 KB of a CU's 160 KB of LDS.
constexpr int64_t SK_LDS_PER_WG = 64 * 1024;

SkinnyPlan skinny_plan(int64_t M, int64_t N, int64_t K, int r,
                       int64_t want_tiles) {
  SkinnyPlan P;
  P.wtiles = (int)cdiv(N, 16);
  P.tps = P.wtiles + rank_tiles(r);
  P.rows_total = 16 * P.tps;
  const int64_t kchunks = cdiv(K, 256);
  int64_t ks_max = (SK_LDS_PER_WG / (2 * (M + 1)) - 8) / 256 * 256;
  ks_max = std::max<int64_t>(256, std::min<int64_t>(ks_max, SK_KS_MAX));
  const int64_t grid_waves = int64_t(SK_WAVES) * SK_WGS_PER_CU * G_CUS;
  const int64_t fewest = cdiv(K, ks_max);
  const int64_t want = cdiv(std::max<int64_t>(want_tiles, 1), P.tps);
  const int64_t cap = std::max(K / (cdiv(128 * M, 256) * 256), cdiv(grid_waves, P.tps));
  int64_t slices = std::max(fewest, std::min(want, cap));
  slices = std::min<int64_t>(slices, kchunks);
  const int64_t ks = cdiv(kchunks, slices) * 256;
  P.ks = (int)ks;
  P.slices = (int)cdiv(K, ks);
  return P;
}

void skinny_plan_batch(const SkinnyJob* jobs, int count, SkinnyPlan* out) {
  double total = 0;
  for (int i = 0; i < count; ++i)
    total += double(jobs[i].w->rows) * double(jobs[i].w->cols);
  for (int i = 0; i < count; ++i) {
    const double share = double(jobs[i].w->rows) * double(jobs[i].w->cols) / total;
    const int64_t want = (int64_t)(share * SK_BATCH_TILES + 0.999);
    out[i] = skinny_plan(jobs[i].M, jobs[i].w->rows, jobs[i].w->cols, jobs[i].r, want);
  }
}

int skinny_bounds(const SkinnyPlan* plans, const int64_t* K, int count,
                  int nslots, int32_t* bound) {
  std::vector<int64_t> tile0(count + 1, 0), cost0(count + 1, 0);
  for (int i = 0; i < count; ++i) {
    tile0[i + 1] = tile0[i] + int64_t(plans[i].tps) * plans[i].slices;
    cost0[i + 1] = cost0[i] + int64_t(plans[i].tps) * cdiv(K[i], 256);
  }
  const int64_t T = cost0[count];
  // first tile whose cost starts at or after x
  auto first_tile = [&](int64_t x) -> int64_t {
    if (x >= T) return tile0[count];
    int p = 0;
    while (p + 1 < count && cost0[p + 1] <= x) ++p;
    const SkinnyPlan& P = plans[p];
    const int64_t kc = P.ks / 256, kchunks = cdiv(K[p], 256);
    const int64_t full = int64_t(P.tps) * kc;              // cost of a slice
    const int64_t local = x - cost0[p];
    const int64_t s = std::min<int64_t>(local / full, P.slices - 1);
    const int64_t c = s < P.slices - 1 ? kc : kchunks - (P.slices - 1) * kc;
    const int64_t t = cdiv(local - s * full, c);
    return tile0[p] + s * P.tps + std::min<int64_t>(t, P.tps);
  };
  for (int c = 0; c <= nslots; ++c)
    bound[c] = (int32_t)first_tile(c * T / nslots);
  return (int)tile0[count];
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
    L.total = align256(skinny_part_bytes(M, P));
    return L;
  }
  // (a general layout also fits the T pass with dropout, whose plan has at
  // least as many column blocks)
  const StreamPlan P = stream_plan(RS_ROWS, M, K, rank_tiles(r), general);
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
  // the dA pass with dropout may have more row blocks
  const StreamPlan Pa = stream_plan(RS_COLS, M, K, jt, true);
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
