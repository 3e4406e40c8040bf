// Host check of the library's planning code (csrc/plan.cpp), built with
// address and undefined-behaviour sanitizers by tests/test_host_sanitizers.py.
//
// * gemm_split_plan: no split with dropout or under 8 reduction steps; with
//   256 x 256 tiles the tiles of a last wave of 1..128 tiles (whole + rem
//   is the tile count, whole a multiple of 256); with 128 x 128 tiles every
//   tile of a grid of at most 256; both pieces get an even number (>= 4) of
//   64-wide reduction steps; known shapes give the documented plans.
// * the split area: status word, 8-byte padding, 2 counter words per split
//   tile, partial tiles 256-byte aligned after them.
// * workspace layouts: every region 256-byte aligned, inside the total, no
//   two regions overlapping, each at least as large as its contents, the
//   split area at offset 0.
// * stream_plan and skinny_plan cover every row and column, and the skinny X
//   slice fits its LDS budget.
// * skinny_bounds: the slots' tile runs are contiguous, cover every tile, and
//   each slot starts at the first tile whose cost starts at or after its
//   share of the total (checked against a walk over every tile).
#include <algorithm>
#include <cstdio>
#include <vector>

#include "qn_internal.h"

using namespace qn;

static int bad = 0;

static void check(bool ok, const char* what, long long a = 0, long long b = 0,
                  long long c = 0) {
  if (!ok) {
    std::fprintf(stderr, "FAIL %s (%lld, %lld, %lld)\n", what, a, b, c);
    bad = 1;
  }
}

struct Region {
  size_t off, bytes;
};

static void check_regions(std::vector<Region> v, size_t total, const char* what,
                          long long M, long long N, long long K) {
  for (size_t i = 0; i < v.size(); ++i) {
    check(v[i].off % 256 == 0, what, M, N, K);
    check(v[i].off + v[i].bytes <= total, what, M, N, K);
    for (size_t j = i + 1; j < v.size(); ++j) {
      const bool disjoint = v[i].off + v[i].bytes <= v[j].off ||
                            v[j].off + v[j].bytes <= v[i].off;
      check(disjoint || v[i].bytes == 0 || v[j].bytes == 0, what, M, N, K);
    }
  }
}

static void split_plan_sweep() {
  const long long Ms[] = {1, 17, 255, 256, 257, 1536, 2048, 2050, 3072, 4096, 8192};
  const long long Ns[] = {8, 1024, 1032, 4096, 8200, 8448, 11008, 28672};
  const long long Ks[] = {64, 128, 192, 1088, 4096, 8256, 11008, 28672};
  for (long long M : Ms)
    for (long long n : Ns)
      for (long long k : Ks) {
        for (int drop = 0; drop < 2; ++drop) {
          const GemmSplit sp = gemm_split_plan(M, n, k, drop != 0);
          const bool big = gemm_big_tiles(M, n);
          const long long tiles = big ? cdiv(M, 256) * cdiv(n, 256)
                                      : cdiv(M, 128) * cdiv(n, 128);
          const long long nsteps = cdiv(k, G_BK);
          if (sp.rem == 0) {
            check(sp.whole == 0, "no-split plan not empty", M, n, k);
            // when a split would apply it is taken
            const long long rem = tiles % G_CUS;
            const bool could = !drop && nsteps >= 8 &&
                               (big ? rem > 0 && 2 * rem <= G_CUS : tiles <= G_CUS);
            check(!could, "split not taken", M, n, k);
            continue;
          }
          check(!drop && nsteps >= 8, "split with dropout or a short reduction", M, n, k);
          if (big) {
            check(sp.tile == 256, "big-tile split edge", M, n, k);
            check(sp.whole + sp.rem == tiles, "whole + rem != tiles", M, n, k);
            check(sp.whole % G_CUS == 0, "whole not a multiple of the CUs", M, n, k);
            check(sp.rem >= 1 && 2 * sp.rem <= G_CUS, "rem out of range", M, n, k);
          } else {
            check(sp.tile == 128, "small-tile split edge", M, n, k);
            check(sp.whole == 0 && sp.rem == tiles && tiles <= G_CUS,
                  "small grid not split whole", M, n, k);
          }
          // the two pieces: [0, h) and [h, nsteps), h even, both >= 4 steps
          const long long h = (nsteps / 2) & ~1LL;
          check(h >= 4 && nsteps - h >= 4, "piece shorter than four steps", M, n, k);
          const size_t part = gemm_split_part_offset(sp);
          check(part % 256 == 0 && part >= G_SPLIT_HDR + 8 * size_t(sp.rem),
                "partials overlap the counters", M, n, k);
          check(gemm_split_bytes(sp) ==
                    part + size_t(sp.rem) * sp.tile * sp.tile * 4,
                "split area size", M, n, k);
        }
      }
  // documented plans
  GemmSplit sp = gemm_split_plan(4096, 11008, 4096, false);   // 688 tiles
  check(sp.rem == 0, "gate7b forward must not split (176 left)", sp.rem);
  sp = gemm_split_plan(2048, 8448, 1024, false);              // 264 tiles
  check(sp.whole == 256 && sp.rem == 8 && sp.tile == 256, "2048x8448x1024 plan",
        sp.whole, sp.rem, sp.tile);
  sp = gemm_split_plan(2048, 28672, 8192, false);             // 896 tiles
  check(sp.whole == 768 && sp.rem == 128 && sp.tile == 256, "70B gate forward plan",
        sp.whole, sp.rem, sp.tile);
  sp = gemm_split_plan(4096, 4096, 11008, false);             // 256 tiles
  check(sp.rem == 0, "gate7b dX must not split", sp.rem);
  sp = gemm_split_plan(2048, 1024, 8192, false);              // 70B k/v forward
  check(sp.whole == 0 && sp.rem == 128 && sp.tile == 128, "70B k forward plan",
        sp.whole, sp.rem, sp.tile);
  check(gemm_split_bytes(GemmSplit{0, 0, 0}) == 256, "status word area");
}

static void layouts() {
  const long long shapes[][3] = {{1, 8, 64},     {8, 28672, 8192}, {16, 64, 4160},
                                 {17, 136, 192}, {37, 200, 192},   {300, 264, 128},
                                 {2048, 8448, 1024}, {2050, 1032, 8256},
                                 {4096, 11008, 4096}, {2048, 1024, 8192}};
  const int ranks[] = {1, 5, 16, 17, 64, 256};
  for (auto& sh : shapes)
    for (int r : ranks) {
      const long long M = sh[0], N = sh[1], K = sh[2];
      const int jt = rank_tiles(r), rpad = 16 * jt;
      check(rpad >= r && rpad <= 256 && (jt & (jt - 1)) == 0, "rank tiles", r);
      for (int general = 0; general < 2; ++general) {
        const FwdWorkspace f = fwd_workspace_layout(M, N, K, r, general != 0);
        if (M <= QN_SKINNY_M && !general) {
          const SkinnyPlan P = skinny_plan(M, N, K, r);
          check(P.ks % 256 == 0 && P.ks <= SK_KS_MAX, "skinny slice width", M, N, K);
          check((long long)P.slices * P.ks >= K && (long long)(P.slices - 1) * P.ks < K,
                "skinny slices cover K", M, N, K);
          check((M + 1) * (P.ks + 8) * 2 <= 64 * 1024, "skinny X tile fits LDS", M, N, K);
          check(P.wtiles * 16 >= N && P.wtiles * 16 < N + 16 &&
                    P.tps == P.wtiles + rank_tiles(r) && P.rows_total == 16 * P.tps &&
                    P.rows_total >= N + r,
                "skinny rows", M, N, K);
          check(f.total >= size_t(P.slices) * M * P.rows_total * 4, "skinny partials",
                M, N, K);
          continue;
        }
        // a general layout holds the T pass of a forward with dropout too
        const StreamPlan P = stream_plan(RS_ROWS, M, K, jt, general != 0);
        check(P.nb >= stream_plan(RS_ROWS, M, K, jt).nb, "dropout T plan has fewer blocks",
              M, N, K);
        check((long long)P.mb * P.rm >= M, "T stream rows", M, N, K);
        check((long long)P.nb * P.cpb * 64 * P.sub >= K, "T stream columns", M, N, K);
        const GemmSplit sp = gemm_split_plan(M, N, K, false);
        check(f.split == 0, "split area not first", M, N, K);
        check_regions({{f.split, gemm_split_bytes(sp)},
                       {f.th, size_t(M) * rpad * 2},
                       {f.tl, size_t(M) * rpad * 2},
                       {f.bp, size_t(N) * rpad * 2},
                       {f.prow, size_t(P.nb) * M * rpad * 4}},
                      f.total, "forward layout", M, N, K);
      }
      const BwdWorkspace b = bwd_workspace_layout(M, N, K, r);
      const StreamPlan Pg = stream_plan(RS_ROWS | RS_COLS, M, N, jt);
      const StreamPlan Pa = stream_plan(RS_COLS, M, K, jt);
      const StreamPlan Pad = stream_plan(RS_COLS, M, K, jt, true);   // with dropout
      check((long long)Pg.mb * Pg.rm >= M && (long long)Pa.mb * Pa.rm >= M &&
                (long long)Pad.mb * Pad.rm >= M,
            "dY / dA stream rows", M, N, K);
      check((long long)Pad.nb * Pad.cpb * 64 * Pad.sub >= K, "dA stream columns", M, N, K);
      check((long long)Pg.nb * Pg.cpb * 64 * Pg.sub >= N, "dY stream columns", M, N, K);
      check(b.mp % 8 == 0 && b.mp >= M, "Mp", M, N, K);
      check(b.split == 0, "split area not first (backward)", M, N, K);
      const size_t pcol = std::max({size_t(Pg.mb) * N, size_t(Pa.mb) * K, size_t(Pad.mb) * K});
      check_regions({{b.split, gemm_split_bytes(gemm_split_plan(M, K, N, false))},
                     {b.bt, size_t(r) * N * 2},
                     {b.uth, size_t(r) * b.mp * 2},
                     {b.utl, size_t(r) * b.mp * 2},
                     {b.atp, size_t(K) * rpad * 2},
                     {b.gh, size_t(M) * rpad * 2},
                     {b.gl, size_t(M) * rpad * 2},
                     {b.ugh, size_t(r) * b.mp * 2},
                     {b.ugl, size_t(r) * b.mp * 2},
                     {b.prow, size_t(Pg.nb) * M * rpad * 4},
                     {b.pcol, pcol * rpad * 4}},
                    b.total, "backward layout", M, N, K);
    }
}

static void skinny_bounds_sweep() {
  // batches: single projections and the seven projections of two layers
  const long long shapes[][3] = {{8, 1024, 8192},  {8, 8192, 8192},   {8, 28672, 8192},
                                 {8, 8192, 28672}, {16, 4096, 11008}, {1, 8, 64},
                                 {3, 136, 192},    {16, 264, 4160},   {5, 11008, 4096}};
  std::vector<std::vector<int>> batches;
  for (int i = 0; i < 9; ++i) batches.push_back({i});
  batches.push_back({1, 0, 0, 1, 2, 2, 3});
  batches.push_back({4, 4, 4, 4, 4, 4, 4, 5});
  batches.push_back({5, 6, 7, 8});
  const int ranks[] = {1, 16, 64, 256};
  for (auto& b : batches)
    for (int r : ranks) {
      const int n = (int)b.size();
      std::vector<SkinnyPlan> P(n);
      std::vector<int64_t> K(n);
      std::vector<nf4_tensor> w(n);
      std::vector<SkinnyJob> J(n);
      for (int i = 0; i < n; ++i) {
        const long long* sh = shapes[b[i]];
        w[i].rows = sh[1];
        w[i].cols = sh[2];
        J[i] = SkinnyJob{nullptr, (int)sh[0], &w[i], nullptr, nullptr, r, 1.f,
                         nullptr, nullptr, 0};
        K[i] = sh[2];
      }
      if (n == 1)
        P[0] = skinny_plan(J[0].M, w[0].rows, w[0].cols, r);
      else
        skinny_plan_batch(J.data(), n, P.data());
      // every tile's cost start, by walking the list
      std::vector<int64_t> start;
      int64_t T = 0;
      for (int i = 0; i < n; ++i) {
        const int64_t kch = cdiv(K[i], 256), kc = P[i].ks / 256;
        for (int s = 0; s < P[i].slices; ++s) {
          const int64_t c = s < P[i].slices - 1 ? kc : kch - (P[i].slices - 1) * kc;
          check(c >= 1 && c <= kc, "slice chunks", b[i], s, c);
          for (int t = 0; t < P[i].tps; ++t) {
            start.push_back(T);
            T += c;
          }
        }
      }
      // one run per CU, and one per workgroup (two per CU, as launched)
      for (const int ns : {G_CUS, SK_WGS_PER_CU * G_CUS}) {
        std::vector<int32_t> bound(ns + 1);
        const int tiles = skinny_bounds(P.data(), K.data(), n, ns, bound.data());
        check(tiles == (int)start.size(), "tile count", tiles, (long long)start.size());
        check(bound[0] == 0 && bound[ns] == tiles, "bounds cover the tiles", bound[0],
              bound[ns], tiles);
        for (int c = 0; c <= ns; ++c) {
          const int64_t x = int64_t(c) * T / ns;
          int64_t want = (int64_t)start.size();
          for (size_t i = 0; i < start.size(); ++i)
            if (start[i] >= x) {
              want = (int64_t)i;
              break;
            }
          check(bound[c] == want, "slot bound", c, bound[c], want);
          if (c > 0) check(bound[c] >= bound[c - 1], "bounds not monotone", c);
        }
      }
    }
}

static void shape_rules() {
  nf4_tensor w{reinterpret_cast<uint8_t*>(0x1000), reinterpret_cast<uint8_t*>(0x2000),
               reinterpret_cast<float*>(0x3000), 256, 512};
  check(valid_linear(16, &w, 8), "tiny shape rejected");
  check(!valid_linear(0, &w, 8), "M = 0 accepted");
  check(!valid_linear(16, &w, 0) && !valid_linear(16, &w, 257), "rank out of range accepted");
  nf4_tensor w2 = w;
  w2.cols = 500;
  check(!valid_linear(16, &w2, 8), "K % 64 != 0 accepted");
  w2 = w;
  w2.rows = 250;
  check(!valid_linear(16, &w2, 8), "N % 8 != 0 accepted");
  w2 = w;
  w2.packed = reinterpret_cast<uint8_t*>(0x1008);
  check(!valid_linear(16, &w2, 8), "misaligned packed accepted");
  w2 = w;
  w2.rows = 65536;
  w2.cols = 65536;   // packed = 2 GiB
  check(!valid_linear(16, &w2, 8), "2 GiB operand accepted");
}

int main() {
  split_plan_sweep();
  layouts();
  skinny_bounds_sweep();
  shape_rules();
  if (!bad) std::printf("ok\n");
  return bad;
}
