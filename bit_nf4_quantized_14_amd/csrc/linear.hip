// C entry points of the fused QLoRA linear layer (forward, backward,
// workspace sizes) and the library's shared host state: the codebook
// kernel argument, argument validation, error strings and the profiling
// hook.  "QLoRA Guide" (Forward pass diagram: W_bf16 x + B(A(x)); only A
// and B get gradients), "QLoRA Implementation Details (2025 Edition)"
// (Step 4: scale alpha / r).
#include <atomic>
#include <cmath>
#include <mutex>

#include "qn_host.h"

namespace qn {

#ifdef QN_PROFILE_HOOK
ProfileHook g_prof;
#endif

const Codebook& codebook() {
  static const Codebook cb = [] {
    Codebook c;
    derive_codebook(c.L, c.T);
    return c;
  }();
  return cb;
}

// A pad job with no valid columns that zeroes the status word and the split
// GEMM's counters (the split area's first G_SPLIT_HDR + 8 rem bytes) before
// the GEMM runs.
void zero_split_counters(FinishPad& p, char* split_ws, const GemmSplit& sp) {
  uint16_t* c = reinterpret_cast<uint16_t*>(split_ws);
  p = FinishPad{c, c, 1, (int)(G_SPLIT_HDR / 2) + 4 * sp.rem, 0, 0, 0};
}

}  // namespace qn

using namespace qn;

extern "C" {

int qn_profile_kernel(const char* name, void** ev_start, void** ev_stop,
                      int32_t capacity) {
#ifdef QN_PROFILE_HOOK
  const int32_t recorded = g_prof.count;
  if (name == nullptr) {
    g_prof = ProfileHook();
    return recorded;
  }
  if (ev_start == nullptr || ev_stop == nullptr || capacity < 0 ||
      std::strlen(name) >= sizeof(g_prof.name))
    return QN_EINVAL;
  g_prof = ProfileHook();
  std::strcpy(g_prof.name, name);
  g_prof.ev_start = ev_start;
  g_prof.ev_stop = ev_stop;
  g_prof.capacity = capacity;
  return recorded;
#else
  (void)name;
  (void)ev_start;
  (void)ev_stop;
  (void)capacity;
  return QN_EINVAL;   // the default build has no hook
#endif
}

const char* qn_strerror(int code) {
  switch (code) {
    case QN_OK: return "success";
    case QN_EINVAL: return "invalid argument";
    case QN_EWORKSPACE: return "workspace too small";
    case QN_EHIP: return "HIP launch error";
    case QN_ENONFINITE: return "non-finite weight";
    case QN_ESYNC: return "split tile partial never became ready";
    default: return "unknown error";
  }
}

size_t qlora_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t r,
                             int32_t which) {
  if (M <= 0 || N <= 0 || K <= 0 || r < 1 || r > QN_MAX_RANK) return 0;
  if (which == QN_FWD) return qn::fwd_workspace_layout(M, N, K, r, false).total;
  if (which == QN_FWD_DROPOUT)
    return qn::fwd_workspace_layout(M, N, K, r, true).total;
  if (which == QN_BWD) return qn::bwd_workspace_layout(M, N, K, r).total;
  return 0;
}

}  // extern "C"

namespace {

// Kernel arguments of a qn_dropout; false for p outside [0, 1).  p == 0
// keeps every element unscaled, which is the layer without dropout, so it
// maps to no dropout at all (*use = false).
bool drop_args(const qn_dropout* d, qn::DropArgs* out, bool* use) {
  *use = false;
  if (d == nullptr) return true;
  if (!(d->p >= 0.0 && d->p < 1.0)) return false;
  if (d->p == 0.0) return true;
  const double t = std::floor(d->p * 4294967296.0);
  out->thresh = t >= 4294967295.0 ? 0xFFFFFFFFu : static_cast<uint32_t>(t);
  out->scale = static_cast<float>(1.0 / (1.0 - d->p));
  out->key0 = static_cast<uint32_t>(d->seed & 0xFFFFFFFFu);
  out->key1 = static_cast<uint32_t>(d->seed >> 32);
  *use = true;
  return true;
}

// allow_split: the GEMM may split a ragged last wave (its partial tiles need
// workspace); without it the workspace is the smaller no-split layout.
int linear_fwd(const uint16_t* x, int64_t M, const nf4_tensor* w,
               const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
               void* y, int32_t y_dtype, float* t_save, const qn_dropout* drop,
               void* ws, size_t ws_bytes, void* stream,
               bool allow_split = true) {
  if (x == nullptr || A == nullptr || B == nullptr || y == nullptr ||
      t_save == nullptr)
    return QN_EINVAL;
  if (!valid_linear(M, w, r)) return QN_EINVAL;
  if (y_dtype != QN_F32 && y_dtype != QN_BF16) return QN_EINVAL;
  if (!aligned16(x) || !aligned16(A) || !aligned16(y) || !aligned16(t_save))
    return QN_EINVAL;
  qn::DropArgs da{};
  bool use_drop = false;
  if (!drop_args(drop, &da, &use_drop)) return QN_EINVAL;
  const int64_t N = w->rows, K = w->cols;
  // a forward with dropout always takes the general path (the skinny
  // kernel shares one X slice between W and A rows)
  const qn::FwdWorkspace L =
      qn::fwd_workspace_layout(M, N, K, r, drop != nullptr, allow_split);
  if (ws == nullptr || ws_bytes < L.total || !aligned16(ws))
    return QN_EWORKSPACE;
  const float s = alpha / (float)r;
  const int Mi = (int)M, Ni = (int)N, Ki = (int)K;
  hipStream_t st = (hipStream_t)stream;
  if (M <= qn::QN_SKINNY_M && !use_drop && drop == nullptr) {
    const SkinnyJob job{x, Mi, w, A, B, (int)r, s, t_save, y,
                        (int)(y_dtype == QN_BF16)};
    const SkinnyPlan plan = skinny_plan(M, N, K, r);
    launch_skinny(st, &job, 1, &plan, ws_at<char>(ws, L.part));
    return check_launch();
  }
  uint16_t* Th = ws_at<uint16_t>(ws, L.th);
  uint16_t* Tl = ws_at<uint16_t>(ws, L.tl);
  uint16_t* Bp = ws_at<uint16_t>(ws, L.bp);
  float* prow = ws_at<float>(ws, L.prow);
  const int jt = rank_tiles(r);
  // T = X A^T: partials over column blocks of X
  const StreamPlan P = stream_plan(RS_ROWS, M, K, jt, use_drop);
  launch_rank_stream<RS_ROWS>(st, "k_rank_stream_t", P, x, Mi, Ki, A, (int)r,
                              nullptr, nullptr, 0, prow, nullptr,
                              use_drop ? &da : nullptr);
  // T (fp32, saved), hi/lo parts of s T, B zero-padded to [N][rpad]
  FinishArgs fa = finish_args();
  fa.R = FinishRows{prow, (int64_t)M * L.rpad, L.rpad, P.nb, Mi, Mi, (int)r,
                    L.rpad, s, t_save, Th, Tl, nullptr, nullptr};
  // B already has rpad columns and 16-byte rows: the GEMM reads it as is
  const bool b_as_is = r == L.rpad && aligned16(B);
  if (!b_as_is)
    fa.P1 = FinishPad{B, Bp, Ni, L.rpad, (int)r, (int64_t)r, (int64_t)1};
  char* split_ws = ws_at<char>(ws, L.split);
  zero_split_counters(fa.P2, split_ws,
                      allow_split ? gemm_split_plan(M, N, K, false)
                                  : GemmSplit{0, 0, 0});
  launch_finish(st, fa);
  launch_gemm<false>(st, x, w, Th, Tl, b_as_is ? B : Bp, Mi, L.rpad, y,
                     (int)(y_dtype == QN_BF16), nullptr,
                     allow_split ? split_ws : nullptr);
  return check_launch();
}

int linear_bwd(const uint16_t* dy, const uint16_t* x, int64_t M,
               const nf4_tensor* w, const uint16_t* A, const uint16_t* B,
               int32_t r, float alpha, const float* t_saved, void* dx,
               int32_t dx_dtype, float* dA, float* dB, const qn_dropout* drop,
               void* ws, size_t ws_bytes, void* stream) {
  if (dy == nullptr || x == nullptr || A == nullptr || B == nullptr ||
      t_saved == nullptr || dx == nullptr || dA == nullptr || dB == nullptr)
    return QN_EINVAL;
  if (!valid_linear(M, w, r)) return QN_EINVAL;
  if (dx_dtype != QN_F32 && dx_dtype != QN_BF16) return QN_EINVAL;
  if (!aligned16(dy) || !aligned16(x) || !aligned16(A) || !aligned16(dx))
    return QN_EINVAL;
  qn::DropArgs da{};
  bool use_drop = false;
  if (!drop_args(drop, &da, &use_drop)) return QN_EINVAL;
  const int64_t N = w->rows, K = w->cols;
  const qn::BwdWorkspace L = qn::bwd_workspace_layout(M, N, K, r);
  if (ws == nullptr || ws_bytes < L.total || !aligned16(ws))
    return QN_EWORKSPACE;
  uint16_t* Bt = ws_at<uint16_t>(ws, L.bt);
  uint16_t* UTh = ws_at<uint16_t>(ws, L.uth);
  uint16_t* UTl = ws_at<uint16_t>(ws, L.utl);
  uint16_t* Atp = ws_at<uint16_t>(ws, L.atp);
  uint16_t* Gh = ws_at<uint16_t>(ws, L.gh);
  uint16_t* Gl = ws_at<uint16_t>(ws, L.gl);
  uint16_t* UGh = ws_at<uint16_t>(ws, L.ugh);
  uint16_t* UGl = ws_at<uint16_t>(ws, L.ugl);
  float* prow = ws_at<float>(ws, L.prow);
  float* pcol = ws_at<float>(ws, L.pcol);
  const float s = alpha / (float)r;
  const int Mi = (int)M, Ni = (int)N, Ki = (int)K, Mp = (int)L.mp;
  const int jt = rank_tiles(r);
  hipStream_t st = (hipStream_t)stream;

  // s T transposed (hi/lo), A^T padded to [K][rpad], B^T
  FinishArgs f0 = finish_args();
  f0.R = FinishRows{t_saved, 0, (int)r, 1, Mi, Mp, (int)r, L.rpad, s,
                    nullptr, nullptr, nullptr, UTh, UTl};
  f0.P1 = FinishPad{A, Atp, Ki, L.rpad, (int)r, (int64_t)1, K};
  f0.P2 = FinishPad{B, Bt, (int)r, Ni, Ni, (int)1, (int64_t)r};
  launch_finish(st, f0);
  // one pass over dY: G = dY B (column-block partials), dB = dY^T (s T)
  // (row-block partials)
  const StreamPlan Pg = stream_plan(RS_ROWS | RS_COLS, M, N, jt);
  launch_rank_stream<RS_ROWS | RS_COLS>(st, "k_rank_stream_dy", Pg, dy, Mi, Ni,
                                        Bt, (int)r, UTh, UTl, Mp, prow, pcol);
  // hi/lo parts of s G (row-major and transposed), dB
  FinishArgs f1 = finish_args();
  f1.R = FinishRows{prow, (int64_t)M * L.rpad, L.rpad, Pg.nb, Mi, Mp, (int)r,
                    L.rpad, s, nullptr, Gh, Gl, UGh, UGl};
  f1.Cc = FinishCols{pcol, Pg.mb, Ni, (int)r, L.rpad, dB, (int64_t)r, 1};
  char* split_ws = ws_at<char>(ws, L.split);
  zero_split_counters(f1.P1, split_ws, gemm_split_plan(M, K, N, use_drop));
  launch_finish(st, f1);
  // dX = dY W' + (s G) A
  launch_gemm<true>(st, dy, w, Gh, Gl, Atp, Mi, L.rpad, dx,
                    (int)(dx_dtype == QN_BF16), use_drop ? &da : nullptr,
                    split_ws);
  // dA = (s G)^T X: row-block partials of out[k][j] -> dA[j][k]
  const StreamPlan Pa = stream_plan(RS_COLS, M, K, jt, use_drop);
  launch_rank_stream<RS_COLS>(st, "k_rank_stream_da", Pa, x, Mi, Ki, nullptr,
                              (int)r, UGh, UGl, Mp, nullptr, pcol,
                              use_drop ? &da : nullptr);
  FinishArgs f2 = finish_args();
  f2.Cc = FinishCols{pcol, Pa.mb, Ki, (int)r, L.rpad, dA, (int64_t)1, K};
  launch_finish(st, f2);
  return check_launch();
}

}  // namespace

extern "C" {

int qlora_linear_fwd(const uint16_t* x, int64_t M, const nf4_tensor* w,
                     const uint16_t* A, const uint16_t* B, int32_t r,
                     float alpha, void* y, int32_t y_dtype, float* t_save,
                     void* ws, size_t ws_bytes, void* stream) {
  return linear_fwd(x, M, w, A, B, r, alpha, y, y_dtype, t_save, nullptr, ws,
                    ws_bytes, stream);
}

int qlora_linear_fwd_dropout(const uint16_t* x, int64_t M,
                             const nf4_tensor* w, const uint16_t* A,
                             const uint16_t* B, int32_t r, float alpha,
                             void* y, int32_t y_dtype, float* t_save,
                             const qn_dropout* drop, void* ws,
                             size_t ws_bytes, void* stream) {
  if (drop == nullptr) return QN_EINVAL;
  return linear_fwd(x, M, w, A, B, r, alpha, y, y_dtype, t_save, drop, ws,
                    ws_bytes, stream);
}

int qlora_linear_bwd(const uint16_t* dy, const uint16_t* x, int64_t M,
                     const nf4_tensor* w, const uint16_t* A,
                     const uint16_t* B, int32_t r, float alpha,
                     const float* t_saved, void* dx, int32_t dx_dtype,
                     float* dA, float* dB, void* ws, size_t ws_bytes,
                     void* stream) {
  return linear_bwd(dy, x, M, w, A, B, r, alpha, t_saved, dx, dx_dtype, dA,
                    dB, nullptr, ws, ws_bytes, stream);
}

int qlora_linear_bwd_dropout(const uint16_t* dy, const uint16_t* x,
                             int64_t M, const nf4_tensor* w,
                             const uint16_t* A, const uint16_t* B, int32_t r,
                             float alpha, const float* t_saved, void* dx,
                             int32_t dx_dtype, float* dA, float* dB,
                             const qn_dropout* drop, void* ws,
                             size_t ws_bytes, void* stream) {
  if (drop == nullptr) return QN_EINVAL;
  return linear_bwd(dy, x, M, w, A, B, r, alpha, t_saved, dx, dx_dtype, dA,
                    dB, drop, ws, ws_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Batched skinny forward: up to QN_FWD_BATCH_MAX projections with M <= 16
// in one launch pair.
// ---------------------------------------------------------------------------
namespace {

// Validates the jobs (each as qlora_linear_fwd would, and M <= 16) and
// fills the internal jobs and plans; returns the workspace bytes, or 0.
size_t fwd_batch_plan(const qlora_fwd_job* jobs, int32_t count,
                      SkinnyJob* out, SkinnyPlan* plans) {
  if (jobs == nullptr || count < 1 || count > QN_FWD_BATCH_MAX) return 0;
  for (int i = 0; i < count; ++i) {
    const qlora_fwd_job& J = jobs[i];
    if (J.x == nullptr || J.A == nullptr || J.B == nullptr || J.y == nullptr ||
        J.t_save == nullptr)
      return 0;
    if (!valid_linear(J.M, J.w, J.r) || J.M > QN_SKINNY_M) return 0;
    if (J.y_dtype != QN_F32 && J.y_dtype != QN_BF16) return 0;
    if (!aligned16(J.x) || !aligned16(J.A) || !aligned16(J.y) ||
        !aligned16(J.t_save))
      return 0;
    out[i] = SkinnyJob{J.x, (int)J.M, J.w, J.A, J.B, J.r,
                       J.alpha / (float)J.r, J.t_save, J.y,
                       (int)(J.y_dtype == QN_BF16)};
  }
  skinny_plan_batch(out, count, plans);
  size_t total = 0;
  for (int i = 0; i < count; ++i) total += align256(skinny_part_bytes(out[i].M, plans[i]));
  return total;
}

}  // namespace

extern "C" size_t qlora_fwd_batch_workspace_bytes(const qlora_fwd_job* jobs,
                                                  int32_t count) {
  SkinnyJob sj[QN_FWD_BATCH_MAX];
  SkinnyPlan sp[QN_FWD_BATCH_MAX];
  return fwd_batch_plan(jobs, count, sj, sp);
}

extern "C" int qlora_linear_fwd_batch(const qlora_fwd_job* jobs, int32_t count,
                                      void* ws, size_t ws_bytes, void* stream) {
  SkinnyJob sj[QN_FWD_BATCH_MAX];
  SkinnyPlan sp[QN_FWD_BATCH_MAX];
  const size_t need = fwd_batch_plan(jobs, count, sj, sp);
  if (need == 0) return QN_EINVAL;
  if (ws == nullptr || ws_bytes < need || !aligned16(ws)) return QN_EWORKSPACE;
  launch_skinny((hipStream_t)stream, sj, count, sp, static_cast<char*>(ws));
  return check_launch();
}

// ---------------------------------------------------------------------------
// Allocation-free forward: the workspace is a file-scope device array, one
// copy per GPU, shared by every call on that GPU.
// ---------------------------------------------------------------------------
namespace {

static __device__ __align__(256) char scratch[QN_NOALLOC_SCRATCH_BYTES];

constexpr int QN_MAX_DEVICES = 64;
std::atomic<void*> g_scratch_addr[QN_MAX_DEVICES];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device, looked up once per
// device with that device current.  The host-side name is only a stand-in
// for the symbol; kernels get this address instead.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= QN_MAX_DEVICES)
    return QN_EHIP;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess ||
          p == nullptr)
        return QN_EHIP;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return QN_OK;
}

}  // namespace

extern "C" int qlora_linear_fwd_noalloc(const uint16_t* x, int64_t M,
                                        const nf4_tensor* w, const uint16_t* A,
                                        const uint16_t* B, int32_t r,
                                        float alpha, void* y, int32_t y_dtype,
                                        float* t_save, void* stream) {
  if (!valid_linear(M, w, r)) return QN_EINVAL;
  // no split of a ragged last wave: its partial tiles would need up to
  // 32 MiB of their own
  const qn::FwdWorkspace L =
      qn::fwd_workspace_layout(M, w->rows, w->cols, r, false, false);
  if (L.total > QN_NOALLOC_SCRATCH_BYTES) return QN_EWORKSPACE;
  void* ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc != QN_OK) return rc;
  return linear_fwd(x, M, w, A, B, r, alpha, y, y_dtype, t_save, nullptr, ws,
                    QN_NOALLOC_SCRATCH_BYTES, stream, false);
}

