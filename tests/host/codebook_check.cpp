// Host check of the library's codebook code, built with address and
// undefined-behaviour sanitizers by tests/test_host_sanitizers.py.
// For every table (NF4, FP4, INT4): 16 sorted levels spanning [-1, 1] with
// an exact 0, 15 fp32 thresholds equal to the midpoints of adjacent levels
// (computed in double and rounded once), and at most one threshold in each
// bucket [(b - 64) / 64, (b - 63) / 64) -- the property the quantizer's
// bucketed threshold search relies on.  Unknown tables are rejected.
#include <cmath>
#include <cstdio>

#include "qlora_nf4.h"
#include "qn_internal.h"

static int fail(const char* what, int code) {
  std::fprintf(stderr, "code table %d: %s\n", code, what);
  return 1;
}

int main() {
  int bad = 0;
  for (int code = QN_CODE_NF4; code <= QN_CODE_INT4; ++code) {
    float lv[16], th[15];
    if (qn_codebook(code, lv, th) != QN_OK) return fail("rejected", code);
    bool zero = false;
    for (int j = 0; j < 16; ++j) zero = zero || lv[j] == 0.0f;
    if (!zero) bad |= fail("no exact zero level", code);
    if (lv[15] != 1.0f) bad |= fail("largest level is not 1", code);
    if (lv[0] < -8.0f / 7.0f - 1e-6f || lv[0] > -1.0f)
      bad |= fail("smallest level outside [-8/7, -1]", code);
    for (int j = 0; j < 15; ++j) {
      if (!(lv[j] <= lv[j + 1])) bad |= fail("levels not sorted", code);
      const float mid = static_cast<float>((double(lv[j]) + double(lv[j + 1])) / 2.0);
      if (th[j] != mid) bad |= fail("threshold is not the fp32 midpoint", code);
    }
    for (int b = 0; b < 129; ++b) {
      const double lo = (b - 64) / 64.0, hi = (b - 63) / 64.0;
      int inside = 0;
      for (int j = 0; j < 15; ++j) inside += (th[j] >= lo && th[j] < hi) ? 1 : 0;
      if (inside > 1) bad |= fail("two thresholds in one 1/64 bucket", code);
    }
  }
  float lv[16], th[15];
  if (qn_codebook(3, lv, th) != QN_EINVAL) bad |= fail("unknown table accepted", 3);
  if (qn_codebook(-1, lv, th) != QN_EINVAL) bad |= fail("unknown table accepted", -1);
  // nf4_codebook is the NF4 table
  float l2[16], t2[15];
  nf4_codebook(l2, t2);
  qn_codebook(QN_CODE_NF4, lv, th);
  for (int j = 0; j < 16; ++j)
    if (l2[j] != lv[j]) bad |= fail("nf4_codebook differs", 0);
  if (!bad) std::printf("ok\n");
  return bad;
}
