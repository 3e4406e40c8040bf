// Host check of the division the 8-bit AdamW kernel uses to encode a block
// of moments: x / s with s = fp32(amax / 448), computed as the block scaled
// by 2^k (k = 64 - exponent(amax), clamped to [-126, 127]), y = RN(1 / s 2^k)
// and two fma corrections q <- q + (x - q s) y.  Claim: the E4M3 code of the
// result equals the code of the IEEE quotient for every x in [-amax, amax],
// and the fp32 quotient itself is equal wherever |x / s| >= 2^-11.  Checked
// on seeded random blocks over every binade of amax, with x spread from
// amax down to ~2^-60 amax; E4M3 here is an independent software encoder
// (round to nearest even, saturate at 448, subnormals m 2^-9, and a value
// that rounds to zero stored as code 0 whatever its sign, as the state
// format does).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

static uint64_t st = 0x2545F4914F6CDD1Dull;
static uint64_t next_u64() {
  st ^= st << 13;
  st ^= st >> 7;
  st ^= st << 17;
  return st;
}

static int e4m3(float x) {
  const int sign = std::signbit(x) ? 1 : 0;
  double a = std::fabs(static_cast<double>(x));
  if (a > 448.0) a = 448.0;
  if (a == 0.0) return 0;
  int e;
  std::frexp(a, &e);               // a = f 2^e, f in [0.5, 1)
  int E = e - 1;                   // a = (2f) 2^E
  if (E < -6) E = -6;              // the subnormal step is 2^-9
  double r = std::nearbyint(a / std::ldexp(1.0, E - 3));   // ties to even
  if (r >= 16.0) {                 // rounded up into the next binade
    ++E;
    r /= 2.0;
  }
  const int code = (E == -6 && r < 8.0) ? static_cast<int>(r)
                                        : ((E + 7) << 3) | (static_cast<int>(r) - 8);
  return code == 0 ? 0 : (sign << 7) | code;
}

static float block_quotient(float x, float s, float sc, float s2, float y) {
  const float a = x * sc;
  const float q0 = a * y;
  const float q1 = std::fma(std::fma(-q0, s2, a), y, q0);
  return std::fma(std::fma(-q1, s2, a), y, q1);
}

int main() {
  long bad_code = 0, bad_fp32 = 0, n = 0;
  for (long it = 0; it < 3000000; ++it) {
    const uint64_t u = next_u64();
    const int e = static_cast<int>(u % 276) - 149;          // binades of amax
    const float amax =
        std::ldexp(1.0f + static_cast<float>((u >> 9) & 0x7FFFFF) / 8388608.0f, e);
    const float s = amax / 448.0f;
    if (amax == 0.0f || s == 0.0f || !std::isfinite(amax)) continue;
    int ea;
    std::frexp(amax, &ea);
    int k = 64 - ea;
    k = k > 127 ? 127 : (k < -126 ? -126 : k);
    const float sc = std::ldexp(1.0f, k);
    const float s2 = s * sc;
    const float y = 1.0f / s2;
    for (int j = 0; j < 8; ++j) {
      const uint64_t v = next_u64();
      float f = static_cast<float>(v & 0xFFFFFF) / 16777216.0f;
      if ((v >> 30) % 4 == 0) f = std::ldexp(f, -static_cast<int>((v >> 40) % 60));
      float x = (v >> 60) & 1 ? -amax * f : amax * f;
      if ((v >> 50) % 64 == 0) x = (v >> 61) & 1 ? -amax : amax;
      const float ref = x / s;
      const float q = block_quotient(x, s, sc, s2, y);
      ++n;
      bad_code += e4m3(ref) != e4m3(q);
      if (std::fabs(ref) >= std::ldexp(1.0f, -11) && std::memcmp(&ref, &q, 4) != 0)
        ++bad_fp32;
    }
  }
  if (bad_code != 0 || bad_fp32 != 0 || n < 10000000) {
    std::printf("FAIL n=%ld code mismatches=%ld fp32 mismatches=%ld\n", n, bad_code,
                bad_fp32);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
