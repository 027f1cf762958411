/* ORACLE (test infrastructure only; nothing of the product links or includes this file).
 *
 * The cast step of the dynamic tensorwise e4m3fn quantisation of the MLP's FP8 GEMMs
 * [hn.213312.xyz translation, 提升吞吐量 / Increasing throughput: FP8 with dynamic scaling;
 * linlog.top article, 吞吐量优化: torch._scaled_mm with dynamic tensorwise scales], in plain C so
 * that every one of the 2^32 fp32 bit patterns can be checked against the device in seconds. It
 * follows the same definitions as oracle/numerics.py (e4m3_round, e4m3_encode), written again
 * from the format's definition:
 *   e4m3fn (OCP FP8 E4M3): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits, no infinities,
 *   S.1111.111 is NaN, largest finite 448 = 1.75 * 2^8, smallest normal 2^-6, subnormals k * 2^-9.
 *   q = e4m3fn_rne(clamp(fl32(x * scale), -448, 448)); a NaN product gives the code 0x7F (the
 *   library's documented convention for non-finite activations; the pages do not cover them).
 * Rounding: a nonzero |v| in [2^(e-1), 2^e) has 4 significant bits, so its quantum is 2^(e-4);
 * below 2^-6 the quantum is the subnormal step 2^-9. |v| / quantum is exact in double and
 * nearbyint rounds half to even in the default rounding mode. The sign of zero is kept.
 * Build: gcc -O2 -fPIC -shared -ffp-contract=off (no fast-math: the fp32 product must be one IEEE
 * multiplication rounded to nearest even). */
#include <math.h>
#include <stdint.h>

static uint8_t cast_one(float x, float scale) {
  const float p = x * scale; /* one fp32 multiplication */
  if (isnan(p)) return 0x7F;
  double v = (double)p;
  if (v > 448.0) v = 448.0;
  if (v < -448.0) v = -448.0;
  const uint8_t sign = signbit(v) ? 0x80 : 0x00;
  const double a = fabs(v);
  int e;
  frexp(a, &e); /* a = m 2^e, 0.5 <= m < 1 (e = 0 for a = 0) */
  if (e < -5) e = -5; /* below 2^-6 the quantum stays 2^-9 */
  const double quantum = ldexp(1.0, e - 4);
  const double r = nearbyint(a / quantum) * quantum; /* the nearest e4m3 magnitude, <= 448 */
  if (r == 0.0) return sign;
  if (r < 0.015625) return sign | (uint8_t)(r * 512.0); /* subnormal: k 2^-9 */
  int er;
  const double mr = frexp(r, &er); /* r = (2 mr) 2^(er - 1), 2 mr in [1, 2) */
  const int exp_field = er - 1 + 7;
  const int mant = (int)((2.0 * mr - 1.0) * 8.0); /* exact: 3 fraction bits */
  return sign | (uint8_t)(exp_field << 3) | (uint8_t)mant;
}

/* q[i] = the e4m3fn code of x[i] at `scale`, for i in [0, n) */
void oracle_e4m3_cast(const float* x, int64_t n, float scale, uint8_t* q) {
  for (int64_t i = 0; i < n; ++i) q[i] = cast_one(x[i], scale);
}

/* The same over the n consecutive fp32 bit patterns first, first + 1, ... (wrapping at 2^32), so
 * that a sweep need not materialise its inputs */
void oracle_e4m3_cast_patterns(uint32_t first, int64_t n, float scale, uint8_t* q) {
  for (int64_t i = 0; i < n; ++i) {
    union {
      uint32_t u;
      float f;
    } b;
    b.u = first + (uint32_t)i;
    q[i] = cast_one(b.f, scale);
  }
}
