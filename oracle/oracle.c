/*
 * Plain CPU oracle for the tiled GEMMs.  TEST INFRASTRUCTURE ONLY: the tests,
 * the smoke check and the benchmark's CPU-baseline leg may load this; the
 * GPU library never does, and this file shares nothing with it.
 *
 * What is computed is the textbook matrix product, with no tiles, stages or
 * buffers: software pipelining only reorders the loads that feed the
 * arithmetic, so the pipelined kernels must reach this same result.
 *   - Croqtile tutorial, ch.6 "Synchronization: pipelines, events and double
 *     buffering", listing "double buffering with swap": out(m,n) accumulates
 *     lhs(m,k) * rhs(k,n) over all k, int32 operands, output starts empty.
 *   - Same page, listing "1P1C kernel with events": lhs f16 [M,K],
 *     rhs f16 [N,K], output f16 [M,N]; the accumulator starts at zero
 *     (mma.fill 0) and row m of lhs meets row n of rhs (both K-contiguous).
 *
 * Readings taken where the pages are silent:
 *   - int32: sums wrap modulo 2^32 (two's complement); int64 products are
 *     accumulated in uint64 and the low 32 bits kept.
 *   - f16/bf16: the oracle keeps the exact products in binary64 and adds them
 *     one after another in k order, multiply and add kept separate (the file
 *     is built with -ffp-contract=off).  It also returns sum_k |a*b|, the
 *     scale of the acceptance bound.
 *   - Output rounding is round-to-nearest-even; the acceptance test for a
 *     GPU element g is |g - ref| <= rel * mag + ulp(RNE(ref)) in the output
 *     type (rel = 1e-3).
 *   - Special values follow IEEE 754: a NaN or infinite exact sum (a NaN
 *     operand, an infinity times zero, infinities of both signs, or one
 *     infinity) must come out as NaN or as that infinity, and a finite sum
 *     past the output format's overflow threshold as the infinity of its
 *     sign; subnormal operands count at their value.  pgo_check_nt gives
 *     the exact rule.
 *
 * Codecs: IEEE-754 binary16 (1 sign, 5 exponent bits with bias 15, 10
 * fraction bits, subnormals) and bfloat16 (the upper half of binary32: 1, 8
 * with bias 127, 7).  They are written here from the field definitions and
 * are independent of any other half-precision code in the repository.
 */
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define PGO_F16 0
#define PGO_BF16 1

/* ---------------------------------------------------------------- codecs */

double pgo_f16_to_f64(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 0x1F, f = h & 0x3FF;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24); /* subnormal: f * 2^-24 */
  else if (e == 0x1F)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + f), e - 25); /* (1 + f/2^10) * 2^(e-15) */
  return s ? -v : v;
}

double pgo_bf16_to_f64(uint16_t h) {
  int s = h >> 15, e = (h >> 7) & 0xFF, f = h & 0x7F;
  double v;
  if (e == 0)
    v = ldexp((double)f, -133); /* subnormal: f/2^7 * 2^-126 */
  else if (e == 0xFF)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(128 + f), e - 134); /* (1 + f/2^7) * 2^(e-127) */
  return s ? -v : v;
}

/* Round |x| to a format with `mbits` fraction bits, minimum normal exponent
 * `emin`, maximum finite exponent `emax`; returns the rounded magnitude (may
 * be INFINITY on overflow).  Ties go to even via nearbyint in the default
 * rounding mode. */
static double round_to_format(double a, int mbits, int emin, int emax) {
  int e2;
  frexp(a, &e2); /* a = m * 2^e2, m in [0.5, 1) */
  int E = e2 - 1;
  if (E < emin) E = emin;                  /* subnormal range: fixed quantum */
  double q = ldexp(1.0, E - mbits);        /* spacing of the binade */
  double r = nearbyint(a / q);             /* a / q is exact (power of two) */
  double y = r * q;
  if (y >= ldexp(1.0, emax + 1)) return INFINITY;
  return y;
}

uint16_t pgo_f64_to_f16(double x) {
  uint16_t s = signbit(x) ? 0x8000 : 0;
  if (isnan(x)) return 0x7E00;
  double a = fabs(x);
  if (a == 0.0) return s;
  double y = isinf(a) ? INFINITY : round_to_format(a, 10, -14, 15);
  if (isinf(y)) return s | 0x7C00;
  if (y == 0.0) return s;
  int e2;
  frexp(y, &e2);
  int E = e2 - 1;
  if (E < -14) return s | (uint16_t)ldexp(y, 24); /* subnormal field */
  uint16_t field_e = (uint16_t)(E + 15);
  uint16_t field_f = (uint16_t)(ldexp(y, 10 - E) - 1024.0);
  return s | (uint16_t)(field_e << 10) | field_f;
}

uint16_t pgo_f64_to_bf16(double x) {
  uint16_t s = signbit(x) ? 0x8000 : 0;
  if (isnan(x)) return 0x7FC0;
  double a = fabs(x);
  if (a == 0.0) return s;
  double y = isinf(a) ? INFINITY : round_to_format(a, 7, -126, 127);
  if (isinf(y)) return s | 0x7F80;
  if (y == 0.0) return s;
  int e2;
  frexp(y, &e2);
  int E = e2 - 1;
  if (E < -126) return s | (uint16_t)ldexp(y, 133);
  uint16_t field_e = (uint16_t)(E + 127);
  uint16_t field_f = (uint16_t)(ldexp(y, 7 - E) - 128.0);
  return s | (uint16_t)(field_e << 7) | field_f;
}

/* Unit in the last place of a value y of the output format: the spacing of
 * the binade that holds y, and the subnormal spacing below the smallest
 * normal (also for y = 0). */
double pgo_ulp_f16(double y) {
  double a = fabs(y);
  if (a < ldexp(1.0, -14)) return ldexp(1.0, -24);
  int e2;
  frexp(a, &e2);
  return ldexp(1.0, e2 - 1 - 10);
}

double pgo_ulp_bf16(double y) {
  double a = fabs(y);
  if (a < ldexp(1.0, -126)) return ldexp(1.0, -133);
  int e2;
  frexp(a, &e2);
  return ldexp(1.0, e2 - 1 - 7);
}

/* Array forms, for checking the codecs against other implementations. */
void pgo_decode(int fmt, const uint16_t *in, double *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    out[i] = fmt == PGO_F16 ? pgo_f16_to_f64(in[i]) : pgo_bf16_to_f64(in[i]);
}

void pgo_encode(int fmt, const double *in, uint16_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    out[i] = fmt == PGO_F16 ? pgo_f64_to_f16(in[i]) : pgo_f64_to_bf16(in[i]);
}

void pgo_ulp(int fmt, const double *in, double *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    out[i] = fmt == PGO_F16 ? pgo_ulp_f16(in[i]) : pgo_ulp_bf16(in[i]);
}

/* Number of threads the OpenMP loops below use. */
int pgo_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ----------------------------------------------------------------- GEMMs */

/* out[m,n] = sum_k lhs[m,k] * rhs[k,n]  (mod 2^32), lhs [M,K], rhs [K,N]. */
void pgo_gemm_s32_nn(const int32_t *lhs, const int32_t *rhs, int32_t *out,
                     int64_t M, int64_t N, int64_t K) {
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      uint64_t acc = 0;
      for (int64_t k = 0; k < K; ++k)
        acc += (uint64_t)((int64_t)lhs[m * K + k] * (int64_t)rhs[k * N + n]);
      uint32_t low = (uint32_t)acc;
      int32_t v;
      memcpy(&v, &low, sizeof v);
      out[m * N + n] = v;
    }
}

static double *decode_table(int fmt) {
  double *t = (double *)malloc(65536 * sizeof(double));
  if (!t) return NULL;
  for (int h = 0; h < 65536; ++h)
    t[h] = fmt == PGO_F16 ? pgo_f16_to_f64((uint16_t)h) : pgo_bf16_to_f64((uint16_t)h);
  return t;
}

/* One output element of the NT product: ref = sum_k a(m,k) * b(n,k) in k
 * order, mag = sum_k |a(m,k) * b(n,k)|. */
static void nt_entry(const double *T, const uint16_t *arow, const uint16_t *brow,
                     int64_t K, double *ref, double *mag) {
  double s = 0.0, t = 0.0;
  for (int64_t k = 0; k < K; ++k) {
    double p = T[arow[k]] * T[brow[k]];
    s = s + p;
    t = t + fabs(p);
  }
  *ref = s;
  *mag = t;
}

/* Full NT product: lhs [M,K], rhs [N,K] (half-precision bits), ref/mag [M,N].
 * Returns 0, or -1 if the decode table could not be allocated. */
int pgo_gemm_nt(int fmt, const uint16_t *lhs, const uint16_t *rhs, double *ref,
                double *mag, int64_t M, int64_t N, int64_t K) {
  double *T = decode_table(fmt);
  if (!T) return -1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n)
      nt_entry(T, lhs + m * K, rhs + n * K, K, ref + m * N + n, mag + m * N + n);
  free(T);
  return 0;
}

/* Selected elements (mi[i], ni[i]) of the NT product. */
int pgo_gemm_nt_entries(int fmt, const uint16_t *lhs, const uint16_t *rhs,
                        int64_t M, int64_t N, int64_t K, const int64_t *mi,
                        const int64_t *ni, int64_t count, double *ref, double *mag) {
  (void)M;
  (void)N;
  double *T = decode_table(fmt);
  if (!T) return -1;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t i = 0; i < count; ++i)
    nt_entry(T, lhs + mi[i] * K, rhs + ni[i] * K, K, ref + i, mag + i);
  free(T);
  return 0;
}

/* Acceptance test, element by element, in the output format (largest finite
 * value MAX, spacing of the top binade TOP, overflow threshold
 * MAX + TOP/2 of round-to-nearest-even).  With r = ref[i] (the exact
 * products summed in binary64, so NaN or an infinity when IEEE arithmetic
 * gives one), g = decode(got[i]) and bound = rel * mag[i] + ulp(RNE(r))
 * (TOP when RNE(r) overflows):
 *   - r NaN: g must be NaN;
 *   - r infinite: g must be the same infinity;
 *   - r finite: g must not be NaN; a finite g must satisfy |g - r| <= bound;
 *     an infinite g must carry the sign of r, with |r| + bound at or above
 *     the overflow threshold (the exact sum rounds to it, or is within the
 *     accumulation error of a sum that does).
 * Returns the number of failures and, in *worst, the largest |g - r| / bound
 * over finite pairs (infinity if any element failed otherwise). */
static double fmt_max(int fmt) { return fmt == PGO_F16 ? 65504.0 : ldexp(255.0, 120); }
static double fmt_top_ulp(int fmt) { return fmt == PGO_F16 ? 32.0 : ldexp(1.0, 120); }

int64_t pgo_check_nt(int fmt, const uint16_t *got, const double *ref,
                     const double *mag, int64_t count, double rel, double *worst) {
  int64_t bad = 0;
  double w = 0.0;
  const double top = fmt_top_ulp(fmt), threshold = fmt_max(fmt) + top / 2;
  for (int64_t i = 0; i < count; ++i) {
    double g = fmt == PGO_F16 ? pgo_f16_to_f64(got[i]) : pgo_bf16_to_f64(got[i]);
    double r = ref[i];
    int ok;
    double ratio = 0.0;
    if (isnan(r)) {
      ok = isnan(g);
    } else if (isinf(r)) {
      ok = g == r;
    } else if (isnan(g)) {
      ok = 0;
    } else {
      double yr = fmt == PGO_F16 ? pgo_f16_to_f64(pgo_f64_to_f16(r))
                                 : pgo_bf16_to_f64(pgo_f64_to_bf16(r));
      double ulp = isinf(yr) ? top : fmt == PGO_F16 ? pgo_ulp_f16(yr) : pgo_ulp_bf16(yr);
      double bound = rel * mag[i] + ulp;
      if (isinf(g)) {
        ok = (signbit(g) == signbit(r)) && fabs(r) + bound >= threshold;
      } else {
        double err = fabs(g - r);
        ok = err <= bound;
        ratio = err / bound;
      }
    }
    if (!ok) {
      ++bad;
      ratio = INFINITY;
    }
    if (ratio > w) w = ratio;
  }
  if (worst) *worst = w;
  return bad;
}
