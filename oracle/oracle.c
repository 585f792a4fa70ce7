/*
 * oracle.c -- the plain CPU oracle for C = epilogue(A . B).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no code, header, table or constant
 * with the HIP library; it reads raw 16-bit patterns and decodes them with
 * conversions written here from the IEEE 754 binary16 and bfloat16 bit
 * layouts.
 *
 * What it computes (page "gizml:tile", the worked example at the top of the
 * page, with Program.zeros, Program.fold, Tile.dot, Tile.relu, Tile.to and
 * Out.put):
 *
 *     for each batch item b, row i < M, column j < N:
 *         acc = +0.0f                                   (Program.zeros)
 *         for k = 0, 1, ..., K-1:                        (Program.fold)
 *             acc = fl32(acc + fl32(f32(A[b,i,k]) * f32(B[b,k,j])))   (Tile.dot: F32)
 *         v = bias ? fl32(acc + bias[j]) : acc          (Tile.add, a [1, N] row broadcast)
 *         y = act(v)                                    (Tile.relu, gelu, geluErf, sigmoid, tanh)
 *         C[b,i,j] = round_to_nearest_even(y, out_dtype) (Tile.to: what storing and reloading the type gives)
 *
 * Activations (codes 0 none, 1 relu, 2 gelu, 3 geluErf, 4 sigmoid, 5 tanh)
 * follow their definitions on the page, evaluated in double precision from
 * the fp32 value v and rounded once to fp32 (the page asks for results
 * within a few ulp; this is the correctly rounded value up to double's own
 * error, except far in the negative tail of the two GELU forms, where
 * 1 + tanh and 1 + erf cancel in double and leave an absolute error of
 * about 1e-16 |v| on results that small):
 *     relu(v)    = v > 0 ? v : +0
 *     gelu(v)    = v/2 * (1 + tanh(sqrt(2/pi) * (v + 0.044715 v^3)))   (tanh form)
 *                  (the page names the tanh form but prints no constants;
 *                  these are the published approximation of x Phi(x) of
 *                  Hendrycks and Gimpel, "Gaussian Error Linear Units", 2016)
 *     geluErf(v) = v/2 * (1 + erf(v / sqrt(2)))                          (erf form)
 *     sigmoid(v) = 1 / (1 + e^-v)
 *     tanh(v)    = tanh(v)
 *
 * Readings taken where the page is silent (each is also listed with the
 * design notes):
 *   - the output conversion rounds to nearest, ties to even; overflow goes
 *     to +-Inf, NaN stays NaN (quiet), subnormals are kept;
 *   - relu(x) is x when x > 0, else +0: -0 and NaN both give +0, because
 *     max(x, 0) returns the operand that is not NaN (Tile.maximum), i.e. 0;
 *   - K = 0 leaves the zero accumulator: C = epilogue(+0) everywhere;
 *   - the product of two fp16 (or two bf16, or two FP8) values is exact in
 *     fp32 except when it over- or underflows fp32's range, so FMA
 *     contraction would be immaterial; the file is still built with
 *     -ffp-contract=off so that the loop is literally fl32(acc + fl32(a*b));
 *   - the page's FP8 storage type is "FP8 E4M3" with no further detail; it
 *     is read as the OCP 8-bit E4M3 format (bias 7, no infinities, NaN only
 *     at S.1111.111, largest finite 448).
 *
 * Storage codes follow the page's constants (F32 = 0, F16 = 4, BF16 = 5,
 * FP8 = 9 for FP8 E4M3 operands).
 *
 * The loop order is i, k, j: every C[b,i,j] still sums k in ascending order,
 * one element per accumulator; the j loop only walks a row of outputs at a
 * time.  Operands are decoded once to fp32 (the f32() step of the formula).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_F32 0
#define ORC_F16 4
#define ORC_BF16 5
#define ORC_FP8 9

#define ORC_OK 0
#define ORC_EARG (-1)
#define ORC_EDTYPE (-2)
#define ORC_ENOMEM (-3)

/* ---------------------------------------------------------------------- */
/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static float orc_f16_decode(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int f = h & 1023;
  float v;
  if (e == 0) {
    v = ldexpf((float)f, -24); /* zero or subnormal: f * 2^-24 */
  } else if (e == 31) {
    if (f == 0) {
      v = INFINITY;
    } else {
      uint32_t u = 0x7fc00000u | ((uint32_t)f << 13); /* quiet NaN, payload kept */
      memcpy(&v, &u, 4);
    }
  } else {
    v = ldexpf((float)(1024 + f), e - 25); /* (1.f) * 2^(e-15) */
  }
  return sign ? -v : v;
}

/* bfloat16: the top 16 bits of an IEEE binary32 pattern. */
static float orc_bf16_decode(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float v;
  memcpy(&v, &u, 4);
  return v;
}

/* FP8 E4M3 (the page's FP8 storage type; read as the OCP 8-bit E4M3 format):
 * 1 sign bit, 4 exponent bits (bias 7), 3 fraction bits; exponent 0 holds
 * zero and the subnormals f * 2^-9; there are no infinities, and the one
 * pattern with all exponent and fraction bits set (0x7f, 0xff) is NaN. */
static float orc_fp8_decode(uint8_t h) {
  int sign = (h >> 7) & 1;
  int e = (h >> 3) & 15;
  int f = h & 7;
  float v;
  if (e == 15 && f == 7) {
    v = NAN;
  } else if (e == 0) {
    v = ldexpf((float)f, -9);
  } else {
    v = ldexpf((float)(8 + f), e - 10); /* (1.f) * 2^(e-7) */
  }
  return sign ? -v : v;
}

/* Element idx of an operand array of storage type dtype. */
static float orc_decode_at(int dtype, const void* base, int64_t idx) {
  if (dtype == ORC_FP8) return orc_fp8_decode(((const uint8_t*)base)[idx]);
  const uint16_t h = ((const uint16_t*)base)[idx];
  return (dtype == ORC_F16) ? orc_f16_decode(h) : orc_bf16_decode(h);
}

/* Round an unsigned magnitude right by `shift` bits, to nearest, ties to even. */
static uint32_t orc_rshift_rne(uint32_t m, int shift) {
  if (shift <= 0) return m;
  if (shift >= 32) return 0; /* m < 2^24 here, so below half of one unit */
  uint32_t q = m >> shift;
  uint32_t rem = m & ((1u << shift) - 1u);
  uint32_t half = 1u << (shift - 1);
  if (rem > half || (rem == half && (q & 1u))) q += 1u;
  return q;
}

static uint16_t orc_f16_encode(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return (uint16_t)(sign | 0x7e00u | ((a >> 13) & 0x1ffu)); /* NaN */
  int e = (int)(a >> 23);         /* biased binary32 exponent */
  uint32_t f = a & 0x7fffffu;
  if (e == 255) return (uint16_t)(sign | 0x7c00u); /* Inf */
  /* Significand as an integer m with value m * 2^(e2) exactly. */
  uint32_t m = (e == 0) ? f : (f | 0x800000u);
  int e2 = (e == 0) ? -149 : e - 150;
  /* binary16 quantum at this magnitude: 2^-24 for subnormals, else 2^(E-10)
   * where E is the unbiased exponent of the value (>= -14). */
  int unb = (e == 0) ? -127 : e - 127; /* exponent of the leading bit (approx. for f32 subnormals) */
  int q_exp = (unb < -14) ? -24 : unb - 10;
  uint32_t q = orc_rshift_rne(m, q_exp - e2); /* value in units of 2^q_exp */
  /* Re-normalise: q may have carried to 2^11 (normal) or to 2^10 (subnormal -> normal). */
  if (unb < -14) {
    /* q in units of 2^-24: q < 1024 is subnormal, q == 1024 is the smallest normal. */
    return (uint16_t)(sign | q); /* q <= 1024; 1024 == 0x0400 encodes 2^-14 */
  }
  int E = unb;
  if (q >= 2048u) { q >>= 1; E += 1; } /* carry; exact since q == 2048 */
  if (E > 15) return (uint16_t)(sign | 0x7c00u);
  return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(q & 1023u));
}

static uint16_t orc_bf16_encode(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u); /* quiet NaN */
  uint32_t hi = u >> 16;
  uint32_t rem = u & 0xffffu;
  /* Carry from the fraction into the exponent is the correct rounding,
   * including the step from the largest finite value to Inf. */
  if (rem > 0x8000u || (rem == 0x8000u && (hi & 1u))) hi += 1u;
  return (uint16_t)hi;
}

/* Exported element-wise conversions (used by the tests that pin them).
 * src holds n elements of dtype (F16, BF16: 16-bit patterns; FP8: bytes). */
void oracle_decode(int dtype, const void* src, float* dst, int64_t n) {
  for (int64_t i = 0; i < n; ++i) dst[i] = orc_decode_at(dtype, src, i);
}

void oracle_encode(int dtype, const float* src, uint16_t* dst, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    dst[i] = (dtype == ORC_F16) ? orc_f16_encode(src[i]) : orc_bf16_encode(src[i]);
}

/* ---------------------------------------------------------------------- */
static int orc_check(int64_t M, int64_t N, int64_t K, int in_dtype, int out_dtype, int epilogue,
                     int64_t batch) {
  if (M < 0 || N < 0 || K < 0 || batch < 1) return ORC_EARG;
  if (epilogue < 0 || epilogue > 5) return ORC_EARG;
  if (in_dtype != ORC_F16 && in_dtype != ORC_BF16 && in_dtype != ORC_FP8) return ORC_EDTYPE;
  if (out_dtype != ORC_F32 && out_dtype != ORC_F16 && out_dtype != ORC_BF16) return ORC_EDTYPE;
  return ORC_OK;
}

static float orc_relu(float v) { return (v > 0.0f) ? v : 0.0f; }

static float orc_activate(float v, int act) {
  const double x = (double)v;
  const double pi = 3.14159265358979323846;
  switch (act) {
    case 0: return v;
    case 1: return orc_relu(v);
    case 2: return (float)(0.5 * x * (1.0 + tanh(sqrt(2.0 / pi) * (x + 0.044715 * x * x * x))));
    case 3: return (float)(0.5 * x * (1.0 + erf(x / sqrt(2.0))));
    case 4: return (float)(1.0 / (1.0 + exp(-x)));
    default: return (float)tanh(x);
  }
}

/* The epilogue of one output: bias (when given), then the activation. */
static float orc_epilogue(float acc, const float* bias, int64_t j, int act) {
  const float v = bias ? acc + bias[j] : acc;
  return orc_activate(v, act);
}

static void orc_store(int out_dtype, void* C, int64_t idx, float y) {
  if (out_dtype == ORC_F32)
    ((float*)C)[idx] = y;
  else if (out_dtype == ORC_F16)
    ((uint16_t*)C)[idx] = orc_f16_encode(y);
  else
    ((uint16_t*)C)[idx] = orc_bf16_encode(y);
}

/* Decode n elements starting at element `first` of an operand array. */
static void orc_decode_batch(int dtype, const void* base, int64_t first, float* dst, int64_t n) {
  for (int64_t i = 0; i < n; ++i) dst[i] = orc_decode_at(dtype, base, first + i);
}

static void orc_set_threads(int threads) {
#ifdef _OPENMP
  if (threads > 0) omp_set_num_threads(threads);
#else
  (void)threads;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * Full GEMM.  A is [batch][M][K], B is [batch][K][N], C is [batch][M][N],
 * each row-major with contiguous rows; stride_* is the element distance
 * between batch items.  bias, when not NULL, holds N fp32 values added to
 * every row.  Y, when not NULL, receives the fp32 value y before the output
 * conversion, as a contiguous [batch][M][N] array.
 */
int oracle_gemm(int64_t M, int64_t N, int64_t K, int in_dtype, int out_dtype, int epilogue,
                const float* bias, int64_t batch, const void* A, int64_t stride_a,
                const void* B, int64_t stride_b, void* C, int64_t stride_c, float* Y,
                int threads) {
  int rc = orc_check(M, N, K, in_dtype, out_dtype, epilogue, batch);
  if (rc) return rc;
  if (M == 0 || N == 0) return ORC_OK;
  orc_set_threads(threads);
  float* bf = (float*)malloc(sizeof(float) * (size_t)(K > 0 ? K * N : 1));
  float* af = (float*)malloc(sizeof(float) * (size_t)(K > 0 ? M * K : 1));
  if (!bf || !af) { free(bf); free(af); return ORC_ENOMEM; }
  for (int64_t b = 0; b < batch; ++b) {
    orc_decode_batch(in_dtype, A, b * stride_a, af, M * K);
    orc_decode_batch(in_dtype, B, b * stride_b, bf, K * N);
    int64_t i;
#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < M; ++i) {
      float* acc = (float*)malloc(sizeof(float) * (size_t)N);
      for (int64_t j = 0; j < N; ++j) acc[j] = 0.0f;
      for (int64_t k = 0; k < K; ++k) {
        const float a = af[i * K + k];
        const float* brow = bf + k * N;
        for (int64_t j = 0; j < N; ++j) acc[j] = acc[j] + a * brow[j];
      }
      for (int64_t j = 0; j < N; ++j) {
        float y = orc_epilogue(acc[j], bias, j, epilogue);
        orc_store(out_dtype, C, b * stride_c + i * N + j, y);
        if (Y) Y[(b * M + i) * N + j] = y;
      }
      free(acc);
    }
  }
  free(af);
  free(bf);
  return ORC_OK;
}

/*
 * The same result for a list of output elements only (for full-size
 * workloads where the whole product would take the CPU too long):
 * element e is C[bi[e], ii[e], jj[e]], written to out (out_dtype storage)
 * and, when Y is not NULL, its fp32 y to Y[e].  Same sum order as above.
 */
int oracle_gemm_sampled(int64_t M, int64_t N, int64_t K, int in_dtype, int out_dtype,
                        int epilogue, const float* bias, int64_t batch, const void* A,
                        int64_t stride_a,
                        const void* B, int64_t stride_b, int64_t count, const int64_t* bi,
                        const int64_t* ii, const int64_t* jj, void* out, float* Y, int threads) {
  int rc = orc_check(M, N, K, in_dtype, out_dtype, epilogue, batch);
  if (rc) return rc;
  for (int64_t e = 0; e < count; ++e)
    if (bi[e] < 0 || bi[e] >= batch || ii[e] < 0 || ii[e] >= M || jj[e] < 0 || jj[e] >= N)
      return ORC_EARG;
  orc_set_threads(threads);
  int64_t e;
#pragma omp parallel for schedule(static)
  for (e = 0; e < count; ++e) {
    const int64_t arow = bi[e] * stride_a + ii[e] * K;
    const int64_t bcol = bi[e] * stride_b + jj[e];
    float acc = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
      float a = orc_decode_at(in_dtype, A, arow + k);
      float bv = orc_decode_at(in_dtype, B, bcol + k * N);
      acc = acc + a * bv;
    }
    float y = orc_epilogue(acc, bias, jj[e], epilogue);
    orc_store(out_dtype, out, e, y);
    if (Y) Y[e] = y;
  }
  return ORC_OK;
}

/*
 * fp64 twin for error bounds: Y64 = the sum in double precision (the
 * products of two 16-bit values are exact in double), before the epilogue;
 * S64 = sum over k of |a_ik| |b_kj| (the scale of the rounding-error bound).
 * Either output may be NULL.  Contiguous [batch][M][N] outputs.
 */
int oracle_gemm_f64(int64_t M, int64_t N, int64_t K, int in_dtype, int64_t batch,
                    const void* A, int64_t stride_a, const void* B, int64_t stride_b,
                    double* Y64, double* S64, int threads) {
  int rc = orc_check(M, N, K, in_dtype, ORC_F32, 0, batch);
  if (rc) return rc;
  if (M == 0 || N == 0) return ORC_OK;
  orc_set_threads(threads);
  float* bf = (float*)malloc(sizeof(float) * (size_t)(K > 0 ? K * N : 1));
  float* af = (float*)malloc(sizeof(float) * (size_t)(K > 0 ? M * K : 1));
  if (!bf || !af) { free(bf); free(af); return ORC_ENOMEM; }
  for (int64_t b = 0; b < batch; ++b) {
    orc_decode_batch(in_dtype, A, b * stride_a, af, M * K);
    orc_decode_batch(in_dtype, B, b * stride_b, bf, K * N);
    int64_t i;
#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < M; ++i) {
      double* acc = (double*)malloc(sizeof(double) * (size_t)N);
      double* sab = (double*)malloc(sizeof(double) * (size_t)N);
      for (int64_t j = 0; j < N; ++j) { acc[j] = 0.0; sab[j] = 0.0; }
      for (int64_t k = 0; k < K; ++k) {
        const double a = (double)af[i * K + k];
        const float* brow = bf + k * N;
        for (int64_t j = 0; j < N; ++j) {
          acc[j] = acc[j] + a * (double)brow[j];
          sab[j] = sab[j] + fabs(a) * fabs((double)brow[j]);
        }
      }
      for (int64_t j = 0; j < N; ++j) {
        if (Y64) Y64[(b * M + i) * N + j] = acc[j];
        if (S64) S64[(b * M + i) * N + j] = sab[j];
      }
      free(acc);
      free(sab);
    }
  }
  free(af);
  free(bf);
  return ORC_OK;
}
