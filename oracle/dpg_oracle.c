/*
 * FP64 CPU oracle for the deterministic BF16 projection GEMM family.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library's product path may call,
 * link or load this file; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no code, header or table
 * with the HIP implementation.
 *
 * What it computes (all in double precision, from the exact input values):
 *
 *   forward          Y[t,n]  = sum_k X[t,k]  * W[n,k]
 *   input gradient   dX[t,k] = sum_n dY[t,n] * W[n,k]
 *   weight gradient  dW[n,k] = sum_t dY[t,n] * X[t,k]
 *
 * These are the three passes of the dense projection GEMM as the pages on
 * "plan the 4096 -> 12288 input gradient with the row-half-release program"
 * and "restore the K1 weight-gradient routes" describe them (forward with a
 * K-major B, input gradient with an MN-major B, weight gradient reducing over
 * the token count T).  The FP32 router GEMM (256 experts) uses the same three
 * formulas on FP32 operands ("cache the router entry points' calls", page
 * description).
 *
 * BF16 -> FP64 and FP32 -> FP64 conversions are exact, and a product of two
 * FP32 values is exact in FP64, so the only rounding in the plain mode is the
 * FP64 summation, done in ascending order of the reduction index.
 *
 * The BF16x3 mode returns the value the three-product emulation would give
 * with exact arithmetic: every FP32 operand a is split as hi = bf16_rne(a),
 * lo = bf16_rne(a - hi) (a - hi is exact in FP32), and each product a*b is
 * replaced by hi_a*hi_b + hi_a*lo_b + lo_a*hi_b (lo*lo dropped).  This is the
 * two-term, three-product scheme of Henry, Tang and Heinecke, "Leveraging the
 * bfloat16 AI datatype for higher-precision computations" (ARITH 2019).
 *
 * Each call describes both operands as strided views so that one routine,
 * C[i,j] = sum_r A(i,r) * B(r,j), serves all passes:
 *   A(i,r) = a[i*a_si + r*a_sr],  B(r,j) = b[r*b_sr + j*b_sj].
 */
#include <stdint.h>
#include <string.h>
#include <stdlib.h>
#include <math.h>

enum { ORC_BF16 = 0, ORC_F32 = 1 };
enum { ORC_MODE_EXACT = 0, ORC_MODE_BF16X3 = 1, ORC_MODE_ABS = 2 };

/* bf16 bit pattern -> float: the bf16 value is the top half of an fp32 word */
static float bf16_bits_to_float(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* fp32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN. */
uint16_t orc_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
    return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t lsb = (u >> 16) & 1u;
  return (uint16_t)((u + 0x7fffu + lsb) >> 16);
}

void orc_f32_to_bf16_array(const float* x, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_bf16(x[i]);
}

/* fp64 -> fp32 (C cast, round to nearest even) -> bf16 (RNE).  Used to state
 * the expected BF16 output where the FP64 value is exact in FP32. */
void orc_f64_to_bf16_via_f32(const double* x, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_bf16((float)x[i]);
}

/* BF16x3 split of one FP32 value: hi = bf16(a), lo = bf16(a - hi). */
static void split3(float a, double* hi, double* lo) {
  float h = bf16_bits_to_float(orc_f32_to_bf16(a));
  float r = a - h; /* exact: a and h share the leading bits */
  float l = bf16_bits_to_float(orc_f32_to_bf16(r));
  *hi = (double)h;
  *lo = (double)l;
}

void orc_split_bf16x3(const float* a, float* hi, float* lo, int64_t n) {
  for (int64_t i = 0; i < n; ++i) {
    double h, l;
    split3(a[i], &h, &l);
    hi[i] = (float)h;
    lo[i] = (float)l;
  }
}

static double load_elem(const void* p, int dtype, int64_t idx) {
  if (dtype == ORC_BF16) return (double)bf16_bits_to_float(((const uint16_t*)p)[idx]);
  return (double)((const float*)p)[idx];
}

/* the contribution of one pair of operand values under the chosen mode */
static double pair_term(const void* a, int adt, int64_t ai, const void* b, int bdt, int64_t bi, int mode) {
  double x = load_elem(a, adt, ai);
  double y = load_elem(b, bdt, bi);
  if (mode == ORC_MODE_EXACT) return x * y;
  if (mode == ORC_MODE_ABS) return fabs(x * y);
  /* BF16x3: hi*hi + hi*lo + lo*hi, each product exact in FP64 */
  double xh, xl, yh, yl;
  split3((float)x, &xh, &xl);
  split3((float)y, &yh, &yl);
  return xh * yh + xh * yl + xl * yh;
}

/*
 * Full output: C[i*ldc + j] for 0 <= i < M, 0 <= j < N, each an ascending-r
 * FP64 sum over 0 <= r < R.  Two loop nests give the same sums in the same
 * order; the second is used when B is contiguous along j (cache friendlier).
 */
int orc_matmul(int64_t M, int64_t N, int64_t R,
               const void* a, int adt, int64_t a_si, int64_t a_sr,
               const void* b, int bdt, int64_t b_sr, int64_t b_sj,
               int mode, double* c, int64_t ldc) {
  if (M < 0 || N < 0 || R < 0 || ldc < N) return 1;
  if (b_sj != 1) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i) {
      for (int64_t j = 0; j < N; ++j) {
        double s = 0.0;
        for (int64_t r = 0; r < R; ++r)
          s += pair_term(a, adt, i * a_si + r * a_sr, b, bdt, r * b_sr + j * b_sj, mode);
        c[i * ldc + j] = s;
      }
    }
  } else {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i) {
      double* row = c + i * ldc;
      for (int64_t j = 0; j < N; ++j) row[j] = 0.0;
      for (int64_t r = 0; r < R; ++r)
        for (int64_t j = 0; j < N; ++j)
          row[j] += pair_term(a, adt, i * a_si + r * a_sr, b, bdt, r * b_sr + j, mode);
    }
  }
  return 0;
}

/* Selected outputs only: out[p] = C[ii[p], jj[p]], for checks at full size. */
int orc_matmul_sampled(int64_t R,
                       const void* a, int adt, int64_t a_si, int64_t a_sr,
                       const void* b, int bdt, int64_t b_sr, int64_t b_sj,
                       int mode, const int64_t* ii, const int64_t* jj, int64_t P, double* out) {
  if (R < 0 || P < 0) return 1;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t p = 0; p < P; ++p) {
    double s = 0.0;
    for (int64_t r = 0; r < R; ++r)
      s += pair_term(a, adt, ii[p] * a_si + r * a_sr, b, bdt, r * b_sr + jj[p] * b_sj, mode);
    out[p] = s;
  }
  return 0;
}

int orc_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Thread count for later calls (timing of the oracle on one thread). */
void orc_set_num_threads(int n) {
#ifdef _OPENMP
  extern void omp_set_num_threads(int);
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
