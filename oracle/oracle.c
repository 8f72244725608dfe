/*
 * oracle.c -- plain, slow, obviously correct CPU reference for the TN GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The GPU library never
 * links, calls or shares code with it, and this file includes nothing from
 * the GPU side.
 *
 * What it computes (cited by page and section):
 *   - "hello-gpu, chapter 11 (GEMM-like)", section 11.1, the dot-product
 *     equation: C[m,n] = sum over k = 0..K-1 of A[m,k] * B[k,n], with no
 *     scaling, transpose or addend; the partial sum starts at 0 and k runs
 *     upwards (Fig. 11.1).
 *   - "FP16 GEMM optimisation on AMD RDNA 3 and RDNA 4", section "What we
 *     compute": A is row-major M x K, B is column-major (each of its N
 *     columns holds K contiguous elements), and C is column-major with
 *     leading dimension ldc (= M for a packed C).
 *   - section 11.4 of the hello-gpu chapter: the reference accumulates in
 *     double precision on the CPU.
 *
 * So the oracle is that definition written out: every input element is
 * decoded exactly to binary64 with this file's own decoders, the products
 * are summed in binary64 with k ascending, and the result is kept in
 * binary64.  For the FP8 path the per-tensor scales are applied afterwards
 * as one binary64 product scale_a * scale_b.
 *
 * Codecs (written from the published format definitions):
 *   IEEE 754 binary16  1-5-10, bias 15, subnormals, Inf/NaN
 *   bfloat16           1-8-7,  bias 127 (the top half of a binary32)
 *   OCP FP8 E4M3FN     1-4-3,  bias 7, subnormal step 2^-9, no Inf,
 *                      S.1111.111 is NaN, largest finite 448
 * Encoders round to nearest, ties to even.  binary16 and bfloat16 overflow
 * to +-Inf as IEEE rounding does; E4M3FN saturates to +-448.
 *
 * Attention (oracle_attention_rows): the chapter summary of the hello-gpu
 * GEMM chapter names the next step as joining the matrix product with softmax
 * so the intermediate result need not be written back; the TileLang attention
 * page motivates the same fusion for QK^T.  The pages define no formula for
 * it, so the oracle is the textbook definition of softmax attention for one
 * query row i of one head:
 *     s_n = scale * sum_d Q[i,d] * K[n,d]            (d ascending, binary64)
 *     w_n = exp(s_n - max_n s_n)                     (libm exp, binary64)
 *     O[i,d] = (sum_n w_n * V[n,d]) / (sum_n w_n)    (n ascending)
 * with V given column-major (Vt[d*ldv + n], the K-contiguous operand of the
 * TN product O = P V).  Subtracting the row maximum changes nothing
 * mathematically and keeps exp in range.
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -pthread (no -ffast-math: the sum
 * order must stay exactly k ascending).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_FMT_F16 = 0, ORACLE_FMT_E4M3FN = 1, ORACLE_FMT_BF16 = 2 };

/* ---------------------------------------------------------------- decoders */

static double decode_f16(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int m = h & 0x3ff;
  double v;
  if (e == 0) {
    v = ldexp((double)m, -24); /* subnormal: m * 2^(1-15-10) */
  } else if (e == 31) {
    v = (m == 0) ? INFINITY : NAN;
  } else {
    v = ldexp((double)(1024 + m), e - 25); /* (1 + m/2^10) * 2^(e-15) */
  }
  return sign ? -v : v;
}

static double decode_bf16(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 7) & 0xff;
  int m = h & 0x7f;
  double v;
  if (e == 0) {
    v = ldexp((double)m, -133); /* m * 2^(1-127-7) */
  } else if (e == 255) {
    v = (m == 0) ? INFINITY : NAN;
  } else {
    v = ldexp((double)(128 + m), e - 134); /* (1 + m/2^7) * 2^(e-127) */
  }
  return sign ? -v : v;
}

static double decode_e4m3fn(uint8_t b) {
  int sign = (b >> 7) & 1;
  int e = (b >> 3) & 0xf;
  int m = b & 0x7;
  double v;
  if (e == 15 && m == 7) {
    v = NAN; /* the only NaN pattern; E4M3FN has no infinities */
  } else if (e == 0) {
    v = ldexp((double)m, -9); /* m * 2^(1-7-3) */
  } else {
    v = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
  }
  return sign ? -v : v;
}

static double decode_one(int fmt, const void *base, int64_t idx) {
  switch (fmt) {
  case ORACLE_FMT_F16: return decode_f16(((const uint16_t *)base)[idx]);
  case ORACLE_FMT_BF16: return decode_bf16(((const uint16_t *)base)[idx]);
  case ORACLE_FMT_E4M3FN: return decode_e4m3fn(((const uint8_t *)base)[idx]);
  default: return NAN;
  }
}

/* ---------------------------------------------------------------- encoders */

/*
 * Round |x| (finite, > 0) to the nearest value with `mbits` fraction bits and
 * minimum normal exponent `emin`; ties go to the even significand.  Returns
 * the rounded magnitude as a double (exact: every target value is a double).
 */
static double round_to_format(double ax, int mbits, int emin) {
  int e2;
  frexp(ax, &e2);          /* ax = f * 2^e2, f in [0.5, 1) */
  int e = e2 - 1;          /* ax in [2^e, 2^(e+1)) */
  if (e < emin) e = emin;  /* subnormal range shares the smallest quantum */
  double quantum = ldexp(1.0, e - mbits);
  double r = ax / quantum; /* exact: division by a power of two */
  double fl = floor(r);
  double frac = r - fl;
  double n;
  if (frac > 0.5) n = fl + 1.0;
  else if (frac < 0.5) n = fl;
  else n = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0; /* tie: to even */
  return n * quantum;
}

/* Pack an exactly representable magnitude into sign/exponent/fraction bits. */
static uint32_t pack_bits(double av, int sign, int ebits, int mbits, int bias) {
  uint32_t s = (uint32_t)sign << (ebits + mbits);
  if (av == 0.0) return s;
  int emin = 1 - bias;
  int e2;
  double f = frexp(av, &e2);
  int e = e2 - 1;
  if (e < emin) { /* subnormal: value = mant * 2^(emin - mbits) */
    uint32_t mant = (uint32_t)ldexp(av, mbits - emin);
    return s | mant;
  }
  uint32_t mant = (uint32_t)ldexp(f * 2.0 - 1.0, mbits);
  return s | ((uint32_t)(e + bias) << mbits) | mant;
}

static uint16_t encode_f16(double x) {
  if (isnan(x)) return 0x7e00;
  int sign = signbit(x) ? 1 : 0;
  double ax = fabs(x);
  if (isinf(ax)) return (uint16_t)((sign << 15) | 0x7c00);
  double r = round_to_format(ax, 10, -14);
  if (r >= 65536.0) return (uint16_t)((sign << 15) | 0x7c00); /* overflow */
  return (uint16_t)pack_bits(r, sign, 5, 10, 15);
}

static uint16_t encode_bf16(double x) {
  if (isnan(x)) return 0x7fc0;
  int sign = signbit(x) ? 1 : 0;
  double ax = fabs(x);
  if (isinf(ax)) return (uint16_t)((sign << 15) | 0x7f80);
  double r = round_to_format(ax, 7, -126);
  if (r >= ldexp(1.0, 128)) return (uint16_t)((sign << 15) | 0x7f80);
  return (uint16_t)pack_bits(r, sign, 8, 7, 127);
}

static uint8_t encode_e4m3fn(double x) {
  if (isnan(x)) return 0x7f;
  int sign = signbit(x) ? 1 : 0;
  double ax = fabs(x);
  double r = isinf(ax) ? 448.0 : round_to_format(ax, 3, -6);
  if (r > 448.0) r = 448.0; /* saturate: 1.1111.110 is the largest finite */
  return (uint8_t)pack_bits(r, sign, 4, 3, 7);
}

/* ------------------------------------------------------------- public codecs */

int oracle_decode(int fmt, const void *in, double *out, int64_t n) {
  if (fmt != ORACLE_FMT_F16 && fmt != ORACLE_FMT_BF16 && fmt != ORACLE_FMT_E4M3FN)
    return 1;
  for (int64_t i = 0; i < n; ++i) out[i] = decode_one(fmt, in, i);
  return 0;
}

int oracle_encode(int fmt, const double *in, void *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) {
    switch (fmt) {
    case ORACLE_FMT_F16: ((uint16_t *)out)[i] = encode_f16(in[i]); break;
    case ORACLE_FMT_BF16: ((uint16_t *)out)[i] = encode_bf16(in[i]); break;
    case ORACLE_FMT_E4M3FN: ((uint8_t *)out)[i] = encode_e4m3fn(in[i]); break;
    default: return 1;
    }
  }
  return 0;
}

/* ------------------------------------------------------------------- GEMM */

typedef struct {
  const double *a; /* M x K, decoded, packed row-major */
  const double *b; /* N x K, decoded, one packed row per column of B */
  double *c;
  int64_t M, K, ldc, n_begin, n_end;
  double scale;
} gemm_job;

static void *gemm_worker(void *arg) {
  const gemm_job *j = (const gemm_job *)arg;
  for (int64_t n = j->n_begin; n < j->n_end; ++n) {
    const double *bcol = j->b + n * j->K;
    for (int64_t m = 0; m < j->M; ++m) {
      const double *arow = j->a + m * j->K;
      double acc = 0.0; /* the partial sum starts at zero ... */
      for (int64_t k = 0; k < j->K; ++k)
        acc += arow[k] * bcol[k]; /* ... and k runs upwards */
      j->c[m + n * j->ldc] = acc * j->scale;
    }
  }
  return NULL;
}

/*
 * General strides (element units, all >= 0):
 *   C(m, n) = scale * sum_k A(m, k) * B(k, n)                      (binary64)
 *   A(m, k) = A[m*sam + k*sak],  B(k, n) = B[k*sbk + n*sbn],
 *   C(m, n) is stored at C[m*scm + n*scn].
 * The row-major storage of section 11.1 of the hello-gpu chapter (A[m*K + k],
 * B[k*N + n], C[m*N + n]) and the TN layout below are special cases.  fmt
 * selects the element format of A and B.  Returns 0 on success.
 */
int oracle_gemm_strided(int fmt, const void *A, int64_t sam, int64_t sak,
                        const void *B, int64_t sbk, int64_t sbn,
                        double *C, int64_t scm, int64_t scn,
                        int64_t M, int64_t N, int64_t K, double scale, int nthreads) {
  if (M < 0 || N < 0 || K < 0 || sam < 0 || sak < 0 || sbk < 0 || sbn < 0 || scm < 0 ||
      scn < 0)
    return 1;
  if (fmt != ORACLE_FMT_F16 && fmt != ORACLE_FMT_BF16 && fmt != ORACLE_FMT_E4M3FN)
    return 1;
  if (M == 0 || N == 0) return 0;
  double *a = (double *)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
  double *b = (double *)malloc(sizeof(double) * (size_t)(N * K > 0 ? N * K : 1));
  double *c = (double *)malloc(sizeof(double) * (size_t)(M * N));
  if (!a || !b || !c) { free(a); free(b); free(c); return 2; }
  for (int64_t m = 0; m < M; ++m)
    for (int64_t k = 0; k < K; ++k) a[m * K + k] = decode_one(fmt, A, m * sam + k * sak);
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) b[n * K + k] = decode_one(fmt, B, k * sbk + n * sbn);

  if (nthreads < 1) nthreads = 1;
  if (nthreads > N) nthreads = (int)N;
  pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
  gemm_job *jobs = (gemm_job *)malloc(sizeof(gemm_job) * (size_t)nthreads);
  int rc = 0;
  if (!tid || !jobs) rc = 2;
  int started = 0;
  for (int t = 0; rc == 0 && t < nthreads; ++t) {
    jobs[t].a = a; jobs[t].b = b; jobs[t].c = c;
    jobs[t].M = M; jobs[t].K = K; jobs[t].ldc = M; jobs[t].scale = scale;
    jobs[t].n_begin = N * t / nthreads;
    jobs[t].n_end = N * (t + 1) / nthreads;
    if (nthreads == 1) { gemm_worker(&jobs[t]); continue; }
    if (pthread_create(&tid[t], NULL, gemm_worker, &jobs[t]) != 0) { rc = 3; break; }
    ++started;
  }
  for (int t = 0; t < started; ++t) pthread_join(tid[t], NULL);
  if (rc == 0)
    for (int64_t n = 0; n < N; ++n)
      for (int64_t m = 0; m < M; ++m) C[m * scm + n * scn] = c[m + n * M];
  free(jobs); free(tid); free(a); free(b); free(c);
  return rc;
}

/*
 * C[m + n*ldc] = scale * sum_k A[m*lda + k] * B[n*ldb + k]  (binary64): the TN
 * layout of "FP16 GEMM optimisation on AMD RDNA 3 and RDNA 4", section "What
 * we compute".  Returns 0 on success.
 */
int oracle_gemm_tn(int fmt, const void *A, const void *B, double *C,
                   int64_t M, int64_t N, int64_t K,
                   int64_t lda, int64_t ldb, int64_t ldc,
                   double scale, int nthreads) {
  if (M < 0 || N < 0 || K < 0 || lda < K || ldb < K || ldc < M) return 1;
  return oracle_gemm_strided(fmt, A, lda, 1, B, 1, ldb, C, 1, ldc, M, N, K, scale, nthreads);
}

/*
 * Individual entries of the same product, for checks at sizes where the full
 * product is too slow: out[i] = scale * sum_k A[ms[i]*lda + k] * B[ns[i]*ldb + k].
 */
int oracle_gemm_tn_entries(int fmt, const void *A, const void *B, int64_t K,
                           int64_t lda, int64_t ldb, const int64_t *ms,
                           const int64_t *ns, int64_t count, double scale,
                           double *out) {
  if (K < 0 || lda < K || ldb < K) return 1;
  if (fmt != ORACLE_FMT_F16 && fmt != ORACLE_FMT_BF16 && fmt != ORACLE_FMT_E4M3FN)
    return 1;
  for (int64_t i = 0; i < count; ++i) {
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k)
      acc += decode_one(fmt, A, ms[i] * lda + k) * decode_one(fmt, B, ns[i] * ldb + k);
    out[i] = acc * scale;
  }
  return 0;
}

/* Individual entries with general strides (see oracle_gemm_strided). */
int oracle_gemm_strided_entries(int fmt, const void *A, int64_t sam, int64_t sak,
                                const void *B, int64_t sbk, int64_t sbn, int64_t K,
                                const int64_t *ms, const int64_t *ns, int64_t count,
                                double scale, double *out) {
  if (K < 0 || sam < 0 || sak < 0 || sbk < 0 || sbn < 0) return 1;
  if (fmt != ORACLE_FMT_F16 && fmt != ORACLE_FMT_BF16 && fmt != ORACLE_FMT_E4M3FN)
    return 1;
  for (int64_t i = 0; i < count; ++i) {
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k)
      acc += decode_one(fmt, A, ms[i] * sam + k * sak) * decode_one(fmt, B, k * sbk + ns[i] * sbn);
    out[i] = acc * scale;
  }
  return 0;
}

/* ---------------------------------------------------------------- attention */

typedef struct {
  const double *q, *k, *vt; /* decoded: rows x D, N x D, D x N */
  double *o;                /* rows x D */
  int64_t N, D, r_begin, r_end;
  double scale;
} attn_job;

static void *attn_worker(void *arg) {
  const attn_job *j = (const attn_job *)arg;
  double *s = (double *)malloc(sizeof(double) * (size_t)(j->N > 0 ? j->N : 1));
  if (!s) return (void *)1;
  for (int64_t r = j->r_begin; r < j->r_end; ++r) {
    const double *qr = j->q + r * j->D;
    double mx = -INFINITY;
    for (int64_t n = 0; n < j->N; ++n) {
      const double *kr = j->k + n * j->D;
      double acc = 0.0;
      for (int64_t d = 0; d < j->D; ++d) acc += qr[d] * kr[d];
      s[n] = acc * j->scale;
      if (s[n] > mx) mx = s[n];
    }
    double z = 0.0;
    for (int64_t n = 0; n < j->N; ++n) {
      s[n] = exp(s[n] - mx);
      z += s[n];
    }
    for (int64_t d = 0; d < j->D; ++d) {
      const double *vr = j->vt + d * j->N;
      double acc = 0.0;
      for (int64_t n = 0; n < j->N; ++n) acc += s[n] * vr[n];
      j->o[r * j->D + d] = acc / z;
    }
  }
  free(s);
  return NULL;
}

/*
 * Softmax attention of the query rows rows[0..count-1] of one head (binary16
 * inputs): O[r*D + d] for r < count, as defined in the header.  Q[i*ldq + d],
 * K[n*ldk + d], Vt[d*ldv + n].  N >= 1.  Returns 0 on success.
 */
int oracle_attention_rows(const void *Q, const void *K, const void *Vt, int64_t N, int64_t D,
                          int64_t ldq, int64_t ldk, int64_t ldv, const int64_t *rows,
                          int64_t count, double scale, double *O, int nthreads) {
  if (N < 1 || D < 1 || count < 0 || ldq < D || ldk < D || ldv < N) return 1;
  double *q = (double *)malloc(sizeof(double) * (size_t)((count > 0 ? count : 1) * D));
  double *k = (double *)malloc(sizeof(double) * (size_t)(N * D));
  double *vt = (double *)malloc(sizeof(double) * (size_t)(N * D));
  if (!q || !k || !vt) { free(q); free(k); free(vt); return 2; }
  for (int64_t r = 0; r < count; ++r)
    for (int64_t d = 0; d < D; ++d) q[r * D + d] = decode_one(ORACLE_FMT_F16, Q, rows[r] * ldq + d);
  for (int64_t n = 0; n < N; ++n)
    for (int64_t d = 0; d < D; ++d) k[n * D + d] = decode_one(ORACLE_FMT_F16, K, n * ldk + d);
  for (int64_t d = 0; d < D; ++d)
    for (int64_t n = 0; n < N; ++n) vt[d * N + n] = decode_one(ORACLE_FMT_F16, Vt, d * ldv + n);

  if (nthreads < 1) nthreads = 1;
  if (nthreads > count) nthreads = (int)(count > 0 ? count : 1);
  pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
  attn_job *jobs = (attn_job *)malloc(sizeof(attn_job) * (size_t)nthreads);
  int rc = 0;
  if (!tid || !jobs) rc = 2;
  int started = 0;
  for (int t = 0; rc == 0 && t < nthreads; ++t) {
    jobs[t].q = q; jobs[t].k = k; jobs[t].vt = vt; jobs[t].o = O;
    jobs[t].N = N; jobs[t].D = D; jobs[t].scale = scale;
    jobs[t].r_begin = count * t / nthreads;
    jobs[t].r_end = count * (t + 1) / nthreads;
    if (nthreads == 1) { if (attn_worker(&jobs[t])) rc = 2; continue; }
    if (pthread_create(&tid[t], NULL, attn_worker, &jobs[t]) != 0) { rc = 3; break; }
    ++started;
  }
  for (int t = 0; t < started; ++t) {
    void *ret = NULL;
    pthread_join(tid[t], &ret);
    if (ret) rc = 2;
  }
  free(jobs); free(tid); free(q); free(k); free(vt);
  return rc;
}
