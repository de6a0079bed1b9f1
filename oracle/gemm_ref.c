/*
 * GEMM oracle (GO): D = A * B^T + C, a plain triple loop in fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Built with gcc (never hipcc), loaded through
 * ctypes by oracle/gemm.py.  It shares no code, header, table or helper with
 * the HIP library; the only thing both sides see is the input bytes.
 *
 * What it computes, and from where:
 *  - "CuTe 中 A、B 如何加载到 MMA 寄存器", section 1: D = A x B + C with A
 *    indexed (M,K) and B indexed (N,K), i.e. D(m,n) = C(m,n) + sum_k
 *    A(m,k) B(n,k).
 *  - "数据布局及其记号", section "Shape-Stride 模型": every operand element is
 *    found by the dot product of its index with the strides (in elements);
 *    transposed and batched views are nothing but other strides.
 *  - same page, section "Replication 与 Offset" (block-scaled MMA):
 *    A_real[m,k] = A_low[m,k] * SFA[m, k // K_blk], B_real likewise with
 *    SFB[n, k // K_blk] (B stored (N,K) here), D = C + A_real x B_real^T.
 *    MXFP8: A_low, B_low are FP8 E4M3 and the scales E8M0 with K_blk = 32.
 *    The pages only name these encodings; the decoders follow the OCP
 *    Microscaling Formats v1.0 definitions (E4M3: bias 7, no infinities,
 *    S.1111.111 is NaN, max 448; E8M0: 2^(b-127), 255 is NaN).
 *  - fp16 is IEEE 754 binary16 (bias 15, subnormals, inf/NaN); encoding
 *    rounds to nearest, ties to even, overflow to infinity.
 *  - NVFP4 (same section): A_low, B_low FP4 E2M1 and one E4M3 scale per 16
 *    consecutive K.  E2M1 follows the OCP MX v1.0 definition (bias 1, one
 *    significand bit, subnormal 0.5, max 6, no infinities or NaN).  E2M1
 *    operands are packed two per byte along K: element offset o (in
 *    elements, from the descriptor's strides) is byte o / 2, low nibble for
 *    even o, high nibble for odd o.
 *  - MXFP6 (the block-scaled product with 6-bit data and E8M0 scales per
 *    32 K): FP6 E2M3 (bias 1, three significand bits, subnormals m/8, max
 *    7.5) or FP6 E3M2 (bias 3, two significand bits, subnormals m/16, max
 *    28), both without infinities or NaN (OCP MX v1.0).  Packed along K as
 *    one little-endian bit stream: element offset o occupies bits 6o ..
 *    6o+5, bit 0 being the least significant bit of byte 0 (four elements
 *    in three bytes).
 *  - bf16 (the same product in the other 16-bit format; the pages name only
 *    fp16) is the upper half of IEEE binary32: bias 127, 7 stored
 *    significand bits, subnormals, inf/NaN; encoded the same way.
 *
 * Summation: fp64, k ascending, one output element at a time.  Alongside the
 * exact-ish value it returns S = sum_k |A(m,k) B(n,k)| (fp64), which the
 * acceptance bound |D - D_ref| <= 2^-10 |D_ref| + 2^-13 S needs (2^-7 in
 * place of 2^-10 for a bf16 result: twice the format's unit roundoff).
 *
 * Parallelism: pthreads over output rows only; the inner loop stays plain.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { GO_F16 = 1, GO_F32 = 2, GO_E4M3 = 3, GO_E8M0 = 4, GO_BF16 = 5, GO_E2M1 = 6, GO_E2M3 = 7, GO_E3M2 = 8 };

typedef struct {
  const void* data; /* NULL: absent (C = 0, or no scales) */
  int32_t dtype;
  int32_t rank;      /* 2: (rows, cols), 3: (batch, rows, cols) */
  int64_t shape[3];
  int64_t stride[3]; /* in elements */
} go_tensor;

/* ------------------------------------------------------------------ codecs */

double go_f16_decode(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 0x1f, f = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24);                 /* subnormal: f * 2^-24 */
  else if (e == 0x1f)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(0x400 | f), e - 25);    /* (1 + f/1024) * 2^(e-15) */
  return s ? -v : v;
}

uint16_t go_f16_encode(double x) {
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  if (isnan(x)) return 0x7e00;
  double a = fabs(x);
  /* 65520 is halfway between the largest finite 65504 (odd significand)
   * and 65536; ties-to-even takes it, and everything above, to infinity. */
  if (a >= 65520.0) return sign | 0x7c00;
  if (a < ldexp(1.0, -14)) {
    /* subnormal range: a multiple of 2^-24; rint() is ties-to-even */
    int q = (int)rint(ldexp(a, 24));           /* q == 1024 is the smallest normal */
    return sign | (uint16_t)q;
  }
  int e2;
  frexp(a, &e2);                               /* a in [2^(e2-1), 2^e2) */
  int E = e2 - 1;
  int q = (int)rint(ldexp(a, 10 - E));         /* significand in [1024, 2048] */
  if (q == 2048) { q = 1024; E += 1; }
  if (E > 15) return sign | 0x7c00;
  return sign | (uint16_t)(((E + 15) << 10) | (q - 1024));
}

double go_e4m3_decode(uint8_t b) {
  int s = b >> 7, e = (b >> 3) & 0xf, m = b & 7;
  double v;
  if (e == 0xf && m == 7)
    return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);                  /* (m/8) * 2^-6 */
  else
    v = ldexp((double)(8 | m), e - 10);        /* (1 + m/8) * 2^(e-7) */
  return s ? -v : v;
}

double go_e8m0_decode(uint8_t b) {
  if (b == 0xff) return NAN;
  return ldexp(1.0, (int)b - 127);
}

/* bf16: sign, 8-bit exponent (bias 127), 7-bit fraction */
double go_bf16_decode(uint16_t h) {
  int sgn = h >> 15, e = (h >> 7) & 0xFF, f = h & 0x7F;
  double v;
  if (e == 0)
    v = ldexp((double)f, -133);                /* subnormal: f * 2^-133 */
  else if (e == 255)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(0x80 | f), e - 134);    /* (1 + f/128) * 2^(e-127) */
  return sgn ? -v : v;
}

uint16_t go_bf16_encode(double x) {
  if (isnan(x)) return 0x7FC0;
  uint16_t sgn = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (a < ldexp(1.0, -126)) {
    /* subnormal range, step 2^-133; q == 128 is the smallest normal */
    int q = (int)rint(ldexp(a, 133));
    return sgn | (uint16_t)q;
  }
  int E;
  frexp(a, &E);                                /* a in [2^(E-1), 2^E) */
  if (E - 1 > 127) return sgn | 0x7F80;
  int q = (int)rint(ldexp(a, 8 - E));          /* significand in [128, 256] */
  int e = E - 1;
  if (q == 256) {
    q = 128;
    e += 1;
  }
  if (e > 127) return sgn | 0x7F80;            /* rounded past the largest finite */
  return sgn | (uint16_t)((e + 127) << 7) | (uint16_t)(q - 128);
}

/* E2M1: sign, 2-bit exponent (bias 1), 1-bit fraction */
double go_e2m1_decode(uint8_t c) {
  int sgn = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
  double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return sgn ? -v : v;
}

/* E2M3: sign, 2-bit exponent (bias 1), 3-bit fraction */
double go_e2m3_decode(uint8_t c) {
  int sgn = (c >> 5) & 1, e = (c >> 3) & 3, m = c & 7;
  double v = e == 0 ? m / 8.0 : ldexp(1.0 + m / 8.0, e - 1);
  return sgn ? -v : v;
}

/* E3M2: sign, 3-bit exponent (bias 3), 2-bit fraction */
double go_e3m2_decode(uint8_t c) {
  int sgn = (c >> 5) & 1, e = (c >> 2) & 7, m = c & 3;
  double v = e == 0 ? ldexp(m / 4.0, -2) : ldexp(1.0 + m / 4.0, e - 3);
  return sgn ? -v : v;
}

/* the 6-bit code at element offset o of a packed bit stream */
uint8_t go_fp6_code(const uint8_t* bytes, int64_t o) {
  const int64_t bit = 6 * o;
  const int sh = (int)(bit & 7);
  unsigned v = bytes[bit >> 3] >> sh;
  if (sh > 2) v |= (unsigned)bytes[(bit >> 3) + 1] << (8 - sh);
  return (uint8_t)(v & 63);
}

/* decoding tables, filled once from the functions above */
static double g_f16_tab[65536];
static double g_bf16_tab[65536];
static double g_e4m3_tab[256];
static double g_e8m0_tab[256];
static double g_e2m1_tab[16];
static double g_e2m3_tab[64];
static double g_e3m2_tab[64];
static pthread_once_t g_tab_once = PTHREAD_ONCE_INIT;

static void fill_tables(void) {
  for (int i = 0; i < 65536; ++i) {
    g_f16_tab[i] = go_f16_decode((uint16_t)i);
    g_bf16_tab[i] = go_bf16_decode((uint16_t)i);
  }
  for (int i = 0; i < 256; ++i) {
    g_e4m3_tab[i] = go_e4m3_decode((uint8_t)i);
    g_e8m0_tab[i] = go_e8m0_decode((uint8_t)i);
  }
  for (int i = 0; i < 16; ++i) g_e2m1_tab[i] = go_e2m1_decode((uint8_t)i);
  for (int i = 0; i < 64; ++i) {
    g_e2m3_tab[i] = go_e2m3_decode((uint8_t)i);
    g_e3m2_tab[i] = go_e3m2_decode((uint8_t)i);
  }
}

/* ------------------------------------------------------- element addressing */

/* address = b*s0 + i*s1 + j*s2 for rank 3, i*s0 + j*s1 for rank 2 (the
 * batch index is ignored: a rank-2 operand is the same matrix for every
 * batch) */
static int64_t offset_of(const go_tensor* t, int64_t b, int64_t i, int64_t j) {
  if (t->rank == 3) return b * t->stride[0] + i * t->stride[1] + j * t->stride[2];
  return i * t->stride[0] + j * t->stride[1];
}

static double element(const go_tensor* t, int64_t b, int64_t i, int64_t j) {
  int64_t o = offset_of(t, b, i, j);
  switch (t->dtype) {
    case GO_F16: return g_f16_tab[((const uint16_t*)t->data)[o]];
    case GO_BF16: return g_bf16_tab[((const uint16_t*)t->data)[o]];
    case GO_F32: return (double)((const float*)t->data)[o];
    case GO_E4M3: return g_e4m3_tab[((const uint8_t*)t->data)[o]];
    case GO_E8M0: return g_e8m0_tab[((const uint8_t*)t->data)[o]];
    case GO_E2M1: {
      const uint8_t byte = ((const uint8_t*)t->data)[o >> 1];
      return g_e2m1_tab[(o & 1) ? byte >> 4 : byte & 15];
    }
    case GO_E2M3: return g_e2m3_tab[go_fp6_code((const uint8_t*)t->data, o)];
    case GO_E3M2: return g_e3m2_tab[go_fp6_code((const uint8_t*)t->data, o)];
    default: return NAN;
  }
}

static int64_t rows_of(const go_tensor* t) { return t->shape[t->rank - 2]; }
static int64_t cols_of(const go_tensor* t) { return t->shape[t->rank - 1]; }

typedef struct {
  const go_tensor *a, *b, *c, *sfa, *sfb;
  int32_t block_k;
  int64_t K;
  int32_t out_dtype; /* GO_F16 or GO_BF16: the format D is rounded to */
} problem;

static uint16_t encode_out(const problem* p, double v) {
  return p->out_dtype == GO_BF16 ? go_bf16_encode(v) : go_f16_encode(v);
}

/* one output element: fp64 sum over k ascending, plus sum of |products| */
static void one_point(const problem* p, int64_t bi, int64_t m, int64_t n,
                      double* value, double* absum) {
  double acc = 0.0, s = 0.0;
  const int mx = p->sfa != NULL;
  for (int64_t k = 0; k < p->K; ++k) {
    double x = element(p->a, bi, m, k);
    double y = element(p->b, bi, n, k);
    if (mx) {
      x *= element(p->sfa, bi, m, k / p->block_k);
      y *= element(p->sfb, bi, n, k / p->block_k);
    }
    double prod = x * y;
    acc += prod;
    s += fabs(prod);
  }
  if (p->c) acc = element(p->c, bi, m, n) + acc;
  *value = acc;
  *absum = s;
}

static int setup(problem* p, const go_tensor* a, const go_tensor* b, const go_tensor* c,
                 const go_tensor* sfa, const go_tensor* sfb, int32_t block_k, int32_t out_dtype) {
  if (out_dtype != GO_F16 && out_dtype != GO_BF16) return -2;
  p->out_dtype = out_dtype;
  pthread_once(&g_tab_once, fill_tables);
  if (!a || !b || !a->data || !b->data) return -1;
  if (a->rank < 2 || a->rank > 3 || b->rank < 2 || b->rank > 3) return -3;
  if (cols_of(a) != cols_of(b)) return -3;
  p->a = a;
  p->b = b;
  p->c = (c && c->data) ? c : NULL;
  p->sfa = (sfa && sfa->data) ? sfa : NULL;
  p->sfb = (sfb && sfb->data) ? sfb : NULL;
  if ((p->sfa == NULL) != (p->sfb == NULL)) return -2;
  if (p->sfa && block_k <= 0) return -3;
  p->block_k = block_k;
  p->K = cols_of(a);
  return 0;
}

/* ---------------------------------------------------------- sampled points */

typedef struct {
  const problem* p;
  const int64_t* pts; /* (count, 3): batch, m, n */
  int64_t lo, hi;
  uint16_t* d;
  double* ref;
  double* absum;
} point_job;

static void* point_worker(void* arg) {
  point_job* j = (point_job*)arg;
  for (int64_t i = j->lo; i < j->hi; ++i) {
    double v, s;
    one_point(j->p, j->pts[3 * i], j->pts[3 * i + 1], j->pts[3 * i + 2], &v, &s);
    if (j->d) j->d[i] = encode_out(j->p, v);
    if (j->ref) j->ref[i] = v;
    if (j->absum) j->absum[i] = s;
  }
  return NULL;
}

static int run_points(const problem* p, const int64_t* pts, int64_t count, uint16_t* d,
                      double* ref, double* absum, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 512) nthreads = 512;
  if ((int64_t)nthreads > count) nthreads = count > 0 ? (int)count : 1;
  pthread_t th[512];
  point_job jobs[512];
  for (int t = 0; t < nthreads; ++t) {
    jobs[t].p = p;
    jobs[t].pts = pts;
    jobs[t].lo = count * t / nthreads;
    jobs[t].hi = count * (t + 1) / nthreads;
    jobs[t].d = d;
    jobs[t].ref = ref;
    jobs[t].absum = absum;
  }
  for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, point_worker, &jobs[t]);
  point_worker(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
  return 0;
}

/* Values at the listed (batch, m, n) points only: d (codes of the result
 * rounded to out_dtype), ref (fp64 before rounding) and absum may each be
 * NULL. */
int go_gemm_points(const go_tensor* a, const go_tensor* b, const go_tensor* c,
                   const go_tensor* sfa, const go_tensor* sfb, int32_t block_k,
                   const int64_t* pts, int64_t count, uint16_t* d, double* ref,
                   double* absum, int32_t nthreads, int32_t out_dtype) {
  problem p;
  int rc = setup(&p, a, b, c, sfa, sfb, block_k, out_dtype);
  if (rc) return rc;
  return run_points(&p, pts, count, d, ref, absum, nthreads);
}

/* ------------------------------------------------------------- full output */

typedef struct {
  const problem* p;
  int64_t batch, M, N;
  int64_t row_lo, row_hi; /* over batch*M */
  uint16_t* d;
  double* ref;
  double* absum;
} row_job;

static void* row_worker(void* arg) {
  row_job* j = (row_job*)arg;
  for (int64_t r = j->row_lo; r < j->row_hi; ++r) {
    int64_t bi = r / j->M, m = r % j->M;
    for (int64_t n = 0; n < j->N; ++n) {
      double v, s;
      one_point(j->p, bi, m, n, &v, &s);
      int64_t o = r * j->N + n;
      if (j->d) j->d[o] = encode_out(j->p, v);
      if (j->ref) j->ref[o] = v;
      if (j->absum) j->absum[o] = s;
    }
  }
  return NULL;
}

/* Every output element, written densely as (batch, M, N) row-major. */
int go_gemm(const go_tensor* a, const go_tensor* b, const go_tensor* c, const go_tensor* sfa,
            const go_tensor* sfb, int32_t block_k, int64_t batch, uint16_t* d, double* ref,
            double* absum, int32_t nthreads, int32_t out_dtype) {
  problem p;
  int rc = setup(&p, a, b, c, sfa, sfb, block_k, out_dtype);
  if (rc) return rc;
  int64_t M = rows_of(a), N = rows_of(b), rows = batch * M;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 512) nthreads = 512;
  if ((int64_t)nthreads > rows) nthreads = rows > 0 ? (int)rows : 1;
  pthread_t th[512];
  row_job jobs[512];
  for (int t = 0; t < nthreads; ++t) {
    jobs[t].p = &p;
    jobs[t].batch = batch;
    jobs[t].M = M;
    jobs[t].N = N;
    jobs[t].row_lo = rows * t / nthreads;
    jobs[t].row_hi = rows * (t + 1) / nthreads;
    jobs[t].d = d;
    jobs[t].ref = ref;
    jobs[t].absum = absum;
  }
  for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, row_worker, &jobs[t]);
  row_worker(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
  return 0;
}

/* ----------------------------------------------------------- acceptance */

/* Per element: |D - D_ref| <= 2^-r |D_ref| + 2^-13 S, where D_ref is the
 * fp64 value rounded to the output format and both D and D_ref are decoded
 * from it; r = 10 for fp16 and 7 for bf16 (twice the format's unit
 * roundoff, 2^-11 and 2^-8).
 * A NaN on either side fails.  Returns the number of violations and
 * writes the index of the worst one (largest excess over the bound) and
 * the excess ratio |D - D_ref| / bound. */
int64_t go_check(const uint16_t* d, const uint16_t* d_ref, const double* absum, int64_t count,
                 int64_t* worst_index, double* worst_ratio, int32_t out_dtype) {
  pthread_once(&g_tab_once, fill_tables);
  const double* tab = out_dtype == GO_BF16 ? g_bf16_tab : g_f16_tab;
  const int rel = out_dtype == GO_BF16 ? -7 : -10;
  int64_t bad = 0, wi = -1;
  double wr = 0.0;
  for (int64_t i = 0; i < count; ++i) {
    double x = tab[d[i]], r = tab[d_ref[i]];
    double bound = ldexp(fabs(r), rel) + ldexp(absum[i], -13);
    double err = fabs(x - r);
    int ok;
    double ratio;
    if (isnan(x) || isnan(r)) {
      ok = 0;
      ratio = INFINITY;
    } else if (isinf(r) || isinf(x)) {
      ok = (x == r);
      ratio = ok ? 0.0 : INFINITY;
    } else {
      ok = err <= bound;
      ratio = bound > 0 ? err / bound : (err > 0 ? INFINITY : 0.0);
    }
    if (!ok) ++bad;
    if (ratio > wr || wi < 0) {
      wr = ratio;
      wi = i;
    }
  }
  if (worst_index) *worst_index = wi;
  if (worst_ratio) *worst_ratio = wr;
  return bad;
}
