/*
 * Seeded synthetic inputs for the fused transform + dynamic quantization
 * operator: activations x[K,M,N] and square transforms P[n,n], stored as
 * raw 16-bit bf16 or fp16 bit patterns.
 *
 * This module holds none of the operator's arithmetic.  It only draws
 * random numbers and rounds them to the storage type, and it is shared as
 * an input source by the GPU library's tests, the oracle's tests and the
 * benchmark.
 *
 * Random source: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014).  SplitMix64 is
 * counter-based: draw i of a stream with state s is mix(s + (i+1)*gamma),
 * so any element can be generated independently, which lets large tensors
 * be filled by many threads with results identical to a serial fill.
 *
 *   - Gaussian: Box-Muller on the pair (2p, 2p+1), in double.
 *   - Laplace(0, 1): inverse CDF  x = -sgn(u) * ln(1 - 2|u|),  u in (-1/2, 1/2).
 *   - Outlier channels: the first round(frac*M*N) positions of a seeded
 *     Fisher-Yates permutation of the flattened hidden index f = m*N + n; the
 *     same channels for every slice k, multiplied in double before rounding.
 *   - Random orthogonal P: Householder QR of an n x n Gaussian matrix, then
 *     Q * diag(sign(R_ii)) (a Haar-distributed orthogonal matrix).
 *   - Storage rounding: double -> fp32 (C cast, round to nearest even) ->
 *     bf16 or fp16 (round to nearest even, fp16 with subnormals).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define FQS_F16 1
#define FQS_BF16 2

#define GAMMA64 0x9E3779B97F4A7C15ull

static inline uint64_t sm64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* Stream base for one tensor of one workload. */
static inline uint64_t stream_base(uint64_t seed, uint64_t tensor_id) {
  return sm64_mix(seed ^ (tensor_id * 0xD1B54A32D192ED03ull)) ;
}

/* Draw i of a stream. */
static inline uint64_t draw(uint64_t base, uint64_t i) { return sm64_mix(base + (i + 1) * GAMMA64); }

/* Uniform in the open interval (0, 1), 53 bits. */
static inline double unif(uint64_t r) { return ((double)(r >> 11) + 0.5) * (1.0 / 9007199254740992.0); }

static uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFF) ? 0x40 : 0));
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

static uint16_t f32_to_f16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  uint32_t a = u & 0x7FFFFFFFu;
  if (a >= 0x7F800000u) return (uint16_t)(sign | 0x7C00u | (a > 0x7F800000u ? 0x200u : 0));
  /* 65520 and above round to infinity */
  if (a >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u);
  int e = (int)(a >> 23) - 127;
  uint32_t mant = (a & 0x7FFFFFu) | 0x800000u;
  if (e >= -14) {
    /* normal fp16: keep 10 mantissa bits */
    uint32_t shift = 13;
    uint32_t q = mant >> shift, rem = mant & ((1u << shift) - 1), half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u))) q++;
    uint32_t he = (uint32_t)(e + 15);
    if (q == 0x800u) { q = 0x400u; he++; }
    return (uint16_t)(sign | (he << 10) | (q & 0x3FFu));
  }
  if (e < -25) return sign; /* below half the smallest subnormal: rounds to zero */
  /* subnormal fp16: value = q * 2^-24 */
  uint32_t shift = (uint32_t)(-e - 14 + 13);
  uint32_t q = mant >> shift, rem = mant & ((1u << shift) - 1), half = 1u << (shift - 1);
  if (rem > half || (rem == half && (q & 1u))) q++;
  return (uint16_t)(sign | q); /* q == 0x400 becomes the smallest normal, as it should */
}

static inline uint16_t round_dt(double v, int dtype) {
  float f = (float)v;
  return dtype == FQS_BF16 ? f32_to_bf16_rne(f) : f32_to_f16_rne(f);
}

/* ---- outlier channels ---------------------------------------------------- */

/* Writes the first `count` entries of a Fisher-Yates permutation of [0, n). */
int fqs_outlier_channels(int64_t n, int64_t count, uint64_t seed, int64_t* out) {
  if (n <= 0 || count < 0 || count > n) return -1;
  int64_t* a = (int64_t*)malloc((size_t)n * sizeof(int64_t));
  if (!a) return -2;
  for (int64_t i = 0; i < n; ++i) a[i] = i;
  uint64_t base = stream_base(seed, 4);
  for (int64_t i = n - 1; i >= 1; --i) {
    uint64_t r = draw(base, (uint64_t)(n - 1 - i));
    int64_t j = (int64_t)(((unsigned __int128)r * (uint64_t)(i + 1)) >> 64);
    int64_t t = a[i];
    a[i] = a[j];
    a[j] = t;
  }
  memcpy(out, a, (size_t)count * sizeof(int64_t));
  free(a);
  return 0;
}

/* ---- activations -------------------------------------------------------- */

typedef struct {
  uint16_t* out;
  int64_t M, N, k0, e_begin, e_end; /* element range, relative to slice k0 */
  int dtype, dist;
  double scale;
  const uint8_t* is_outlier;
  uint64_t base;
} fill_job;

static void* fill_worker(void* arg) {
  const fill_job* j = (const fill_job*)arg;
  const int64_t MN = j->M * j->N;
  const uint64_t g0 = (uint64_t)j->k0 * (uint64_t)MN; /* global index of the first element */
  for (int64_t e = j->e_begin; e < j->e_end; ++e) {
    uint64_t g = g0 + (uint64_t)e;
    double v;
    if (j->dist == 0) {
      uint64_t p = g >> 1;
      double u1 = unif(draw(j->base, 2 * p)), u2 = unif(draw(j->base, 2 * p + 1));
      double r = sqrt(-2.0 * log(u1));
      double t = 6.283185307179586 * u2;
      v = (g & 1) ? r * sin(t) : r * cos(t);
    } else {
      double u = unif(draw(j->base, g)) - 0.5;
      double a = fabs(u);
      v = -log1p(-2.0 * a);
      if (u < 0) v = -v;
    }
    int64_t f = (int64_t)(g % (uint64_t)MN);
    if (j->is_outlier && j->is_outlier[f]) v *= j->scale;
    j->out[e] = round_dt(v, j->dtype);
  }
  return NULL;
}

/*
 * Fill slices [k0, k1) of x[K, M, N] (row-major) into out[(k1-k0)*M*N].
 * dist: 0 = standard Gaussian, 1 = Laplace(0, 1).
 * Outlier channels: round(outlier_frac*M*N) channels scaled by outlier_scale.
 */
int fqs_fill_x(uint16_t* out, int64_t M, int64_t N, int dtype, int dist, double outlier_frac,
               double outlier_scale, uint64_t seed, int64_t k0, int64_t k1, int nthreads) {
  if (!out || M <= 0 || N <= 0 || k1 < k0 || (dtype != FQS_F16 && dtype != FQS_BF16)) return -1;
  if (dist != 0 && dist != 1) return -1;
  const int64_t MN = M * N;
  int64_t count = llround(outlier_frac * (double)MN);
  uint8_t* is_out = NULL;
  if (count > 0) {
    int64_t* ch = (int64_t*)malloc((size_t)count * sizeof(int64_t));
    is_out = (uint8_t*)calloc((size_t)MN, 1);
    if (!ch || !is_out) { free(ch); free(is_out); return -2; }
    if (fqs_outlier_channels(MN, count, seed, ch) != 0) { free(ch); free(is_out); return -1; }
    for (int64_t i = 0; i < count; ++i) is_out[ch[i]] = 1;
    free(ch);
  }
  const int64_t total = (k1 - k0) * MN;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (total < 65536) nthreads = 1;
  pthread_t th[256];
  fill_job jobs[256];
  int joinable[256] = {0};
  uint64_t base = stream_base(seed, 1);
  int64_t chunk = (total + nthreads - 1) / nthreads;
  for (int t = 0; t < nthreads; ++t) {
    int64_t b = (int64_t)t * chunk, e = b + chunk;
    if (b >= total) break;
    if (e > total) e = total;
    jobs[t] = (fill_job){out, M, N, k0, b, e, dtype, dist, outlier_scale, is_out, base};
    if (nthreads > 1 && pthread_create(&th[t], NULL, fill_worker, &jobs[t]) == 0)
      joinable[t] = 1;
    else
      fill_worker(&jobs[t]);
  }
  for (int t = 0; t < nthreads; ++t)
    if (joinable[t]) pthread_join(th[t], NULL);
  free(is_out);
  return 0;
}

/* ---- random orthogonal transforms ---------------------------------------- */

/*
 * Haar-random orthogonal n x n matrix, row-major, rounded to dtype.
 * tensor_id separates the streams of different matrices of one workload.
 * If q64 is not NULL the unrounded double matrix is written there too.
 */
int fqs_orthogonal(uint16_t* out, double* q64, int64_t n, int dtype, uint64_t seed, uint64_t tensor_id) {
  if (n <= 0 || n > 4096 || (dtype != FQS_F16 && dtype != FQS_BF16)) return -1;
  double* A = (double*)malloc((size_t)(n * n) * sizeof(double));
  double* V = (double*)calloc((size_t)(n * n), sizeof(double)); /* V[k*n + i]: reflector k */
  double* vn = (double*)calloc((size_t)n, sizeof(double));
  double* sg = (double*)malloc((size_t)n * sizeof(double));
  double* Q = (double*)calloc((size_t)(n * n), sizeof(double));
  if (!A || !V || !vn || !sg || !Q) { free(A); free(V); free(vn); free(sg); free(Q); return -2; }
  uint64_t base = stream_base(seed, tensor_id);
  for (int64_t e = 0; e < n * n; ++e) {
    uint64_t p = (uint64_t)e >> 1;
    double u1 = unif(draw(base, 2 * p)), u2 = unif(draw(base, 2 * p + 1));
    double r = sqrt(-2.0 * log(u1)), t = 6.283185307179586 * u2;
    A[e] = (e & 1) ? r * sin(t) : r * cos(t);
  }
  for (int64_t k = 0; k < n; ++k) {
    double nrm = 0.0;
    for (int64_t i = k; i < n; ++i) nrm += A[i * n + k] * A[i * n + k];
    nrm = sqrt(nrm);
    if (nrm == 0.0) { sg[k] = 1.0; vn[k] = 0.0; continue; }
    double alpha = A[k * n + k] > 0 ? -nrm : nrm; /* R_kk */
    sg[k] = alpha > 0 ? 1.0 : -1.0;
    double* v = V + k * n;
    for (int64_t i = k; i < n; ++i) v[i] = A[i * n + k];
    v[k] -= alpha;
    double v2 = 0.0;
    for (int64_t i = k; i < n; ++i) v2 += v[i] * v[i];
    vn[k] = v2;
    if (v2 == 0.0) continue;
    for (int64_t j = k; j < n; ++j) {
      double s = 0.0;
      for (int64_t i = k; i < n; ++i) s += v[i] * A[i * n + j];
      double f = 2.0 * s / v2;
      for (int64_t i = k; i < n; ++i) A[i * n + j] -= f * v[i];
    }
  }
  /* Q = H_0 H_1 ... H_{n-1}, accumulated from the right-most factor */
  for (int64_t i = 0; i < n; ++i) Q[i * n + i] = 1.0;
  for (int64_t k = n - 1; k >= 0; --k) {
    if (vn[k] == 0.0) continue;
    const double* v = V + k * n;
    for (int64_t j = 0; j < n; ++j) {
      double s = 0.0;
      for (int64_t i = k; i < n; ++i) s += v[i] * Q[i * n + j];
      double f = 2.0 * s / vn[k];
      for (int64_t i = k; i < n; ++i) Q[i * n + j] -= f * v[i];
    }
  }
  for (int64_t i = 0; i < n; ++i)
    for (int64_t j = 0; j < n; ++j) {
      double q = Q[i * n + j] * sg[j];
      if (q64) q64[i * n + j] = q;
      out[i * n + j] = round_dt(q, dtype);
    }
  free(A); free(V); free(vn); free(sg); free(Q);
  return 0;
}

/* Round an array of doubles to the 16-bit storage type (hand-made test inputs). */
int fqs_round(const double* in, uint16_t* out, int64_t n, int dtype) {
  if (dtype != FQS_F16 && dtype != FQS_BF16) return -1;
  for (int64_t i = 0; i < n; ++i) out[i] = round_dt(in[i], dtype);
  return 0;
}
