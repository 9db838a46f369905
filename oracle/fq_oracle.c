/*
 * ORACLE -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, scalar CPU implementation of the fused transform + dynamic
 * quantization operator, written from the page "aclnnFlatQuantV2 算子拆解：
 * 两步矩阵乘 + 动态量化，CANN 上怎么写一次讲清" (cited below as [FQV2], by
 * section).  Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg may load it.  It shares no code with the GPU library.
 *
 * Other pages cited, for conventions the operator page leaves open:
 *   [MOCONV] the ModelOpt Conv3D implicit-GEMM page, section 6.1 (the eight
 *            E2M1 magnitudes and the seven decision points between them);
 *   [DSQ]    the dequant_swiglu_quant Triton-Ascend page, section 6.1
 *            (round-half-to-even, 2.5 -> 2 and 3.5 -> 4);
 *   [APT]    the APT-LLM page, section 2.1 (symmetric b-bit integer
 *            quantization clamped to [-2^(b-1), 2^(b-1)-1]);
 *   [DSQ 3.4] the same dequant_swiglu_quant page, section 3.4 (dynamic
 *            per-row quantization: scale = max|out| / max_val, codes
 *            clamp(round(out / scale), -max_val, max_val), max_val 127 for
 *            INT8, 448 for FP8 E4M3FN, 57344 for FP8 E5M2).
 *
 * What is computed for one slice x_k [M, N] (readings of silent or garbled
 * points are marked "reading"):
 *   T = RNE_dt(fl32(x_k . P2))       [FQV2] 第1步; reading: the intermediate is
 *                                    rounded to the activation dtype, the
 *                                    matrices' own dtype (they may not be mixed)
 *   y = fl32(P1 . T)                 [FQV2] 第2步; y stays fp32.  With an empty
 *                                    [0,0] P2 the first step is skipped.
 *   per token:  scale = fl32(max|y| / fl32(7/clipRatio)),
 *               code  = clamp(RNE(fl32(y / scale)), -8, 7)    [FQV2] 第3步 pertoken
 *   per token, 8-bit codes ([DSQ 3.4] with this operator's per-token clip; reading:
 *     the divisor is fl32(max_val / clipRatio), which is the page's max_val at
 *     clipRatio 1):  scale = fl32(max|y| / fl32(max_val/clipRatio)),  q = fl32(y/scale);
 *     INT8: code = clamp(RNE(q), -127, 127);  FP8: code = the representable value
 *     nearest clamp(q, -max_val, max_val), a tie to the even code; the code keeps the
 *     sign of q (reading: the OCP FP8 encodings, E4M3FN = 1.4.3 bias 7 without
 *     infinities, E5M2 = 1.5.2 bias 15; their largest finite values are the page's
 *     max_val 448 and 57344)
 *   per group of 32 over the flattened index f = m*N + n ([FQV2] 第3步 pergroup):
 *     V1 (dstTypeMax == 0): e8m0 = clamp(floor(log2 amax) - 2 + 127, 0, 254),
 *        reading: emax = 2, the exponent of E2M1's largest value 6 = 1.5 * 2^2;
 *     V2 (dstTypeMax in [6,12]): S = fl32(amax / dstTypeMax), split into the
 *        biased exponent E and mantissa; E += 1 when S is normal, E < 254 and
 *        the mantissa is non-zero; e8m0 = E                     [FQV2] 第4步
 *     element code = E2M1_RNE_saturating(y * 2^(127 - e8m0))
 *
 * All sums are accumulated in double (bf16/fp16 products are exact in double)
 * and rounded once.  Scale arithmetic is IEEE fp32 (C float, no contraction).
 *
 * Besides the codes the oracle reports, per element, the range of codes that
 * any correct fp32 implementation can reach: fp32 sums in any order carry an
 * error of at most gamma(n) * sum|terms| (gamma(n) = n u / (1 - n u),
 * u = 2^-24, Higham, "Accuracy and Stability of Numerical Algorithms",
 * Lemma 3.1 / eq. 3.5), which can flip the dtype rounding of T and, through
 * it and through the scale, move y/scale across a code boundary.  The range
 * also covers the stated tolerance window of 1e-6 relative around a tie.
 */
#include <float.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define FQO_F16 1
#define FQO_BF16 2
#define FQO_PER_TOKEN 0
#define FQO_PER_GROUP 1
/* per-token code formats */
#define FQO_Q_INT4 0
#define FQO_Q_INT8 1
#define FQO_Q_E4M3 2
#define FQO_Q_E5M2 3

#define TIE_REL 1e-6 /* the stated tie window, relative */

/* ---- exact decoding of the 16-bit inputs --------------------------------- */

static double bf16_value(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static double f16_value(uint16_t h) {
  int s = (h >> 15) & 1, e = (h >> 10) & 0x1F, m = h & 0x3FF;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + m), e - 25);
  return s ? -v : v;
}

static double dt_value(uint16_t h, int dtype) { return dtype == FQO_BF16 ? bf16_value(h) : f16_value(h); }

/* The decoding above over an array, exported for the pins (every bit pattern of both
 * formats is checked against independent decoders). */
int fqo_decode16(const uint16_t* bits, int64_t n, int dtype, double* out) {
  if (dtype != FQO_F16 && dtype != FQO_BF16) return -1;
  for (int64_t i = 0; i < n; ++i) out[i] = dt_value(bits[i], dtype);
  return 0;
}

/* ---- round to nearest even into a binary format -------------------------
 * A format with `frac` fraction bits, minimum normal exponent `emin` and
 * largest finite value `maxv`.  Textbook construction: scale so that the
 * quantum of v's binade becomes 1, round to an integer (nearbyint, default
 * round-to-nearest-even mode), scale back.  Subnormals use the quantum of
 * the smallest binade.  Magnitudes beyond the last finite value round to
 * infinity when they reach maxv + half a quantum.
 */
static double rne_format(double v, int frac, int emin, double maxv) {
  if (v == 0.0 || isnan(v) || isinf(v)) return v;
  int ex;
  frexp(v, &ex);           /* |v| = m * 2^ex, m in [0.5, 1): floor(log2|v|) = ex - 1 */
  int e = ex - 1;
  if (e < emin) e = emin;
  int q = e - frac;        /* exponent of the quantum */
  double r = ldexp(nearbyint(ldexp(v, -q)), q);
  if (fabs(r) > maxv) return v > 0 ? INFINITY : -INFINITY;
  return r;
}

double fqo_round_f32(double v) { return rne_format(v, 23, -126, FLT_MAX); }
double fqo_round_bf16(double v) { return rne_format(v, 7, -126, 3.3895313892515355e38); }
double fqo_round_f16(double v) { return rne_format(v, 10, -14, 65504.0); }
static double round_dt(double v, int dtype) { return dtype == FQO_BF16 ? fqo_round_bf16(v) : fqo_round_f16(v); }

/* gamma(n) of the error analysis of recursive/any-order summation */
static double gamma_n(int64_t n) {
  const double u = 5.9604644775390625e-08; /* 2^-24 */
  return (double)n * u / (1.0 - (double)n * u);
}

/* ---- int4 encoder ([FQV2] 第3步 pertoken; [APT] 2.1 clamp; [DSQ] 6.1 RNE) -- */

int fqo_int4_code(float q) {
  float r = nearbyintf(q); /* round half to even (default rounding mode) */
  if (r < -8.0f) r = -8.0f;
  if (r > 7.0f) r = 7.0f;
  return (int)r;
}

/* ---- 8-bit per-token encoders ([DSQ 3.4]) ---------------------------------- */

/* max_val of a per-token code format: int4 7 ([FQV2] 第3步 pertoken), the others [DSQ 3.4] */
double fqo_qmax(int fmt) {
  switch (fmt) {
    case FQO_Q_INT8: return 127.0;
    case FQO_Q_E4M3: return 448.0;
    case FQO_Q_E5M2: return 57344.0;
    default: return 7.0;
  }
}

int fqo_int8_code(float q) {
  float r = nearbyintf(q); /* round half to even ([DSQ] 6.1) */
  if (r < -127.0f) r = -127.0f;
  if (r > 127.0f) r = 127.0f;
  return (int)r;
}

/* Value of a non-negative FP8 code (bit 7 clear): sign-less 1.4.3 (bias 7) or 1.5.2
 * (bias 15); exponent field 0 is subnormal (no implicit one, exponent 1 - bias). */
double fqo_fp8_value(int code, int fmt) {
  const int mb = fmt == FQO_Q_E4M3 ? 3 : 2, bias = fmt == FQO_Q_E4M3 ? 7 : 15;
  const int e = (code & 0x7F) >> mb, m = code & ((1 << mb) - 1);
  const double v = e == 0 ? ldexp((double)m, 1 - bias - mb) : ldexp(1.0 + ldexp((double)m, -mb), e - bias);
  return (code & 0x80) ? -v : v;
}

/* the largest finite code: E4M3FN 0x7E (0x7F is NaN), E5M2 0x7B (0x7C is infinity) */
static int fp8_max_code(int fmt) { return fmt == FQO_Q_E4M3 ? 0x7E : 0x7B; }

/* Index (= code) of the FP8 magnitude nearest a >= 0, a <= max; the values grow with the
 * code, so the two candidates are the largest code whose value is <= a and the next one.
 * tie: 0 = even code, 1 = lower, 2 = upper. */
static int fp8_index(double a, int fmt, int tie) {
  int lo = 0, hi = fp8_max_code(fmt);
  if (a >= fqo_fp8_value(hi, fmt)) return hi;
  while (hi - lo > 1) { /* value(lo) <= a < value(hi) */
    const int mid = (lo + hi) / 2;
    if (fqo_fp8_value(mid, fmt) <= a) lo = mid; else hi = mid;
  }
  const double dl = a - fqo_fp8_value(lo, fmt), dh = fqo_fp8_value(hi, fmt) - a;
  if (dl < dh) return lo;
  if (dh < dl) return hi;
  return tie == 1 ? lo : tie == 2 ? hi : ((lo & 1) ? hi : lo);
}

int fqo_fp8_code(double q, int fmt) {
  const double mx = fqo_fp8_value(fp8_max_code(fmt), fmt);
  double a = fabs(q);
  if (a > mx) a = mx; /* clamp to +-max_val ([DSQ 3.4]) */
  return (signbit(q) ? 0x80 : 0) | fp8_index(a, fmt, 0);
}

static int fp8_level(int code) { return (code & 0x80) ? -(code & 0x7F) : (code & 0x7F); }
static double fp8_clamp(double v, int fmt) {
  const double mx = fqo_fp8_value(fp8_max_code(fmt), fmt);
  return v > mx ? mx : (v < -mx ? -mx : v);
}
static int fp8_level_down(double v, int fmt) {
  v = fp8_clamp(v, fmt);
  return v >= 0 ? fp8_index(v, fmt, 1) : -fp8_index(-v, fmt, 2);
}
static int fp8_level_up(double v, int fmt) {
  v = fp8_clamp(v, fmt);
  return v >= 0 ? fp8_index(v, fmt, 2) : -fp8_index(-v, fmt, 1);
}
/* |q| within TIE_REL of a midpoint between two adjacent FP8 magnitudes */
static int fp8_near_tie(double q, int fmt) {
  const double a = fabs(q);
  const int c = fp8_index(a, fmt, 1);
  for (int k = c - 1; k <= c; ++k) {
    if (k < 0 || k + 1 > fp8_max_code(fmt)) continue;
    const double mid = 0.5 * (fqo_fp8_value(k, fmt) + fqo_fp8_value(k + 1, fmt));
    if (fabs(a - mid) <= TIE_REL * mid) return 1;
  }
  return 0;
}

/* ---- E2M1 encoder ----------------------------------------------------------
 * The eight magnitudes of [MOCONV] 6.1; the code is sign<<3 | index, the
 * index being the position in the magnitude list (1 exponent pair + 1
 * mantissa bit: s e1 e0 m).  Nearest magnitude by exhaustive distance; an
 * exact tie goes to the even index, which is round-half-to-even on the
 * format's mantissa bit.  Magnitudes above 6 therefore map to 6
 * (saturation; E2M1 has no infinity or NaN).
 */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* tie: 0 = even index, 1 = lower index, 2 = upper index */
static int e2m1_index(double a, int tie) {
  int best = 0;
  double bd = fabs(a - E2M1_MAG[0]);
  for (int i = 1; i < 8; ++i) {
    double d = fabs(a - E2M1_MAG[i]);
    if (d < bd) {
      bd = d;
      best = i;
    } else if (d == bd) { /* tie between best (lower) and i (upper) */
      if (tie == 2 || (tie == 0 && (i % 2 == 0))) best = i;
    }
  }
  return best;
}

int fqo_e2m1_code(double v) {
  int s = signbit(v) ? 1 : 0;
  return (s << 3) | e2m1_index(fabs(v), 0);
}

double fqo_e2m1_value(int code) {
  double m = E2M1_MAG[code & 7];
  return (code & 8) ? -m : m;
}

/* signed level: +index for a positive code, -index for a negative one */
static int level_of_code(int code) { return (code & 8) ? -(code & 7) : (code & 7); }
static int e2m1_level_down(double v) { return v >= 0 ? e2m1_index(v, 1) : -e2m1_index(-v, 2); }
static int e2m1_level_up(double v) { return v >= 0 ? e2m1_index(v, 2) : -e2m1_index(-v, 1); }

/* ---- e8m0 scale codes ------------------------------------------------------ */

/* V1, [FQV2] 第3步 pergroup: sharedExp = floor(log2(amax)) - emax, emax = 2. */
int fqo_e8m0_v1(float amax) {
  if (!(amax > 0.0f)) return 0;
  int ex;
  frexp((double)amax, &ex);
  int code = (ex - 1) - 2 + 127;
  if (code < 0) code = 0;
  if (code > 254) code = 254;
  return code;
}

/* V2, [FQV2] 第4步, from the fp32 bit fields of S. */
int fqo_e8m0_v2_bits(float amax, float dmax) {
  float S = amax / dmax;
  uint32_t b;
  memcpy(&b, &S, 4);
  uint32_t E = (b >> 23) & 0xFF, mant = b & 0x7FFFFF;
  if (E >= 1 && E < 254 && mant != 0) E += 1;
  return (int)E;
}

/* V2 again, from frexp, as an independent cross-check of the bit version. */
int fqo_e8m0_v2_frexp(float amax, float dmax) {
  float S = amax / dmax;
  if (S == 0.0f) return 0;
  if (S < FLT_MIN) return 0; /* subnormal: biased exponent 0, never incremented */
  int ex;
  double m = frexp((double)S, &ex); /* S = m 2^ex, m in [0.5, 1) */
  int E = (ex - 1) + 127;
  if (m != 0.5 && E < 254) E += 1;
  return E;
}

static int e8m0_code(float amax, double dst_max) {
  if (dst_max == 0.0) return fqo_e8m0_v1(amax); /* [FQV2] V1 还是 V2: 0.0 behaves as V1 */
  return fqo_e8m0_v2_bits(amax, (float)dst_max);
}

/* 2^(127 - code) as a double (exact) */
static double inv_scale_of_code(int code) { return ldexp(1.0, 127 - code); }

/* ---- batch interface ---------------------------------------------------- */

typedef struct {
  int32_t dtype;        /* FQO_F16 | FQO_BF16 */
  int32_t mode;         /* FQO_PER_TOKEN | FQO_PER_GROUP */
  int64_t M, N;
  int32_t two_sided;    /* 0: the right transform is skipped ([0,0] P2) */
  int32_t qfmt;         /* per token: FQO_Q_INT4 | _INT8 | _E4M3 | _E5M2 */
  double clip_ratio;
  double dst_type_max;
} fqo_params;

/* Per-slice outputs; every array holds nslices consecutive slices.  Any pointer
 * may be NULL when that output is not wanted.  Levels: the int4 value for per
 * token; the signed E2M1 magnitude index for per group. */
typedef struct {
  uint8_t* packed;   /* M*N/2 bytes per slice: 4-bit codes, low nibble = lower index */
  float* scale;      /* per token: 1 per slice */
  uint8_t* e8m0;     /* per group: 2*ceil(M*N/64) bytes per slice (odd pad byte = 0) */
  float* y;          /* M*N fp32 per slice */
  uint16_t* t;       /* M*N dtype bits per slice (the rounded intermediate) */
  int8_t* lvl;       /* M*N: the oracle's level */
  int8_t* lo;        /* M*N: lowest reachable level */
  int8_t* hi;        /* M*N: highest reachable level */
  uint8_t* zsign;    /* M*N: a zero code may carry either sign */
  uint8_t* ns_tie;   /* M*N: within 1e-6 relative of a rounding tie */
  int8_t* alt_lvl;   /* per group: the same four under the alternative e8m0 code */
  int8_t* alt_lo;
  int8_t* alt_hi;
  uint8_t* alt_zsign;
  uint8_t* g_lo;     /* per group: reachable e8m0 code range */
  uint8_t* g_hi;
  uint8_t* g_alt;    /* per group: the alternative e8m0 code (== the code if none) */
  float* scale_lo;   /* per token: reachable scale range */
  float* scale_hi;
} fqo_out;

typedef struct {
  const fqo_params* p;
  const uint16_t *x, *p1, *p2;
  const fqo_out* o;
  int64_t s_begin, s_end;
  int want_ranges;
  int status;
} job_t;

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

static void put_nibble(uint8_t* packed, int64_t f, int code) {
  uint8_t c = (uint8_t)(code & 0xF);
  if (f & 1)
    packed[f >> 1] = (uint8_t)((packed[f >> 1] & 0x0F) | (c << 4));
  else
    packed[f >> 1] = (uint8_t)((packed[f >> 1] & 0xF0) | c);
}

static int slice(const fqo_params* p, const uint16_t* xs, const double* P1, const double* P2,
                 const fqo_out* o, int64_t s, int want, double* ws) {
  const int64_t M = p->M, N = p->N, MN = M * N;
  double* X = ws;              /* M*N */
  double* T = X + MN;          /* M*N  rounded intermediate */
  double* Tlo = T + MN;        /* M*N  reachable range of the GPU's rounded intermediate */
  double* Thi = Tlo + MN;
  double* Y = Thi + MN;        /* M*N  fp32 y (as double) */
  double* Ylo = Y + MN;        /* M*N  bounds on any fp32 implementation's y */
  double* Yhi = Ylo + MN;
  for (int64_t f = 0; f < MN; ++f) X[f] = dt_value(xs[f], p->dtype);

  /* [FQV2] 第1步: right-multiply by P2 along the trailing axis */
  if (p->two_sided) {
    const double gN = gamma_n(N);
    for (int64_t m = 0; m < M; ++m)
      for (int64_t n = 0; n < N; ++n) {
        double s = 0.0, sa = 0.0;
        for (int64_t j = 0; j < N; ++j) {
          double pr = X[m * N + j] * P2[j * N + n];
          s += pr;
          sa += fabs(pr);
        }
        T[m * N + n] = round_dt(fqo_round_f32(s), p->dtype);
        if (want) {
          double r = gN * sa;
          Tlo[m * N + n] = round_dt(s - r, p->dtype);
          Thi[m * N + n] = round_dt(s + r, p->dtype);
        }
      }
  } else {
    for (int64_t f = 0; f < MN; ++f) T[f] = Tlo[f] = Thi[f] = X[f];
  }
  if (o->t)
    for (int64_t f = 0; f < MN; ++f) {
      /* store the rounded intermediate as dtype bits */
      double v = T[f];
      uint16_t bits;
      if (p->dtype == FQO_BF16) {
        float fv = (float)v;
        uint32_t u;
        memcpy(&u, &fv, 4);
        bits = (uint16_t)(u >> 16); /* exact: v is a bf16 value */
      } else {
        /* exact fp16 encoding of an fp16 value */
        double a = fabs(v);
        uint16_t sg = signbit(v) ? 0x8000 : 0;
        if (a == 0.0)
          bits = sg;
        else if (isinf(a))
          bits = sg | 0x7C00;
        else if (a < ldexp(1.0, -14))
          bits = sg | (uint16_t)ldexp(a, 24);
        else {
          int ex;
          double mm = frexp(a, &ex); /* a = mm 2^ex */
          int e = ex - 1;
          uint16_t frac = (uint16_t)(ldexp(mm * 2.0, 10) - 1024.0);
          bits = sg | (uint16_t)((e + 15) << 10) | frac;
        }
      }
      o->t[s * MN + f] = bits;
    }

  /* [FQV2] 第2步: left-multiply by P1 along axis 1 */
  const double gM = gamma_n(M);
  for (int64_t i = 0; i < M; ++i)
    for (int64_t n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int64_t m = 0; m < M; ++m) acc += P1[i * M + m] * T[m * N + n];
      Y[i * N + n] = fqo_round_f32(acc);
      if (want) {
        double lo = 0.0, hi = 0.0, sa = 0.0;
        for (int64_t m = 0; m < M; ++m) {
          double a = P1[i * M + m] * Tlo[m * N + n], b = P1[i * M + m] * Thi[m * N + n];
          lo += a < b ? a : b;
          hi += a < b ? b : a;
          sa += fabs(a) > fabs(b) ? fabs(a) : fabs(b);
        }
        double r = gM * sa;
        Ylo[i * N + n] = lo - r;
        Yhi[i * N + n] = hi + r;
      }
    }
  if (o->y)
    for (int64_t f = 0; f < MN; ++f) o->y[s * MN + f] = (float)Y[f];

  const int fmt = p->mode == FQO_PER_TOKEN ? p->qfmt : FQO_Q_INT4;
  const int wide = fmt != FQO_Q_INT4; /* one byte per code */
  uint8_t* packed = o->packed ? o->packed + s * (wide ? MN : MN / 2) : NULL;

  if (p->mode == FQO_PER_TOKEN) {
    /* [FQV2] 第3步 pertoken: one fp32 scale per slice k */
    float amax = 0.0f;
    for (int64_t f = 0; f < MN; ++f) {
      float a = fabsf((float)Y[f]);
      if (a > amax) amax = a;
    }
    const float d = (float)(fqo_qmax(fmt) / p->clip_ratio);
    const float scale = amax / d;
    if (o->scale) o->scale[s] = scale;
    double Alo = 0.0, Ahi = 0.0, slo = 0.0, shi = 0.0;
    if (want) {
      for (int64_t f = 0; f < MN; ++f) {
        double lo = Ylo[f], hi = Yhi[f];
        double amin = lo > 0 ? lo : (hi < 0 ? -hi : 0.0);
        double amx = fabs(lo) > fabs(hi) ? fabs(lo) : fabs(hi);
        if (amin > Alo) Alo = amin;
        if (amx > Ahi) Ahi = amx;
      }
      /* the stated window also applies to the scale's own tie-free rounding */
      slo = Alo / (double)d * (1.0 - 2.4e-7);
      shi = Ahi / (double)d * (1.0 + 2.4e-7);
      if (amax == 0.0f) slo = shi = 0.0;
      if (o->scale_lo) o->scale_lo[s] = (float)slo;
      if (o->scale_hi) o->scale_hi[s] = (float)shi;
    }
    /* level range of the format: int4 [-8, 7] ([APT] 2.1), INT8 +-127 ([DSQ 3.4]), FP8
     * +- the largest finite code; a level is the code's signed value (int) or signed
     * magnitude index (FP8), which grows with the value it encodes */
    const int lmin = fmt == FQO_Q_INT4 ? -8 : fmt == FQO_Q_INT8 ? -127 : -fp8_max_code(fmt);
    const int lmax = fmt == FQO_Q_INT4 ? 7 : fmt == FQO_Q_INT8 ? 127 : fp8_max_code(fmt);
    for (int64_t f = 0; f < MN; ++f) {
      int code = 0, level = 0;
      float q = 0.0f;
      if (scale > 0.0f) q = (float)Y[f] / scale;
      if (fmt == FQO_Q_INT4) {
        if (scale > 0.0f) code = fqo_int4_code(q);
        level = code;
        if (packed) put_nibble(packed, f, code);
      } else if (fmt == FQO_Q_INT8) {
        if (scale > 0.0f) code = fqo_int8_code(q);
        level = code;
        if (packed) packed[f] = (uint8_t)(code & 0xFF);
      } else {
        if (scale > 0.0f) code = fqo_fp8_code(q, fmt);
        level = fp8_level(code);
        if (packed) packed[f] = (uint8_t)code;
      }
      if (o->lvl) o->lvl[s * MN + f] = (int8_t)level;
      /* an integer zero is unsigned; an FP8 zero carries the sign of y, either of which
       * is reachable when y's reachable interval contains 0 */
      if (o->zsign)
        o->zsign[s * MN + f] = (fmt == FQO_Q_E4M3 || fmt == FQO_Q_E5M2) && want && Ylo[f] <= 0.0 && Yhi[f] >= 0.0;
      int tie = 0;
      if (scale > 0.0f) {
        if (fmt == FQO_Q_E4M3 || fmt == FQO_Q_E5M2) {
          tie = fp8_near_tie(q, fmt);
        } else {
          double t = floor((double)q) + 0.5;
          if (t >= lmin + 0.5 && t <= lmax - 0.5 && fabs((double)q - t) <= TIE_REL * fabs(t)) tie = 1;
        }
      }
      if (o->ns_tie) o->ns_tie[s * MN + f] = (uint8_t)tie;
      if (want && (o->lo || o->hi)) {
        int lo, hi;
        if (amax == 0.0f) {
          lo = hi = 0;
        } else if (!(slo > 0.0)) {
          lo = lmin;
          hi = lmax;
        } else {
          double c[4] = {Ylo[f] / slo, Ylo[f] / shi, Yhi[f] / slo, Yhi[f] / shi};
          double qlo = c[0], qhi = c[0];
          for (int i = 1; i < 4; ++i) {
            if (c[i] < qlo) qlo = c[i];
            if (c[i] > qhi) qhi = c[i];
          }
          /* two fp32 roundings (reciprocal and product) and the stated window */
          double w = 2.4e-7 + TIE_REL;
          qlo -= fabs(qlo) * w;
          qhi += fabs(qhi) * w;
          if (fmt == FQO_Q_E4M3 || fmt == FQO_Q_E5M2) {
            lo = fp8_level_down(qlo, fmt);
            hi = fp8_level_up(qhi, fmt);
          } else {
            double dl = ceil(qlo - 0.5), dh = floor(qhi + 0.5);
            if (dl < lmin) dl = lmin;
            if (dl > lmax) dl = lmax;
            if (dh < lmin) dh = lmin;
            if (dh > lmax) dh = lmax;
            lo = (int)dl;
            hi = (int)dh;
          }
          if (lo > level) lo = level;
          if (hi < level) hi = level;
        }
        if (o->lo) o->lo[s * MN + f] = (int8_t)lo;
        if (o->hi) o->hi[s * MN + f] = (int8_t)hi;
      }
    }
    return 0;
  }

  /* [FQV2] 第3步 pergroup / 第4步: groups of 32 over the flattened slice */
  const int64_t G = ceil_div(MN, 32);
  const int64_t GS = 2 * ceil_div(MN, 64);
  uint8_t* e8 = o->e8m0 ? o->e8m0 + s * GS : NULL;
  if (e8)
    for (int64_t g = 0; g < GS; ++g) e8[g] = 0;
  for (int64_t g = 0; g < G; ++g) {
    const int64_t f0 = g * 32, f1 = (f0 + 32 < MN) ? f0 + 32 : MN;
    float amax = 0.0f;
    for (int64_t f = f0; f < f1; ++f) {
      float a = fabsf((float)Y[f]);
      if (a > amax) amax = a;
    }
    const int code = e8m0_code(amax, p->dst_type_max);
    if (e8) e8[g] = (uint8_t)code;
    int glo = code, ghi = code, alt = code;
    if (want) {
      double Alo = 0.0, Ahi = 0.0;
      for (int64_t f = f0; f < f1; ++f) {
        double lo = Ylo[f], hi = Yhi[f];
        double amin = lo > 0 ? lo : (hi < 0 ? -hi : 0.0);
        double amx = fabs(lo) > fabs(hi) ? fabs(lo) : fabs(hi);
        if (amin > Alo) Alo = amin;
        if (amx > Ahi) Ahi = amx;
      }
      /* the stated window around a power-of-two boundary */
      if ((double)amax * (1.0 - TIE_REL) < Alo) Alo = (double)amax * (1.0 - TIE_REL);
      if ((double)amax * (1.0 + TIE_REL) > Ahi) Ahi = (double)amax * (1.0 + TIE_REL);
      /* the code is monotone in amax; a real bound maps through the float
         values next to it */
      float flo = (float)Alo, fhi = (float)Ahi;
      if ((double)flo > Alo) flo = nextafterf(flo, 0.0f);
      if ((double)fhi < Ahi) fhi = nextafterf(fhi, INFINITY);
      if (Alo <= 0.0) flo = 0.0f;
      glo = e8m0_code(flo, p->dst_type_max);
      ghi = e8m0_code(fhi, p->dst_type_max);
      if (glo > code) glo = code;
      if (ghi < code) ghi = code;
      alt = (glo < code) ? glo : (ghi > code ? ghi : code);
      if (o->g_lo) o->g_lo[s * G + g] = (uint8_t)glo;
      if (o->g_hi) o->g_hi[s * G + g] = (uint8_t)ghi;
      if (o->g_alt) o->g_alt[s * G + g] = (uint8_t)alt;
    }
    for (int pass = 0; pass < 2; ++pass) {
      const int c = pass == 0 ? code : alt;
      if (pass == 1 && !want) break;
      const double R = inv_scale_of_code(c);
      for (int64_t f = f0; f < f1; ++f) {
        const double v = Y[f] * R; /* exact power-of-two scaling */
        const int ec = fqo_e2m1_code(v);
        if (pass == 0) {
          if (packed) put_nibble(packed, f, ec);
          int tie = 0;
          static const double mids[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
          for (int i = 0; i < 7; ++i)
            if (fabs(fabs(v) - mids[i]) <= TIE_REL * mids[i]) tie = 1;
          if (o->ns_tie) o->ns_tie[s * MN + f] = (uint8_t)tie;
        }
        int8_t* L = pass == 0 ? o->lvl : o->alt_lvl;
        int8_t* Lo = pass == 0 ? o->lo : o->alt_lo;
        int8_t* Hi = pass == 0 ? o->hi : o->alt_hi;
        uint8_t* Z = pass == 0 ? o->zsign : o->alt_zsign;
        if (L) L[s * MN + f] = (int8_t)level_of_code(ec);
        if (want) {
          double vlo = Ylo[f] * R, vhi = Yhi[f] * R;
          double w = TIE_REL * fabs(v);
          if (v - w < vlo) vlo = v - w;
          if (v + w > vhi) vhi = v + w;
          int lo = e2m1_level_down(vlo), hi = e2m1_level_up(vhi);
          int lv = level_of_code(ec);
          if (lo > lv) lo = lv;
          if (hi < lv) hi = lv;
          if (Lo) Lo[s * MN + f] = (int8_t)lo;
          if (Hi) Hi[s * MN + f] = (int8_t)hi;
          if (Z) Z[s * MN + f] = (uint8_t)(Ylo[f] <= 0.0 && Yhi[f] >= 0.0);
        }
      }
    }
  }
  return 0;
}

static void* worker(void* arg) {
  job_t* j = (job_t*)arg;
  const fqo_params* p = j->p;
  const int64_t M = p->M, N = p->N, MN = M * N;
  double* P1 = (double*)malloc((size_t)(M * M) * sizeof(double));
  double* P2 = p->two_sided ? (double*)malloc((size_t)(N * N) * sizeof(double)) : NULL;
  double* ws = (double*)malloc((size_t)(7 * MN) * sizeof(double));
  if (!P1 || !ws || (p->two_sided && !P2)) {
    j->status = -2;
    free(P1); free(P2); free(ws);
    return NULL;
  }
  for (int64_t i = 0; i < M * M; ++i) P1[i] = dt_value(j->p1[i], p->dtype);
  if (P2)
    for (int64_t i = 0; i < N * N; ++i) P2[i] = dt_value(j->p2[i], p->dtype);
  for (int64_t s = j->s_begin; s < j->s_end; ++s)
    if (slice(p, j->x + s * MN, P1, P2, j->o, s, j->want_ranges, ws) != 0) j->status = -3;
  free(P1); free(P2); free(ws);
  return NULL;
}

/*
 * Run the oracle on nslices consecutive slices x[nslices, M, N] (dtype bits).
 * p2 is ignored when two_sided == 0.  Returns 0, or a negative value on a bad
 * argument.  nthreads worker threads split the slices.
 */
int fqo_run(const fqo_params* p, const uint16_t* x, const uint16_t* p1, const uint16_t* p2,
            int64_t nslices, const fqo_out* o, int nthreads) {
  if (!p || !x || !p1 || !o || nslices < 0) return -1;
  if (p->dtype != FQO_F16 && p->dtype != FQO_BF16) return -1;
  if (p->M < 1 || p->N < 1 || p->M > 4096 || p->N > 4096) return -1;
  if (p->mode == FQO_PER_TOKEN && !(p->clip_ratio > 0.0 && p->clip_ratio <= 1.0)) return -1;
  if (p->mode == FQO_PER_TOKEN && (p->qfmt < FQO_Q_INT4 || p->qfmt > FQO_Q_E5M2)) return -1;
  if (p->two_sided && !p2) return -1;
  /* two 4-bit codes a byte need an even M*N; the 8-bit codes take one byte each */
  if ((p->M * p->N) % 2 != 0 && o->packed && !(p->mode == FQO_PER_TOKEN && p->qfmt != FQO_Q_INT4)) return -1;
  const int want = (o->lo || o->hi || o->zsign || o->alt_lvl || o->alt_lo || o->alt_hi ||
                    o->g_lo || o->g_hi || o->g_alt || o->scale_lo || o->scale_hi) ? 1 : 0;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (nthreads > nslices) nthreads = (int)(nslices > 0 ? nslices : 1);
  pthread_t th[256];
  job_t jobs[256];
  int joinable[256] = {0};
  int64_t per = nslices / nthreads, extra = nslices % nthreads, b = 0;
  for (int t = 0; t < nthreads; ++t) {
    int64_t n = per + (t < extra ? 1 : 0);
    jobs[t] = (job_t){p, x, p1, p2, o, b, b + n, want, 0};
    b += n;
    if (nthreads > 1 && pthread_create(&th[t], NULL, worker, &jobs[t]) == 0)
      joinable[t] = 1;
    else
      worker(&jobs[t]);
  }
  int status = 0;
  for (int t = 0; t < nthreads; ++t) {
    if (joinable[t]) pthread_join(th[t], NULL);
    if (jobs[t].status) status = jobs[t].status;
  }
  return status;
}

/* ---- dequantization (the second half of a fake-quant round trip) ---------
 * The APT-LLM page, section 2.1: the symmetric integer format dequantizes as
 * q * scale.  Per group, an element is the value of its E2M1 code ([MOCONV]
 * 6.1's magnitudes, sign bit on top) times the group's e8m0 power of two
 * 2^(e - 127) ([FQV2] 第3步 pergroup).  The ModelOpt page, section 6.4, uses
 * such a quantize -> dequantize round trip as a reference, and the APT-LLM
 * page, section 5.2, checks the RMS of dequantize(quantize(x)) - x.
 * Readings: the product is formed in IEEE fp32 (per token a C float
 * multiply; per group the exact product rounded once to fp32, so 6 * 2^127
 * overflows to inf) and rounded once, to nearest even, to the output dtype
 * (overflow to inf).  An e8m0 byte 0xFF is NaN (the OCP MX encoding), and so
 * is every element of its group.  Codes are read from the packed layouts the
 * quantizer writes: [S, M*N/2] bytes, low nibble = lower flattened index
 * (INT32 and INT4 outputs are byte-identical); e8m0 [S, 2*ceil(M*N/64)].
 */

/* bits of a value already representable in the format (after round_dt) */
static uint16_t bf16_bits(double v) {
  float f = (float)v; /* exact: v is a bf16 value, and bf16 values are fp32 values */
  uint32_t u;
  memcpy(&u, &f, 4);
  if (isnan(v)) return 0x7FC0;
  return (uint16_t)(u >> 16);
}

static uint16_t f16_bits(double v) {
  if (isnan(v)) return 0x7E00;
  uint16_t s = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (isinf(a)) return s | 0x7C00;
  if (a == 0.0) return s;
  if (a < ldexp(1.0, -14)) return s | (uint16_t)ldexp(a, 24); /* subnormal: multiple of 2^-24 */
  int ex;
  double m = frexp(a, &ex);  /* a = m 2^ex, m in [0.5, 1) */
  int e = ex - 1;            /* a = (2m) 2^e, 2m in [1, 2) */
  uint16_t mant = (uint16_t)ldexp(2.0 * m - 1.0, 10);
  return s | (uint16_t)((e + 15) << 10) | mant;
}

int fqo_dequant8(int dtype, int qfmt, int64_t S, int64_t M, int64_t N, const uint8_t* codes,
                 const float* scale, uint16_t* out) {
  /* 8-bit per-token codes: value = RNE_dt(fl32(v * scale_k)), v the INT8 integer or the FP8
   * value of the code (the same rule as the int4 codes) */
  if (dtype != FQO_F16 && dtype != FQO_BF16) return -1;
  if (qfmt != FQO_Q_INT8 && qfmt != FQO_Q_E4M3 && qfmt != FQO_Q_E5M2) return -1;
  const int64_t MN = M * N;
  if (M < 1 || N < 1) return -1;
  for (int64_t k = 0; k < S; ++k)
    for (int64_t f = 0; f < MN; ++f) {
      const int c = codes[k * MN + f];
      const double q = qfmt == FQO_Q_INT8 ? (double)(int8_t)c : fqo_fp8_value(c, qfmt);
      const float prod = (float)q * scale[k]; /* IEEE fp32 product (q is exact in fp32) */
      const double r = round_dt((double)prod, dtype);
      out[k * MN + f] = dtype == FQO_BF16 ? bf16_bits(r) : f16_bits(r);
    }
  return 0;
}

int fqo_dequant(int dtype, int mode, int64_t S, int64_t M, int64_t N, const uint8_t* packed,
                const void* scale, uint16_t* out) {
  if (dtype != FQO_F16 && dtype != FQO_BF16) return -1;
  if (mode != FQO_PER_TOKEN && mode != FQO_PER_GROUP) return -1;
  const int64_t MN = M * N;
  if (M < 1 || N < 1 || MN % 2 != 0) return -1;
  const int64_t gs = 2 * ceil_div(MN, 64); /* e8m0 bytes per slice */
  for (int64_t k = 0; k < S; ++k) {
    const uint8_t* pk = packed + k * (MN / 2);
    for (int64_t f = 0; f < MN; ++f) {
      const int nib = (pk[f >> 1] >> (4 * (f & 1))) & 15;
      double v;
      if (mode == FQO_PER_TOKEN) {
        const int q = nib >= 8 ? nib - 16 : nib;          /* two's complement nibble */
        const float prod = (float)q * ((const float*)scale)[k]; /* IEEE fp32 product */
        v = (double)prod;
      } else {
        const int e = ((const uint8_t*)scale)[k * gs + f / 32];
        v = e == 255 ? NAN : fqo_round_f32(ldexp(fqo_e2m1_value(nib), e - 127));
      }
      const double r = round_dt(v, dtype);
      out[k * MN + f] = dtype == FQO_BF16 ? bf16_bits(r) : f16_bits(r);
    }
  }
  return 0;
}

/* ---- MXFP4 consumer GEMM (the product that follows the quantizer) ----------
 * C[t, o] = sum_h value(a[t, h]) * value(w[o, h]), value() the dequantization above
 * (E2M1 code times its 32-group's 2^(e8m0 - 127)), both operands in the quantizer's
 * per-group layout: codes [rows, H/2] bytes (low nibble first), e8m0 [rows, 2*ceil(H/64)].
 * The products are exact in double and the H-term sums are accumulated in double (error
 * below H 2^-53 sum|terms|); `c` receives the sums, `cabs` (if non-NULL) sum|terms|, from
 * which the comparison derives the bound any fp32 accumulation order can reach.  e8m0
 * bytes 0xFF are outside this function's domain (the quantizer never writes them). */
/* int4 consumer GEMM (the per-token int4 codes as A, per-output-channel int4 weights as W):
 *   acc[t,o] = sum_h qa[t,h] * qw[o,h]          exact (an int64 sum of int4 products)
 *   C[t,o]   = fl32( fl32(acc) * fl32(sa[t] * sw[o]) )
 * reading: the integer dot product is exact (any implementation accumulating in int32 reaches
 * it, |acc| <= 64 H), the two scales are multiplied first, then the product with acc; both in
 * IEEE fp32 ([APT] 2.1: the symmetric integer format dequantizes as q * scale, so the product
 * of two such values is qa qw sa sw).  Codes two a byte, low nibble first, two's complement. */
int fqo_int4_gemm(int64_t T, int64_t O, int64_t H, const uint8_t* a, const float* sa, const uint8_t* w,
                  const float* sw, float* c) {
  if (T < 1 || O < 1 || H < 2 || H % 2) return -1;
  for (int64_t t = 0; t < T; ++t)
    for (int64_t o = 0; o < O; ++o) {
      int64_t acc = 0;
      for (int64_t h = 0; h < H; ++h) {
        const int na = (a[t * (H / 2) + h / 2] >> (4 * (h & 1))) & 15, nw = (w[o * (H / 2) + h / 2] >> (4 * (h & 1))) & 15;
        acc += (int64_t)(na >= 8 ? na - 16 : na) * (int64_t)(nw >= 8 ? nw - 16 : nw);
      }
      const float s = sa[t] * sw[o];
      c[t * O + o] = (float)acc * s;
    }
  return 0;
}

int fqo_mx_gemm(int64_t T, int64_t O, int64_t H, const uint8_t* a, const uint8_t* a_e8, const uint8_t* w,
                const uint8_t* w_e8, double* c, double* cabs) {
  if (T < 1 || O < 1 || H < 2 || H % 32 != 0) return -1;
  const int64_t gs = 2 * ceil_div(H, 64);
  double* av = (double*)malloc(sizeof(double) * (size_t)H);
  double* wv = (double*)malloc(sizeof(double) * (size_t)(O * H));
  if (!av || !wv) { free(av); free(wv); return -2; }
  for (int64_t o = 0; o < O; ++o)
    for (int64_t h = 0; h < H; ++h) {
      const int nib = (w[o * (H / 2) + h / 2] >> (4 * (h & 1))) & 15;
      wv[o * H + h] = ldexp(fqo_e2m1_value(nib), (int)w_e8[o * gs + h / 32] - 127);
    }
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t h = 0; h < H; ++h) {
      const int nib = (a[t * (H / 2) + h / 2] >> (4 * (h & 1))) & 15;
      av[h] = ldexp(fqo_e2m1_value(nib), (int)a_e8[t * gs + h / 32] - 127);
    }
    for (int64_t o = 0; o < O; ++o) {
      double s = 0.0, sa = 0.0;
      const double* wr = wv + o * H;
      for (int64_t h = 0; h < H; ++h) {
        const double p = av[h] * wr[h];
        s += p;
        sa += fabs(p);
      }
      c[t * O + o] = s;
      if (cabs) cabs[t * O + o] = sa;
    }
  }
  free(av);
  free(wv);
  return 0;
}
