/*
 * oracle.c -- plain fp64 CPU oracle for the fused row operators.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path loads this file or
 * the library built from it: only the test-suite, the package smoke check and
 * the benchmark's CPU-baseline leg do.  It shares no code, header, table or
 * helper with the HIP library; the two meet only through the bits of the
 * seeded inputs and outputs.
 *
 * Source pages (cited by title and section):
 *   [EW]  "TileLang tutorial, ch. 13: elementwise, normalisation and RoPE
 *          operators" (tilelang-tutorial.huandu.me/13-operators-elementwise-norm-rope/)
 *
 * How it computes: every input value is decoded exactly to double; every
 * formula is evaluated in double in the order the definitions state; every
 * 16-bit output and every scale is rounded ONCE, directly from double, to its
 * storage format with round-to-nearest-even, by the encoders below (written
 * from the IEEE-754 binary16 layout, the bfloat16 layout (the top half of
 * binary32) and the OCP 8-bit floating point spec for E4M3FN).  The one
 * exception is the FP8 codes, whose quotient is rounded to binary32 first
 * (next point).  There is no fusion, blocking or reordering: one row at a
 * time, one element at a time, single thread.
 *
 * Readings of points the pages leave open:
 *  - FP8 is OCP E4M3FN (bias 7, max finite 448 = 0x7E, S.1111.111 is NaN, no
 *    infinities); the quantisation divides by the scale and clamps to +-448
 *    before encoding, as the per-token cast in [EW] s3.1.5 does.  That cast
 *    divides in float32 fragments, so the code is decided on the binary32
 *    quotient.  Where the dividend is a stored 16-bit value (the per-token
 *    and per-group cast, the v cache) (float)(v / (double)scale) is the
 *    correctly rounded binary32 quotient (a double quotient of two binary32
 *    values rounds innocuously).  Where it is the unrounded double z of the
 *    fused operators, the same expression rounds z / scale twice, first to
 *    53 bits, far below the binary32 decision it feeds.  A diagnostic switch
 *    (quotient64) encodes the double quotient directly instead; it is not
 *    used for parity.
 *  - The per-token scale is max(amax, floor)/448 with the floor 1e-4 taken as
 *    the binary32 constant the kernels hold; the scale is stored as binary32.
 *  - The fused operator does not round between the norm and the rotation.
 *  - eps enters as the binary32 value the caller passes.
 *  - The elementwise family computes x * alpha + b with one rounding at the
 *    output (the fused kernel's fp32 arithmetic, not eager PyTorch's rounding
 *    after each step).
 *  - The quantised KV-cache write of the QK-norm fusion ([EW] s2.4) uses the
 *    per-token cast with each (token, head) of k and of v as its own group,
 *    k after its norm and rotation (unrounded), v as stored; cache rows are
 *    addressed through a slot per token, and slots outside the cache are
 *    skipped.
 *
 * Every function below has a pin in tests/ (brute force, closed forms or
 * invariants); none is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F16 1
#define OR_BF16 2
#define OR_F32 3

/* ------------------------------------------------------------------ */
/* decoders: storage bits -> exact double                               */
/* ------------------------------------------------------------------ */

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double oracle_decode_f16(uint16_t h) {
  int s = h >> 15;
  int e = (h >> 10) & 0x1F;
  int m = h & 0x3FF;
  double v;
  if (e == 0) {
    v = ldexp((double)m, -24); /* subnormal: m * 2^-14 * 2^-10 */
  } else if (e == 31) {
    v = m ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
  }
  return s ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
double oracle_decode_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 fraction bits; no infinities;
 * exponent 15 with fraction 7 is NaN; exponent 0 is subnormal (m * 2^-9). */
double oracle_decode_e4m3(uint8_t c) {
  int s = c >> 7;
  int e = (c >> 3) & 0xF;
  int m = c & 0x7;
  double v;
  if (e == 0xF && m == 7) {
    v = NAN;
  } else if (e == 0) {
    v = ldexp((double)m, -9);
  } else {
    v = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
  }
  return s ? -v : v;
}

/* ------------------------------------------------------------------ */
/* encoders: double -> storage bits, one round-to-nearest-even step     */
/* ------------------------------------------------------------------ */

/*
 * Round |v| to a binary format with `mbits` stored fraction bits and minimum
 * normal exponent `emin`.  Returns the magnitude as (biased exponent field,
 * fraction field) packed as (E << mbits) | M, or -1 if the rounded value
 * exceeds `maxfield` (the largest finite packed magnitude).
 *
 * Method: pick the binade of |v| (clamped below at emin so subnormals share
 * the emin quantum), divide by that binade's quantum 2^(e - mbits) -- exact in
 * double -- round the quotient to an integer with ties to even, and re-encode.
 */
static int64_t round_mag(double a, int mbits, int emin, int bias, int64_t maxfield) {
  if (a == 0.0) return 0;
  int k;
  frexp(a, &k);        /* a = f * 2^k, f in [0.5, 1) */
  int e = k - 1;       /* a in [2^e, 2^(e+1)) */
  if (e < emin) e = emin;
  double q = ldexp(1.0, e - mbits);
  double n = a / q;    /* exact: scaling by a power of two */
  double r = nearbyint(n); /* default rounding mode: to nearest, ties to even */
  /* r * q is the rounded magnitude.  r lies in [0, 2^(mbits+1)]. */
  int64_t ri = (int64_t)r;
  int64_t field;
  if (ri >= ((int64_t)1 << mbits)) {
    /* normal (possibly carried into the next binade when ri == 2^(mbits+1)) */
    int64_t E = e + bias;
    if (ri == ((int64_t)1 << (mbits + 1))) { E += 1; ri >>= 1; }
    field = (E << mbits) | (ri - ((int64_t)1 << mbits));
  } else {
    /* subnormal (only reachable when e == emin); the hidden bit is 0 */
    field = ri;
  }
  if (field > maxfield) return -1;
  return field;
}

uint16_t oracle_encode_f16(double v) {
  if (isnan(v)) return 0x7E00;
  uint16_t s = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (isinf(a)) return s | 0x7C00;
  int64_t f = round_mag(a, 10, -14, 15, 0x7BFF);
  if (f < 0) return s | 0x7C00; /* rounds past 65504 -> infinity */
  return s | (uint16_t)f;
}

uint16_t oracle_encode_bf16(double v) {
  if (isnan(v)) return 0x7FC0;
  uint16_t s = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (isinf(a)) return s | 0x7F80;
  int64_t f = round_mag(a, 7, -126, 127, 0x7F7F);
  if (f < 0) return s | 0x7F80;
  return s | (uint16_t)f;
}

/* Magnitudes above 464 (the midpoint between 448 and the next step, 480)
 * round past the largest finite value and give NaN, the non-saturating OCP
 * conversion; 464 itself ties to the even 448.  The quantiser clamps first. */
uint8_t oracle_encode_e4m3(double v) {
  if (isnan(v)) return 0x7F;
  uint8_t s = signbit(v) ? 0x80 : 0;
  double a = fabs(v);
  if (isinf(a)) return s | 0x7F;
  int64_t f = round_mag(a, 3, -6, 7, 0x7E);
  if (f < 0) return s | 0x7F;
  return s | (uint8_t)f;
}

/* ------------------------------------------------------------------ */
/* element access by dtype code                                         */
/* ------------------------------------------------------------------ */

static double load_el(const void* base, int64_t i, int dtype) {
  if (dtype == OR_F32) {
    float f;
    memcpy(&f, (const char*)base + 4 * i, 4);
    return (double)f;
  }
  uint16_t h;
  memcpy(&h, (const char*)base + 2 * i, 2);
  return dtype == OR_F16 ? oracle_decode_f16(h) : oracle_decode_bf16(h);
}

static void store_el(void* base, int64_t i, int dtype, double v) {
  if (dtype == OR_F32) {
    float f = (float)v; /* C conversion under the default mode: nearest-even */
    memcpy((char*)base + 4 * i, &f, 4);
    return;
  }
  uint16_t h = dtype == OR_F16 ? oracle_encode_f16(v) : oracle_encode_bf16(v);
  memcpy((char*)base + 2 * i, &h, 2);
}

static void copy_el(const void* src, int64_t si, void* dst, int64_t di, int dtype) {
  int w = dtype == OR_F32 ? 4 : 2;
  memcpy((char*)dst + w * di, (const char*)src + w * si, w);
}

/* The value an FP8 code is decided on: the binary32 quotient of v by the */
/* scale (the per-token cast divides in float32, [EW] s3.1.5), or with     */
/* quotient64 (a diagnostic, not used for parity) the double quotient.     */
static double fp8_quotient(double v, float scale, int quotient64) {
  double q = v / (double)scale;
  return quotient64 ? q : (double)(float)q;
}

/* ------------------------------------------------------------------ */
/* RMSNorm  ([EW] s3.2.1 reference definition)                           */
/*   rstd = 1/sqrt(mean_j x_j^2 + eps);  y_j = x_j * rstd * w_j          */
/*   weight optional (absent = 1); one rounding, at the output.          */
/* `u_out` (nullable, [rows, n] packed) receives x_j * rstd * w_j as      */
/* double, before the rounding.                                           */
/* ------------------------------------------------------------------ */
void oracle_rmsnorm(const void* x, const void* w, void* y, int64_t rows, int64_t n,
                    int64_t x_stride, int64_t y_stride, int dtype, float eps, double* u_out) {
  for (int64_t r = 0; r < rows; ++r) {
    double ss = 0.0;
    for (int64_t j = 0; j < n; ++j) {
      double v = load_el(x, r * x_stride + j, dtype);
      ss += v * v;
    }
    double rstd = 1.0 / sqrt(ss / (double)n + (double)eps);
    for (int64_t j = 0; j < n; ++j) {
      double v = load_el(x, r * x_stride + j, dtype);
      double wj = w ? load_el(w, j, dtype) : 1.0;
      double u = v * rstd * wj;
      if (u_out) u_out[r * n + j] = u;
      store_el(y, r * y_stride + j, dtype, u);
    }
  }
}

/* ------------------------------------------------------------------ */
/* LayerNorm  ([EW] s3.2.1: torch.nn.functional.layer_norm semantics)    */
/*   mu = mean x;  var = mean (x - mu)^2 (biased);                       */
/*   y = (x - mu) / sqrt(var + eps) * gamma + beta                       */
/* ------------------------------------------------------------------ */
void oracle_layernorm(const void* x, const void* gamma, const void* beta, void* y,
                      int64_t rows, int64_t n, int64_t x_stride, int64_t y_stride,
                      int dtype, float eps) {
  for (int64_t r = 0; r < rows; ++r) {
    double s = 0.0;
    for (int64_t j = 0; j < n; ++j) s += load_el(x, r * x_stride + j, dtype);
    double mu = s / (double)n;
    double d2 = 0.0;
    for (int64_t j = 0; j < n; ++j) {
      double d = load_el(x, r * x_stride + j, dtype) - mu;
      d2 += d * d;
    }
    double var = d2 / (double)n;
    double rstd = 1.0 / sqrt(var + (double)eps);
    for (int64_t j = 0; j < n; ++j) {
      double d = load_el(x, r * x_stride + j, dtype) - mu;
      double g = gamma ? load_el(gamma, j, dtype) : 1.0;
      double b = beta ? load_el(beta, j, dtype) : 0.0;
      store_el(y, r * y_stride + j, dtype, d * rstd * g + b);
    }
  }
}

/* ------------------------------------------------------------------ */
/* RoPE  ([EW] s3.3.1 conventions, s3.3.2 reference)                     */
/*   x viewed as [tokens, heads, head_dim]; each head rotates its tail    */
/*   span of rope_dim channels starting at head_dim - rope_dim; the rest  */
/*   is copied unchanged.  cos/sin are [tokens, rope_dim/2], one row per  */
/*   position, one column per pair p.                                     */
/*   interleaved: pair (2p, 2p+1);  NeoX half-split: pair (p, p + R/2).   */
/*   y_a = x_a c - x_b s;  y_b = x_a s + x_b c   (a first, b second).     */
/* `z_out` (nullable, [tokens, heads * head_dim] packed) receives every   */
/* output as double before its rounding (a pass-through channel: x).      */
/* ------------------------------------------------------------------ */
static void rope_pair_index(int64_t p, int64_t half, int neox, int64_t* a, int64_t* b) {
  if (neox) {
    *a = p;
    *b = p + half;
  } else {
    *a = 2 * p;
    *b = 2 * p + 1;
  }
}

void oracle_rope(const void* x, const void* cosv, const void* sinv, void* y,
                 int64_t tokens, int64_t heads, int64_t head_dim, int64_t rope_dim,
                 int64_t x_stride, int64_t y_stride, int dtype, int cs_dtype, int neox,
                 double* z_out) {
  int64_t half = rope_dim / 2;
  int64_t start = head_dim - rope_dim;
  for (int64_t t = 0; t < tokens; ++t) {
    for (int64_t h = 0; h < heads; ++h) {
      int64_t xb = t * x_stride + h * head_dim;
      int64_t yb = t * y_stride + h * head_dim;
      int64_t zb = (t * heads + h) * head_dim;
      for (int64_t j = 0; j < start; ++j) {
        copy_el(x, xb + j, y, yb + j, dtype);
        if (z_out) z_out[zb + j] = load_el(x, xb + j, dtype);
      }
      for (int64_t p = 0; p < half; ++p) {
        int64_t a, b;
        rope_pair_index(p, half, neox, &a, &b);
        double c = load_el(cosv, t * half + p, cs_dtype);
        double s = load_el(sinv, t * half + p, cs_dtype);
        double xa = load_el(x, xb + start + a, dtype);
        double xb_ = load_el(x, xb + start + b, dtype);
        double za = xa * c - xb_ * s, zb2 = xa * s + xb_ * c;
        if (z_out) {
          z_out[zb + start + a] = za;
          z_out[zb + start + b] = zb2;
        }
        store_el(y, yb + start + a, dtype, za);
        store_el(y, yb + start + b, dtype, zb2);
      }
    }
  }
}

/* ------------------------------------------------------------------ */
/* Fused RMSNorm -> RoPE -> per-token FP8  ([EW] s3.3.4, with the         */
/* per-token cast of s3.1.5)                                               */
/*   z = RoPE(x * rstd * w)          (double, no intermediate rounding)    */
/*   amax = max_j |z_j|;  scale = binary32(max(amax, 1e-4f) / 448)         */
/*   q_j = E4M3FN(clamp(binary32(z_j / scale), -448, 448))                 */
/* The row is the whole token: n = heads * head_dim; the norm and amax     */
/* run over all of it; the rotation acts on each head's tail span.         */
/* `z_out` (nullable) receives z as double, for the tests' composition pin. */
/* ------------------------------------------------------------------ */
void oracle_rmsnorm_rope_fp8(const void* x, const void* w, const void* cosv, const void* sinv,
                             uint8_t* q, float* scales, int64_t tokens, int64_t heads,
                             int64_t head_dim, int64_t rope_dim, int64_t x_stride,
                             int64_t q_stride, int dtype, int cs_dtype, int neox, float eps,
                             double* z_out, int quotient64) {
  int64_t n = heads * head_dim;
  int64_t half = rope_dim / 2;
  int64_t start = head_dim - rope_dim;
  const double fp8_max = 448.0;
  const double floor_amax = (double)1e-4f;
  for (int64_t t = 0; t < tokens; ++t) {
    /* pass 1: RMSNorm statistics */
    double ss = 0.0;
    for (int64_t j = 0; j < n; ++j) {
      double v = load_el(x, t * x_stride + j, dtype);
      ss += v * v;
    }
    double rstd = 1.0 / sqrt(ss / (double)n + (double)eps);
    /* pass 2: z = RoPE(normed), element by element, in double */
    double amax = 0.0;
    for (int64_t h = 0; h < heads; ++h) {
      int64_t xb = t * x_stride + h * head_dim;
      int64_t zb = t * n + h * head_dim;
      for (int64_t j = 0; j < start; ++j) {
        double wj = w ? load_el(w, h * head_dim + j, dtype) : 1.0;
        double z = load_el(x, xb + j, dtype) * rstd * wj;
        if (z_out) z_out[zb + j] = z;
        if (fabs(z) > amax) amax = fabs(z);
      }
      for (int64_t p = 0; p < half; ++p) {
        int64_t a, b;
        rope_pair_index(p, half, neox, &a, &b);
        double wa = w ? load_el(w, h * head_dim + start + a, dtype) : 1.0;
        double wb = w ? load_el(w, h * head_dim + start + b, dtype) : 1.0;
        double na = load_el(x, xb + start + a, dtype) * rstd * wa;
        double nb = load_el(x, xb + start + b, dtype) * rstd * wb;
        double c = load_el(cosv, t * half + p, cs_dtype);
        double s = load_el(sinv, t * half + p, cs_dtype);
        double za = na * c - nb * s;
        double zb2 = na * s + nb * c;
        if (z_out) {
          z_out[zb + start + a] = za;
          z_out[zb + start + b] = zb2;
        }
        if (fabs(za) > amax) amax = fabs(za);
        if (fabs(zb2) > amax) amax = fabs(zb2);
      }
    }
    float scale = (float)(fmax(amax, floor_amax) / fp8_max);
    scales[t] = scale;
    /* pass 3: quantise.  Recompute z from x (same double expression). */
    for (int64_t h = 0; h < heads; ++h) {
      int64_t xb = t * x_stride + h * head_dim;
      int64_t qb = t * q_stride + h * head_dim;
      for (int64_t j = 0; j < start; ++j) {
        double wj = w ? load_el(w, h * head_dim + j, dtype) : 1.0;
        double z = load_el(x, xb + j, dtype) * rstd * wj;
        double v = fp8_quotient(z, scale, quotient64);
        if (v > fp8_max) v = fp8_max;
        if (v < -fp8_max) v = -fp8_max;
        q[qb + j] = oracle_encode_e4m3(v);
      }
      for (int64_t p = 0; p < half; ++p) {
        int64_t a, b;
        rope_pair_index(p, half, neox, &a, &b);
        double wa = w ? load_el(w, h * head_dim + start + a, dtype) : 1.0;
        double wb = w ? load_el(w, h * head_dim + start + b, dtype) : 1.0;
        double na = load_el(x, xb + start + a, dtype) * rstd * wa;
        double nb = load_el(x, xb + start + b, dtype) * rstd * wb;
        double c = load_el(cosv, t * half + p, cs_dtype);
        double s = load_el(sinv, t * half + p, cs_dtype);
        double zz[2] = {na * c - nb * s, na * s + nb * c};
        int64_t idx[2] = {a, b};
        for (int k = 0; k < 2; ++k) {
          double v = fp8_quotient(zz[k], scale, quotient64);
          if (v > fp8_max) v = fp8_max;
          if (v < -fp8_max) v = -fp8_max;
          q[qb + start + idx[k]] = oracle_encode_e4m3(v);
        }
      }
    }
  }
}

/* ------------------------------------------------------------------ */
/* Activation quantisation to E4M3FN, per token or per group            */
/* ([EW] s3.1.5: amax per group -> scale = max(amax, 1e-4) / fp8_max -> */
/* q = clamp(x / scale, -fp8_max, fp8_max) -> fp8).  `group` consecutive */
/* channels share a scale (group == n: one scale per row).  scales is    */
/* [rows, n / group], packed.                                            */
/* ------------------------------------------------------------------ */
void oracle_act_quant_fp8(const void* x, uint8_t* q, float* scales, int64_t rows, int64_t n,
                          int64_t group, int64_t x_stride, int64_t q_stride, int dtype,
                          int quotient64) {
  const double fp8_max = 448.0;
  const double floor_amax = (double)1e-4f;
  const int64_t groups = n / group;
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t k = 0; k < groups; ++k) {
      double amax = 0.0;
      for (int64_t j = k * group; j < (k + 1) * group; ++j) {
        double v = fabs(load_el(x, r * x_stride + j, dtype));
        if (v > amax) amax = v;
      }
      float scale = (float)(fmax(amax, floor_amax) / fp8_max);
      scales[r * groups + k] = scale;
      for (int64_t j = k * group; j < (k + 1) * group; ++j) {
        double v = fp8_quotient(load_el(x, r * x_stride + j, dtype), scale, quotient64);
        if (v > fp8_max) v = fp8_max;
        if (v < -fp8_max) v = -fp8_max;
        q[r * q_stride + j] = oracle_encode_e4m3(v);
      }
    }
  }
}

/* ------------------------------------------------------------------ */
/* Per-head QK RMSNorm followed by RoPE, as one operator ([EW] s2.4:     */
/* each q/k value gets a weighted RMSNorm and then RoPE; q/k columns are  */
/* read and written back, v columns are not touched).                    */
/* A token row holds q_heads query heads, then kv_heads key heads, then   */
/* kv_heads value heads, each of head_dim channels.  For every q (k)      */
/* head: r = 1/sqrt(mean over the head of x^2 + eps); z = RoPE(x * r * w) */
/* with w = q_weight (k_weight) of length head_dim (nullable), RoPE on the */
/* head's tail span; one rounding at the output.  v is copied.            */
/* ------------------------------------------------------------------ */
void oracle_qk_norm_rope(const void* x, const void* q_weight, const void* k_weight,
                         const void* cosv, const void* sinv, void* y, int64_t tokens,
                         int64_t q_heads, int64_t kv_heads, int64_t head_dim, int64_t rope_dim,
                         int64_t x_stride, int64_t y_stride, int dtype, int cs_dtype, int neox,
                         float eps) {
  int64_t half = rope_dim / 2;
  int64_t start = head_dim - rope_dim;
  int64_t heads = q_heads + 2 * kv_heads;
  for (int64_t t = 0; t < tokens; ++t) {
    for (int64_t h = 0; h < heads; ++h) {
      int64_t xb = t * x_stride + h * head_dim;
      int64_t yb = t * y_stride + h * head_dim;
      if (h >= q_heads + kv_heads) { /* value head: untouched */
        for (int64_t j = 0; j < head_dim; ++j) copy_el(x, xb + j, y, yb + j, dtype);
        continue;
      }
      const void* w = h < q_heads ? q_weight : k_weight;
      double ss = 0.0;
      for (int64_t j = 0; j < head_dim; ++j) {
        double v = load_el(x, xb + j, dtype);
        ss += v * v;
      }
      double rstd = 1.0 / sqrt(ss / (double)head_dim + (double)eps);
      for (int64_t j = 0; j < start; ++j) {
        double wj = w ? load_el(w, j, dtype) : 1.0;
        store_el(y, yb + j, dtype, load_el(x, xb + j, dtype) * rstd * wj);
      }
      for (int64_t p = 0; p < half; ++p) {
        int64_t a, b;
        rope_pair_index(p, half, neox, &a, &b);
        double wa = w ? load_el(w, start + a, dtype) : 1.0;
        double wb = w ? load_el(w, start + b, dtype) : 1.0;
        double na = load_el(x, xb + start + a, dtype) * rstd * wa;
        double nb = load_el(x, xb + start + b, dtype) * rstd * wb;
        double c = load_el(cosv, t * half + p, cs_dtype);
        double s = load_el(sinv, t * half + p, cs_dtype);
        store_el(y, yb + start + a, dtype, na * c - nb * s);
        store_el(y, yb + start + b, dtype, na * s + nb * c);
      }
    }
  }
}

/* ------------------------------------------------------------------ */
/* One head's values quantised as in the per-token cast ([EW] s3.1.5)   */
/* with the head as the group: scale = max(amax, 1e-4) / 448, codes of  */
/* the binary32 quotient z / scale, clamped to +-448.                   */
/* ------------------------------------------------------------------ */
static void quant_head_e4m3(const double* z, int64_t n, uint8_t* codes, float* scale_out) {
  const double fp8_max = 448.0;
  double amax = 0.0;
  for (int64_t j = 0; j < n; ++j)
    if (fabs(z[j]) > amax) amax = fabs(z[j]);
  float scale = (float)(fmax(amax, (double)1e-4f) / fp8_max);
  *scale_out = scale;
  for (int64_t j = 0; j < n; ++j) {
    double v = fp8_quotient(z[j], scale, 0);
    if (v > fp8_max) v = fp8_max;
    if (v < -fp8_max) v = -fp8_max;
    codes[j] = oracle_encode_e4m3(v);
  }
}

/* ------------------------------------------------------------------ */
/* QK RMSNorm + RoPE with the quantised KV-cache write ([EW] s2.4: the  */
/* cross-module fusion Q/K RMSNorm + RoPE + quantised write of the KV   */
/* cache).  Per token t (row layout as in oracle_qk_norm_rope):         */
/*   q heads: q_out = round_T(RoPE(x * r * q_weight))                   */
/*   k heads: z = RoPE(x * r * k_weight), unrounded; v heads: z = x     */
/*   k and v heads are each quantised with one scale per (token, head)  */
/*   and written to cache row slot = slots[t] (t when slots is NULL):   */
/*   k_cache[slot * cache_stride + h * head_dim + j],                   */
/*   k_scales[slot * kv_heads + h]; likewise v.  A slot outside          */
/*   [0, num_slots) writes nothing to the caches (q is still written).  */
/* ------------------------------------------------------------------ */
void oracle_qk_norm_rope_fp8_kv(const void* x, const void* q_weight, const void* k_weight,
                                const void* cosv, const void* sinv, void* q_out,
                                uint8_t* k_cache, uint8_t* v_cache, float* k_scales,
                                float* v_scales, const int64_t* slots, int64_t num_slots,
                                int64_t tokens, int64_t q_heads, int64_t kv_heads,
                                int64_t head_dim, int64_t rope_dim, int64_t x_stride,
                                int64_t q_stride, int64_t cache_stride, int dtype, int cs_dtype,
                                int neox, float eps) {
  int64_t half = rope_dim / 2;
  int64_t start = head_dim - rope_dim;
  double* z = (double*)malloc((size_t)head_dim * sizeof(double));
  uint8_t* codes = (uint8_t*)malloc((size_t)head_dim);
  for (int64_t t = 0; t < tokens; ++t) {
    int64_t slot = slots ? slots[t] : t;
    int cached = slot >= 0 && slot < num_slots;
    for (int64_t h = 0; h < q_heads + 2 * kv_heads; ++h) {
      int64_t xb = t * x_stride + h * head_dim;
      if (h < q_heads + kv_heads) {
        const void* w = h < q_heads ? q_weight : k_weight;
        double ss = 0.0;
        for (int64_t j = 0; j < head_dim; ++j) {
          double v = load_el(x, xb + j, dtype);
          ss += v * v;
        }
        double rstd = 1.0 / sqrt(ss / (double)head_dim + (double)eps);
        for (int64_t j = 0; j < head_dim; ++j)
          z[j] = load_el(x, xb + j, dtype) * rstd * (w ? load_el(w, j, dtype) : 1.0);
        for (int64_t p = 0; p < half; ++p) {
          int64_t a, b;
          rope_pair_index(p, half, neox, &a, &b);
          double na = z[start + a], nb = z[start + b];
          double c = load_el(cosv, t * half + p, cs_dtype);
          double s = load_el(sinv, t * half + p, cs_dtype);
          z[start + a] = na * c - nb * s;
          z[start + b] = na * s + nb * c;
        }
        if (h < q_heads) {
          for (int64_t j = 0; j < head_dim; ++j)
            store_el(q_out, t * q_stride + h * head_dim + j, dtype, z[j]);
          continue;
        }
      } else {
        for (int64_t j = 0; j < head_dim; ++j) z[j] = load_el(x, xb + j, dtype);
      }
      if (!cached) continue;
      int is_k = h < q_heads + kv_heads;
      int64_t hk = h - q_heads - (is_k ? 0 : kv_heads);
      float scale;
      quant_head_e4m3(z, head_dim, codes, &scale);
      uint8_t* dst = (is_k ? k_cache : v_cache) + slot * cache_stride + hk * head_dim;
      for (int64_t j = 0; j < head_dim; ++j) dst[j] = codes[j];
      (is_k ? k_scales : v_scales)[slot * kv_heads + hk] = scale;
    }
  }
  free(z);
  free(codes);
}

/* ------------------------------------------------------------------ */
/* p + b for doubles, returned ROUNDED TO ODD at double precision: the   */
/* truncation of the exact sum, with its last bit forced to 1 when the  */
/* sum is inexact.  A value rounded to odd with at least two more bits  */
/* than a target format rounds to nearest in that format exactly as the */
/* exact sum would (Boldo and Melquiond, "Emulation of FMA and correctly */
/* rounded sums: proved algorithms using rounding to odd", IEEE TC 2008). */
/* The exact error of the rounded sum comes from Knuth's TwoSum.         */
/* ------------------------------------------------------------------ */
static double sum_round_odd(double p, double b) {
  double s = p + b;
  if (isinf(s) || isnan(s)) return s;
  double bv = s - p;
  double e = (p - (s - bv)) + (b - bv); /* p + b == s + e exactly */
  if (e == 0.0) return s;
  /* truncation toward zero of s + e: s itself when e points away from zero */
  double t = ((s > 0.0) == (e > 0.0)) ? s : nextafter(s, 0.0);
  uint64_t bits;
  memcpy(&bits, &t, 8);
  if ((bits & 1u) == 0) t = nextafter(t, s > 0.0 ? INFINITY : -INFINITY);
  return t;
}

/* ------------------------------------------------------------------ */
/* Elementwise add / scale / cast ([EW] s3.1.1: a + b, and (x * alpha)  */
/* cast to the output dtype; s1.2's scale+add scenario y = x * a + b):  */
/*   y_i = round_out(x_i * alpha + b_i)     (b_i = 0 when b is NULL)    */
/* rounded once from the exact value: the product of two binary32 values */
/* is exact in double, and the sum is carried rounded to odd.  x and b   */
/* share x_dtype; y has y_dtype.  Flat arrays of n elements.            */
/* ------------------------------------------------------------------ */
void oracle_ew_scale_add(const void* x, const void* b, void* y, int64_t n, float alpha,
                         int x_dtype, int y_dtype) {
  for (int64_t i = 0; i < n; ++i) {
    double v = load_el(x, i, x_dtype) * (double)alpha;
    if (b) v = sum_round_odd(v, load_el(b, i, x_dtype));
    store_el(y, i, y_dtype, v);
  }
}
