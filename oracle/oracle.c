/*
 * oracle.c -- plain, slow CPU reference for the group-scaled 1-bit / ternary
 * y = W.x path.  TEST INFRASTRUCTURE ONLY: it is used by the tests, by the
 * smoke check and by the benchmark's CPU-baseline leg, never by the product
 * path.  It shares no code, header or table with the HIP library; it follows
 * the byte layout documented in include/lowbit.h by re-deriving every index
 * from that text.
 *
 * Scalar loops, double precision, no intrinsics, no blocking and no
 * reordering beyond the definitions below.
 *
 * Sources (page title and section):
 *   [P1] 7minutos.es, "Un tutorial de codificacion para ejecutar PrismML Bonsai
 *        1-bit LLM en CUDA con GGUF", section 7 "Q1_0_g128 Cuantizacion":
 *        1 bit per weight, 0 -> -scale, 1 -> +scale, one FP16 scale shared by
 *        every 128 weights; the demonstration sets the scale to the largest
 *        absolute weight of the group and the bit to 1 for weights >= 0.
 *   [P2] 7minutos.es, "PrismML lanza Bonsai 27B ...", section "Como funciona la
 *        compresion": effective weight w_i = s_g * t_i, one FP16 scale per group
 *        of 128; ternary t in {-1, 0, +1}.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - groups run along K (the reduction axis), K % 128 == 0;
 *   - FP16 inputs: max|w| of FP16 values is itself an FP16 value, so the scale
 *     needs no rounding; NaN groups take the NaN pattern with the largest
 *     magnitude bits; the bit is the IEEE comparison w >= 0 (+0, -0 -> 1,
 *     NaN -> 0);
 *   - ternary values are stored as (pos, neg) bit planes, t = pos - neg;
 *   - the output y is the exact sum, evaluated here in double precision.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORC_Q1 1
#define ORC_T2 2

/* ---------------------------------------------------------------------- */
/* Number formats (IEEE 754 binary16 and the bfloat16 truncation of binary32) */

/* binary16 -> double, exact: sign, 5-bit exponent (bias 15), 10-bit fraction. */
double orc_fp16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1F;
  int f = h & 0x3FF;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -24); /* subnormal: f * 2^-24 */
  } else if (e == 31) {
    v = (f == 0) ? INFINITY : NAN;
  } else {
    v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
  }
  return sign ? -v : v;
}

/* bfloat16 -> double, exact: the pattern is the high half of a binary32. */
double orc_bf16_to_f64(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* double -> bfloat16, round to nearest, ties to even, in one step (no
 * intermediate binary32 rounding).  8 significant bits, exponent range of
 * binary32, subnormal spacing 2^-133; overflow rounds to infinity. */
uint16_t orc_f64_to_bf16_rne(double v) {
  if (isnan(v)) return 0x7FC0;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (isinf(a)) return sign | 0x7F80;
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);   /* a = f * 2^e with f in [0.5, 1) */
  int E = e - 1;  /* a = 1.xxx * 2^E */
  if (E < -126) E = -126;
  double ulp = ldexp(1.0, E - 7);
  double q = a / ulp; /* exact: division by a power of two */
  double r = rint(q); /* default rounding mode: nearest, ties to even */
  double res = r * ulp;
  if (res >= ldexp(1.0, 128)) return sign | 0x7F80;
  float f = (float)res; /* exact: at most 8 significant bits, in range */
  uint32_t u;
  memcpy(&u, &f, 4);
  return sign | (uint16_t)(u >> 16);
}

/* double -> binary16, round to nearest, ties to even, in one step.  11
 * significant bits, normal exponents -14..15, subnormal spacing 2^-24; a
 * result of 2^16 or more (i.e. |v| >= 65520) is infinity. */
uint16_t orc_f64_to_fp16_rne(double v) {
  if (isnan(v)) return 0x7E00;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (isinf(a)) return sign | 0x7C00;
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);   /* a = f * 2^e with f in [0.5, 1) */
  int E = e - 1;  /* a = 1.xxx * 2^E */
  if (E < -14) E = -14;
  double ulp = ldexp(1.0, E - 10);
  double res = rint(a / ulp) * ulp; /* a / ulp is exact (power of two) */
  if (res >= 65536.0) return sign | 0x7C00;
  if (res < ldexp(1.0, -14)) /* subnormal: res = f * 2^-24, f < 1024 */
    return sign | (uint16_t)ldexp(res, 24);
  int e2;
  double m = frexp(res, &e2); /* res = m * 2^e2, m in [0.5, 1) */
  uint16_t biased = (uint16_t)(e2 - 1 + 15);
  uint16_t frac = (uint16_t)ldexp(2.0 * m - 1.0, 10); /* exact, < 1024 */
  return sign | (uint16_t)(biased << 10) | frac;
}

/* SiLU(v) = v * sigmoid(v) = v / (1 + e^-v), in double. */
double orc_silu(double v) { return v / (1.0 + exp(-v)); }

/* ---------------------------------------------------------------------- */
/* Layout, re-derived from the text of include/lowbit.h (version 1).       */

static int64_t padded_rows(int64_t n) { return (n + 15) / 16 * 16; }

int64_t orc_codes_bytes(int fmt, int64_t n, int64_t k) {
  if (n < 1 || k < 128 || k % 128 != 0) return 0;
  if (fmt == ORC_Q1) return padded_rows(n) * k / 8;
  if (fmt == ORC_T2) return padded_rows(n) * k / 4;
  return 0;
}

int64_t orc_scales_count(int64_t n, int64_t k) {
  if (n < 1 || k < 128 || k % 128 != 0) return 0;
  return padded_rows(n) * (k / 128);
}

/* Byte that holds the Q1 bit (or the T2 "pos" bit) of weight (row, col);
 * the T2 "neg" bit is 16 bytes further.  The bit inside it is col % 8. */
static int64_t code_byte(int fmt, int64_t k, int64_t row, int64_t col) {
  int64_t tile = row / 16, r = row % 16, chunk = col / 8;
  int64_t cell = tile * (k / 8) + chunk;
  return cell * (fmt == ORC_Q1 ? 16 : 32) + r;
}

static int64_t scale_elem(int64_t k, int64_t row, int64_t group) {
  return ((row / 16) * (k / 128) + group) * 16 + row % 16;
}

/* Ternary value t in {-1, 0, +1} of weight (row, col): Q1 bit 1 -> +1,
 * bit 0 -> -1 [P1 s.7]; T2 t = pos - neg. */
int orc_code_value(int fmt, const uint8_t* codes, int64_t k, int64_t row,
                   int64_t col) {
  int64_t b = code_byte(fmt, k, row, col);
  int bit = (int)(col % 8);
  if (fmt == ORC_Q1) return ((codes[b] >> bit) & 1) ? 1 : -1;
  int pos = (codes[b] >> bit) & 1;
  int neg = (codes[b + 16] >> bit) & 1;
  return pos - neg;
}

uint16_t orc_scale_bits(const uint16_t* scales, int64_t k, int64_t row,
                        int64_t group) {
  return scales[scale_elem(k, row, group)];
}

/* ---------------------------------------------------------------------- */
/* Q1 quantisation [P1 s.7]: scale = largest |w| in the group of 128,
 * bit = 1 if w >= 0 else 0.  Inputs are FP16 patterns. */

/* |w| as an ordered integer key: for every non-NaN FP16 value, larger
 * magnitude <=> larger (h & 0x7FFF); the key is the pattern of |w| itself. */
static uint16_t magnitude_bits(uint16_t h) { return h & 0x7FFF; }

static int is_nan16(uint16_t h) { return (h & 0x7FFF) > 0x7C00; }

void orc_q1_quantize(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes,
                     uint16_t* scales) {
  int64_t np = padded_rows(n), groups = k / 128;
  memset(codes, 0, (size_t)(np * k / 8));
  memset(scales, 0, (size_t)(np * groups) * sizeof(uint16_t));
  for (int64_t row = 0; row < n; ++row) {
    for (int64_t g = 0; g < groups; ++g) {
      /* scale: max |w| over the group.  For groups without NaN this is the
       * largest absolute value (computed on doubles and mapped back to its
       * exact FP16 pattern); a group with a NaN keeps the NaN pattern with the
       * largest magnitude bits. */
      int has_nan = 0;
      uint16_t nan_key = 0;
      double best = 0.0;
      uint16_t best_bits = 0;
      for (int64_t i = 0; i < 128; ++i) {
        uint16_t h = w[row * k + g * 128 + i];
        if (is_nan16(h)) {
          has_nan = 1;
          if (magnitude_bits(h) > nan_key) nan_key = magnitude_bits(h);
          continue;
        }
        double a = fabs(orc_fp16_to_f64(h));
        if (a > best) {
          best = a;
          best_bits = magnitude_bits(h);
        }
      }
      scales[scale_elem(k, row, g)] = has_nan ? nan_key : best_bits;
      /* bits: 1 iff w >= 0 (IEEE comparison; NaN compares false) */
      for (int64_t i = 0; i < 128; ++i) {
        int64_t col = g * 128 + i;
        double v = orc_fp16_to_f64(w[row * k + col]);
        if (v >= 0.0) codes[code_byte(ORC_Q1, k, row, col)] |= (uint8_t)(1u << (col % 8));
      }
    }
  }
}

/* Ternary pack [P2]: code = sign(t) as (pos, neg) bits; scales copied. */
void orc_t2_pack(const int8_t* t, const uint16_t* s, int64_t n, int64_t k,
                 uint8_t* codes, uint16_t* scales) {
  int64_t np = padded_rows(n), groups = k / 128;
  memset(codes, 0, (size_t)(np * k / 4));
  memset(scales, 0, (size_t)(np * groups) * sizeof(uint16_t));
  for (int64_t row = 0; row < n; ++row) {
    for (int64_t g = 0; g < groups; ++g)
      scales[scale_elem(k, row, g)] = s[row * groups + g];
    for (int64_t col = 0; col < k; ++col) {
      int8_t v = t[row * k + col];
      int64_t b = code_byte(ORC_T2, k, row, col);
      if (v > 0) codes[b] |= (uint8_t)(1u << (col % 8));
      if (v < 0) codes[b + 16] |= (uint8_t)(1u << (col % 8));
    }
  }
}

/* Dequantise to FP16 patterns [P1 s.7: scale if bit == 1 else -scale; P2:
 * w = s * t].  -s is s with its sign bit flipped; t = 0 gives +0.0. */
void orc_unpack(int fmt, const uint8_t* codes, const uint16_t* scales,
                int64_t n, int64_t k, uint16_t* w) {
  for (int64_t row = 0; row < n; ++row) {
    for (int64_t col = 0; col < k; ++col) {
      uint16_t s = scales[scale_elem(k, row, col / 128)];
      int t = orc_code_value(fmt, codes, k, row, col);
      uint16_t out;
      if (t > 0) out = s;
      else if (t < 0) out = (uint16_t)(s ^ 0x8000);
      else out = 0;
      w[row * k + col] = out;
    }
  }
}

/* ---------------------------------------------------------------------- */
/* Products, in double precision.                                          */

/* y[i][r] = sum_g s[row][g] * sum_{k in g} t[row][k] * x[i][k]
 * for rows row0 .. row0+nrows-1 and 0 <= i < b.  x is [b][k] doubles,
 * y is [b][nrows]. */
void orc_gemv_rows_f64x(int fmt, const uint8_t* codes, const uint16_t* scales,
                        int64_t n, int64_t k, const double* x, int64_t b,
                        int64_t row0, int64_t nrows, double* y) {
  (void)n;
  int64_t groups = k / 128;
  for (int64_t i = 0; i < b; ++i) {
    for (int64_t r = 0; r < nrows; ++r) {
      int64_t row = row0 + r;
      double total = 0.0;
      for (int64_t g = 0; g < groups; ++g) {
        double part = 0.0;
        for (int64_t j = 0; j < 128; ++j) {
          int64_t col = g * 128 + j;
          int t = orc_code_value(fmt, codes, k, row, col);
          part += (double)t * x[i * k + col];
        }
        total += orc_fp16_to_f64(scales[scale_elem(k, row, g)]) * part;
      }
      y[i * nrows + r] = total;
    }
  }
}

/* Same with x given as FP16 patterns ([b][k]); x is converted exactly. */
void orc_gemv_rows(int fmt, const uint8_t* codes, const uint16_t* scales,
                   int64_t n, int64_t k, const uint16_t* x_fp16, int64_t b,
                   int64_t row0, int64_t nrows, double* xbuf, double* y) {
  for (int64_t i = 0; i < b * k; ++i) xbuf[i] = orc_fp16_to_f64(x_fp16[i]);
  orc_gemv_rows_f64x(fmt, codes, scales, n, k, xbuf, b, row0, nrows, y);
}

/* GEMM: Y[i][r] for X rows i in [m0, m0+mrows) and weight rows
 * [row0, row0+nrows); X is BF16 [*][k]; Y is [mrows][nrows] doubles.
 * Each output is the GEMV sum of one X row. */
void orc_gemm_rows(int fmt, const uint8_t* codes, const uint16_t* scales,
                   int64_t n, int64_t k, const uint16_t* x_bf16, int64_t m0,
                   int64_t mrows, int64_t row0, int64_t nrows, double* xbuf,
                   double* y) {
  for (int64_t i = 0; i < mrows; ++i) {
    for (int64_t c = 0; c < k; ++c) xbuf[c] = orc_bf16_to_f64(x_bf16[(m0 + i) * k + c]);
    orc_gemv_rows_f64x(fmt, codes, scales, n, k, xbuf, 1, row0, nrows,
                       y + i * nrows);
  }
}

/* Decode FFN, hidden part.  h = W_gu x with W_gu [2f][k]: rows 0..f-1 are
 * the gate projection, rows f..2f-1 the up projection; then
 *   z[i][j] = RNE_fp16( SiLU(h[i][j]) * h[i][f + j] ),  0 <= j < f,
 * the activation that the down projection (W_dn [k][f]) reads.  x is FP16
 * [b][k]; xbuf holds b*k doubles, hbuf b*2f doubles; z is FP16 [b][f]. */
void orc_ffn_hidden(int fmt, const uint8_t* gu_codes, const uint16_t* gu_scales,
                    int64_t k, int64_t f, const uint16_t* x_fp16, int64_t b,
                    double* xbuf, double* hbuf, uint16_t* z_fp16) {
  orc_gemv_rows(fmt, gu_codes, gu_scales, 2 * f, k, x_fp16, b, 0, 2 * f, xbuf, hbuf);
  for (int64_t i = 0; i < b; ++i)
    for (int64_t j = 0; j < f; ++j) {
      double gate = hbuf[i * 2 * f + j];
      double up = hbuf[i * 2 * f + f + j];
      z_fp16[i * f + j] = orc_f64_to_fp16_rne(orc_silu(gate) * up);
    }
}

/* ---------------------------------------------------------------------- */
/* Ternary quantiser and base-3 storage.                                  */
/* [P2] "Como funciona la compresion": a ternary weight carries log2(3)   */
/* bits, ~1.71 bits per weight with one FP16 scale per 128.  The pages    */
/* give no ternary rounding rule; the rule here is this build's reading:  */
/* s = max |w| of the group (as the 1-bit worked example), and t is the   */
/* nearest of {-1, 0, +1} to w / s, ties going to 0: t = sign(w) when     */
/* 2 |w| > s (IEEE comparison in double, exact for FP16 inputs; false for */
/* a NaN, and for 2 |w| = s), else 0.                                     */

void orc_t2_quantize(const uint16_t* w, int64_t n, int64_t k, int8_t* t_out,
                     uint16_t* s_out) {
  int64_t groups = k / 128;
  for (int64_t row = 0; row < n; ++row)
    for (int64_t g = 0; g < groups; ++g) {
      uint16_t smax = 0;
      for (int64_t j = 0; j < 128; ++j) {
        uint16_t m = magnitude_bits(w[row * k + g * 128 + j]);
        if (m > smax) smax = m;
      }
      s_out[row * groups + g] = smax;
      double s = orc_fp16_to_f64(smax);
      for (int64_t j = 0; j < 128; ++j) {
        uint16_t h = w[row * k + g * 128 + j];
        double v = orc_fp16_to_f64(h);
        int8_t t = 0;
        if (2.0 * fabs(v) > s) t = (h & 0x8000) ? -1 : 1;
        t_out[row * k + g * 128 + j] = t;
      }
    }
}

/* Base-3 storage: five trits per byte, byte = sum_i (t_i + 1) * 3^i for the
 * weights 5j + i of a row (i = 0..4), rows packed one after another with
 * ceil(k / 5) bytes each; positions past k hold t = 0.  8/5 + 16/128 =
 * 1.725 bits per weight with the FP16 scales. */
int64_t orc_base3_row_bytes(int64_t k) { return (k + 4) / 5; }

void orc_base3_pack(const int8_t* t, int64_t n, int64_t k, uint8_t* out) {
  int64_t rb = orc_base3_row_bytes(k);
  for (int64_t row = 0; row < n; ++row)
    for (int64_t j = 0; j < rb; ++j) {
      int v = 0, p = 1;
      for (int i = 0; i < 5; ++i) {
        int64_t col = 5 * j + i;
        int tv = col < k ? t[row * k + col] : 0;
        v += (tv + 1) * p;
        p *= 3;
      }
      out[row * rb + j] = (uint8_t)v;
    }
}

/* Inverse; a byte of 243..255 (never written by the packer) decodes with
 * its fifth digit taken mod 3. */
void orc_base3_unpack(const uint8_t* in, int64_t n, int64_t k, int8_t* t) {
  int64_t rb = orc_base3_row_bytes(k);
  for (int64_t row = 0; row < n; ++row)
    for (int64_t col = 0; col < k; ++col) {
      int v = in[row * rb + col / 5];
      int i = (int)(col % 5);
      for (int q = 0; q < i; ++q) v /= 3;
      t[row * k + col] = (int8_t)(v % 3 - 1);
    }
}
