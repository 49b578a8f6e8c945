/*
 * fp4_oracle.c -- scalar CPU oracle.  TEST INFRASTRUCTURE ONLY (see the
 * header for who may load it and for the page tags used in citations).
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -fopenmp -ffp-contract=off
 *        -fno-fast-math fp4_oracle.c -o libfp4_oracle.so -lm
 */
#include "fp4_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------
 * Element grids.
 * E2M1: sign, 2 exponent bits, 1 mantissa bit; magnitudes 0, .5, 1, 1.5, 2,
 * 3, 4, 6 ([UFP4] "Declaracion del Problema" and Metodologia 1 name E2M1;
 * [TJ2] Riepilogo 1 has 0 and 0.5 as neighbouring bins; [MXFP4] 2.A gives
 * the FP4 limit 6.0).  Uniform grid: equal spacing l_i = r_i ([UFP4]
 * Metodologia 2, "Rejilla Uniforme"), read as the integers 0..7 times the
 * block scale (E1M2 with bias 1 is k/4; the factor 4 lives in the scale).
 * ---------------------------------------------------------------------- */
static const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
static const double kUniform[8] = {0.0, 1.0, 2.0, 3.0, 4.0, 5.0, 6.0, 7.0};

static const double* grid_levels(int grid) {
  return grid == FP4R_GRID_UNIFORM ? kUniform : kE2M1;
}

/* The largest code a grid rounds to: 7, or 4 (magnitude 2) for the E2M1
 * grid cut at 2 ([UFP4] Ablacion: E2M1 with its maximum limited, which the
 * page tried as an emulation of a uniform grid; cut at 2 the levels 0, .5,
 * 1, 1.5, 2 are equally spaced).  Codes above the top still decode through
 * the E2M1 table. */
static int grid_top(int grid) { return grid == FP4R_GRID_E2M1_CAP2 ? 4 : 7; }

float fp4r_level(int grid, int k) { return (float)grid_levels(grid)[k & 7]; }

/* ------------------------------------------------------------------------
 * Philox4x32-10 (Salmon et al., SC'11).  One round maps counter c under key
 * k: the two 32x32 -> 64-bit products M0*c0 and M1*c2 are split into high
 * and low words, and the new counter is
 *   (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0));
 * the key is bumped by the Weyl constants between rounds.
 * ---------------------------------------------------------------------- */
#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

void fp4r_philox4x32_10(uint32_t k0, uint32_t k1, const uint32_t ctr[4],
                        uint32_t out[4]) {
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += PHILOX_W0;
      k1 += PHILOX_W1;
    }
    uint64_t p0 = (uint64_t)PHILOX_M0 * (uint64_t)c0;
    uint64_t p1 = (uint64_t)PHILOX_M1 * (uint64_t)c2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    uint32_t n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

uint16_t fp4r_rht_signs(uint64_t seed) {
  uint32_t ctr[4] = {0u, 0u, 1u, 0u};
  uint32_t out[4];
  fp4r_philox4x32_10((uint32_t)seed, (uint32_t)(seed >> 32), ctr, out);
  return (uint16_t)(out[0] & 0xFFFFu);
}

/* Draw for logical element n: one Philox call per 8 consecutive elements,
 * counter (g_lo, g_hi, 0, 0) with g = n / 8; element l = n % 8 takes the
 * 16-bit half (l % 2) of word (l / 2). */
uint32_t fp4r_sr_u16(uint64_t seed, uint64_t n) {
  uint64_t g = n >> 3;
  unsigned l = (unsigned)(n & 7u);
  uint32_t ctr[4] = {(uint32_t)g, (uint32_t)(g >> 32), 0u, 0u};
  uint32_t out[4];
  fp4r_philox4x32_10((uint32_t)seed, (uint32_t)(seed >> 32), ctr, out);
  return (out[l >> 1] >> (16u * (l & 1u))) & 0xFFFFu;
}

/* ------------------------------------------------------------------------
 * Random Hadamard transform on one group of 16 ([UFP4] Metodologia 1-2 and
 * "Eficiencia"; [TJ2] 2.C): a random +-1 diagonal D followed by the
 * Sylvester-ordered Hadamard matrix, scaled by 1/4 so that it is orthogonal.
 * The butterfly runs the stages h = 1, 2, 4, 8; at each stage every pair
 * (j, j+h) with j & h == 0 becomes (t_j + t_{j+h}, t_j - t_{j+h}).
 * ---------------------------------------------------------------------- */
static void fwht16(float t[16]) {
  for (int h = 1; h < 16; h <<= 1) {
    for (int j = 0; j < 16; ++j) {
      if (j & h) continue;
      float u = t[j], v = t[j + h];
      t[j] = u + v;
      t[j + h] = u - v;
    }
  }
}

void fp4r_rht16(const float in[16], uint16_t signs, int inverse,
                float out[16]) {
  float t[16];
  if (!inverse) {
    for (int j = 0; j < 16; ++j) t[j] = ((signs >> j) & 1u) ? -in[j] : in[j];
    fwht16(t);
    for (int j = 0; j < 16; ++j) out[j] = t[j] * 0.25f;
  } else {
    for (int j = 0; j < 16; ++j) t[j] = in[j];
    fwht16(t);
    for (int j = 0; j < 16; ++j) {
      float s = t[j] * 0.25f;
      out[j] = ((signs >> j) & 1u) ? -s : s;
    }
  }
}

/* ------------------------------------------------------------------------
 * E4M3 scale byte (NVFP4's 8-bit block scale, [TJ2] 2.A; named E4M3 in
 * [MXFP4] 2): bias 7, 3 mantissa bits, subnormal step 2^-9, largest finite
 * 448 (byte 0x7E; 0x7F is NaN).  Values are listed by byte, which orders
 * them by magnitude; encoding picks the nearest, ties to the even byte.
 * ---------------------------------------------------------------------- */
static double e4m3_value_def(unsigned b) {
  unsigned e = (b >> 3) & 15u, m = b & 7u;
  if (e == 0) return ldexp((double)m, -9);
  return ldexp(1.0 + (double)m / 8.0, (int)e - 7);
}

/* The 127 non-negative finite values, filled from the definition above
 * when the library is loaded. */
static double kE4M3[127];

__attribute__((constructor)) static void e4m3_table_init(void) {
  for (unsigned b = 0; b < 127u; ++b) kE4M3[b] = e4m3_value_def(b);
}

/* ------------------------------------------------------------------------
 * HiF4's E6M2 block scale ([HIF] 2. Metodologia: the shared scale of a
 * 64-element block; reading: unsigned, exponent bias 2^5 - 1 = 31 as in the
 * IEEE layouts, subnormals at exponent field 0, every byte finite).  The
 * 256 values are listed by byte, which orders them by magnitude.
 * ---------------------------------------------------------------------- */
static double e6m2_value_def(unsigned b) {
  unsigned e = (b >> 2) & 63u, m = b & 3u;
  if (e == 0) return ldexp((double)m / 4.0, 1 - 31);
  return ldexp(1.0 + (double)m / 4.0, (int)e - 31);
}

static double kE6M2[256];

__attribute__((constructor)) static void e6m2_table_init(void) {
  for (unsigned b = 0; b < 256u; ++b) kE6M2[b] = e6m2_value_def(b);
}

float fp4r_e6m2_decode(uint8_t b) { return (float)kE6M2[b]; }

uint8_t fp4r_e6m2_encode(float r) {
  double x = (double)r;
  if (x >= kE6M2[255]) return 0xFF; /* saturating */
  if (!(x > 0.0)) return 0x00;
  unsigned c = 0;
  while (c + 1 <= 0xFFu && kE6M2[c + 1] <= x) ++c;
  if (kE6M2[c] == x) return (uint8_t)c;
  double dl = x - kE6M2[c], dh = kE6M2[c + 1] - x; /* exact in binary64 */
  if (dl < dh) return (uint8_t)c;
  if (dh < dl) return (uint8_t)(c + 1);
  return (uint8_t)((c & 1u) ? c + 1 : c);
}

float fp4r_e4m3_decode(uint8_t b) {
  if ((b & 0x7Fu) == 0x7Fu) return NAN;
  double v = kE4M3[b & 0x7Fu];
  return (float)((b & 0x80u) ? -v : v);
}

uint8_t fp4r_e4m3_encode(float r) {
  double x = (double)r;
  if (x >= 448.0) return 0x7E; /* saturating: 448 is the largest finite */
  if (!(x > 0.0)) return 0x00; /* zero (and negative zero) */
  unsigned c = 0;
  while (c + 1 <= 0x7Eu && kE4M3[c + 1] <= x) ++c;
  double lo = kE4M3[c];
  if (lo == x) return (uint8_t)c;
  double hi = kE4M3[c + 1];
  double dl = x - lo, dh = hi - x; /* both exact in binary64 */
  if (dl < dh) return (uint8_t)c;
  if (dh < dl) return (uint8_t)(c + 1);
  return (uint8_t)((c & 1u) ? c + 1 : c);
}

/* ------------------------------------------------------------------------
 * MX (E8M0) scale exponent ([MXFP4] 2: a power-of-two scale; 2.A: the
 * block amax lands near the top of the E2M1 range and saturates at 6).
 * e = floor(log2 amax) - 2, where 2 is E2M1's largest exponent.
 * ---------------------------------------------------------------------- */
/* ------------------------------------------------------------------------
 * Macro-block scaling, static ([MXFP4] 2.B): a scale of higher precision
 * (an 8-bit mantissa) per 128-element macro block, taken directly from the
 * macro block's maximum, over the 16-element blocks.  Reading: M =
 * round8(amax / 6) in binary32 (the largest element then sits at the top
 * E2M1 level 6), kept as FP32; round8 rounds the significand to 8 fraction
 * bits.  Done here in binary64, where every step is exact: scaling by a
 * power of two into [256, 512) and rint (ties to even).
 * ---------------------------------------------------------------------- */
float fp4r_round8(float x) {
  if (x == 0.0f || !isfinite(x)) return x;
  int ex;
  (void)frexp((double)x, &ex); /* |x| = f * 2^ex, f in [0.5, 1) */
  double scaled = ldexp((double)x, 9 - ex); /* [256, 512) */
  return (float)ldexp(rint(scaled), ex - 9);
}

float fp4r_mbs_macro_scale(float amax) { return fp4r_round8(amax / 6.0f); }

int fp4r_e8m0_exponent(float amax) {
  if (!(amax > 0.0f)) return -127;
  int ex;
  (void)frexp((double)amax, &ex); /* amax = f * 2^ex, f in [0.5, 1) */
  int e = (ex - 1) - 2;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return e;
}

/* [MXFP4] 2.A (overflow-aware scaling): the block amax is mapped into
 * (3.5, 7] instead of [4, 8), so the largest element no longer lands past
 * the top level 6 by up to a third.  Search upward from an exponent that is
 * certainly too small; amax <= 7 * 2^e is exact in binary64. */
int fp4r_e8m0_exponent_oas(float amax) {
  if (!(amax > 0.0f)) return -127;
  int ex;
  (void)frexp((double)amax, &ex); /* 2^(ex-1) <= amax < 2^ex */
  int e = ex - 5;                 /* 7 * 2^(ex-5) < 2^(ex-1) <= amax */
  while ((double)amax > 7.0 * ldexp(1.0, e)) ++e;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return e;
}

/* ------------------------------------------------------------------------
 * Rounding a magnitude m >= 0 to a grid.  k is the bin with
 * L[k] <= m < L[k+1]; m >= L[top] saturates at the grid's top code (7, or 4
 * for the cut E2M1; [MXFP4] 2.A: saturation at the FP4 limit).  RTNE compares m with the exact midpoint, ties to the even
 * code ([UFP4] Metodologia 1: RTNE bins).  SR rounds up with probability
 * p = (m - L[k]) / (L[k+1] - L[k]) using a 16-bit draw ([TJ2] 2.A:
 * stochastic rounding so that E[round(x)] = x; [UFP4] Metodologia 2: SR on
 * dY): up iff p * 2^22 >= 64 * u16 + 1, i.e. iff the draw, read as the
 * fixed-point number (u16 + 2^-6) * 2^-16, does not exceed p.  Of the 2^16
 * draws, min(2^16, floor((p * 2^22 - 1) / 64) + 1) round up (none when
 * p * 2^22 < 1), which is within one of p * 2^16: E[round(m)] equals m to
 * within 2^-16 of a bin width.
 * ---------------------------------------------------------------------- */
static int bin_below(double m, const double* L, int top) {
  int k = 0;
  while (k < top && L[k + 1] <= m) ++k;
  return k;
}

int fp4r_round_rtne(float mf, int grid) {
  const double* L = grid_levels(grid);
  const int top = grid_top(grid);
  double m = (double)mf;
  if (m >= L[top]) return top;
  int k = bin_below(m, L, top);
  double mid = 0.5 * (L[k] + L[k + 1]);
  if (m < mid) return k;
  if (m > mid) return k + 1;
  return (k & 1) ? k + 1 : k;
}

int fp4r_round_sr(float mf, int grid, uint32_t u16) {
  const double* L = grid_levels(grid);
  const int top = grid_top(grid);
  double m = (double)mf;
  if (m >= L[top]) return top;
  int k = bin_below(m, L, top);
  double p = (m - L[k]) / (L[k + 1] - L[k]);
  /* p * 2^22 and 64 * u16 + 1 are exact in binary64 */
  return (p * 4194304.0 >= 64.0 * (double)(u16 & 0xFFFFu) + 1.0) ? k + 1 : k;
}

/* ------------------------------------------------------------------------
 * Tensor helpers.
 * ---------------------------------------------------------------------- */
static float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
    return (uint16_t)((u >> 16) | 0x0040u); /* quiet NaN */
  uint32_t bias = 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)((u + bias) >> 16);
}

static float load_elem(const void* x, int dt, int64_t idx) {
  if (dt == FP4R_BF16) return bf16_to_f32(((const uint16_t*)x)[idx]);
  return ((const float*)x)[idx];
}

/* A[i][j] of the logical operand: x[i][j] for ROW, x[j][i] for COL. */
static int64_t a_index(int axis, int64_t i, int64_t j, int64_t ld) {
  return axis == FP4R_ROW ? i * ld + j : j * ld + i;
}

static int grid_of(int format) {
  if (format == FP4R_UFP4 || format == FP4R_HIF4) return FP4R_GRID_UNIFORM;
  return format == FP4R_E2M1_CAP2 ? FP4R_GRID_E2M1_CAP2 : FP4R_GRID_E2M1;
}

/* G, the largest grid level, used by the two-level tensor scale and the
 * block scale's target. */
static float grid_max(int format) {
  if (format == FP4R_UFP4) return 7.0f;
  return format == FP4R_E2M1_CAP2 ? 2.0f : 6.0f;
}

static int is_mx(int format) {
  return format == FP4R_MXFP4 || format == FP4R_MXFP4_OAS || format == FP4R_MXFP4_OAS16;
}

/* Elements per block scale: 32 for MXFP4 and MXFP4-OAS ([MXFP4] 2), 16 for
 * the rest (NVFP4's groups; [MXFP4] 2: its techniques at a granularity of 16). */
static int block_of(int format) {
  if (format == FP4R_HIF4) return 64;
  return (format == FP4R_MXFP4 || format == FP4R_MXFP4_OAS) ? 32 : 16;
}

/* Formats with a tensor (or outer) scale: the two-level E4M3 formats and
 * MBS-Static's macro scales.  The MX formats and HiF4 carry all their
 * scales per block. */
static int has_tensor_scale(int format) { return !is_mx(format) && format != FP4R_HIF4; }

static int check_params(const fp4r_params* p, int64_t rows, int64_t cols,
                        int64_t ld) {
  if (!p) return -1;
  if (p->format < 0 || p->format > 7) return -1;
  if (p->format == FP4R_MXFP4_MBS && p->ts_mode != FP4R_TS_OUTER128) return -1;
  if (p->block != block_of(p->format)) return -1;
  if (has_tensor_scale(p->format) && (p->ts_mode < 0 || p->ts_mode > 2)) return -1;
  if (p->axis != FP4R_ROW && p->axis != FP4R_COL) return -1;
  if (p->rounding != FP4R_RTNE && p->rounding != FP4R_SR) return -1;
  if (rows < 0 || cols < 0 || ld < cols) return -1;
  int64_t W = p->axis == FP4R_ROW ? cols : rows;
  if (W % p->block) return -1;
  if (p->rht && (W % 16)) return -1;
  if (has_tensor_scale(p->format) && p->ts_mode == FP4R_TS_OUTER128 && (W % FP4R_OUTER))
    return -1;
  return 0;
}

/* One row of the logical operand, widened and (optionally) rotated. */
static void load_row(const void* x, int dt, int axis, int64_t ld, int64_t i,
                     int64_t W, int rht, uint16_t signs, float* y) {
  for (int64_t j = 0; j < W; ++j) y[j] = load_elem(x, dt, a_index(axis, i, j, ld));
  if (rht)
    for (int64_t j = 0; j < W; j += 16) fp4r_rht16(y + j, signs, 0, y + j);
}

/* ------------------------------------------------------------------------
 * Block scale and element quantization.
 *
 * NVFP4 / uniform grid (two-level scaling: FP32 tensor scale, E4M3 block
 * scale per 16 elements; [TJ2] 2.A, [NGPT] "Enunciato del Problema" on
 * per-tensor dynamic scaling):
 *   s_t = amax_t / (G * 448);  r_b = amax_b / (s_t * G);  S_b = E4M3(r_b);
 *   d_b = s_t * decode(S_b);  v = y * (1 / d_b).
 * MXFP4 ([MXFP4] 2): d_b = 2^e with e = floor(log2 amax_b) - 2; with
 * overflow-aware scaling ([MXFP4] 2.A) e places amax_b / 2^e in (3.5, 7].
 * Double block ([TJ2] 2.A): s_t is replaced by the outer scale of the
 * 128-element piece of the A-row that holds the block.
 * A block whose scale decodes to zero codes every element as a signed zero.
 * ---------------------------------------------------------------------- */
static float block_decode_scale(const fp4r_params* p, uint8_t sbyte, float s_t) {
  if (is_mx(p->format)) return ldexpf(1.0f, (int)sbyte - 127);
  /* MBS: d_b = M * 2^e_b in binary32 (s_t holds the macro scale M) */
  if (p->format == FP4R_MXFP4_MBS) return ldexpf(s_t, (int)sbyte - 127);
  if (sbyte == 0) return 0.0f;
  return s_t * fp4r_e4m3_decode(sbyte);
}

static uint8_t block_scale_byte(const fp4r_params* p, float amax_b, float s_t) {
  if (p->format == FP4R_MXFP4) return (uint8_t)(fp4r_e8m0_exponent(amax_b) + 127);
  if (p->format == FP4R_MXFP4_OAS || p->format == FP4R_MXFP4_OAS16)
    return (uint8_t)(fp4r_e8m0_exponent_oas(amax_b) + 127);
  /* MBS: the MX exponent rule applied to amax_b / M, so the block's largest
   * element lands in [4, 8) times d_b = M * 2^e_b (e_b = 0 for the block
   * holding the macro maximum: amax / M is then about 6). */
  if (p->format == FP4R_MXFP4_MBS) {
    if (s_t == 0.0f || amax_b == 0.0f) return 0x00;
    return (uint8_t)(fp4r_e8m0_exponent(amax_b / s_t) + 127);
  }
  if (s_t == 0.0f || amax_b == 0.0f) return 0x00;
  float den = s_t * grid_max(p->format);
  float r = amax_b / den;
  return fp4r_e4m3_encode(r);
}

void fp4r_quantize_block(const float* y, const fp4r_params* p,
                         uint8_t scale_byte, float tensor_scale,
                         int64_t row_a, int64_t col_a0, int64_t W,
                         uint8_t* codes_out) {
  int grid = grid_of(p->format);
  float d = block_decode_scale(p, scale_byte, tensor_scale);
  float inv = d != 0.0f ? 1.0f / d : 0.0f;
  for (int i = 0; i < p->block; ++i) {
    float yi = y[i];
    unsigned s = signbit(yi) ? 1u : 0u;
    int k = 0;
    if (d != 0.0f && yi != 0.0f) {
      float v = yi * inv;
      float m = fabsf(v);
      if (p->rounding == FP4R_SR) {
        uint64_t n = (uint64_t)row_a * (uint64_t)W + (uint64_t)(col_a0 + i);
        k = fp4r_round_sr(m, grid, fp4r_sr_u16(p->sr_seed, n));
      } else {
        k = fp4r_round_rtne(m, grid);
      }
    }
    codes_out[i] = (uint8_t)((s << 3) | (unsigned)k);
  }
}

/* ------------------------------------------------------------------------
 * HiF4 ([HIF] 2. Metodologia): a 64-element block shares an E6M2 scale S;
 * each of its eight 8-element sub-blocks refines it by an E1M0 factor f8,
 * each of its sixteen 4-element micro-blocks by another, f4; elements are
 * E1M2, magnitudes k/4.  The block's largest magnitude is mapped to the top
 * element level 7/4: S = E6M2(amax / 1.75).  A refinement halves the scale
 * when the piece's maximum still fits under the top level after halving:
 * f8 = 1/2 iff amax_8 <= 0.875 * S, f4 = 1/2 iff amax_4 <= 0.875 * S * f8
 * (products of powers of two and 3-bit significands: exact in binary32).
 * The element step is d = S * f8 * f4 / 4; v = y * (1 / d) is rounded on
 * the uniform grid 0..7 (RTNE or SR, saturating at 7), as for UFP4.
 * ---------------------------------------------------------------------- */
static float hif4_step(float S, uint32_t word, int e) {
  const int sub = e / 8, micro = e / 4;
  const float f8 = ((word >> (8 + sub)) & 1u) ? 1.0f : 0.5f;
  const float f4 = ((word >> (16 + micro)) & 1u) ? 1.0f : 0.5f;
  return S * f8 * f4 * 0.25f;
}

static uint32_t hif4_block(const float* y, const fp4r_params* p, int64_t row_a,
                           int64_t col_a0, int64_t W, uint8_t* kb) {
  float amax = 0.0f;
  for (int e = 0; e < 64; ++e)
    if (fabsf(y[e]) > amax) amax = fabsf(y[e]);
  const uint8_t sb = fp4r_e6m2_encode(amax / 1.75f);
  const float S = fp4r_e6m2_decode(sb);
  uint32_t word = sb;
  for (int s = 0; s < 8; ++s) {
    float a8 = 0.0f;
    for (int e = 8 * s; e < 8 * s + 8; ++e)
      if (fabsf(y[e]) > a8) a8 = fabsf(y[e]);
    const int keep8 = !(a8 <= 0.875f * S);
    if (keep8) word |= 1u << (8 + s);
    const float f8 = keep8 ? 1.0f : 0.5f;
    for (int u = 2 * s; u < 2 * s + 2; ++u) {
      float a4 = 0.0f;
      for (int e = 4 * u; e < 4 * u + 4; ++e)
        if (fabsf(y[e]) > a4) a4 = fabsf(y[e]);
      if (!(a4 <= 0.875f * S * f8)) word |= 1u << (16 + u);
    }
  }
  for (int e = 0; e < 64; ++e) {
    const float d = hif4_step(S, word, e);
    const float yi = y[e];
    unsigned sgn = signbit(yi) ? 1u : 0u;
    int k = 0;
    if (d != 0.0f && yi != 0.0f) {
      const float inv = 1.0f / d;
      const float m = fabsf(yi * inv);
      if (p->rounding == FP4R_SR) {
        uint64_t n = (uint64_t)row_a * (uint64_t)W + (uint64_t)(col_a0 + e);
        k = fp4r_round_sr(m, FP4R_GRID_UNIFORM, fp4r_sr_u16(p->sr_seed, n));
      } else {
        k = fp4r_round_rtne(m, FP4R_GRID_UNIFORM);
      }
    }
    kb[e] = (uint8_t)((sgn << 3) | (unsigned)k);
  }
  return word;
}

int fp4r_quantize(const void* x, int in_dtype, int64_t rows, int64_t cols,
                  int64_t ld, const fp4r_params* p, uint8_t* codes,
                  uint8_t* scales, float* tensor_scale) {
  if (check_params(p, rows, cols, ld)) return -1;
  if (in_dtype != FP4R_BF16 && in_dtype != FP4R_F32) return -1;
  const int axis = p->axis, B = p->block;
  const int64_t RA = axis == FP4R_ROW ? rows : cols;
  const int64_t W = axis == FP4R_ROW ? cols : rows;
  const uint16_t signs = p->rht ? fp4r_rht_signs(p->rht_seed) : 0;
  const int two_level = has_tensor_scale(p->format);
  const int outer = two_level && p->ts_mode == FP4R_TS_OUTER128;

  /* tensor scale: amax over the whole (rotated) operand */
  float s_t = 0.0f;
  if (two_level) {
    if (!tensor_scale) return -1;
    if (outer) {
      /* double block: one scale per 128-element piece, in the row loop */
    } else if (p->ts_mode == FP4R_TS_GIVEN) {
      s_t = *tensor_scale;
    } else {
      float amax = 0.0f;
#pragma omp parallel
      {
        float* y = (float*)malloc(sizeof(float) * (size_t)(W > 0 ? W : 1));
        float local = 0.0f;
#pragma omp for schedule(static)
        for (int64_t i = 0; i < RA; ++i) {
          load_row(x, in_dtype, axis, ld, i, W, p->rht, signs, y);
          for (int64_t j = 0; j < W; ++j)
            if (fabsf(y[j]) > local) local = fabsf(y[j]);
        }
#pragma omp critical
        if (local > amax) amax = local;
        free(y);
      }
      s_t = amax / (grid_max(p->format) * 448.0f);
      *tensor_scale = s_t;
    }
  }

  const int64_t nblk = W / B;
  const int64_t nout = W / FP4R_OUTER;
#pragma omp parallel
  {
    float* y = (float*)malloc(sizeof(float) * (size_t)(W > 0 ? W : 1));
    uint8_t kb[64];
#pragma omp for schedule(static)
    for (int64_t i = 0; i < RA; ++i) {
      load_row(x, in_dtype, axis, ld, i, W, p->rht, signs, y);
      if (p->format == FP4R_HIF4) {
        for (int64_t b = 0; b < nblk; ++b) {
          const uint32_t word = hif4_block(y + b * 64, p, i, b * 64, W, kb);
          for (int j = 0; j < 4; ++j) scales[(i * nblk + b) * 4 + j] = (uint8_t)(word >> (8 * j));
          for (int e = 0; e < 64; e += 2)
            codes[i * (W / 2) + (b * 64 + e) / 2] = (uint8_t)(kb[e] | (kb[e + 1] << 4));
        }
        continue;
      }
      if (outer) {
        /* [TJ2] 2.A double block: the outer scale of a 128-element piece
         * takes the place of the tensor scale, from that piece's amax. */
        for (int64_t o = 0; o < nout; ++o) {
          float amax_o = 0.0f;
          for (int e = 0; e < FP4R_OUTER; ++e)
            if (fabsf(y[o * FP4R_OUTER + e]) > amax_o) amax_o = fabsf(y[o * FP4R_OUTER + e]);
          tensor_scale[i * nout + o] = p->format == FP4R_MXFP4_MBS
                                           ? fp4r_mbs_macro_scale(amax_o)
                                           : amax_o / (grid_max(p->format) * 448.0f);
        }
      }
      for (int64_t b = 0; b < nblk; ++b) {
        const float* yb = y + b * B;
        const float s_b = outer ? tensor_scale[i * nout + (b * B) / FP4R_OUTER] : s_t;
        float amax_b = 0.0f;
        for (int e = 0; e < B; ++e)
          if (fabsf(yb[e]) > amax_b) amax_b = fabsf(yb[e]);
        uint8_t sbyte = block_scale_byte(p, amax_b, s_b);
        scales[i * nblk + b] = sbyte;
        fp4r_quantize_block(yb, p, sbyte, s_b, i, b * B, W, kb);
        for (int e = 0; e < B; e += 2) {
          int64_t c = b * B + e; /* even column: low nibble */
          codes[i * (W / 2) + c / 2] = (uint8_t)(kb[e] | (kb[e + 1] << 4));
        }
      }
    }
    free(y);
  }
  return 0;
}

int fp4r_dequantize(const uint8_t* codes, const uint8_t* scales,
                    const float* tensor_scale, int64_t rows, int64_t cols,
                    const fp4r_params* p, int inverse_rht, void* out,
                    int out_dtype, int64_t ld_out) {
  if (check_params(p, rows, cols, ld_out)) return -1;
  if (out_dtype != FP4R_BF16 && out_dtype != FP4R_F32) return -1;
  if (inverse_rht && !p->rht) return -1;
  const int axis = p->axis, B = p->block, grid = grid_of(p->format);
  const int64_t RA = axis == FP4R_ROW ? rows : cols;
  const int64_t W = axis == FP4R_ROW ? cols : rows;
  const int64_t nblk = W / B;
  const uint16_t signs = p->rht ? fp4r_rht_signs(p->rht_seed) : 0;
  const int outer = has_tensor_scale(p->format) && p->ts_mode == FP4R_TS_OUTER128;
  const int hif4 = p->format == FP4R_HIF4;
  float s_t = 0.0f;
  if (has_tensor_scale(p->format)) {
    if (!tensor_scale) return -1;
    if (!outer) s_t = *tensor_scale;
  }
#pragma omp parallel
  {
    float* v = (float*)malloc(sizeof(float) * (size_t)(W > 0 ? W : 1));
#pragma omp for schedule(static)
    for (int64_t i = 0; i < RA; ++i) {
      for (int64_t b = 0; b < nblk; ++b) {
        uint32_t word = 0;
        float S = 0.0f, d = 0.0f;
        if (hif4) {
          const uint8_t* sw = scales + (i * nblk + b) * 4;
          word = sw[0] | (sw[1] << 8) | ((uint32_t)sw[2] << 16) | ((uint32_t)sw[3] << 24);
          S = fp4r_e6m2_decode(sw[0]);
        } else {
          const float s_b =
              outer ? tensor_scale[i * (W / FP4R_OUTER) + (b * B) / FP4R_OUTER] : s_t;
          d = block_decode_scale(p, scales[i * nblk + b], s_b);
        }
        for (int e = 0; e < B; ++e) {
          int64_t c = b * B + e;
          uint8_t byte = codes[i * (W / 2) + c / 2];
          unsigned code = (c & 1) ? (byte >> 4) : (byte & 15u);
          /* HiF4: k * d with d the element's step, S * f8 * f4 / 4 */
          float mag = hif4 ? (float)(code & 7u) * hif4_step(S, word, e)
                           : fp4r_level(grid, (int)(code & 7u)) * d;
          v[c] = (code & 8u) ? -mag : mag;
        }
      }
      if (inverse_rht)
        for (int64_t j = 0; j < W; j += 16) fp4r_rht16(v + j, signs, 1, v + j);
      for (int64_t j = 0; j < W; ++j) {
        int64_t o = a_index(axis, i, j, ld_out);
        if (out_dtype == FP4R_F32) ((float*)out)[o] = v[j];
        else ((uint16_t*)out)[o] = f32_to_bf16_rne(v[j]);
      }
    }
    free(v);
  }
  return 0;
}

int fp4r_rht(const void* x, int in_dtype, int64_t rows, int64_t cols,
             int64_t ld, int axis, uint64_t seed, int inverse, float* y) {
  if (in_dtype != FP4R_BF16 && in_dtype != FP4R_F32) return -1;
  if (axis != FP4R_ROW && axis != FP4R_COL) return -1;
  if (rows < 0 || cols < 0 || ld < cols) return -1;
  const int64_t RA = axis == FP4R_ROW ? rows : cols;
  const int64_t W = axis == FP4R_ROW ? cols : rows;
  if (W % 16) return -1;
  const uint16_t signs = fp4r_rht_signs(seed);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < RA; ++i) {
    for (int64_t j = 0; j < W; j += 16) {
      float a[16], t[16];
      for (int e = 0; e < 16; ++e) a[e] = load_elem(x, in_dtype, a_index(axis, i, j + e, ld));
      fp4r_rht16(a, signs, inverse, t);
      for (int e = 0; e < 16; ++e) y[a_index(axis, i, j + e, cols)] = t[e];
    }
  }
  return 0;
}

/* ---- array forms ------------------------------------------------------- */
void fp4r_e4m3_encode_n(const float* r, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = fp4r_e4m3_encode(r[i]);
}

void fp4r_round_n(const float* m, int64_t n, int grid, int rounding,
                  const uint32_t* u16, uint8_t* k_out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    k_out[i] = (uint8_t)(rounding == FP4R_SR ? fp4r_round_sr(m[i], grid, u16[i])
                                             : fp4r_round_rtne(m[i], grid));
}

void fp4r_e6m2_encode_n(const float* r, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = fp4r_e6m2_encode(r[i]);
}

void fp4r_f32_to_bf16_n(const float* in, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne(in[i]);
}

void fp4r_sr_u16_n(uint64_t seed, const uint64_t* idx, int64_t n,
                   uint32_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = fp4r_sr_u16(seed, idx[i]);
}

int fp4r_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
