/*
 * fp4_oracle.h -- scalar CPU oracle for block-scaled 4-bit quantization with
 * an optional 16-point random Hadamard transform (RHT).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no source,
 * header, table or helper with the HIP library; the two meet only through
 * the seeded input generators and the comparison in the tests.
 *
 * The oracle is deliberately plain: one element at a time, in the order the
 * method is described, with linear scans instead of bit tricks.  Rows of the
 * logical operand are independent, so an OpenMP "parallel for" over rows is
 * the only concession to speed; it does not change any result.
 *
 * Pages cited (each is a summary of one paper):
 *   [UFP4]  gist.science/es/paper/2606.20381, "Replanteamiento del Sesgo de
 *           Contraccion en el Preentrenamiento de LLM en FP4"
 *   [NGPT]  gist.science/it/paper/2605.06067, "Le Architetture Normalizzate
 *           sono Nativamente a 4 Bit"
 *   [TJ2]   gist.science/it/paper/2510.27527, "TetraJet-v2: Accurate NVFP4
 *           Training for Large Language Models ..."
 *   [MXFP4] gist.science/fr/paper/2603.08713, "Unveiling the Potential of
 *           Quantization with MXFP4 ..."
 *   [HIF]   gist.science/es/paper/2602.12635, "Unleashing Low-Bit Inference
 *           on Ascend NPUs ..."
 * Published definitions used where the pages name a thing without defining
 * it: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers:
 * as easy as 1, 2, 3", SC'11); OCP FP8 E4M3 and OCP Microscaling (MX) v1.0
 * for the E4M3 and E8M0 scale bytes; the Sylvester-ordered Hadamard matrix.
 *
 * Arithmetic model: every float operation that feeds a decision is an IEEE
 * binary32 operation with round-to-nearest-even, in the order written
 * (built with -ffp-contract=off, no fast-math, denormals kept).  Rounding
 * decisions that are exact in binary64 are taken in binary64.
 */
#ifndef FP4_ORACLE_H
#define FP4_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* enumerations (values mirror the product's C-ABI by convention only) */
/* FP4R_E2M1_CAP2: E2M1 codes restricted to magnitudes <= 2 ([UFP4]
 * Metodologia 2, Ablacion: an E2M1 whose range is cut to emulate a uniform
 * grid), NVFP4's two-level scaling with the block amax mapped to 2. */
/* FP4R_MXFP4_MBS: MXFP4 with macro-block scaling, static variant ([MXFP4]
 * 2.B): one scale with an 8-bit mantissa per 128-element macro block,
 * computed from the macro block's maximum, over 16-element blocks with
 * E8M0 scales relative to it.  Always with 128-element outer scales. */
/* FP4R_MXFP4_OAS16: overflow-aware MX scaling ([MXFP4] 2.A) on 16-element
 * blocks, the granularity at which [MXFP4] 2 applies its techniques. */
/* FP4R_HIF4: the three-level HiF4 format ([HIF] 2. Metodologia): per
 * 64-element block an E6M2 scale, per 8-element sub-block and per 4-element
 * micro-block a one-bit E1M0 refinement, E1M2 elements.  Reading: element
 * magnitudes k/4 (k = 0..7); E6M2 unsigned with bias 31 and subnormals,
 * S = RNE(amax_64 / 1.75) saturating at 1.75 * 2^32; E1M0 with bias 1 is a
 * factor 1/2 (bit 0) or 1 (bit 1): a sub-block takes 1/2 iff its maximum is
 * at most 0.875 * S, a micro-block iff its maximum is at most
 * 0.875 * S * (its sub-block's factor); step d = S * f8 * f4 / 4, v = y *
 * (1 / d) rounded on the uniform grid 0..7.  Scales: 4 bytes per block
 * (byte 0 = S, byte 1 = the 8 sub-block bits, bytes 2-3 = the 16
 * micro-block bits, bit i for the i-th piece, little-endian). */
enum { FP4R_NVFP4 = 0, FP4R_MXFP4 = 1, FP4R_UFP4 = 2, FP4R_MXFP4_OAS = 3, FP4R_E2M1_CAP2 = 4,
       FP4R_MXFP4_MBS = 5, FP4R_MXFP4_OAS16 = 6, FP4R_HIF4 = 7 };
enum { FP4R_ROW = 0, FP4R_COL = 1 };
enum { FP4R_RTNE = 0, FP4R_SR = 1 };
enum { FP4R_BF16 = 0, FP4R_F32 = 1 };
enum { FP4R_TS_COMPUTE = 0, FP4R_TS_GIVEN = 1, FP4R_TS_OUTER128 = 2 };
/* Outer blocks of the double-block mode ([TJ2] 2.A): 128 elements. */
enum { FP4R_OUTER = 128 };
enum { FP4R_GRID_E2M1 = 0, FP4R_GRID_UNIFORM = 1, FP4R_GRID_E2M1_CAP2 = 2 };

typedef struct {
  int32_t format;   /* FP4R_NVFP4 / _MXFP4 / _UFP4 / _MXFP4_OAS / _E2M1_CAP2 / _MXFP4_MBS /
                       _MXFP4_OAS16 / _HIF4 */
  int32_t block;    /* 16 (NVFP4, UFP4, E2M1_CAP2, MXFP4_MBS, MXFP4_OAS16), 32 (MXFP4,
                       MXFP4_OAS) or 64 (HIF4) */
  int32_t axis;     /* FP4R_ROW: quantize along rows of x; FP4R_COL: of x^T */
  int32_t rounding; /* FP4R_RTNE or FP4R_SR (elements only; scales are RTNE) */
  int32_t rht;      /* 0: off, 1: 16-point RHT before quantization */
  int32_t ts_mode;  /* FP4R_TS_COMPUTE, _GIVEN or _OUTER128 (two-level formats) */
  uint64_t rht_seed;
  uint64_t sr_seed;
} fp4r_params;

/* ---- primitives -------------------------------------------------------- */

/* Philox4x32-10 block function (SC'11): 10 rounds of the 4x32 Philox
 * bijection of counter ctr under key (k0, k1). */
void fp4r_philox4x32_10(uint32_t k0, uint32_t k1, const uint32_t ctr[4],
                        uint32_t out[4]);

/* The 16 RHT signs of a seed: low 16 bits of Philox(key = seed,
 * counter = (0, 0, 1, 0)) word 0.  Bit j set means d_j = -1. */
uint16_t fp4r_rht_signs(uint64_t seed);

/* The 16-bit stochastic-rounding draw of logical element n = row*W + col. */
uint32_t fp4r_sr_u16(uint64_t seed, uint64_t n);

/* Forward: y = (1/4) H16 D a.  Inverse: a = D (1/4) H16 y.  Butterfly
 * stages h = 1, 2, 4, 8 in binary32, then the exact scaling by 1/4. */
void fp4r_rht16(const float in[16], uint16_t signs, int inverse, float out[16]);

/* OCP E4M3 (FN: bias 7, max 448, no infinities), round to nearest even,
 * saturating to 448 for r >= 448.  r must be >= 0. */
uint8_t fp4r_e4m3_encode(float r);
float fp4r_e4m3_decode(uint8_t b);

/* MX scale exponent for a block amax: floor(log2 amax) - 2 clamped to
 * [-127, 127]; amax == 0 gives -127. */
int fp4r_e8m0_exponent(float amax);
/* A binary32 value rounded to 8 fraction bits (9 significant bits counted
 * from its leading one, normal or subnormal), ties to even. */
float fp4r_round8(float x);
/* MBS-Static macro scale of a 128-element piece: round8(amax / 6). */
float fp4r_mbs_macro_scale(float amax);

/* HiF4's E6M2 block scale (unsigned, 6 exponent bits with bias 31, 2
 * mantissa bits, subnormals, all 256 bytes finite): round to nearest even,
 * saturating at byte 0xFF = 1.75 * 2^32.  r must be >= 0. */
uint8_t fp4r_e6m2_encode(float r);
float fp4r_e6m2_decode(uint8_t b);

/* Overflow-aware MX exponent ([MXFP4] 2.A): the e that places amax / 2^e
 * in (3.5, 7], i.e. the smallest e with amax <= 7 * 2^e, clamped to
 * [-127, 127]; amax == 0 gives -127. */
int fp4r_e8m0_exponent_oas(float amax);

/* Magnitude code k (0..7) of m >= 0 on a grid, RTNE or SR with draw u16. */
int fp4r_round_rtne(float m, int grid);
int fp4r_round_sr(float m, int grid, uint32_t u16);
float fp4r_level(int grid, int k);

/* ---- tensor entry points (host pointers) ------------------------------- */

/* Quantize x (rows x cols, leading dimension ld, BF16 bits or FP32).
 * codes: rows_A * W / 2 bytes, scales: rows_A * W / block bytes, where the
 * logical operand A is x (ROW) or x^T (COL) and W its row length.
 * tensor_scale (NVFP4/UFP4): one float, written (COMPUTE) or read (GIVEN);
 * with OUTER128, rows_A * W / 128 floats written, the outer scale of each
 * 128-element piece of an A-row (W must be a multiple of 128).
 * Returns 0 on success, -1 on invalid arguments. */
int fp4r_quantize(const void* x, int in_dtype, int64_t rows, int64_t cols,
                  int64_t ld, const fp4r_params* p, uint8_t* codes,
                  uint8_t* scales, float* tensor_scale);

/* Dequantize back into x's layout (rows x cols, leading dimension ld_out),
 * optionally undoing the RHT.  out_dtype FP4R_F32 or FP4R_BF16 (RNE). */
int fp4r_dequantize(const uint8_t* codes, const uint8_t* scales,
                    const float* tensor_scale, int64_t rows, int64_t cols,
                    const fp4r_params* p, int inverse_rht, void* out,
                    int out_dtype, int64_t ld_out);

/* Standalone RHT along the axis; y is rows x cols FP32, contiguous. */
int fp4r_rht(const void* x, int in_dtype, int64_t rows, int64_t cols,
             int64_t ld, int axis, uint64_t seed, int inverse, float* y);

/* Quantize one block of already-transformed values y[0..block) with a
 * given scale byte and tensor scale; element (row_a, col_a0 + i) of a
 * logical operand with row length W supplies the SR draw.  codes_out gets
 * one 4-bit code per byte.  Used by the tests' boundary rule. */
void fp4r_quantize_block(const float* y, const fp4r_params* p,
                         uint8_t scale_byte, float tensor_scale,
                         int64_t row_a, int64_t col_a0, int64_t W,
                         uint8_t* codes_out);

/* ---- array forms of the primitives, for the tests' pins ---------------- */
void fp4r_e6m2_encode_n(const float* r, int64_t n, uint8_t* out);
void fp4r_e4m3_encode_n(const float* r, int64_t n, uint8_t* out);
void fp4r_round_n(const float* m, int64_t n, int grid, int rounding,
                  const uint32_t* u16, uint8_t* k_out);
void fp4r_sr_u16_n(uint64_t seed, const uint64_t* idx, int64_t n,
                   uint32_t* out);
/* The binary32 -> BF16 conversion of fp4r_dequantize's BF16 output (round
 * to nearest even; NaN stays NaN), element by element. */
void fp4r_f32_to_bf16_n(const float* in, int64_t n, uint16_t* out);
int fp4r_max_threads(void);

#ifdef __cplusplus
}
#endif
#endif /* FP4_ORACLE_H */
