/*
 * fp4.h -- C ABI of the gfx950 (MI355X) fused RHT + block-scaled 4-bit codec.
 *
 * One shared library, libfp4.so, exports the functions below.  Every tensor
 * argument is a plain device pointer (HIP device memory, e.g. a torch
 * tensor's data_ptr()) and every size is an element count; no C++ or torch
 * type crosses this boundary.  `stream` is a hipStream_t passed as void*
 * (NULL = the default stream).
 *
 * Method (summaries on gist.science; the page title and section are given):
 *  - Block-scaled FP4 with the E2M1 element grid and a random Hadamard
 *    transform (RHT) before quantization: "Replanteamiento del Sesgo de
 *    Contraccion en el Preentrenamiento de LLM en FP4" (es/paper/2606.20381),
 *    "Declaracion del Problema", "Metodologia" 1-2 and "Eficiencia" (RHT and
 *    quantization fused in one pass).
 *  - The uniform E1M2/INT4 grid (UFP4) with RHT on every training GEMM and
 *    stochastic rounding on dY: same page, "Metodologia" 2.
 *  - NVFP4 (16-element groups, 8-bit E4M3 scale), stochastic rounding so
 *    that E[round(x)] = x, 1x16 groups realigned for the transposed weight,
 *    RHT on the backward GEMMs: "TetraJet-v2: Accurate NVFP4 Training for
 *    Large Language Models ..." (it/paper/2510.27527), Riepilogo Tecnico
 *    2.A and 2.C.
 *  - Per-tensor dynamic scaling as part of the NVFP4 recipe: "Le
 *    Architetture Normalizzate sono Nativamente a 4 Bit"
 *    (it/paper/2605.06067), "Enunciato del Problema".
 *  - MXFP4 (32-element blocks, power-of-two E8M0 scale, saturation at the
 *    FP4 limit 6): "Unveiling the Potential of Quantization with MXFP4 ..."
 *    (fr/paper/2603.08713), "2. Methodologie et Analyse" and 2.A; its
 *    overflow-aware scaling (OAS, block amax mapped into (3.5, 7]): same
 *    page, 2.A.
 *  - Double-block scaling (an outer scale per 128 elements, inner 16-element
 *    E4M3 scales, no whole-tensor amax): TetraJet-v2 page, Riepilogo
 *    Tecnico 2.A.
 *  - Macro-block scaling, static variant (a scale with an 8-bit mantissa
 *    per 128 elements over 16-element E8M0 blocks): the MXFP4 page, 2.B.
 *  - E2M1 with its range cut to emulate a uniform grid: the shrinkage-bias
 *    page, Metodologia 2 (Ablacion).
 *
 * Numerics (one output per input; any launch geometry gives the same bytes):
 *  - A is the logical operand: x (FP4_AXIS_ROW) or x^T (FP4_AXIS_COL); W is
 *    the length of A's rows; blocks are B consecutive elements of an A-row.
 *  - RHT: per aligned 16-group of an A-row, y = (1/4) H16 D a, H16 the
 *    Sylvester-ordered Hadamard matrix, D = diag(+-1) from fp4_rht_signs(),
 *    computed in binary32 as butterfly stages h = 1, 2, 4, 8, then * 0.25.
 *  - NVFP4 (G = 6) / UFP4 (G = 7): s_t = amax|y| / (G * 448) (binary32);
 *    per block S = E4M3_RNE_satfinite(amax_b / (s_t * G)), d = s_t * S;
 *    elements v = y * (1/d) rounded to the grid.  S = 0 or d = 0 gives
 *    signed-zero codes.  With FP4_TS_OUTER128, each 128-element piece of an
 *    A-row has its own s_o = amax_piece / (G * 448), used in place of s_t.
 *    E2M1_CAP2 is NVFP4 with G = 2.
 *    MXFP4: d = 2^e, e = floor(log2 amax_b) - 2 clamped to [-127, 127],
 *    scale byte e + 127.  MXFP4_OAS: e is the integer with
 *    3.5 < amax_b / 2^e <= 7, same clamp and byte.  MXFP4_MBS: see its
 *    #define below (macro scale in the outer-scale slot, E8M0 per 16).
 *  - Grids: E2M1 {0, .5, 1, 1.5, 2, 3, 4, 6}; E2M1_CAP2 {0, .5, 1, 1.5, 2};
 *    UFP4 {0, 1, ..., 7}; values past the top level saturate.  RTNE ties
 *    go to the even code.  SR (unbiased: E[round(m)] = m, TetraJet-v2 page,
 *    Riepilogo Tecnico 2.A) rounds m in [L[k], L[k+1]) up iff the draw
 *    U = (u16 + 2^-6) * 2^-16 is at most p = (m - L[k]) / (L[k+1] - L[k]),
 *    i.e. iff p * 2^22 >= 64 * u16 + 1; u16 is half of a Philox4x32-10 word
 *    (Salmon et al., SC'11) with key = sr_seed and counter (g, 0, 0),
 *    g = n / 8, n = row_A * W + col_A; element n % 8 takes half (n % 2) of
 *    word (n % 8) / 2.
 *  - Codes: 4 bits, bit 3 = sign of y, bits 0-2 = level index.
 *
 * Layouts (all row-major, owned and allocated by the caller):
 *  - x: rows x cols, leading dimension ld (elements), BF16 or FP32.
 *  - codes: rows_A x (W / 2) bytes; byte (i, j/2) holds A[i][j], even j in
 *    the low nibble.  rows_A = rows (ROW) or cols (COL); W = cols or rows.
 *  - scales: rows_A x (W / B) bytes (HiF4: 4 bytes per block).
 *  - tensor_scale (two-level formats only): one float; with FP4_TS_OUTER128,
 *    rows_A x (W / 128) floats, row-major (requires W % 128 == 0).
 *
 * Ownership and concurrency: the library allocates no memory and keeps no
 * state between calls; all work is enqueued asynchronously on `stream` and
 * the call never synchronizes (unless FP4_DEBUG_SYNC=1 is set in the
 * environment, which synchronizes and checks after each launch).  Calls on
 * different streams that share an output or a workspace race.
 *
 * Errors: arguments are validated on the host before anything is launched;
 * an invalid call returns a negative fp4_status and enqueues nothing.  A
 * launch failure returns FP4_ERR_DEVICE.  Faults inside a kernel surface at
 * the caller's next synchronization.  Inputs containing NaN or Inf, or whose
 * RHT overflows binary32, are outside the contract.
 */
#ifndef FP4_H
#define FP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t fp4_status;
#define FP4_OK 0
#define FP4_ERR_NULL (-1)      /* a required pointer is NULL */
#define FP4_ERR_FORMAT (-2)    /* bad format / block / axis / rounding / mode */
#define FP4_ERR_SHAPE (-3)     /* negative size, ld < cols, W not divisible */
#define FP4_ERR_ALIGN (-4)     /* pointer or leading dimension misaligned */
#define FP4_ERR_DTYPE (-5)     /* unknown element type */
#define FP4_ERR_WORKSPACE (-6) /* workspace missing or too small */
#define FP4_ERR_DEVICE (-7)    /* HIP launch failed */

#define FP4_NVFP4 0     /* E2M1, 16-element blocks, E4M3 scale, FP32 tensor scale */
#define FP4_MXFP4 1     /* E2M1, 32-element blocks, E8M0 scale */
#define FP4_UFP4 2      /* uniform 0..7 grid, 16-element blocks, E4M3 + FP32 */
#define FP4_MXFP4_OAS 3 /* MXFP4 with overflow-aware E8M0 scales */
/* E2M1 with its range cut at 2 ("Replanteamiento del Sesgo de Contraccion
 * en el Preentrenamiento de LLM en FP4", Metodologia 2, Ablacion: limiting
 * E2M1's maximum to emulate a uniform grid): codes 0..4 only (levels 0, .5,
 * 1, 1.5, 2, equally spaced), values past 2 saturate at 2; NVFP4's
 * 16-element blocks, E4M3 scale and FP32 tensor (or outer) scale, with the
 * block amax mapped to 2 (s_t = amax / (2 * 448)).  Dequantizes as NVFP4. */
#define FP4_E2M1_CAP2 4
/* MXFP4 with static macro-block scaling ("Unveiling the Potential of
 * Quantization with MXFP4", 2.B MBS-Static): for each 128-element piece of
 * a row of A, a macro scale M = amax / 6 rounded to 8 fraction bits (FP32,
 * stored where the double block stores its outer scales); for each
 * 16-element block an E8M0 byte e_b + 127 with e_b = floor(log2(amax_b /
 * M)) - 2 clamped to [-127, 127] (-127 when M or amax_b is 0), d_b = M *
 * 2^e_b (binary32); E2M1 elements, saturating at 6.  Requires ts_mode =
 * FP4_TS_OUTER128 and block 16. */
#define FP4_MXFP4_MBS 5
/* MXFP4 with overflow-aware scales on 16-element blocks: the granularity at
 * which the MXFP4 page applies its techniques ("Unveiling the Potential of
 * Quantization with MXFP4", 2. Methodologie et Analyse; OAS in 2.A): an
 * E8M0 byte per 16 elements with 3.5 < amax_b / 2^e <= 7, E2M1 elements
 * saturating at 6, no tensor scale.  Block 16. */
#define FP4_MXFP4_OAS16 6
/* HiF4 ("Unleashing Low-Bit Inference on Ascend NPUs: A Comprehensive
 * Evaluation of HiFloat Formats", 2. Metodologia: an E6M2 scale per 64
 * elements, E1M0 scales per 8 and per 4 elements, E1M2 elements).  The page
 * gives no selection or rounding rule; reading: element magnitudes k/4
 * (k = 0..7, the E1M2 values with bias 1); S = E6M2 (unsigned, bias 31,
 * subnormal step 2^-32, saturating at 1.75 * 2^32) of amax_64 / 1.75,
 * rounded to nearest even; an 8-element sub-block takes factor 1/2 iff its
 * maximum <= 0.875 * S, else 1; a 4-element micro-block takes 1/2 iff its
 * maximum <= 0.875 * S * (its sub-block's factor), else 1; step d = S *
 * f8 * f4 / 4; codes k = the uniform-grid rounding (RTNE or SR, saturating
 * at 7) of |y| * (1/d), sign in bit 3.  No tensor scale.  Block 64 (W %
 * 64 == 0).  Scales: 4 bytes per block, rows_A x (W / 16) bytes: byte 0 =
 * S, byte 1 = the 8 sub-block bits, bytes 2-3 = the 16 micro-block bits
 * (bit i for the i-th piece of the block, little-endian; set: factor 1). */
#define FP4_HIF4 7

#define FP4_AXIS_ROW 0 /* quantize along rows of x */
#define FP4_AXIS_COL 1 /* quantize along columns of x (output is x^T-major) */

#define FP4_RTNE 0 /* round to nearest, ties to even code */
#define FP4_SR 1   /* stochastic rounding with Philox draws */

#define FP4_BF16 0
#define FP4_F32 1

#define FP4_TS_COMPUTE 0  /* tensor scale computed from the data, written out */
#define FP4_TS_GIVEN 1    /* tensor scale read from *tensor_scale */
#define FP4_TS_OUTER128 2 /* double block (MBS: macro scale): one FP32 per 128 elements */

typedef struct {
  int32_t format;   /* FP4_NVFP4 / _MXFP4 / _UFP4 / _MXFP4_OAS / _E2M1_CAP2 / _MXFP4_MBS /
                       _MXFP4_OAS16 / _HIF4 */
  int32_t block;    /* 16 for NVFP4, UFP4, E2M1_CAP2, MXFP4_MBS, MXFP4_OAS16; 32 for MXFP4,
                       MXFP4_OAS; 64 for HIF4 */
  int32_t axis;     /* FP4_AXIS_ROW / FP4_AXIS_COL */
  int32_t rounding; /* FP4_RTNE / FP4_SR (elements only; scales are RTNE) */
  int32_t rht;      /* 0 = off, 1 = 16-point RHT before quantization */
  int32_t ts_mode;  /* FP4_TS_COMPUTE / _GIVEN / _OUTER128 (ignored for MXFP4, MXFP4_OAS,
                       MXFP4_OAS16 and HIF4;
                       MXFP4_MBS requires _OUTER128) */
  uint64_t rht_seed;
  uint64_t sr_seed;
} fp4_params;

/* Bytes of device workspace fp4_quantize needs for this call (0 when none:
 * the MX formats, a given tensor scale, outer scales).  Contents need no
 * initialization.  A computed tensor scale takes the tensor maximum of the
 * (rotated) operand before any block is coded.  On the row axis, with W a
 * multiple of 32 and an operand that fits the registers of one
 * resident grid (about 16M elements with the RHT on MI355X), one kernel
 * reads x once: its workgroups exchange partial maxima through 16-byte
 * records in the workspace, tagged per call so that earlier contents are
 * never taken for this call's.  A larger BF16 row operand whose rows are
 * back to back (ld == cols), up to about 84M elements with the RHT, also
 * takes one kernel with the same exchange: it holds part of x in
 * registers and LDS and reads only the rest a second time.  Otherwise, when
 * ws_bytes is below the returned size but at least 4096 (1024 floats), or
 * when the stream is being captured into a HIP graph (a replayed launch
 * would carry the tag it was captured with), a tensor-maximum pass precedes
 * the quantize pass.  All give the same bytes.  A workgroup that waits
 * longer than FP4_AMAX_WAIT_US microseconds (environment; by default 10 plus
 * the time to read x at 2.5 TB/s) for the others computes what it misses
 * from x itself, so a call whose workgroups are not all resident at once
 * still finishes. */
size_t fp4_workspace_bytes(int64_t rows, int64_t cols, const fp4_params* p);

/* Quantize x (rows x cols, leading dimension ld, in_dtype) into codes and
 * scales (layouts above).  tensor_scale is written (COMPUTE, OUTER128) or
 * read (GIVEN) for the two-level formats (NVFP4, UFP4, E2M1_CAP2; MXFP4_MBS
 * writes its macro scales there, as OUTER128) and may be NULL for the MX
 * formats and HiF4.
 * workspace holds ws_bytes bytes: at least 4096 for a computed tensor scale,
 * fp4_workspace_bytes() for the single-pass kernel.  Requirements: block
 * matches the format; W divisible by the block (and by 16 when rht, by 128
 * with OUTER128); ld >= cols; x, codes, scales 16-byte aligned; ld *
 * element size a multiple of 16 bytes.  rows == 0 or cols == 0 is valid
 * (COMPUTE writes s_t = 0). */
fp4_status fp4_quantize(const void* x, int32_t in_dtype, int64_t rows, int64_t cols,
                        int64_t ld, const fp4_params* p, uint8_t* codes, uint8_t* scales,
                        float* tensor_scale, void* workspace, size_t ws_bytes,
                        void* stream);

/* Host-side query, no launch: the bytes of x that fp4_quantize with these
 * arguments reads on the current device, outside graph capture, stored in
 * *bytes.  A computed tensor scale needs the maximum of the whole operand
 * before any block is coded (per-tensor scaling: "Le Architetture
 * Normalizzate ...", "Enunciato del Problema"): the single pass reads x
 * once (rows * cols elements), the wide single pass
 * reads the units it does not hold twice, and the two-pass path (a
 * tensor-maximum pass, then the quantize pass) reads x twice.  Every other
 * mode reads x once.  Same argument checks as fp4_quantize apart from the
 * pointers; FP4_ERR_NULL if bytes is NULL, FP4_ERR_WORKSPACE if a computed
 * tensor scale's ws_bytes is below 4096.  Without a device (or when the
 * occupancy query fails) it reports the two-pass path, which fp4_quantize
 * then takes too. */
fp4_status fp4_quantize_input_bytes(int32_t in_dtype, int64_t rows, int64_t cols, int64_t ld,
                                    const fp4_params* p, size_t ws_bytes, int64_t* bytes);

/* Allocation-free fp4_quantize, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, checks and results as fp4_quantize
 * without the workspace: the computed tensor scale's records (single-pass
 * exchange, or two-pass partial maxima) go to a fixed array of
 * FP4_NOALLOC_SCRATCH_BYTES bytes in the library's device memory, one per
 * device, held until the process ends; its address is looked up on the
 * first call on each device.  The call allocates nothing (no hipMalloc or
 * allocating library routine).  The array needs no clearing between calls:
 * single-pass records carry a per-call tag and the two-pass partial maxima
 * are all rewritten by each call.  Every call on one device shares the
 * array, so calls that overlap in time on one device (different streams,
 * or different host threads) race and may produce wrong tensor scales:
 * serialize them.  Returns FP4_ERR_WORKSPACE if a call would need more than
 * the array (none does: the exchange takes fp4_workspace_bytes(), at most
 * 16400 bytes) and FP4_ERR_DEVICE if the array's address cannot be found. */
#define FP4_NOALLOC_SCRATCH_BYTES 16640
fp4_status fp4_quantize_noalloc(const void* x, int32_t in_dtype, int64_t rows, int64_t cols,
                                int64_t ld, const fp4_params* p, uint8_t* codes,
                                uint8_t* scales, float* tensor_scale, void* stream);

/* Bytes of device workspace fp4_quantize_dual needs (0 when none). */
size_t fp4_workspace_bytes_dual(int64_t rows, int64_t cols, const fp4_params* p);

/* Both quantizations of x in one call: the row axis (codes_row, scales_row,
 * ts_row, as fp4_quantize with p->axis = FP4_AXIS_ROW) and the column axis
 * (codes_col, scales_col, ts_col, as with FP4_AXIS_COL); p->axis is
 * ignored.  The outputs are byte for byte those of the two single calls.
 * The forward and the weight-gradient GEMM both need an operand this way
 * (TetraJet-v2 page, Riepilogo Tecnico 2.A: the 1x16 groups realigned for
 * the transposed matrix; the [UFP4] page, Metodologia 2: quantized
 * operands of all three GEMMs).  With BF16 input, a two-level format
 * (NVFP4, uniform grid, cut E2M1), rows and cols multiples of 128 and 256 * ld < 2^31 (a
 * 128-row tile's byte extent), x is read once per pass
 * (once in all with a given tensor scale or outer scales, twice with
 * computed tensor scales instead of four times); otherwise the call runs
 * the two single-axis quantizations in turn.  ts_row / ts_col follow the
 * tensor_scale rules of fp4_quantize for their axis; workspace must hold
 * fp4_workspace_bytes_dual() bytes.  Same alignment rules and errors as
 * fp4_quantize, checked for both axes. */
fp4_status fp4_quantize_dual(const void* x, int32_t in_dtype, int64_t rows, int64_t cols,
                             int64_t ld, const fp4_params* p, uint8_t* codes_row,
                             uint8_t* scales_row, float* ts_row, uint8_t* codes_col,
                             uint8_t* scales_col, float* ts_col, void* workspace,
                             size_t ws_bytes, void* stream);

/* Rebuild x from codes, scales and tensor_scale (as produced by
 * fp4_quantize with the same rows, cols and params, including ts_mode for
 * the outer-scale layout) into out, in x's
 * layout (rows x cols, leading dimension ld_out), FP32 or BF16 (RNE).
 * inverse_rht = 1 undoes the RHT (requires p->rht).  Each value is
 * sign * L[k] * d, one binary32 product per element. */
fp4_status fp4_dequantize(const uint8_t* codes, const uint8_t* scales,
                          const float* tensor_scale, int64_t rows, int64_t cols,
                          const fp4_params* p, int32_t inverse_rht, void* out,
                          int32_t out_dtype, int64_t ld_out, void* stream);

/* Standalone RHT (inverse = 0) or its inverse (inverse = 1) along `axis`,
 * per aligned 16-group; y is rows x cols FP32, dense (leading dimension
 * cols), in x's layout. */
fp4_status fp4_rht(const void* x, int32_t in_dtype, int64_t rows, int64_t cols, int64_t ld,
                   int32_t axis, uint64_t rht_seed, int32_t inverse, float* y, void* stream);

/* C = A * B^T for MXFP4 (or MXFP4-OAS) operands quantized along K: A is
 * M x K, B is N x K, each as fp4_quantize writes it with axis FP4_AXIS_ROW
 * (codes [rows][K/2], element 2j in the low nibble of byte j; E8M0 scales
 * [rows][K/32]).  The GEMM consumer of the quantized operands, for the
 * single-GEMM output quality the [UFP4] page measures per path
 * ("Diagnosticos de Cuantizacion y GEMM") and the quantize overhead
 * relative to the GEMM the [MXFP4] page reports ("4. Resultats
 * Experimentaux").  An RHT applied to both operands along K cancels in the
 * product (the 16-point transform is orthogonal).  Each product of two
 * codes is exact; accumulation is in binary32 inside gfx950's scaled
 * matrix instruction (v_mfma_scale_f32_32x32x64_f8f6f4), in its order, so
 * results match an exact reference within a binary32 accumulation bound,
 * not bit for bit.  C is M x N, FP32 or BF16 (round to nearest even), row
 * leading dimension ldc >= N.  M, N and K must be multiples of 128, K > 0,
 * and each operand's codes under 4 GiB (M * K / 2 and N * K / 2 bytes),
 * else FP4_ERR_SHAPE; codes and C 16-byte aligned, scales 4-byte
 * aligned (else FP4_ERR_ALIGN).  No workspace; nothing allocated. */
fp4_status fp4_gemm_mx(const uint8_t* a_codes, const uint8_t* a_scales,
                       const uint8_t* b_codes, const uint8_t* b_scales, int64_t M, int64_t N,
                       int64_t K, void* c, int32_t c_dtype, int64_t ldc, void* stream);

/* The RHT sign mask of a seed (host function): low 16 bits of word 0 of
 * Philox4x32-10(key = seed, counter = (0, 0, 1, 0)); bit j set: d_j = -1. */
uint16_t fp4_rht_signs(uint64_t rht_seed);

/* Static description of a status code. */
const char* fp4_status_str(fp4_status s);

#ifdef __cplusplus
}
#endif
#endif /* FP4_H */
