// fp4_quantize.h -- gfx950 kernels of the quantize path and their launcher,
// instantiated per format by fp4_quantize_<format>.hip (parallel builds).
//
// Terms: x is the caller's rows x cols tensor (row-major, leading dimension
// ld).  The logical operand A is x (row axis) or x^T (column axis); W is the
// length of A's rows, B the block size (16 or 32).  Codes are A-row-major,
// two per byte (even column in the low nibble); scales are one byte per
// block, A-row-major.  SR draws are keyed on the logical A coordinate, so
// every tiling gives the same bytes.
//
// Two-level formats (NVFP4, uniform grid) need the tensor amax of the
// rotated operand before any block can be coded: a first kernel writes one
// partial maximum per workgroup, and every workgroup of the quantize kernel
// reduces them.  The MX formats, a given tensor scale and outer scales (one
// per 128-piece of an A-row, reduced across the lanes that hold the piece)
// skip that pass.
//
// Row axis: a lane owns a 32-element (or 16-element) piece of an A-row,
// read with 16-byte loads; the next piece's loads are issued before the
// current piece is coded.  Column axis: a lane owns C adjacent columns of x
// (A-rows) and a run of NB consecutive blocks down them; each row of a
// block is one 2C- or 4C-byte load, so a wave reads one contiguous segment
// per row, and each lane writes NB*B/2 contiguous code bytes per column.
#pragma once

#include <mutex>
#include <type_traits>
#include <unordered_map>

#include "fp4_device.h"
#include "fp4_launch.h"
#include "fp4_tiles.h"

#ifndef FP4_UNIFORM_PACK
#define FP4_UNIFORM_PACK 1
#endif

using namespace fp4dev;

namespace {

// ------------------------------------------------------------ tensor amax
// Partial maxima of |A| or, with the RHT, of |H16 D a| before the exact
// scaling by 1/4 (monotone, so it is applied once to each partial).
template <bool RHT, typename T>
__global__ __launch_bounds__(kThreads) void amax_row_kernel(
    const T* __restrict__ x, int64_t ld, int64_t n_major, int64_t M, int64_t sq, int64_t sr,
    uint32_t signs, float* __restrict__ partials) {
  Walk w;
  w.init((int64_t)blockIdx.x * kThreads + threadIdx.x, M);
  float m = 0.0f;
  while (w.major < n_major) {
    RowRaw<T, 16> raw;
    raw.load(x + w.major * ld + w.minor * 16);
    float t[16];
    raw.template group<RHT>(0, t, signs);
    if (RHT) {
      m = fmaxf(m, fwht16_absmax(t));
    } else {
#pragma unroll
      for (int j = 0; j < 16; j += 2) m = fmaxf(m, fmaxf(fabsf(t[j]), fabsf(t[j + 1])));
    }
    w.advance(sq, sr, M);
  }
  m = block_max_256(m);
  if (threadIdx.x == 0) partials[blockIdx.x] = RHT ? m * 0.25f : m;
}

// Column axis: units are (16-row group, C-column group), column group fastest.
template <bool RHT, typename T, int C>
__global__ __launch_bounds__(kThreads) void amax_col_kernel(
    const T* __restrict__ x, int64_t ld, int64_t n_major, int64_t M, int64_t sq, int64_t sr,
    uint32_t signs, float* __restrict__ partials) {
  Walk w;
  w.init((int64_t)blockIdx.x * kThreads + threadIdx.x, M);
  float m = 0.0f;
  while (w.major < n_major) {
    ColRaw<T, C> raw;
    raw.load(x + w.major * 16 * ld + w.minor * C, ld);
    if (RHT) raw.flip_rows(signs);
#pragma unroll
    for (int k = 0; k < C; ++k) {
      float t[16];
      raw.column(k, t);
      if (RHT) {
        m = fmaxf(m, fwht16_absmax(t));
      } else {
#pragma unroll
        for (int j = 0; j < 16; j += 2) m = fmaxf(m, fmaxf(fabsf(t[j]), fabsf(t[j + 1])));
      }
    }
    w.advance(sq, sr, M);
  }
  m = block_max_256(m);
  if (threadIdx.x == 0) partials[blockIdx.x] = RHT ? m * 0.25f : m;
}

// ---------------------------------------------------------- quantize core
struct QuantArgs {
  int64_t ld, W;
  int64_t n_major, M, sq, sr;  // unit walk
  int64_t nblk_axis;           // column axis: blocks down the rows (W / B)
  int64_t blk_begin, blk_end;  // column axis: row-block range of this launch
  int64_t col_begin;           // column axis: first column of this launch
  uint8_t* codes;
  uint8_t* scales;
  const float* ts_in;      // given tensor scale (kTsGiven)
  float* ts_out;           // computed tensor scale, or outer scales (kTsOuter)
  const float* partials;   // amax partials (kTsCompute)
  int npartials;
  uint32_t signs;
  uint32_t sr_k0, sr_k1;
};

// Per-workgroup constants of the two-level scale: s_t, den = s_t * G, and
// rden, den's binary32 reciprocal for the block-scale selection (0: not
// set, or den's reciprocal not a normal number; the quotient is then
// always divided out).  Outer scales (one per 128-piece) leave rden unused.
struct ScaleCtx {
  float s_t, den, rden;
};

__device__ __forceinline__ float recip_of_den(float den) {
  return (den >= 0x1p-125f && den <= 0x1p125f) ? 1.0f / den : 0.0f;
}

// Tensor-scale inputs of a workgroup: the amax partial maxima (4 per lane)
// or the given scale.  Fetched before the lane's first data loads: loads
// complete in issue order, so the prologue then waits only for these and
// not for the data behind them.
// Scale of a 128-element outer piece from its amax: the double block's
// amax / (G * 448) ([TJ2] 2.A), or the MBS-Static macro scale.
template <int FMT>
__device__ __forceinline__ float outer_scale(float amax) {
  if constexpr (FMT == kMBS) return mbs_macro_scale(amax);
  else return amax / (grid_max<FMT>() * 448.0f);
}

constexpr int kFetch = kAmaxPartials / kThreads;
static_assert(kAmaxPartials % kThreads == 0, "partials per lane");
struct ScaleFetch {
  float v[kFetch];
};

template <int FMT, int TSM>
__device__ __forceinline__ ScaleFetch scale_fetch(const float* partials, int npartials,
                                                  const float* ts_in) {
  ScaleFetch f;
#pragma unroll
  for (int k = 0; k < kFetch; ++k) f.v[k] = 0.0f;
  if constexpr (has_tensor_scale(FMT) && TSM == kTsCompute) {
#pragma unroll
    for (int k = 0; k < kFetch; ++k) {
      const int i = threadIdx.x + k * kThreads;
      if (i < npartials) f.v[k] = partials[i];
    }
  } else if constexpr (has_tensor_scale(FMT) && TSM == kTsGiven) {
    f.v[0] = ts_in[0];
  }
  return f;
}

// Tensor scale s_t = amax / (G * 448) and, in LDS, the reciprocal of every
// decoded block scale: inv[S] = 1 / (s_t * decode(S)), 0 where that is 0.
// Nothing for the MX formats and for outer scales (per 128-piece, coded
// with the blocks).
template <int FMT, int TSM>
__device__ __forceinline__ ScaleCtx scale_prologue(const ScaleFetch& f, float* ts_out,
                                                   float* inv_tab) {
  ScaleCtx c{0.0f, 0.0f, 0.0f};
  if constexpr (has_tensor_scale(FMT) && TSM != kTsOuter) {
    if (TSM == kTsGiven) {
      c.s_t = f.v[0];
    } else {
      float m = f.v[0];
#pragma unroll
      for (int k = 1; k < kFetch; ++k) m = fmaxf(m, f.v[k]);
      m = block_max_256(m);
      c.s_t = m / (grid_max<FMT>() * 448.0f);
      if (blockIdx.x == 0 && threadIdx.x == 0) ts_out[0] = c.s_t;
    }
    c.den = c.s_t * grid_max<FMT>();
    c.rden = recip_of_den(c.den);
    if (threadIdx.x < 128) {
      const uint32_t S = threadIdx.x < 127 ? threadIdx.x : 126u;
      const float d = S ? c.s_t * e4m3_decode(S) : 0.0f;
      inv_tab[threadIdx.x] = d != 0.0f ? 1.0f / d : 0.0f;
    }
    __syncthreads();
  }
  return c;
}

// Stochastic E2M1 conversion of one pair into byte J of `word`, the other
// bytes kept.  The convert writes only the byte its selector names; the
// compiler's builtin does not carry the other bytes of its first operand
// through to the result, so the instruction is written out with `word` as
// an input-output operand (byte 0, converted first, starts the word: its
// other bytes are written by the next three).  Pair order (odd element,
// even element); scale operand 1.0 (no rescaling).  Wait states, which the
// compiler does not add around inline assembly: one before each convert,
// which reads the word (or the draw register it may share) the previous
// instruction may have just written (the compiler puts one between two such
// converts of its own), and two after the last one, before other
// instructions read the word.
typedef float f32x2 __attribute__((ext_vector_type(2)));
template <int J>
__device__ __forceinline__ void cvt_sr_pk_fp4_byte(uint32_t& word, f32x2 p, uint32_t rnd) {
  if constexpr (J == 0)
    asm("s_nop 0\n\tv_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0" : "=v"(word) : "v"(p), "v"(rnd));
  else if constexpr (J == 1)
    asm("s_nop 0\n\tv_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 op_sel:[0,0,1,0]"
        : "+v"(word) : "v"(p), "v"(rnd));
  else if constexpr (J == 2)
    asm("s_nop 0\n\tv_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 op_sel:[0,0,0,1]"
        : "+v"(word) : "v"(p), "v"(rnd));
  else
    asm("s_nop 0\n\tv_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 op_sel:[0,0,1,1]\n\ts_nop 1"
        : "+v"(word) : "v"(p), "v"(rnd));
}

// Elements 2J and 2J + 1 of a group of 8, stochastically rounded in
// hardware with the draws of Philox word w (element 2J its low half, 2J + 1
// its high half), into byte J of `odd` and of `even`.  Both converts take
// the pair (odd element first); the first uses the odd element's draw and
// keeps its code in the low nibble of its byte, the second the even
// element's draw and keeps its code in the high nibble; the caller swaps
// the nibbles into place.
template <int J>
__device__ __forceinline__ void sr_pair_e2m1(float ve, float vo, uint32_t w, uint32_t& odd,
                                             uint32_t& even) {
  // first slot, bits 31..10: ~(high half) then six ones = ~w | 0xFFFF
  // (three-input op, truth table 0xCF = ~a | b)
  const uint32_t r0 = __builtin_amdgcn_bitop3_b32(w, 0xFFFFu, 0u, 0xCF);
  // second slot, bits 30..9: ~(low half) then six ones = ~(w << 15)
  // = w * -2^15 - 1 in 24-bit signed multiply-add (only w's low 17 bits
  // reach bits 31..15), one instruction where the compiler would emit a
  // shift and a not
  uint32_t r1;
  asm("v_mad_i32_i24 %0, %1, %2, -1" : "=v"(r1) : "v"(w), "s"(-32768));
  f32x2 p;
  p.x = vo;
  p.y = ve;
  cvt_sr_pk_fp4_byte<J>(odd, p, r0);
  cvt_sr_pk_fp4_byte<J>(even, p, r1);
}

// Encode 8 scaled values (all finite) into one word of 4-bit codes.
template <int FMT, bool SR>
__device__ __forceinline__ uint32_t encode8_fast(const float* v_in, const uint32_t (&r)[4]) {
  uint32_t word = 0;
  // The cut E2M1 saturates at 2: clamp first (sign, and the sign of zero,
  // kept), then the E2M1 converts below see no value past their level 2
  // except 2 itself.  Other formats code the values as they are.
  float vc[8];
  const float* v = v_in;
  if constexpr (FMT == kCAP2) {
#pragma unroll
    for (int l = 0; l < 8; ++l) vc[l] = fminf(fmaxf(v_in[l], -2.0f), 2.0f);
    v = vc;
  }
  if constexpr (FMT == kUFP4 && !SR && FP4_UNIFORM_PACK) {
    // Uniform grid, round to nearest even: k = rint(min(|v|, 7)), an exact
    // integer 0..7, written into a byte by the float -> u8 pack convert
    // (exact for integers): element 2j into byte j of lo, element 2j + 1
    // into byte j of hi, so that lo | hi << 4 holds element l in nibble l.
    // Signs: byte selectors 9 and 11 of the byte permute give 0xFF where bit
    // 31 of its second or first source is set; the even elements' sign
    // bytes masked to bit 3 of each byte, the odd ones' to bit 7.
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo = __builtin_amdgcn_cvt_pk_u8_f32(rintf(fminf(fabsf(v[2 * j]), 7.0f)), j, lo);
      hi = __builtin_amdgcn_cvt_pk_u8_f32(rintf(fminf(fabsf(v[2 * j + 1]), 7.0f)), j, hi);
    }
    const uint32_t b[8] = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                           __float_as_uint(v[3]), __float_as_uint(v[4]), __float_as_uint(v[5]),
                           __float_as_uint(v[6]), __float_as_uint(v[7])};
    // bytes 0, 1 = signs of (b[p], b[p + 2]); bytes 2, 3 = signs of (b[p + 4], b[p + 6])
    const uint32_t se0 = __builtin_amdgcn_perm(b[2], b[0], 0x0C0C0B09u);
    const uint32_t se1 = __builtin_amdgcn_perm(b[6], b[4], 0x0B090C0Cu);
    const uint32_t so0 = __builtin_amdgcn_perm(b[3], b[1], 0x0C0C0B09u);
    const uint32_t so1 = __builtin_amdgcn_perm(b[7], b[5], 0x0B090C0Cu);
    word = (lo | (hi << 4)) | ((se0 | se1) & 0x08080808u) | ((so0 | so1) & 0x80808080u);
  } else if constexpr (FMT == kUFP4 && !SR) {
    // Uniform grid, round to nearest even: adding 2^23 to min(m, 7) rounds
    // it to an integer (binary32 addition, ties to even) held in the low
    // mantissa bits; the sign bit of v becomes bit 3.
#pragma unroll
    for (int l = 0; l < 8; ++l) {
      const float m = fminf(fabsf(v[l]), 7.0f);
      const uint32_t k = __float_as_uint(m + 8388608.0f) & 7u;
      word |= (k | ((__float_as_uint(v[l]) >> 28) & 8u)) << (4 * l);
    }
  } else if constexpr (FMT != kUFP4 && !SR) {
    // E2M1 round-to-nearest-even in hardware: two values per instruction,
    // sign and saturation included; scale operand 1.0 (no rescaling).
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, v[0], v[1], 1.0f, 0);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, v[2], v[3], 1.0f, 1);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, v[4], v[5], 1.0f, 2);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, v[6], v[7], 1.0f, 3);
  } else if constexpr (FMT != kUFP4) {
    // E2M1 stochastic rounding in hardware.  The SR convert adds 22 random
    // fraction bits to the value's position p between its two levels and
    // keeps the carry: up iff p * 2^22 + r >= 2^22, with r = bits 31..10 of
    // its random word for the first element of the pair and bits 30..9 for
    // the second.  r = (~u16 << 6) | 0b111111 makes that p * 2^22 >=
    // 64 * u16 + 1, the rounding rule.  The two elements of a byte need
    // independent draws, so each pair is converted twice, once with each
    // element's draw, and each element's nibble is taken from its convert.
    // The pair enters odd element first: each slot then takes its draw from
    // w in one instruction (above), and the nibbles swap back in the merge.
    uint32_t wo, we;  // odd codes in low nibbles, even codes in high nibbles
    sr_pair_e2m1<0>(v[0], v[1], r[0], wo, we);
    sr_pair_e2m1<1>(v[2], v[3], r[1], wo, we);
    sr_pair_e2m1<2>(v[4], v[5], r[2], wo, we);
    sr_pair_e2m1<3>(v[6], v[7], r[3], wo, we);
    word = ((we >> 4) & 0x0F0F0F0Fu) | ((wo << 4) & 0xF0F0F0F0u);
  } else {
#pragma unroll
    for (int l = 0; l < 8; ++l) {
      const float m = fabsf(v[l]);
      uint32_t k;
      if constexpr (SR) k = round_sr_sw<FMT>(m, (r[l >> 1] >> (16 * (l & 1))) & 0xFFFFu);
      else k = round_rtne_sw<FMT>(m);
      word |= (((__float_as_uint(v[l]) >> 28) & 8u) | k) << (4 * l);
    }
  }
  return word;
}

// Per-element path for blocks whose reciprocal scale, or its product with
// the block amax, is not finite: zero elements code as signed zeros and the
// rest follow v = y * inv exactly as in the scalar definition.
template <int FMT, bool SR>
__device__ __forceinline__ uint32_t encode8_careful(const float* y, float inv,
                                                    const uint32_t (&r)[4]) {
  uint32_t word = 0;
#pragma unroll
  for (int l = 0; l < 8; ++l) {
    const float yi = y[l];
    uint32_t k = 0;
    if (yi != 0.0f) {
      const float m = fabsf(yi * inv);
      if constexpr (SR) k = round_sr_sw<FMT>(m, (r[l >> 1] >> (16 * (l & 1))) & 0xFFFFu);
      else k = round_rtne_sw<FMT>(m);
    }
    word |= (((__float_as_uint(yi) >> 28) & 8u) | k) << (4 * l);
  }
  return word;
}

// One HiF4 block of 64 ([HIF] 2. Metodologia: an E6M2 scale per 64
// elements, E1M0 scales per 8 and per 4, E1M2 elements).  Reading: the
// block maximum maps to the top element level 7/4, S = E6M2(amax / 1.75);
// a sub-block (micro-block) halves its scale when its maximum still fits
// under the top level after halving: factor 1/2 iff max <= 0.875 * S
// (times the sub-block's factor); codes k of |y| / d on the uniform grid
// 0..7 with d = S * f8 * f4 / 4.  Scale word: byte 0 = S, bits 8..15 the
// sub-block factors, bits 16..31 the micro-block factors (bit set: factor
// 1; clear: 1/2).  1/d = (1/S) * 4 / (f8 * f4): the binary32 reciprocal
// scaled by a power of two, exact (nothing leaves the normal range), so one
// division serves the sixteen micro-blocks.  The maxima compare in the y
// domain (t / 4 with the RHT, exact).
// NS sub-blocks (8 elements each) of a HiF4 block, the block's largest
// magnitude (before the 1/4 with the RHT) given: the whole block (NS = 8)
// or one half (NS = 4, sub-blocks s0 .. s0 + 3, when two lanes share a
// block).  Writes the lane's code words and its part of the scale word:
// byte 0 and the bits of its own sub-blocks and micro-blocks.
template <int NS, bool SR, bool RHT, bool BF16IN, bool PRE>
__device__ __forceinline__ void encode_hif4_part(const float* t, float amax_t, int s0,
                                                 uint32_t k0, uint32_t k1, uint64_t n0,
                                                 uint32_t* packed, uint32_t& sword,
                                                 const uint32_t* pre) {
  constexpr bool kFold = RHT && BF16IN;
  const float amax = RHT ? amax_t * 0.25f : amax_t;
  const uint32_t S = e6m2_encode(amax / 1.75f);
  const float D = e6m2_decode(S);
  const float thr = 0.875f * D;
  const float invD = D != 0.0f ? 1.0f / D : 0.0f;
  uint32_t word = S;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    float a4[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const float* tp = t + 8 * s + 4 * m;
      const float mx = fmaxf(fmaxf(fabsf(tp[0]), fabsf(tp[1])), fmaxf(fabsf(tp[2]), fabsf(tp[3])));
      a4[m] = RHT ? mx * 0.25f : mx;
    }
    const bool keep8 = !(fmaxf(a4[0], a4[1]) <= thr);
    word |= (uint32_t)keep8 << (8 + s0 + s);
    const float thr4 = keep8 ? thr : thr * 0.5f;
    float v[8];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const bool keep4 = !(a4[m] <= thr4);
      word |= (uint32_t)keep4 << (16 + 2 * (s0 + s) + m);
      const float inv = invD * (keep8 ? 4.0f : 8.0f) * (keep4 ? 1.0f : 2.0f);
#pragma unroll
      for (int l = 0; l < 4; ++l) {
        const float tv = t[8 * s + 4 * m + l];
        v[4 * m + l] = kFold ? tv * (inv * 0.25f) : (RHT ? tv * 0.25f : tv) * inv;
      }
    }
    uint32_t r[4] = {0u, 0u, 0u, 0u};
    if constexpr (SR && PRE) {
      r[0] = pre[4 * s]; r[1] = pre[4 * s + 1]; r[2] = pre[4 * s + 2]; r[3] = pre[4 * s + 3];
    } else if constexpr (SR) {
      const uint64_t g = (n0 >> 3) + (uint64_t)s;
      const u32x4 o = philox4x32_10(k0, k1, (uint32_t)g, (uint32_t)(g >> 32), 0u, 0u);
      r[0] = o.x; r[1] = o.y; r[2] = o.z; r[3] = o.w;
    }
    packed[s] = encode8_fast<kUFP4, SR>(v, r);
  }
  sword = word;
}

// One HiF4 block of 64 ([HIF] 2. Metodologia: an E6M2 scale per 64
// elements, E1M0 scales per 8 and per 4, E1M2 elements).  Reading: the
// block maximum maps to the top element level 7/4, S = E6M2(amax / 1.75);
// a sub-block (micro-block) halves its scale when its maximum still fits
// under the top level after halving: factor 1/2 iff max <= 0.875 * S
// (times the sub-block's factor); codes k of |y| / d on the uniform grid
// 0..7 with d = S * f8 * f4 / 4.  Scale word: byte 0 = S, bits 8..15 the
// sub-block factors, bits 16..31 the micro-block factors (bit set: factor
// 1; clear: 1/2).  1/d = (1/S) * 4 / (f8 * f4): the binary32 reciprocal
// scaled by a power of two, exact (nothing leaves the normal range), so one
// division serves the sixteen micro-blocks.  The maxima compare in the y
// domain (t / 4 with the RHT, exact).
template <bool SR, bool RHT, bool BF16IN, bool PRE>
__device__ __forceinline__ void encode_hif4(const float (&t)[64], float amax_t, uint32_t k0,
                                            uint32_t k1, uint64_t n0, uint32_t (&packed)[8],
                                            uint32_t& sword, const uint32_t* pre) {
  encode_hif4_part<8, SR, RHT, BF16IN, PRE>(t, amax_t, 0, k0, k1, n0, packed, sword, pre);
}

// Code one block.  t[] holds the rotated values before the 1/4 (RHT) or the
// plain values, amax_t their largest magnitude, n0 the logical index of the
// first element (SR draws).
// Two-level formats ([TJ2] 2.A; [NGPT] per-tensor dynamic scaling):
//   r = amax_b / (s_t * G), S = E4M3(r), d = s_t * decode(S), v = y * (1/d);
// with outer scales ([TJ2] 2.A double block) c holds the 128-piece's scale
// in place of s_t and 1/d is computed here instead of read from the table.
// MXFP4 ([MXFP4] 2): d = 2^e, e = floor(log2 amax_b) - 2; overflow-aware
// ([MXFP4] 2.A): e places amax_b / 2^e in (3.5, 7].
// With BF16 input every RHT partial sum is a multiple of 2^-133, so y = t/4
// is exact and, while inv >= 2^-124, v = t * (inv / 4) equals y * inv.
// SR draws: computed here from (k0, k1, n0), or with PRE taken from pre[],
// the Philox words of the block's B/8 groups, drawn earlier by the caller.
template <int FMT, bool SR, bool RHT, bool BF16IN, int B, int TSM, bool PRE = false>
__device__ __forceinline__ void encode_block(const float (&t)[B], float amax_t, const ScaleCtx& c,
                                             const float* inv_tab, uint32_t k0, uint32_t k1,
                                             uint64_t n0, uint32_t (&packed)[B / 8],
                                             uint32_t& sbyte, const uint32_t* pre = nullptr) {
  if constexpr (FMT == kHIF4) {
    encode_hif4<SR, RHT, BF16IN, PRE>(t, amax_t, k0, k1, n0, packed, sbyte, pre);
    return;
  }
  constexpr bool kFold = RHT && BF16IN;
  const float amax_b = RHT ? amax_t * 0.25f : amax_t;
  float inv;
  if constexpr (is_mx(FMT)) {
    const int e = is_oas(FMT) ? e8m0_exponent_oas(amax_b) : e8m0_exponent(amax_b);
    sbyte = (uint32_t)(e + 127);
    inv = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, exact
  } else if constexpr (FMT == kMBS) {
    // [MXFP4] 2.B static macro-block scaling: the MX exponent rule on
    // amax_b / M (M, the macro scale, in c.s_t), d_b = M * 2^e_b
    const int e = (c.s_t != 0.0f && amax_b != 0.0f) ? e8m0_exponent(amax_b / c.s_t) : -127;
    sbyte = (uint32_t)(e + 127);
    const float d = __builtin_ldexpf(c.s_t, e);
    inv = d != 0.0f ? 1.0f / d : 0.0f;
  } else {
    if constexpr (TSM == kTsOuter)
      sbyte = (c.s_t != 0.0f && amax_b != 0.0f) ? e4m3_encode(amax_b / c.den) : 0u;
    else
      sbyte = (c.s_t != 0.0f && amax_b != 0.0f) ? e4m3_encode_quotient(amax_b, c.den, c.rden)
                                                : 0u;
    if constexpr (TSM == kTsOuter) {
      const float d = sbyte ? c.s_t * e4m3_decode(sbyte) : 0.0f;
      inv = d != 0.0f ? 1.0f / d : 0.0f;
    } else {
      inv = inv_tab[sbyte];
    }
  }
  const float limit = __builtin_inff();
  float mul;
  bool fast;
  if constexpr (kFold) {
    mul = inv * 0.25f;
    fast = inv >= 4.70197740328915e-38f && amax_t * mul < limit;
  } else {
    mul = inv;
    fast = amax_b * inv < limit;
  }
#pragma unroll
  for (int q = 0; q < B / 8; ++q) {
    uint32_t r[4] = {0u, 0u, 0u, 0u};
    if constexpr (SR && PRE) {
      r[0] = pre[4 * q]; r[1] = pre[4 * q + 1]; r[2] = pre[4 * q + 2]; r[3] = pre[4 * q + 3];
    } else if constexpr (SR) {
      const uint64_t g = (n0 >> 3) + (uint64_t)q;
      const u32x4 o = philox4x32_10(k0, k1, (uint32_t)g, (uint32_t)(g >> 32), 0u, 0u);
      r[0] = o.x; r[1] = o.y; r[2] = o.z; r[3] = o.w;
    }
    const float* tq = t + 8 * q;
    if (fast) {
      float v[8];
#pragma unroll
      for (int l = 0; l < 8; ++l) v[l] = ((RHT && !kFold) ? tq[l] * 0.25f : tq[l]) * mul;
      packed[q] = encode8_fast<FMT, SR>(v, r);
    } else {
      float y[8];
#pragma unroll
      for (int l = 0; l < 8; ++l) y[l] = RHT ? tq[l] * 0.25f : tq[l];
      packed[q] = encode8_careful<FMT, SR>(y, inv, r);
    }
  }
}

// ------------------------------------------------------------- row axis
// Store the codes and block scales of one unit of U elements of an A-row
// (SB scale bytes per block: a HiF4 scale word is one 4-byte store).
template <int B, int U, int SB = 1>
__device__ __forceinline__ void store_row_unit(const uint32_t (&packed)[U / 8],
                                               const uint32_t (&sb)[U / B], int64_t row,
                                               int64_t minor, const QuantArgs& a) {
  constexpr int NBU = U / B;
  uint8_t* cp = a.codes + row * (a.W / 2) + minor * (U / 2);
  if constexpr (U >= 32) {
#pragma unroll
    for (int i = 0; i < U / 32; ++i)
      store16<true>(cp + 16 * i, packed[4 * i], packed[4 * i + 1], packed[4 * i + 2],
                    packed[4 * i + 3]);
  } else {
    store8<true>(cp, packed[0], packed[1]);
  }
  uint8_t* sp = a.scales + row * (a.W / B * SB) + minor * NBU * SB;
  if constexpr (SB == 4)
    *reinterpret_cast<uint32_t*>(sp) = sb[0];
  else if constexpr (NBU == 4)
    *reinterpret_cast<uint32_t*>(sp) = sb[0] | (sb[1] << 8) | (sb[2] << 16) | (sb[3] << 24);
  else if constexpr (NBU == 2)
    *reinterpret_cast<uint16_t*>(sp) = (uint16_t)(sb[0] | (sb[1] << 8));
  else
    sp[0] = (uint8_t)sb[0];
}

// Code one unit of an A-row held in `cur` (A-row `row`, unit `minor` of U
// elements within it) and store its codes and block scales.
template <int FMT, bool SR, bool RHT, int TSM, typename T, int U>
__device__ __forceinline__ void code_row_unit(const RowRaw<T, U>& cur, int64_t row, int64_t minor,
                                              const QuantArgs& a, const ScaleCtx& c,
                                              const float* inv_tab) {
  if constexpr (FMT == kHIF4 && U == 32) {
    // two lanes per HiF4 block (units 2i and 2i + 1 of an A-row sit in
    // lanes 2j and 2j + 1): the block maximum and the scale word combine by
    // a lane-pair exchange; the even lane stores the word
    float t[32], am = 0.0f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float g[16];
      cur.template group<RHT>(h, g, a.signs);
      if (RHT) fwht16(g);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        t[16 * h + j] = g[j];
        am = fmaxf(am, fabsf(g[j]));
      }
    }
    am = group_max<2>(am);
    const int half = (int)(minor & 1);
    const uint64_t n0 = (uint64_t)row * (uint64_t)a.W + (uint64_t)(minor * 32);
    uint32_t pk[4], part;
    encode_hif4_part<4, SR, RHT, sizeof(T) == 2, false>(t, am, 4 * half, a.sr_k0, a.sr_k1, n0,
                                                        pk, part, nullptr);
    const uint32_t word = part | swap_lane_pair(part);
    store16<true>(a.codes + row * (a.W / 2) + minor * 16, pk[0], pk[1], pk[2], pk[3]);
    if (!half)
      *reinterpret_cast<uint32_t*>(a.scales + row * (a.W / 16) + (minor >> 1) * 4) = word;
  } else {
    constexpr int B = block_of<FMT>();
    constexpr int NBU = U / B;  // blocks per unit
    uint32_t packed[U / 8];
    uint32_t sb[NBU];
    // widened (and rotated) block bi of the unit, with its largest magnitude
    auto block_values = [&](int bi, float (&t)[B], float& amax_t) {
      amax_t = 0.0f;
#pragma unroll
      for (int h = 0; h < B / 16; ++h) {
        float g[16];
        cur.template group<RHT>(bi * (B / 16) + h, g, a.signs);
        if (RHT) fwht16(g);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          t[16 * h + j] = g[j];
          amax_t = fmaxf(amax_t, fabsf(g[j]));
        }
      }
    };
    auto code = [&](int bi, const float (&t)[B], float amax_t, const ScaleCtx& cc) {
      const uint64_t n0 = (uint64_t)row * (uint64_t)a.W + (uint64_t)(minor * U + bi * B);
      uint32_t pk[B / 8];
      encode_block<FMT, SR, RHT, sizeof(T) == 2, B, TSM>(t, amax_t, cc, inv_tab, a.sr_k0,
                                                         a.sr_k1, n0, pk, sb[bi]);
#pragma unroll
      for (int q = 0; q < B / 8; ++q) packed[bi * (B / 8) + q] = pk[q];
    };
    if constexpr (TSM == kTsOuter) {
      // kOuter / U consecutive lanes hold one 128-piece of an A-row (the
      // walk keeps them in step): their maxima combine by lane exchange.
      constexpr int LPO = kOuter / U;
      float t[NBU][B], am[NBU];
      float ao = 0.0f;
#pragma unroll
      for (int bi = 0; bi < NBU; ++bi) {
        block_values(bi, t[bi], am[bi]);
        ao = fmaxf(ao, am[bi]);
      }
      ao = group_max<LPO>(ao);
      ScaleCtx co;
      co.s_t = outer_scale<FMT>(RHT ? ao * 0.25f : ao);
      co.den = co.s_t * grid_max<FMT>();
      if (minor % LPO == 0) a.ts_out[row * (a.W / kOuter) + minor / LPO] = co.s_t;
#pragma unroll
      for (int bi = 0; bi < NBU; ++bi) code(bi, t[bi], am[bi], co);
    } else {
#pragma unroll
      for (int bi = 0; bi < NBU; ++bi) {
        float t[B], amax_t;
        block_values(bi, t, amax_t);
        code(bi, t, amax_t, c);
      }
    }
    store_row_unit<B, U, scale_bytes<FMT>()>(packed, sb, row, minor, a);
  }
}

// Units: major = A-row, minor = piece of U elements within it.
template <int FMT, bool SR, bool RHT, int TSM, typename T, int U>
__global__ __launch_bounds__(kThreads) void quantize_row_kernel(const T* __restrict__ x,
                                                                QuantArgs a) {
  __shared__ float inv_tab[128];
  Walk w;
  w.init((int64_t)blockIdx.x * kThreads + threadIdx.x, a.M);
  RowRaw<T, U> cur;
  // After a tensor-amax pass the rows are taken last to first: the end of
  // the input, read last by that pass, is then still in the memory-side
  // cache when this pass starts.
  constexpr bool kRev = TSM == kTsCompute && has_tensor_scale(FMT);
  auto row_of = [&](int64_t m) { return kRev ? a.n_major - 1 - m : m; };
  bool have = w.major < a.n_major;
  const ScaleFetch sf = scale_fetch<FMT, TSM>(a.partials, a.npartials, a.ts_in);
  if (have) cur.load(x + row_of(w.major) * a.ld + w.minor * U);  // in flight during the prologue
  const ScaleCtx c = scale_prologue<FMT, TSM>(sf, a.ts_out, inv_tab);
  while (have) {
    Walk nw = w;
    nw.advance(a.sq, a.sr, a.M);
    const bool have_next = nw.major < a.n_major;
    RowRaw<T, U> nxt;
    if (have_next) nxt.load(x + row_of(nw.major) * a.ld + nw.minor * U);
    code_row_unit<FMT, SR, RHT, TSM, T, U>(cur, row_of(w.major), w.minor, a, c, inv_tab);
    cur = nxt;
    w = nw;
    have = have_next;
  }
}


// ------------------------------------------------ row axis, single pass
// Two-level formats with a computed tensor scale, when every unit of the
// operand fits in the registers of one resident grid: each lane loads its
// NU units once (unit u = global lane + k * lanes of the grid), the
// workgroups exchange their partial maxima through the workspace, and the
// lanes then code the units they still hold.  The input is read once, in
// one launch, where the two-pass path reads it twice in two.
//
// Exchange: workgroup b posts its partial maximum in slot b; workgroup 0
// gathers the slots and posts the tensor maximum in the result slot; the
// others wait for it.  A slot is two 64-bit words, each holding one half of
// the call's 64-bit tag above the (masked) maximum, written and read as relaxed
// device-scope atomics: a slot counts as posted when both words carry this
// call's halves and the same maximum, so no fence (and no cache write-back
// or invalidation) is needed, and a slot half-written by a racing read is
// simply not posted yet.  Tags are unique per call, so nothing a slot held
// before (an earlier call's record, or any other bytes, but with chance
// 2^-64) reads as posted, and the workspace needs no clearing.  Every wait
// is bounded in time: a workgroup that has not seen what it waits for
// computes the missing partial maxima from the input itself.  They are the
// same values, so the tensor scale is the same, and the call ends even
// when not all of its workgroups are resident at once.
// Each word's low half is the maximum XOR the other word's tag half, so a
// 64-bit access torn into its dwords cannot pass for a record.  When one word
// reads whole, a slot is accepted only with that word's maximum.  When both
// read as new tag half over an earlier record's value, they decode to two
// maxima that differ unless the halves of (old tag XOR new tag) are equal:
// never for two tags of one process with the same high half, with chance
// 2^-32 otherwise.
struct AmaxSlot {
  uint64_t hi;  // tag bits 63..32 | maximum ^ tag bits 31..0
  uint64_t lo;  // tag bits 31..0  | maximum ^ tag bits 63..32
};
static_assert(sizeof(AmaxSlot) == kAmaxSlotBytes, "slot size");

__device__ __forceinline__ void post_slot(AmaxSlot* s, float v, uint64_t tag) {
  const uint32_t m = __float_as_uint(v), th = (uint32_t)(tag >> 32), tl = (uint32_t)tag;
  __hip_atomic_store(&s->hi, ((uint64_t)th << 32) | (m ^ tl), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(&s->lo, ((uint64_t)tl << 32) | (m ^ th), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// The slot's maximum if both words hold this call's record.
__device__ __forceinline__ bool read_slot(AmaxSlot* s, uint64_t tag, float& v) {
  const uint32_t th = (uint32_t)(tag >> 32), tl = (uint32_t)tag;
  const uint64_t hi = __hip_atomic_load(&s->hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t lo = __hip_atomic_load(&s->lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t m = (uint32_t)hi ^ tl;
  if ((uint32_t)(hi >> 32) != th || (uint32_t)(lo >> 32) != tl || ((uint32_t)lo ^ th) != m)
    return false;
  v = __uint_as_float(m);
  return true;
}

// Largest |H16 D a| (before the 1/4) or |a| of a row unit.
template <bool RHT, typename T, int U>
__device__ __forceinline__ float unit_absmax(const RowRaw<T, U>& r, uint32_t signs) {
  float m = 0.0f;
#pragma unroll
  for (int h = 0; h < U / 16; ++h) {
    float t[16];
    r.template group<RHT>(h, t, signs);
    if (RHT) {
      m = fmaxf(m, fwht16_absmax(t));
    } else {
#pragma unroll
      for (int j = 0; j < 16; j += 2) m = fmaxf(m, fmaxf(fabsf(t[j]), fabsf(t[j + 1])));
    }
  }
  return m;
}

// Partial maximum of workgroup j, recomputed from the input by the whole
// calling workgroup (the value workgroup j posts); nu units per lane.
template <bool RHT, typename T, int U, int NT>
__device__ float partial_of(const T* __restrict__ x, const QuantArgs& a, int64_t j,
                            int64_t stride, int nu) {
  const int64_t units = a.n_major * a.M;
  float m = 0.0f;
#pragma unroll 1
  for (int k = 0; k < nu; ++k) {
    const int64_t u = j * NT + threadIdx.x + k * stride;
    if (u < units) {
      const int64_t row = u / a.M, minor = u - row * a.M;
      RowRaw<T, U> r;
      r.load(x + row * a.ld + minor * U);
      m = fmaxf(m, unit_absmax<RHT, T, U>(r, a.signs));
    }
  }
  m = block_max<NT>(m);
  return RHT ? m * 0.25f : m;
}

// Tensor maximum from the posted slots [0, n), waiting up to wait_ticks of
// the constant-rate clock; slots still missing then are computed here (nu
// units per lane).  Block-uniform control flow (partial_of synchronises the
// workgroup).
template <bool RHT, typename T, int U, int NT>
__device__ float gather_slots(const T* __restrict__ x, const QuantArgs& a, AmaxSlot* slots, int n,
                              uint64_t tag, uint64_t wait_ticks, int64_t stride, int nu) {
  constexpr int kPer = (kAmaxPartials + NT - 1) / NT;
  __shared__ int missing[kAmaxPartials];
  __shared__ int nmissing;
  float m = 0.0f;
  uint32_t pending = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if ((int)threadIdx.x + i * NT < n) pending |= 1u << i;
  const uint64_t t0 = wall_clock64();
  while (true) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      float v;
      if ((pending >> i) & 1u && read_slot(slots + threadIdx.x + i * NT, tag, v)) {
        m = fmaxf(m, v);
        pending &= ~(1u << i);
      }
    }
    if (!__syncthreads_or(pending != 0)) break;
    if (__syncthreads_or(wall_clock64() - t0 >= wait_ticks)) break;
    __builtin_amdgcn_s_sleep(2);
  }
  if (threadIdx.x == 0) nmissing = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if ((pending >> i) & 1u) missing[atomicAdd(&nmissing, 1)] = threadIdx.x + i * NT;
  __syncthreads();
  const int nm = nmissing;
  for (int i = 0; i < nm; ++i)
    m = fmaxf(m, partial_of<RHT, T, U, NT>(x, a, missing[i], stride, nu));
  return block_max<NT>(m);
}

// The exchange: this workgroup's partial maximum m (before the 1/4 with the
// RHT) is posted in its slot; workgroup 0 gathers the slots and posts the
// tensor maximum in the result slot, and the others wait for it.  nu units
// per lane, for the recomputation of partial maxima that never arrive.
//
// Waits: workgroup 0 waits wait_ticks for every slot, then computes the
// missing partial maxima itself and posts the tensor maximum; the other
// workgroups wait up to long_ticks (longer) for that result, so that in the
// normal course only workgroup 0 recomputes anything, and compute what they
// miss themselves only if it never comes (workgroup 0 not resident).
template <bool RHT, typename T, int U, int NT>
__device__ float exchange_amax(const T* __restrict__ x, const QuantArgs& a, AmaxSlot* slots,
                               uint64_t tag, float m, uint64_t wait_ticks, uint64_t long_ticks,
                               int64_t stride, int nu) {
  __shared__ float shared_amax;
  __shared__ int shared_have;
  m = block_max<NT>(m);
  if (threadIdx.x == 0) post_slot(slots + blockIdx.x, RHT ? m * 0.25f : m, tag);
  AmaxSlot* result = slots + kAmaxPartials;
  float amax;
  if (blockIdx.x == 0) {
    amax = gather_slots<RHT, T, U, NT>(x, a, slots, gridDim.x, tag, wait_ticks, stride, nu);
    if (threadIdx.x == 0) post_slot(result, amax, tag);
  } else {
    if (threadIdx.x == 0) {
      const uint64_t t0 = wall_clock64();
      float v = 0.0f;
      bool ok;
      while (!(ok = read_slot(result, tag, v)) && wall_clock64() - t0 < long_ticks)
        __builtin_amdgcn_s_sleep(2);
      shared_amax = v;
      shared_have = ok;
    }
    __syncthreads();
    amax = shared_amax;
    if (!shared_have)  // workgroup 0 never posted: take what is posted, compute the rest
      amax = gather_slots<RHT, T, U, NT>(x, a, slots, gridDim.x, tag, 0, stride, nu);
  }
  return amax;
}

// The two-level scale from the tensor maximum, as in scale_prologue: s_t,
// written once by the grid's first lane, and the reciprocal step table.
template <int FMT>
__device__ __forceinline__ ScaleCtx scale_from_amax(float amax, const QuantArgs& a,
                                                    float* inv_tab) {
  ScaleCtx c;
  c.s_t = amax / (grid_max<FMT>() * 448.0f);
  if (blockIdx.x == 0 && threadIdx.x == 0) a.ts_out[0] = c.s_t;
  c.den = c.s_t * grid_max<FMT>();
  c.rden = recip_of_den(c.den);
  if (threadIdx.x < 128) {
    const uint32_t S = threadIdx.x < 127 ? threadIdx.x : 126u;
    const float d = S ? c.s_t * e4m3_decode(S) : 0.0f;
    inv_tab[threadIdx.x] = d != 0.0f ? 1.0f / d : 0.0f;
  }
  __syncthreads();
  return c;
}

// NT lanes per workgroup, NU units of U elements per lane.  With stochastic
// rounding the Philox words of a lane's units are drawn into LDS (dynamic,
// NT * NU * U / 8 * 16 bytes) right after its loads are issued: that VALU
// work then runs while the loads are in flight instead of after the
// exchange.  Layout [group of 8 elements][lane], 16 bytes per entry, so the
// writes and reads of a wave are contiguous.
// The exchange and its waits: exchange_amax.
template <int FMT, bool SR, bool RHT, typename T, int U, int NU, int NT>
__global__ __launch_bounds__(NT) void quantize_row_single_kernel(
    const T* __restrict__ x, QuantArgs a, AmaxSlot* slots, uint64_t tag, uint64_t wait_ticks,
    uint64_t long_ticks) {
  constexpr int B = block_of<FMT>();
  constexpr int NBU = U / B;
  constexpr int GPU = U / 8;  // Philox groups (8 elements each) per unit
  extern __shared__ uint4 draws[];
  __shared__ float inv_tab[128];
  const int64_t units = a.n_major * a.M;
  const int64_t stride = (int64_t)gridDim.x * NT;
  const int64_t u0 = (int64_t)blockIdx.x * NT + threadIdx.x;
  // Everything that does not depend on the tensor scale is done before the
  // exchange: the units' widened (and rotated) values and their block
  // maxima stay in registers for the coding after it.
  // A lane's units past the last one load a copy of the last unit (its
  // values are in the operand, so the partial maximum is unchanged, and
  // nothing is stored for them): every load is unconditional, so none
  // waits for the one before (a zero fill on the other side of a branch
  // would rewrite the load's registers, and the load would be waited for
  // first).  Rows back to back (ld = W): unit u starts at element 32u, no
  // division.
  RowRaw<T, U> raw[NU];
  const bool dense = a.ld == a.W;
#pragma unroll
  for (int k = 0; k < NU; ++k) {
    const int64_t u = u0 + k * stride;
    const int64_t uc = u < units ? u : units - 1;
    if (dense) {
      raw[k].load(x + uc * U);
    } else {
      const int64_t row = uc / a.M;
      raw[k].load(x + row * a.ld + (uc - row * a.M) * U);
    }
  }
  if constexpr (SR) {
#pragma unroll
    for (int k = 0; k < NU; ++k) {
      const uint64_t g0 = ((uint64_t)(u0 + k * stride) * (uint64_t)U) >> 3;
#pragma unroll
      for (int q = 0; q < GPU; ++q) {
        const uint64_t g = g0 + (uint64_t)q;
        const u32x4 o = philox4x32_10(a.sr_k0, a.sr_k1, (uint32_t)g, (uint32_t)(g >> 32), 0u, 0u);
        draws[(k * GPU + q) * NT + threadIdx.x] = make_uint4(o.x, o.y, o.z, o.w);
      }
    }
  }
  // With the RHT the rotated values are kept (the butterfly is not redone);
  // without it the raw words are kept and widened again for the coding
  // (half the registers for BF16).
  float t[NU][NBU][B];
  float bam[NU][NBU];
#pragma unroll
  for (int k = 0; k < NU; ++k) {
#pragma unroll
    for (int bi = 0; bi < NBU; ++bi) {
      bam[k][bi] = 0.0f;
#pragma unroll
      for (int h = 0; h < B / 16; ++h) {
        float g[16];
        raw[k].template group<RHT>(bi * (B / 16) + h, g, a.signs);
        if (RHT) fwht16(g);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          if (RHT) t[k][bi][16 * h + j] = g[j];
          bam[k][bi] = fmaxf(bam[k][bi], fabsf(g[j]));
        }
      }
    }
  }
  float m = 0.0f;
#pragma unroll
  for (int k = 0; k < NU; ++k)
#pragma unroll
    for (int bi = 0; bi < NBU; ++bi) m = fmaxf(m, bam[k][bi]);
  const float amax = exchange_amax<RHT, T, U, NT>(x, a, slots, tag, m, wait_ticks, long_ticks,
                                                   stride, NU);

  if constexpr (!RHT) {
    // opaque to the compiler, so that it widens the raw words again below
    // instead of keeping the widened values of the first pass alive
#pragma unroll
    for (int k = 0; k < NU; ++k)
#pragma unroll
      for (int i = 0; i < RowRaw<T, U>::kVec; ++i)
        asm volatile("" : "+v"(raw[k].q[i].x), "+v"(raw[k].q[i].y), "+v"(raw[k].q[i].z),
                     "+v"(raw[k].q[i].w));
  }

  const ScaleCtx c = scale_from_amax<FMT>(amax, a, inv_tab);
#pragma unroll
  for (int k = 0; k < NU; ++k) {
    const int64_t u = u0 + k * stride;
    if (u < units) {
      // rows back to back in the outputs: (row 0, piece u) is unit u
      const int64_t row = 0, minor = u;
      uint32_t packed[U / 8];
      uint32_t sb[NBU];
#pragma unroll
      for (int bi = 0; bi < NBU; ++bi) {
        const uint64_t n0 = (uint64_t)row * (uint64_t)a.W + (uint64_t)(minor * U + bi * B);
        uint32_t pre[B / 2];
        if constexpr (SR) {
#pragma unroll
          for (int q = 0; q < B / 8; ++q) {
            const uint4 w = draws[(k * GPU + bi * (B / 8) + q) * NT + threadIdx.x];
            pre[4 * q] = w.x; pre[4 * q + 1] = w.y; pre[4 * q + 2] = w.z; pre[4 * q + 3] = w.w;
          }
        }
        uint32_t pk[B / 8];
        if constexpr (RHT) {
          encode_block<FMT, SR, RHT, sizeof(T) == 2, B, kTsCompute, true>(
              t[k][bi], bam[k][bi], c, inv_tab, a.sr_k0, a.sr_k1, n0, pk, sb[bi], pre);
        } else {
          float tb[B];
#pragma unroll
          for (int h = 0; h < B / 16; ++h) {
            float g[16];
            raw[k].template group<false>(bi * (B / 16) + h, g, 0u);
#pragma unroll
            for (int j = 0; j < 16; ++j) tb[16 * h + j] = g[j];
          }
          encode_block<FMT, SR, RHT, sizeof(T) == 2, B, kTsCompute, true>(
              tb, bam[k][bi], c, inv_tab, a.sr_k0, a.sr_k1, n0, pk, sb[bi], pre);
        }
#pragma unroll
        for (int q = 0; q < B / 8; ++q) packed[bi * (B / 8) + q] = pk[q];
      }
      store_row_unit<B, U>(packed, sb, row, minor, a);
    }
  }
}


// ----------------------------------------- row axis, wide single pass
// Two-level formats with a computed tensor scale, contiguous BF16 operands
// too large for the registers of one resident grid: one workgroup of NT
// lanes per compute unit.  Units of a lane: u0 + k * stride, k = 0 .. nu - 1
// (unit u: elements [32u, 32u + 32) of the operand, rows back to back);
// the first NR stay raw in registers, the next NL raw in LDS, the rest are
// streamed.  Pass 1 reads every unit once and rotates it for the partial
// maximum, keeping the held units; after the exchange the lanes code the
// held units (rotated again from the raw words) and read the streamed ones
// a second time.  Only the streamed share of the input is read twice,
// where the two-pass path reads all of it twice; the second rotation is
// vector work that overlaps the streamed reads and the stores.
// LDS layout [slot][16-byte piece][lane]: the writes and reads of one piece
// by a wave are contiguous.
template <int FMT, bool SR, bool RHT, typename T, int U, int NR, int NL, int NT>
__global__ __launch_bounds__(NT) void quantize_row_wide_kernel(
    const T* __restrict__ x, QuantArgs a, AmaxSlot* slots, uint64_t tag, uint64_t wait_ticks,
    uint64_t long_ticks, int nu) {
  using Raw = RowRaw<T, U>;
  constexpr int KV = Raw::kVec;
  extern __shared__ uint4 held[];
  __shared__ float inv_tab[128];
  const int64_t units = a.n_major * a.M;
  const int64_t stride = (int64_t)gridDim.x * NT;
  const int64_t u0 = (int64_t)blockIdx.x * NT + threadIdx.x;
  auto unit = [&](int k) { return u0 + (int64_t)k * stride; };
  // Past the last unit a lane loads a copy of the last unit: the partial
  // maximum is unchanged and nothing is stored for it.  The loads are
  // unconditional, so none is waited for before the next is issued (a
  // zero fill on the other side of a branch would rewrite the registers of
  // a load in flight and force a wait on it).
  auto load = [&](int k, Raw& r) { r.load(x + (unit(k) < units ? unit(k) : units - 1) * U); };
  auto lds_at = [&](int slot, int i) -> uint4& { return held[(slot * KV + i) * NT + threadIdx.x]; };

  // ---- pass 1: every unit read once.  The held units' loads are issued
  // first; each of the next NR loads is in flight while a held unit is
  // rotated, and the rest stream one at a time.
  Raw raw[NR];
#pragma unroll
  for (int k = 0; k < NR; ++k) load(k, raw[k]);
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const int k = NR + j;
    Raw cur;
    if (k < nu) load(k, cur);
    m = fmaxf(m, unit_absmax<RHT, T, U>(raw[j], a.signs));
    if (k < nu) {
      m = fmaxf(m, unit_absmax<RHT, T, U>(cur, a.signs));
      if (j < NL) {
#pragma unroll
        for (int i = 0; i < KV; ++i) lds_at(j, i) = cur.q[i];
      }
    }
  }
#pragma unroll 1
  for (int k = 2 * NR; k < nu; ++k) {
    Raw cur;
    load(k, cur);
    m = fmaxf(m, unit_absmax<RHT, T, U>(cur, a.signs));
  }

  const float amax = exchange_amax<RHT, T, U, NT>(x, a, slots, tag, m, wait_ticks, long_ticks,
                                                   stride, nu);
  // opaque to the compiler, so that the held words are rotated again below
  // instead of the first rotation being kept alive across the exchange
#pragma unroll
  for (int k = 0; k < NR; ++k)
#pragma unroll
    for (int i = 0; i < KV; ++i)
      asm volatile("" : "+v"(raw[k].q[i].x), "+v"(raw[k].q[i].y), "+v"(raw[k].q[i].z),
                   "+v"(raw[k].q[i].w));
  const ScaleCtx c = scale_from_amax<FMT>(amax, a, inv_tab);

  // ---- pass 2: held units, then the streamed ones read again (the first
  // two streamed loads are issued as soon as registers free up).  With
  // the rows back to back, (row 0, piece u) addresses unit u.
  const int ns = nu - NR - NL;
  auto code = [&](int k, const Raw& r) {
    if (unit(k) < units)
      code_row_unit<FMT, SR, RHT, kTsCompute, T, U>(r, 0, unit(k), a, c, inv_tab);
  };
  Raw sa, sb;
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    code(k, raw[k]);
    if (k == NR - 1 && ns > 0) load(NR + NL, sa);
  }
#pragma unroll
  for (int l = 0; l < NL; ++l) {
    if (NR + l < nu) {
      Raw r;
#pragma unroll
      for (int i = 0; i < KV; ++i) r.q[i] = lds_at(l, i);
      code(NR + l, r);
    }
    if (l == 0 && ns > 1) load(NR + NL + 1, sb);
  }
#pragma unroll 1
  for (int j = 0; j < ns; j += 2) {
    const int k = NR + NL + j;
    code(k, sa);
    if (j + 2 < ns) load(k + 2, sa);
    if (j + 1 < ns) {
      code(k + 1, sb);
      if (j + 3 < ns) load(k + 3, sb);
    }
  }
}


// ---------------------------------------------------------- column axis
// Units: major = run of NB blocks down the rows, minor = group of C columns.
template <int FMT, bool SR, bool RHT, int TSM, typename T, int C, int NB>
__global__ __launch_bounds__(kThreads) void quantize_col_kernel(const T* __restrict__ x,
                                                                QuantArgs a) {
  constexpr int B = block_of<FMT>();
  constexpr int WPB = B / 8;  // code words per block
  __shared__ float inv_tab[128];
  const ScaleCtx c =
      scale_prologue<FMT, TSM>(scale_fetch<FMT, TSM>(a.partials, a.npartials, a.ts_in),
                               a.ts_out, inv_tab);
  const bool vec_codes = (a.W % 32) == 0;  // 16-byte aligned A-rows of codes

  Walk w;
  w.init((int64_t)blockIdx.x * kThreads + threadIdx.x, a.M);
  while (w.major < a.n_major) {
    const int64_t col = a.col_begin + w.minor * C;
    const int64_t blk0 = a.blk_begin + w.major * NB;
    const int nb = (int)min((int64_t)NB, a.blk_end - blk0);
    uint32_t codes[C][NB * WPB];
    uint32_t sbw[C][(NB + 3) / 4];  // scale bytes, four per word
#pragma unroll
    for (int k = 0; k < C; ++k)
#pragma unroll
      for (int i = 0; i < (NB + 3) / 4; ++i) sbw[k][i] = 0u;
    const T* base = x + blk0 * B * a.ld + col;
    // outer scales: the run is one 128-piece of each of the C A-rows; a
    // first pass over it takes the piece maxima
    ScaleCtx co[C];
    if constexpr (TSM == kTsOuter) {
      static_assert(NB * B == kOuter, "one outer piece per run");
      float ao[C];
#pragma unroll
      for (int k = 0; k < C; ++k) ao[k] = 0.0f;
#pragma unroll 1
      for (int j = 0; j < NB; ++j) {
        ColRaw<T, C> g;
        g.load(base + (int64_t)j * B * a.ld, a.ld);
        if (RHT) g.flip_rows(a.signs);
#pragma unroll
        for (int k = 0; k < C; ++k) {
          float t[16];
          g.column(k, t);
          if (RHT) fwht16(t);
#pragma unroll
          for (int i = 0; i < 16; ++i) ao[k] = fmaxf(ao[k], fabsf(t[i]));
        }
      }
#pragma unroll
      for (int k = 0; k < C; ++k) {
        co[k].s_t = outer_scale<FMT>(RHT ? ao[k] * 0.25f : ao[k]);
        co[k].den = co[k].s_t * grid_max<FMT>();
        a.ts_out[(col + k) * (a.W / kOuter) + blk0 * B / kOuter] = co[k].s_t;
      }
    } else {
#pragma unroll
      for (int k = 0; k < C; ++k) co[k] = c;
    }
    ColRaw<T, C> cur[B / 16];
#pragma unroll
    for (int h = 0; h < B / 16; ++h) cur[h].load(base + (int64_t)h * 16 * a.ld, a.ld);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (j < nb) {
        ColRaw<T, C> nxt[B / 16];
        if (j + 1 < nb) {
#pragma unroll
          for (int h = 0; h < B / 16; ++h)
            nxt[h].load(base + ((int64_t)(j + 1) * B + h * 16) * a.ld, a.ld);
        }
#pragma unroll
        for (int k = 0; k < C; ++k) {
          float t[B];
          float amax_t = 0.0f;
#pragma unroll
          for (int h = 0; h < B / 16; ++h) {
            float g[16];
            cur[h].column(k, g);
            if (RHT) { apply_signs(g, a.signs); fwht16(g); }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              t[16 * h + i] = g[i];
              amax_t = fmaxf(amax_t, fabsf(g[i]));
            }
          }
          const uint64_t n0 = (uint64_t)(col + k) * (uint64_t)a.W + (uint64_t)((blk0 + j) * B);
          uint32_t pk[WPB];
          uint32_t sbyte;
          encode_block<FMT, SR, RHT, sizeof(T) == 2, B, TSM>(t, amax_t, co[k], inv_tab, a.sr_k0,
                                                              a.sr_k1, n0, pk, sbyte);
          sbw[k][j / 4] |= sbyte << (8 * (j % 4));
#pragma unroll
          for (int q = 0; q < WPB; ++q) codes[k][j * WPB + q] = pk[q];
        }
#pragma unroll
        for (int h = 0; h < B / 16; ++h) cur[h] = nxt[h];
      }
    }
    // stores: NB*B/2 contiguous code bytes and NB scale bytes per column
#pragma unroll
    for (int k = 0; k < C; ++k) {
      constexpr int SB = scale_bytes<FMT>();
      uint8_t* cp = a.codes + (col + k) * (a.W / 2) + blk0 * (B / 2);
      uint8_t* sp = a.scales + (col + k) * a.nblk_axis * SB + blk0 * SB;
      if (nb == NB && vec_codes) {
#pragma unroll
        for (int q = 0; q < NB * WPB; q += 4)
          store16<true>(cp + 4 * q, codes[k][q], codes[k][q + 1], codes[k][q + 2],
                        codes[k][q + 3]);
      } else {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          if (j < nb) {
#pragma unroll
            for (int q = 0; q < WPB; q += 2)
              store8<true>(cp + 4 * (j * WPB + q), codes[k][j * WPB + q],
                           codes[k][j * WPB + q + 1]);
          }
        }
      }
      if constexpr (SB == 4) {
        static_assert(NB == 1, "one HiF4 block per run");
        *reinterpret_cast<uint32_t*>(sp) = sbw[k][0];
      } else {
#pragma unroll
        for (int j = 0; j < NB; ++j)
          if (j < nb) sp[j] = (uint8_t)(sbw[k][j / 4] >> (8 * (j % 4)));
      }
    }
    w.advance(a.sq, a.sr, a.M);
  }
}


// Column axis, interior tiles: TR x-rows by TC x-columns (TC * sizeof(T) =
// 128 bytes), staged through LDS.  Every global load is a 16-byte piece of a
// row (8 lanes read one 128-byte row segment); the tile is written to LDS
// transposed (A-row-major, packed row pairs for BF16; layout in ColTile);
// each lane then codes whole blocks of one A-row, and the lanes of one A-row
// write its TR/2 code bytes as one contiguous run.  A workgroup walks tiles
// with a grid stride and loads its next tile while coding the current one.

template <int FMT, bool SR, bool RHT, int TSM, typename T>
__global__ __launch_bounds__(kThreads, block_of<FMT>() == 64 ? 2 : 4) void quantize_col_tile_kernel(
    const T* __restrict__ x, QuantArgs a) {
  using Tile = ColTile<T>;
  constexpr int B = block_of<FMT>();
  constexpr int TR = Tile::TR, TC = Tile::TC;
  constexpr int kLoads = TR * TC * (int)sizeof(T) / 16 / kThreads;  // 16-byte loads per lane
  constexpr int kUnits = TC * (TR / B) / kThreads;                  // blocks coded per lane
  constexpr int LPR = TR / B;              // lanes per A-row of a tile (its blocks)
  constexpr int kRowStep = kThreads / LPR;  // A-rows between a lane's units
  __shared__ float inv_tab[128];
  __shared__ __align__(16) uint32_t lds[Tile::kWords];
  const int64_t ntile = a.n_major * a.M;  // row tiles x column tiles, column tile fastest

  // Load i of a lane reads 16 bytes of tile row lane_row + row_i at byte
  // lane_col: lane_row and lane_col depend on the lane only, row_i on i
  // only, so every address is a wave-uniform base plus one per-lane 32-bit
  // offset (the launcher keeps a tile's extent below 2^31 bytes).  For BF16,
  // loads i and i + kLoads/2 are the two rows of one pair.
  const int seg = threadIdx.x & 7;
  const uint32_t lane_off = (uint32_t)(((sizeof(T) == 2 ? 2 : 1) * (threadIdx.x >> 3)) * a.ld +
                                       seg * (16 / (int)sizeof(T))) * (uint32_t)sizeof(T);
  // After a tensor-amax pass the row tiles are taken last to first (the end
  // of the input, read last by that pass, is still in the memory-side cache)
  constexpr bool kRev = TSM == kTsCompute && has_tensor_scale(FMT);
  auto rt = [&](int64_t t) { return kRev ? a.n_major - 1 - t : t; };
  auto load_tile = [&](int64_t tr, int64_t tc, uint4 (&buf)[kLoads]) {
    const char* base = reinterpret_cast<const char*>(x + rt(tr) * TR * a.ld + tc * TC);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int row_i = sizeof(T) == 2 ? 64 * (i % (kLoads / 2)) + (i >= kLoads / 2 ? 1 : 0)
                                       : 32 * i;
      const char* p = base + (int64_t)row_i * a.ld * (int64_t)sizeof(T);
      buf[i] = *reinterpret_cast<const uint4*>(p + lane_off);
    }
  };

  // (row tile, column tile) walk with a grid stride, no division in the loop
  const int64_t step_r = gridDim.x / a.M, step_c = gridDim.x - step_r * a.M;
  int64_t tile = blockIdx.x;
  int64_t tr = tile / a.M, tc = tile - tr * a.M;
  bool have = tile < ntile;
  uint4 buf[kLoads];
  const ScaleFetch sf = scale_fetch<FMT, TSM>(a.partials, a.npartials, a.ts_in);
  if (have) load_tile(tr, tc, buf);  // in flight during the prologue
  const ScaleCtx c = scale_prologue<FMT, TSM>(sf, a.ts_out, inv_tab);
  // a lane's units: A-rows lane_ra + kRowStep * i of the tile, block j
  const int lane_ra = threadIdx.x / LPR, j = threadIdx.x % LPR;
  while (have) {
    const int64_t r0 = rt(tr) * TR, c0 = tc * TC;
    __syncthreads();  // previous tile's LDS reads are done
    // ---- registers -> LDS, transposed
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int i = 0; i < kLoads / 2; ++i) {
        const int pr = (threadIdx.x >> 3) + 32 * i;  // row pair
        const uint4 e = buf[i], o = buf[i + kLoads / 2];
        const uint32_t ev[4] = {e.x, e.y, e.z, e.w}, od[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int col = seg * 8 + 2 * k;
          // (even row, odd row) of column col, then of col + 1: byte picks
          lds[Tile::at(col, pr)] = __builtin_amdgcn_perm(od[k], ev[k], 0x05040100u);
          lds[Tile::at(col + 1, pr)] = __builtin_amdgcn_perm(od[k], ev[k], 0x07060302u);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const int row = (threadIdx.x >> 3) + 32 * i;
        const uint32_t v[4] = {buf[i].x, buf[i].y, buf[i].z, buf[i].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) lds[Tile::at(seg * 4 + k, row)] = v[k];
      }
    }
    __syncthreads();
    // ---- the next tile's loads fly while this one is coded
    const int64_t next = tile + gridDim.x;
    const bool have_next = next < ntile;
    int64_t ntr = tr + step_r, ntc = tc + step_c;
    if (ntc >= a.M) { ntc -= a.M; ntr += 1; }
    if (have_next) load_tile(ntr, ntc, buf);
    // ---- code blocks: unit i -> (A-row lane_ra + kRowStep * i, block j);
    // units one at a time for 32-element blocks (register pressure)
    const int64_t ra0 = c0 + lane_ra;  // A-row = column of x
    const int64_t rb = r0 / B + j;     // block index along the A-row
    constexpr int SB = scale_bytes<FMT>();
    uint8_t* cp0 = a.codes + ra0 * (a.W / 2) + rb * (B / 2);
    uint8_t* sp0 = a.scales + ra0 * a.nblk_axis * SB + rb * SB;
    const uint64_t n00 = (uint64_t)ra0 * (uint64_t)a.W + (uint64_t)(rb * B);
    constexpr int kUnroll = B == 32 ? 1 : kUnits;
#pragma unroll kUnroll
    for (int i = 0; i < kUnits; ++i) {
      const int cl = lane_ra + kRowStep * i;
      float t[B];
      float amax_t = 0.0f;
#pragma unroll
      for (int h = 0; h < B / 16; ++h) {
        float g[16];
        if constexpr (sizeof(T) == 2) {
          const int pr0 = (j * B + h * 16) / 2;
          const uint4 lo = *reinterpret_cast<const uint4*>(lds + Tile::at(cl, pr0));
          const uint4 hi = *reinterpret_cast<const uint4*>(lds + Tile::at(cl, pr0 + 4));
          const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
          widen_bf16_group<RHT>(w, a.signs, g);
        } else {
          const uint32_t* src = lds + Tile::at(cl, j * B + h * 16);
#pragma unroll
          for (int e = 0; e < 16; ++e) g[e] = __uint_as_float(src[e]);
          if (RHT) apply_signs(g, a.signs);
        }
        if (RHT) fwht16(g);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          t[16 * h + e] = g[e];
          amax_t = fmaxf(amax_t, fabsf(g[e]));
        }
      }
      const int64_t di = (int64_t)kRowStep * i;  // A-rows past the lane's first
      const uint64_t n0 = n00 + (uint64_t)di * (uint64_t)a.W;
      ScaleCtx cc = c;
      if constexpr (TSM == kTsOuter) {
        // kOuter / B consecutive lanes hold the blocks of one 128-piece
        constexpr int LPO = kOuter / B;
        const float ao = group_max<LPO>(amax_t);
        cc.s_t = outer_scale<FMT>(RHT ? ao * 0.25f : ao);
        cc.den = cc.s_t * grid_max<FMT>();
        if (j % LPO == 0) a.ts_out[(ra0 + di) * (a.W / kOuter) + rb / LPO] = cc.s_t;
      }
      uint32_t pk[B / 8];
      uint32_t sbyte;
      encode_block<FMT, SR, RHT, sizeof(T) == 2, B, TSM>(t, amax_t, cc, inv_tab, a.sr_k0,
                                                         a.sr_k1, n0, pk, sbyte);
      uint8_t* cp = cp0 + di * (a.W / 2);
      if constexpr (B == 16) {
        store8<true>(cp, pk[0], pk[1]);
      } else {
#pragma unroll
        for (int q = 0; q < B / 32; ++q)
          store16<true>(cp + 16 * q, pk[4 * q], pk[4 * q + 1], pk[4 * q + 2], pk[4 * q + 3]);
      }
      if constexpr (SB == 4)
        *reinterpret_cast<uint32_t*>(sp0 + di * a.nblk_axis * 4) = sbyte;
      else
        sp0[di * a.nblk_axis] = (uint8_t)sbyte;
    }
    tile = next;
    tr = ntr;
    tc = ntc;
    have = have_next;
  }
}

// ------------------------------------------- dual output (row and column)
// One read of a BF16 x emits both the row-axis and the column-axis
// quantization (the forward and the weight-gradient operands), for the
// 16-element-block formats.  Tiles are kDT x kDT: the column part goes
// through LDS as in the column tiles; the row part is coded straight from
// the load registers, where lanes 2m and 2m + 1 of a 16-lane row group hold
// columns 16m..16m+15 of two adjacent rows and one lane-pair swap gives each
// a whole 16-column block.  A 128-piece is a whole tile row (row part) or a
// whole tile column (column part), so outer scales stay inside a tile.  The
// tensor-amax pass is the same kernel with AMAX = true: it writes one
// row-axis and one column-axis partial maximum per workgroup.
constexpr int kDT = 128;          // tile rows and columns
constexpr int kDP = kDT / 2 + 4;  // LDS words per A-row of the column part

// LDS word of (x column col, row pair pr): XOR-swizzled in 4-word units
// as in ColTile (conflict-free stores per half wave, conflict-free 128-bit
// reads by the 8 lanes of one column).
__device__ __forceinline__ int dual_at(int col, int pr) {
  return col * kDP + (pr ^ (((col >> 3) & 7) << 2) ^ (((pr >> 5) & 1) << 2));
}

struct DualArgs {
  int64_t ld, rows, cols, n_ct, ntile;
  uint8_t* codes_r;
  uint8_t* scales_r;
  uint8_t* codes_c;
  uint8_t* scales_c;
  const float* ts_in_r;  // given tensor scales (kTsGiven)
  const float* ts_in_c;
  float* ts_out_r;       // computed tensor scales, or outer scales (kTsOuter)
  float* ts_out_c;
  float* partials;       // [row-axis maxima | column-axis maxima], npartials each
  int npartials;
  uint32_t signs, sr_k0, sr_k1;
};

// Both axes' tensor scales and reciprocal tables (nothing for outer scales).
template <int FMT, int TSM>
__device__ __forceinline__ void dual_prologue(const DualArgs& a, const ScaleFetch& fr,
                                              const ScaleFetch& fc, float* inv_r, float* inv_c,
                                              ScaleCtx& cr, ScaleCtx& cc) {
  cr = ScaleCtx{0.0f, 0.0f};
  cc = ScaleCtx{0.0f, 0.0f};
  if constexpr (TSM != kTsOuter) {
    if (TSM == kTsGiven) {
      cr.s_t = fr.v[0];
      cc.s_t = fc.v[0];
    } else {
      float mr = fr.v[0], mc = fc.v[0];
#pragma unroll
      for (int k = 1; k < kFetch; ++k) {
        mr = fmaxf(mr, fr.v[k]);
        mc = fmaxf(mc, fc.v[k]);
      }
      mr = block_max_256(mr);
      mc = block_max_256(mc);
      cr.s_t = mr / (grid_max<FMT>() * 448.0f);
      cc.s_t = mc / (grid_max<FMT>() * 448.0f);
      if (blockIdx.x == 0 && threadIdx.x == 0) {
        a.ts_out_r[0] = cr.s_t;
        a.ts_out_c[0] = cc.s_t;
      }
    }
    cr.den = cr.s_t * grid_max<FMT>();
    cc.den = cc.s_t * grid_max<FMT>();
    cr.rden = recip_of_den(cr.den);
    cc.rden = recip_of_den(cc.den);
    if (threadIdx.x < 128) {
      const uint32_t S = threadIdx.x < 127 ? threadIdx.x : 126u;
      const float dr = S ? cr.s_t * e4m3_decode(S) : 0.0f;
      const float dc = S ? cc.s_t * e4m3_decode(S) : 0.0f;
      inv_r[threadIdx.x] = dr != 0.0f ? 1.0f / dr : 0.0f;
      inv_c[threadIdx.x] = dc != 0.0f ? 1.0f / dc : 0.0f;
    }
    __syncthreads();
  }
}

template <int FMT, bool SR, bool RHT, int TSM, bool AMAX>
__global__ __launch_bounds__(kThreads, 4) void dual_tile_kernel(const uint16_t* __restrict__ x,
                                                                DualArgs a) {
  static_assert(!is_mx(FMT), "16-element blocks");
  constexpr int kLoads = kDT * kDT * 2 / 16 / kThreads;  // 8 loads of 16 bytes per lane
  __shared__ float inv_r[128], inv_c[128];
  __shared__ __align__(16) uint32_t lds[kDT * kDP];
  const int seg = threadIdx.x & 15;  // 16-byte column segment (8 columns)
  const int q = threadIdx.x >> 4;    // row pair within a pass
  // load i: rows 2p and 2p + 1 (p = q + 16 * (i % 4)) are loads i and i + 4;
  // a wave-uniform base per load plus one per-lane 32-bit offset (the
  // launcher keeps a tile's byte extent below 2^31)
  const uint32_t lane_off = (uint32_t)(2 * q * a.ld + seg * 8) * 2u;
  // After the tensor-amax pass the row tiles are taken last to first (the
  // end of the input, read last by that pass, is still in the memory-side
  // cache)
  constexpr bool kRev = TSM == kTsCompute && !AMAX;
  const int64_t n_rt = a.rows / kDT;
  auto rt = [&](int64_t t) { return kRev ? n_rt - 1 - t : t; };
  auto load_tile = [&](int64_t tr, int64_t tc, uint4 (&buf)[kLoads]) {
    const char* base = reinterpret_cast<const char*>(x + rt(tr) * kDT * a.ld + tc * kDT);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int row_i = 32 * (i & 3) + (i >> 2);
      buf[i] = *reinterpret_cast<const uint4*>(base + (int64_t)row_i * a.ld * 2 + lane_off);
    }
  };

  // (row tile, column tile) walk with a grid stride, no division in the loop
  const int64_t step_r = gridDim.x / a.n_ct, step_c = gridDim.x - step_r * a.n_ct;
  int64_t tile = blockIdx.x;
  int64_t tr = tile / a.n_ct, tc = tile - tr * a.n_ct;
  bool have = tile < a.ntile;
  uint4 buf[kLoads];
  ScaleFetch fr{}, fc{};
  if constexpr (!AMAX) {
    fr = scale_fetch<FMT, TSM>(a.partials, a.npartials, a.ts_in_r);
    fc = scale_fetch<FMT, TSM>(a.partials + a.npartials, a.npartials, a.ts_in_c);
  }
  if (have) load_tile(tr, tc, buf);  // in flight during the prologue
  ScaleCtx cr, cc;
  if constexpr (!AMAX) dual_prologue<FMT, TSM>(a, fr, fc, inv_r, inv_c, cr, cc);
  float mr = 0.0f, mc = 0.0f;  // AMAX: running maxima of the two axes
  while (have) {
    const int64_t r0 = rt(tr) * kDT, c0 = tc * kDT;
    __syncthreads();  // previous tile's LDS reads are done
    // ---- registers -> LDS, transposed, for the column part
#pragma unroll
    for (int i = 0; i < kLoads / 2; ++i) {
      const int pr = q + 16 * i;
      const uint4 e = buf[i], o = buf[i + kLoads / 2];
      const uint32_t ev[4] = {e.x, e.y, e.z, e.w}, od[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int col = seg * 8 + 2 * k;
        // (even row, odd row) of column col, then of col + 1: byte picks
        lds[dual_at(col, pr)] = __builtin_amdgcn_perm(od[k], ev[k], 0x05040100u);
        lds[dual_at(col + 1, pr)] = __builtin_amdgcn_perm(od[k], ev[k], 0x07060302u);
      }
    }
    // ---- row part, from the registers
    const bool odd = seg & 1;
    const int64_t row0 = r0 + 2 * q + (odd ? 1 : 0);  // the lane's row in pass 0
    const int64_t b = c0 / 16 + (seg >> 1);           // block along the row
    uint8_t* cpr = a.codes_r + row0 * (a.cols / 2) + b * 8;
    uint8_t* spr = a.scales_r + row0 * (a.cols / 16) + b;
    const uint64_t nr0 = (uint64_t)row0 * (uint64_t)a.cols + (uint64_t)(b * 16);
#pragma unroll
    for (int i = 0; i < kLoads / 2; ++i) {
      const uint4 send = odd ? buf[i] : buf[i + kLoads / 2];
      uint4 recv;
      recv.x = swap_lane_pair(send.x);
      recv.y = swap_lane_pair(send.y);
      recv.z = swap_lane_pair(send.z);
      recv.w = swap_lane_pair(send.w);
      const uint4 lo = odd ? recv : buf[i];
      const uint4 hi = odd ? buf[i + kLoads / 2] : recv;
      const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      float t[16];
      widen_bf16_group<RHT>(w, a.signs, t);
      if constexpr (AMAX && RHT) {
        mr = fmaxf(mr, fwht16_absmax(t));
      } else {
        if (RHT) fwht16(t);
        float amax_t = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) amax_t = fmaxf(amax_t, fabsf(t[j]));
        if constexpr (AMAX) {
          mr = fmaxf(mr, amax_t);
        } else {
          const int64_t dr = 32 * i;  // rows past the lane's pass-0 row
          ScaleCtx c = cr;
          if constexpr (TSM == kTsOuter) {
            // the 8 lanes of this parity hold the row's 128-piece
            const float ao = parity_max16(amax_t);
            c.s_t = outer_scale<FMT>(RHT ? ao * 0.25f : ao);
            c.den = c.s_t * grid_max<FMT>();
            if (seg < 2) a.ts_out_r[(row0 + dr) * (a.cols / kOuter) + c0 / kOuter] = c.s_t;
          }
          uint32_t pk[2];
          uint32_t sbyte;
          encode_block<FMT, SR, RHT, true, 16, TSM>(t, amax_t, c, inv_r, a.sr_k0, a.sr_k1,
                                                    nr0 + (uint64_t)dr * (uint64_t)a.cols, pk,
                                                    sbyte);
          store8<true>(cpr + dr * (a.cols / 2), pk[0], pk[1]);
          spr[dr * (a.cols / 16)] = (uint8_t)sbyte;
        }
      }
    }
    __syncthreads();
    // ---- the next tile's loads fly while the column part is coded
    const int64_t next = tile + gridDim.x;
    const bool have_next = next < a.ntile;
    int64_t ntr = tr + step_r, ntc = tc + step_c;
    if (ntc >= a.n_ct) { ntc -= a.n_ct; ntr += 1; }
    if (have_next) load_tile(ntr, ntc, buf);
    // ---- column part: unit i -> (x column (tid >> 3) + 32 i, block j = tid & 7)
    const int j = threadIdx.x & 7;
    const int64_t ra0 = c0 + (threadIdx.x >> 3);  // A-row = column of x
    const int64_t rb = r0 / 16 + j;               // block down the column
    uint8_t* cpc = a.codes_c + ra0 * (a.rows / 2) + rb * 8;
    uint8_t* spc = a.scales_c + ra0 * (a.rows / 16) + rb;
    const uint64_t nc0 = (uint64_t)ra0 * (uint64_t)a.rows + (uint64_t)(rb * 16);
#pragma unroll
    for (int i = 0; i < kDT * (kDT / 16) / kThreads; ++i) {
      const int cl = (threadIdx.x >> 3) + 32 * i;
      const uint4 lo = *reinterpret_cast<const uint4*>(lds + dual_at(cl, 8 * j));
      const uint4 hi = *reinterpret_cast<const uint4*>(lds + dual_at(cl, 8 * j + 4));
      const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      float t[16];
      widen_bf16_group<RHT>(w, a.signs, t);
      if constexpr (AMAX && RHT) {
        mc = fmaxf(mc, fwht16_absmax(t));
      } else {
        if (RHT) fwht16(t);
        float amax_t = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) amax_t = fmaxf(amax_t, fabsf(t[e]));
        if constexpr (AMAX) {
          mc = fmaxf(mc, amax_t);
        } else {
          const int64_t da = 32 * i;  // A-rows past the lane's first
          ScaleCtx c = cc;
          if constexpr (TSM == kTsOuter) {
            const float ao = group_max<8>(amax_t);
            c.s_t = outer_scale<FMT>(RHT ? ao * 0.25f : ao);
            c.den = c.s_t * grid_max<FMT>();
            if (j == 0) a.ts_out_c[(ra0 + da) * (a.rows / kOuter) + r0 / kOuter] = c.s_t;
          }
          uint32_t pk[2];
          uint32_t sbyte;
          encode_block<FMT, SR, RHT, true, 16, TSM>(t, amax_t, c, inv_c, a.sr_k0, a.sr_k1,
                                                    nc0 + (uint64_t)da * (uint64_t)a.rows, pk,
                                                    sbyte);
          store8<true>(cpc + da * (a.rows / 2), pk[0], pk[1]);
          spc[da * (a.rows / 16)] = (uint8_t)sbyte;
        }
      }
    }
    tile = next;
    tr = ntr;
    tc = ntc;
    have = have_next;
  }
  if constexpr (AMAX) {
    mr = block_max_256(mr);
    mc = block_max_256(mc);
    if (threadIdx.x == 0) {
      a.partials[blockIdx.x] = RHT ? mr * 0.25f : mr;
      a.partials[a.npartials + blockIdx.x] = RHT ? mc * 0.25f : mc;
    }
  }
}

// ------------------------------------------------------------ dispatch
// Launch geometry (measured on MI355X; overridable at build time for sweeps).
#ifndef FP4_ROW_GRID
#define FP4_ROW_GRID 1024
#endif
#ifndef FP4_COL_GRID
#define FP4_COL_GRID 4096
#endif
#ifndef FP4_COL_BLOCKS
#define FP4_COL_BLOCKS 8
#endif
#ifndef FP4_ROW_UNIT
#define FP4_ROW_UNIT 32
#endif
#ifndef FP4_COL_PAIR
#define FP4_COL_PAIR 1
#endif
constexpr int64_t kRowGrid = FP4_ROW_GRID;  // workgroups of the row kernel (cap)
constexpr int64_t kColGrid = FP4_COL_GRID;  // workgroups of the column kernel (cap)
constexpr int kColBlocks = FP4_COL_BLOCKS;  // NB for 16-element blocks (half for 32)

#ifndef FP4_RESIDENT_CAP
#define FP4_RESIDENT_CAP 1
#endif

// Workgroups of `kernel` (kThreads lanes, static LDS only) that the current
// device holds at once over all its CUs; cached per kernel and device.
// Grids no larger than this run as a single wave of workgroups, with no
// partial last wave.  0 when the runtime cannot tell.
int64_t resident_wgs(const void* kernel) {
  static std::mutex mu;
  static std::unordered_map<const void*, int64_t> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache[dev].find(kernel);
  if (it != cache[dev].end()) return it->second;
  int per_cu = 0, cus = 0;
  int64_t n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
    n = (int64_t)per_cu * cus;
  cache[dev][kernel] = n;
  return n;
}

// Grid cap for `kernel`: the fixed cap, lowered to one resident wave.
int64_t grid_cap(const void* kernel, int64_t cap) {
  if (!FP4_RESIDENT_CAP) return cap;
  const int64_t r = resident_wgs(kernel);
  return r > 0 && r < cap ? r : cap;
}

struct WalkPlan {
  unsigned grid;
  int64_t sq, sr;
};
// Grid of at most `cap` workgroups over n_major x M units, one unit per
// lane per round, sized so that every round but the last is whole and the
// rounds are spread evenly (no lone partial round).
inline WalkPlan plan_walk(int64_t n_major, int64_t M, int64_t cap) {
  const int64_t units = n_major * M;
  if (cap < 1) cap = 1;
  const int64_t rounds = (units + cap * kThreads - 1) / (cap * kThreads);
  int64_t g = rounds > 0 ? (units + rounds * kThreads - 1) / (rounds * kThreads) : 1;
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  const int64_t stride = g * kThreads;
  return {(unsigned)g, stride / M, stride % M};
}


template <bool RHT, typename T>
void launch_amax(const QuantLaunch& q, hipStream_t s) {
  const T* x = static_cast<const T*>(q.x);
  const int64_t stride = (int64_t)kAmaxPartials * kThreads;
  if (q.axis == 0) {
    const int64_t nmaj = q.rows, M = q.cols / 16;
    hipLaunchKernelGGL((amax_row_kernel<RHT, T>), dim3(kAmaxPartials), dim3(kThreads), 0, s, x,
                       q.ld, nmaj, M, stride / M, stride % M, q.signs, q.workspace);
  } else if (q.cols % 2 == 0) {
    // (16-byte row pieces, C = 8 for BF16, measured slower)
    const int64_t nmaj = q.rows / 16, M = q.cols / 2;
    hipLaunchKernelGGL((amax_col_kernel<RHT, T, 2>), dim3(kAmaxPartials), dim3(kThreads), 0, s,
                       x, q.ld, nmaj, M, stride / M, stride % M, q.signs, q.workspace);
  } else {
    const int64_t nmaj = q.rows / 16, M = q.cols;
    hipLaunchKernelGGL((amax_col_kernel<RHT, T, 1>), dim3(kAmaxPartials), dim3(kThreads), 0, s,
                       x, q.ld, nmaj, M, stride / M, stride % M, q.signs, q.workspace);
  }
}

// Ticks of the constant-rate clock (wall_clock64) per microsecond.
uint64_t wall_ticks_per_us() {
  static std::mutex mu;
  static int64_t cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 100;
  std::lock_guard<std::mutex> lock(mu);
  if (!cache[dev]) {
    int khz = 0;
    cache[dev] = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) == hipSuccess &&
                         khz > 0
                     ? (khz + 999) / 1000
                     : 100;
  }
  return (uint64_t)cache[dev];
}

#ifndef FP4_SINGLE_PASS
#define FP4_SINGLE_PASS 1
#endif
#ifndef FP4_WIDE_PASS
#define FP4_WIDE_PASS 1
#endif

// Dynamic LDS of the single-pass kernel: the SR draws of every lane.
template <bool SR, int U, int NU, int NT>
constexpr size_t single_pass_lds() {
  return SR ? (size_t)NT * NU * (U / 8) * 16 : 0;
}

// Workgroups of a kernel with NT lanes and `lds` bytes of dynamic LDS that
// the device holds at once; cached per kernel and device (0: unknown).
int64_t resident_wgs_nt(const void* kernel, int nt, size_t lds) {
  static std::mutex mu;
  static std::unordered_map<const void*, int64_t> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache[dev].find(kernel);
  if (it != cache[dev].end()) return it->second;
  if (lds > 65536 &&
      hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) !=
          hipSuccess)
    (void)hipGetLastError();  // the launch itself reports a real limit
  int per_cu = 0, cus = 0;
  int64_t n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, nt, lds) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
    n = (int64_t)per_cu * cus;
  else
    (void)hipGetLastError();
  cache[dev][kernel] = n;
  return n;
}

// The single-pass row path with NT lanes per workgroup and NU units per
// lane, when its grid (one unit per lane per k) is resident at once and has
// at most kAmaxPartials workgroups.  False when the operand does not fit;
// nothing is launched then.
template <int FMT, bool SR, bool RHT, typename T, int NU, int NT>
bool try_single_pass(const QuantLaunch& q, QuantArgs a, hipStream_t s) {
  constexpr int U = 32;
  auto kernel = quantize_row_single_kernel<FMT, SR, RHT, T, U, NU, NT>;
  constexpr size_t lds = single_pass_lds<SR, U, NU, NT>();
  const int64_t units = q.rows * (q.cols / U);
  const int64_t grid = (units + (int64_t)NT * NU - 1) / ((int64_t)NT * NU);
  const int64_t cap = resident_wgs_nt(reinterpret_cast<const void*>(kernel), NT, lds);
  if (grid < 1 || grid > kAmaxPartials || grid > cap) return false;
  if (q.plan_reads) {  // every element read once
    *q.plan_reads = q.rows * q.cols;
    return true;
  }
  a.W = q.cols;
  a.n_major = q.rows;
  a.M = q.cols / U;
  AmaxSlot* slots = reinterpret_cast<AmaxSlot*>(q.workspace);
  const uint64_t per_us = wall_ticks_per_us();
  const uint64_t ticks = (uint64_t)q.wait_us * per_us;
  // the other workgroups wait for workgroup 0's result past its own
  // deadline plus time to recompute up to every partial maximum
  const uint64_t long_ticks = 4 * ticks + 64 * per_us;
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(NT), lds, s,
                     static_cast<const T*>(q.x), a, slots, q.call_tag, ticks, long_ticks);
  return true;
}

// The wide single pass (contiguous BF16 row operands past the single
// pass's reach): one workgroup of 1024 lanes per compute unit, NR units
// held in registers and NL in LDS per lane.  False when one such workgroup per
// compute unit is not resident at once, or when fewer than half of a lane's
// units would be held; nothing is launched then.
template <int FMT, bool SR, bool RHT, typename T>
bool try_wide_pass(const QuantLaunch& q, QuantArgs a, hipStream_t s) {
  if constexpr (sizeof(T) != 2) {
    return false;
  } else {
  constexpr int U = 32, NR = RHT ? 3 : 4, NL = 2, NT = 1024;
  static_assert(NL <= NR, "LDS units are taken with the held ones");
  auto kernel = quantize_row_wide_kernel<FMT, SR, RHT, T, U, NR, NL, NT>;
  constexpr size_t lds = (size_t)NL * RowRaw<T, U>::kVec * 16 * NT;
  const int64_t units = q.rows * (q.cols / U);
  if (q.ld != q.cols) return false;
  const int64_t grid = resident_wgs_nt(reinterpret_cast<const void*>(kernel), NT, lds);
  if (grid < 1 || grid > kAmaxPartials) return false;
  const int64_t stride = grid * NT;
  const int64_t nu = (units + stride - 1) / stride;
  // Only while at least half of a lane's units are held: past that the
  // second pass reads nearly all of the operand again anyway, and the two
  // kernels of the two-pass path, each with its loads spread over four
  // workgroups per compute unit, stream it faster (measured on an
  // 8192 x 28672 operand, 28 units per lane: 190 us wide, 173 us two-pass).
  if (nu > 2 * (NR + NL)) return false;
  if (q.plan_reads) {  // units past the first NR + NL of every lane are read twice
    const int64_t held = units < stride * (NR + NL) ? units : stride * (NR + NL);
    *q.plan_reads = (2 * units - held) * U;
    return true;
  }
  a.W = q.cols;
  a.n_major = q.rows;
  a.M = q.cols / U;
  AmaxSlot* slots = reinterpret_cast<AmaxSlot*>(q.workspace);
  const uint64_t per_us = wall_ticks_per_us();
  const uint64_t ticks = (uint64_t)q.wait_us * per_us;
  const uint64_t long_ticks = 4 * ticks + 64 * per_us;
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(NT), lds, s, static_cast<const T*>(q.x), a,
                     slots, q.call_tag, ticks, long_ticks, (int)nu);
  return true;
  }
}

template <int FMT, bool SR, bool RHT, int TSM, typename T>
hipError_t launch_quantize_t(const QuantLaunch& q, hipStream_t s) {
  constexpr int B = block_of<FMT>();
  const T* x = static_cast<const T*>(q.x);
  QuantArgs a{};
  a.ld = q.ld;
  a.codes = q.codes;
  a.scales = q.scales;
  a.ts_in = q.tensor_scale;
  a.ts_out = q.tensor_scale;
  a.partials = q.workspace;
  a.npartials = kAmaxPartials;
  a.signs = q.signs;
  a.sr_k0 = q.sr_k0;
  a.sr_k1 = q.sr_k1;
  if constexpr (has_tensor_scale(FMT) && FMT != kMBS && TSM == kTsCompute) {
    if (FP4_SINGLE_PASS && q.axis == 0 && q.cols % 32 == 0 && q.call_tag != 0 &&
        q.ws_bytes >= kSinglePassWsBytes &&
        (try_single_pass<FMT, SR, RHT, T, 1, 1024>(q, a, s) ||
         (sizeof(T) == 2 && try_single_pass<FMT, SR, RHT, T, 2, 1024>(q, a, s)) ||
         try_single_pass<FMT, SR, RHT, T, 4, 256>(q, a, s) ||
         (FP4_WIDE_PASS && try_wide_pass<FMT, SR, RHT, T>(q, a, s))))
      return hipGetLastError();
  }
  if (q.plan_reads) {  // a tensor-amax pass reads x once more
    *q.plan_reads = (has_tensor_scale(FMT) && TSM == kTsCompute ? 2 : 1) * q.rows * q.cols;
    return hipSuccess;
  }
  if constexpr (has_tensor_scale(FMT) && TSM == kTsCompute) launch_amax<RHT, T>(q, s);
  if (q.axis == 0) {
    a.W = q.cols;
    const bool wide = q.cols % 32 == 0;
    // (HiF4: two lanes of 32 elements per 64-element block)
    const bool wider = FP4_ROW_UNIT >= 64 && FMT != kHIF4 && q.cols % 64 == 0;
    const int U = wider ? 64 : (wide ? 32 : 16);
    a.n_major = q.rows;
    a.M = q.cols / U;
    auto launch = [&](auto kernel) {
      const WalkPlan wp =
          plan_walk(a.n_major, a.M, grid_cap(reinterpret_cast<const void*>(kernel), kRowGrid));
      a.sq = wp.sq;
      a.sr = wp.sr;
      hipLaunchKernelGGL(kernel, dim3(wp.grid), dim3(kThreads), 0, s, x, a);
    };
    if constexpr (FMT == kHIF4) {
      launch(quantize_row_kernel<FMT, SR, RHT, TSM, T, 32>);  // W % 64 == 0
    } else if (wider) {
      launch(quantize_row_kernel<FMT, SR, RHT, TSM, T, 64>);
    } else if constexpr (B <= 32) {
      if (wide)
        launch(quantize_row_kernel<FMT, SR, RHT, TSM, T, 32>);
      else if constexpr (B == 16)
        launch(quantize_row_kernel<FMT, SR, RHT, TSM, T, 16>);
    }
  } else {
    a.W = q.rows;
    a.nblk_axis = q.rows / B;
    using Tile = ColTile<T>;
    // interior: whole tiles; edges (bottom rows, right columns): run kernel
    const int64_t nrt = q.rows / Tile::TR, nct = q.cols / Tile::TC;
    // (a tile's byte extent below 2^31 keeps its per-lane load offsets in 32 bits)
    // (a HiF4 FP32 tile holds fewer blocks than lanes: runs only)
    const bool tiles = nrt > 0 && nct > 0 && (q.ld * (int64_t)sizeof(T)) % 16 == 0 &&
                       q.ld * (int64_t)sizeof(T) * Tile::TR < ((int64_t)1 << 31) &&
                       !(FMT == kHIF4 && sizeof(T) == 4);
    const int64_t rows_main = tiles ? nrt * Tile::TR : 0;
    const int64_t cols_main = tiles ? nct * Tile::TC : 0;
    if constexpr (!(FMT == kHIF4 && sizeof(T) == 4)) {
      if (tiles) {
        QuantArgs t = a;
        t.n_major = nrt;
        t.M = nct;
        const int64_t ntile = nrt * nct;
        // more workgroups than fit at once measured faster here than one
        // resident wave
        const unsigned grid = (unsigned)(ntile < kColGrid ? ntile : kColGrid);
        hipLaunchKernelGGL((quantize_col_tile_kernel<FMT, SR, RHT, TSM, T>), dim3(grid),
                           dim3(kThreads), 0, s, x, t);
      }
    }
    // runs of 128 rows (64 with SR, whose Philox state needs the registers)
    // (one 128-piece per run with outer scales)
    // (one 64-element block per run for HiF4: its registers)
    constexpr int NB = TSM == kTsOuter ? kOuter / B
                       : B == 64       ? 1
                                       : (B == 16 ? kColBlocks : kColBlocks / 2) / (SR ? 2 : 1);
    auto run = [&](int64_t blk_begin, int64_t blk_end, int64_t col_begin, int64_t col_end) {
      if (blk_end <= blk_begin || col_end <= col_begin) return;
      QuantArgs r = a;
      r.blk_begin = blk_begin;
      r.blk_end = blk_end;
      r.col_begin = col_begin;
      r.n_major = (blk_end - blk_begin + NB - 1) / NB;
      const int C = (FP4_COL_PAIR && B < 64 && (col_end - col_begin) % 2 == 0) ? 2 : 1;
      r.M = (col_end - col_begin) / C;
      const WalkPlan wp = plan_walk(r.n_major, r.M, kColGrid);
      r.sq = wp.sq;
      r.sr = wp.sr;
      if constexpr (B < 64) {
        if (C == 2) {
          hipLaunchKernelGGL((quantize_col_kernel<FMT, SR, RHT, TSM, T, 2, NB>), dim3(wp.grid),
                             dim3(kThreads), 0, s, x, r);
          return;
        }
      }
      hipLaunchKernelGGL((quantize_col_kernel<FMT, SR, RHT, TSM, T, 1, NB>), dim3(wp.grid),
                         dim3(kThreads), 0, s, x, r);
    };
    // right strip over the tiled rows, then the bottom strip over all columns
    run(0, rows_main / B, cols_main, q.cols);
    run(rows_main / B, a.nblk_axis, 0, q.cols);
  }
  return hipGetLastError();
}

template <int FMT, bool SR, bool RHT, int TSM>
hipError_t pick_dtype(const QuantLaunch& q, hipStream_t s) {
  return q.in_dtype == 0 ? launch_quantize_t<FMT, SR, RHT, TSM, uint16_t>(q, s)
                         : launch_quantize_t<FMT, SR, RHT, TSM, float>(q, s);
}
template <int FMT, bool SR, bool RHT>
hipError_t pick_tsm(const QuantLaunch& q, hipStream_t s) {
  if constexpr (is_mx(FMT) || FMT == kHIF4) {
    return pick_dtype<FMT, SR, RHT, kTsCompute>(q, s);  // no tensor scale
  } else if constexpr (FMT == kMBS) {
    return pick_dtype<FMT, SR, RHT, kTsOuter>(q, s);  // macro scales only
  } else {
    switch (q.ts_mode) {
      case kTsGiven: return pick_dtype<FMT, SR, RHT, kTsGiven>(q, s);
      case kTsOuter: return pick_dtype<FMT, SR, RHT, kTsOuter>(q, s);
      default: return pick_dtype<FMT, SR, RHT, kTsCompute>(q, s);
    }
  }
}
template <int FMT, bool SR>
hipError_t pick_rht(const QuantLaunch& q, hipStream_t s) {
  return q.rht ? pick_tsm<FMT, SR, true>(q, s) : pick_tsm<FMT, SR, false>(q, s);
}
template <int FMT>
hipError_t quantize_format(const QuantLaunch& q, hipStream_t s) {
  return q.sr ? pick_rht<FMT, true>(q, s) : pick_rht<FMT, false>(q, s);
}

// Dual output: BF16, rows and cols multiples of kDT (checked by the caller).
template <int FMT, bool SR, bool RHT, int TSM>
hipError_t launch_dual_t(const DualLaunch& q, hipStream_t s) {
  DualArgs a{};
  a.ld = q.ld;
  a.rows = q.rows;
  a.cols = q.cols;
  a.n_ct = q.cols / kDT;
  a.ntile = (q.rows / kDT) * a.n_ct;
  a.codes_r = q.codes_row;
  a.scales_r = q.scales_row;
  a.codes_c = q.codes_col;
  a.scales_c = q.scales_col;
  a.ts_in_r = q.ts_row;
  a.ts_in_c = q.ts_col;
  a.ts_out_r = q.ts_row;
  a.ts_out_c = q.ts_col;
  a.partials = q.workspace;
  a.npartials = kAmaxPartials;
  a.signs = q.signs;
  a.sr_k0 = q.sr_k0;
  a.sr_k1 = q.sr_k1;
  const uint16_t* x = static_cast<const uint16_t*>(q.x);
  if constexpr (TSM == kTsCompute)  // every partial slot is written
    hipLaunchKernelGGL((dual_tile_kernel<FMT, false, RHT, kTsCompute, true>),
                       dim3(kAmaxPartials), dim3(kThreads), 0, s, x, a);
  const unsigned grid = (unsigned)(a.ntile < kColGrid ? a.ntile : kColGrid);
  hipLaunchKernelGGL((dual_tile_kernel<FMT, SR, RHT, TSM, false>), dim3(grid), dim3(kThreads), 0,
                     s, x, a);
  return hipGetLastError();
}
template <int FMT, bool SR, bool RHT>
hipError_t dual_pick_tsm(const DualLaunch& q, hipStream_t s) {
  if constexpr (FMT == kMBS) return launch_dual_t<FMT, SR, RHT, kTsOuter>(q, s);
  switch (q.ts_mode) {
    case kTsGiven: return launch_dual_t<FMT, SR, RHT, kTsGiven>(q, s);
    case kTsOuter: return launch_dual_t<FMT, SR, RHT, kTsOuter>(q, s);
    default: return launch_dual_t<FMT, SR, RHT, kTsCompute>(q, s);
  }
}
template <int FMT, bool SR>
hipError_t dual_pick_rht(const DualLaunch& q, hipStream_t s) {
  return q.rht ? dual_pick_tsm<FMT, SR, true>(q, s) : dual_pick_tsm<FMT, SR, false>(q, s);
}
template <int FMT>
hipError_t quantize_dual_format(const DualLaunch& q, hipStream_t s) {
  return q.sr ? dual_pick_rht<FMT, true>(q, s) : dual_pick_rht<FMT, false>(q, s);
}

}  // namespace
