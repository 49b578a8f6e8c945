// fp4_device.h -- device-side building blocks of the gfx950 FP4 codec.
//
// Everything here runs per lane in registers.  The arithmetic is binary32
// with round-to-nearest-even in the order of the method's description (the
// library is built with -ffp-contract=off and correctly rounded division),
// so codes and scales are reproducible bit for bit on any launch geometry.
//
// Pages cited (summaries on gist.science):
//   [UFP4]  es/paper/2606.20381  shrinkage bias and the uniform E1M2 grid
//   [NGPT]  it/paper/2605.06067  normalized transformers under NVFP4
//   [TJ2]   it/paper/2510.27527  TetraJet-v2 NVFP4 training
//   [MXFP4] fr/paper/2603.08713  MXFP4 error reduction (OAS, MBS)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fp4dev {

// kCAP2: E2M1 codes cut at magnitude 2 (levels 0, .5, 1, 1.5, 2, equally
// spaced), NVFP4's two-level scaling with the block amax mapped to 2 -- the
// range-restricted E2M1 of [UFP4] Metodologia 2 (Ablacion).
// kMBS: MXFP4 with static macro-block scaling ([MXFP4] 2.B): a scale with
// an 8-bit mantissa per 128-element macro block (carried like the outer
// scales), 16-element blocks with E8M0 scales relative to it, E2M1 codes.
// kMXOAS16: overflow-aware MX scaling on 16-element blocks, the granularity
// at which [MXFP4] 2 applies its techniques (E8M0 per 16 elements).
// kHIF4: HiF4 ([HIF] 2. Metodologia): per 64-element block an E6M2 scale,
// per 8 and per 4 elements a one-bit E1M0 refinement, E1M2 elements (k/4);
// its scale word (4 bytes per block) is described at encode_hif4.
enum : int { kNVFP4 = 0, kMXFP4 = 1, kUFP4 = 2, kMXOAS = 3, kCAP2 = 4, kMBS = 5, kMXOAS16 = 6,
             kHIF4 = 7 };
// Tensor-scale modes of the two-level formats: computed from the data,
// given by the caller, or one outer scale per kOuter elements of an A-row.
enum : int { kTsCompute = 0, kTsGiven = 1, kTsOuter = 2 };
constexpr int kOuter = 128;

// E8M0-scaled formats (power-of-two block scales, no tensor scale).
constexpr bool is_mx(int fmt) { return fmt == kMXFP4 || fmt == kMXOAS || fmt == kMXOAS16; }
// Overflow-aware MX exponents ([MXFP4] 2.A).
constexpr bool is_oas(int fmt) { return fmt == kMXOAS || fmt == kMXOAS16; }
// A tensor scale (computed or given) or outer scales per 128 elements: the
// E4M3 two-level formats and MBS-Static.  The MX formats and HiF4 carry
// every scale per block.
constexpr bool has_tensor_scale(int fmt) { return !is_mx(fmt) && fmt != kHIF4; }
template <int FMT>
constexpr int block_of() {
  return FMT == kHIF4 ? 64 : ((is_mx(FMT) && FMT != kMXOAS16) ? 32 : 16);
}
// Scale bytes per block: 4 for HiF4's scale word, 1 otherwise.
template <int FMT>
constexpr int scale_bytes() { return FMT == kHIF4 ? 4 : 1; }

// ---------------------------------------------------------------- widening
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Sign flips of the RHT's D on packed BF16: word e of a 16-group holds
// elements 2e (low half) and 2e + 1 (high half), so one xor with bits 15
// and 31 flips both before widening.
__device__ __forceinline__ uint32_t pair_sign_mask(uint32_t signs, int e) {
  return (((signs >> (2 * e)) & 1u) << 15) | (((signs >> (2 * e + 1)) & 1u) << 31);
}

// Half H (0 low, 1 high) of w xor the same half of the wave-uniform m,
// moved to bits 31..16 of a word whose low half is zero: one BF16 element
// with its sign flipped, widened exactly to binary32, in one SDWA
// instruction that reads m from a scalar register.  (Written out as C, the
// high half compiles to a three-input op that needs m copied to a vector
// register first.)
template <int H>
__device__ __forceinline__ uint32_t xor_widen_bf16(uint32_t w, uint32_t m) {
  uint32_t r;
  if constexpr (H == 0)
    asm("v_xor_b32_sdwa %0, %1, %2 dst_sel:WORD_1 dst_unused:UNUSED_PAD src0_sel:WORD_0 "
        "src1_sel:WORD_0" : "=v"(r) : "v"(w), "s"(m));
  else
    asm("v_xor_b32_sdwa %0, %1, %2 dst_sel:WORD_1 dst_unused:UNUSED_PAD src0_sel:WORD_1 "
        "src1_sel:WORD_1" : "=v"(r) : "v"(w), "s"(m));
  return r;
}

// Widen the 8 words of a BF16 16-group, flipping signs when SIGN (signs is
// wave-uniform: the RHT's one sign vector).
template <bool SIGN>
__device__ __forceinline__ void widen_bf16_group(const uint32_t (&w)[8], uint32_t signs,
                                                 float (&t)[16]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if constexpr (SIGN) {
      const uint32_t m = pair_sign_mask(signs, e);
      t[2 * e] = __uint_as_float(xor_widen_bf16<0>(w[e], m));
      t[2 * e + 1] = __uint_as_float(xor_widen_bf16<1>(w[e], m));
    } else {
      t[2 * e] = bf16_lo(w[e]);
      t[2 * e + 1] = bf16_hi(w[e]);
    }
  }
}

// ------------------------------------------------------------ Philox4x32-10
// Counter-based generator of Salmon et al. (SC'11): ten rounds of
// 32x32->64-bit products of counter words with the two round multipliers,
// high halves xor-ed with the other counter words and the key, key bumped
// by the Weyl constants between rounds.  One 64-bit product per multiplier
// maps to a single v_mad_u64_u32.
struct u32x4 { uint32_t x, y, z, w; };

__device__ __forceinline__ u32x4 philox4x32_10(uint32_t k0, uint32_t k1, uint32_t c0,
                                               uint32_t c1, uint32_t c2, uint32_t c3) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    // three-input exclusive or (truth table 0x96): one instruction each
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
    c0 = n0; c1 = (uint32_t)p1; c2 = n2; c3 = (uint32_t)p0;
    k0 += 0x9E3779B9u; k1 += 0xBB67AE85u;
  }
  return {c0, c1, c2, c3};
}

// ------------------------------------------------------------ RHT butterfly
// 16-point Walsh-Hadamard butterfly in natural (Sylvester) order, stages
// h = 1, 2, 4, 8 ([UFP4] Metodologia 1-2, "Eficiencia"; [TJ2] 2.C).  The
// stage order is fixed so that the binary32 result does not depend on the
// launch geometry.
__device__ __forceinline__ void fwht16(float (&t)[16]) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j & h) continue;
      const float u = t[j], v = t[j + h];
      t[j] = u + v;
      t[j + h] = u - v;
    }
  }
}

// Largest magnitude of fwht16(t), without its outputs: after the stages
// h = 1, 2, 4 the last stage would give u + v and u - v for each pair
// (u, v) = (t[j], t[j + 8]), and max(|fl(u + v)|, |fl(u - v)|) =
// fl(|u| + |v|) exactly: one of the two is that sum up to sign and the
// other's magnitude, |u| - |v| rounded, is not larger (rounding to nearest
// is monotone and odd).  NaN and infinity propagate as in the full form
// under fmaxf.  t is left holding the stage-4 inputs.
__device__ __forceinline__ float fwht16_absmax(float (&t)[16]) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j & h) continue;
      const float u = t[j], v = t[j + h];
      t[j] = u + v;
      t[j + h] = u - v;
    }
  }
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(t[j]) + fabsf(t[j + 8]));
  return m;
}

// Sign flip d_j a_j for a group (bit j of `signs` set: d_j = -1).
__device__ __forceinline__ void apply_signs(float (&t)[16], uint32_t signs) {
#pragma unroll
  for (int j = 0; j < 16; ++j)
    t[j] = __uint_as_float(__float_as_uint(t[j]) ^ (((signs >> j) & 1u) << 31));
}

// Forward RHT of one group: y = (1/4) H16 D a.
__device__ __forceinline__ void rht16_forward(float (&t)[16], uint32_t signs) {
  apply_signs(t, signs);
  fwht16(t);
#pragma unroll
  for (int j = 0; j < 16; ++j) t[j] = t[j] * 0.25f;
}

// Inverse: a = D (1/4) H16 y.
__device__ __forceinline__ void rht16_inverse(float (&t)[16], uint32_t signs) {
  fwht16(t);
#pragma unroll
  for (int j = 0; j < 16; ++j) t[j] = t[j] * 0.25f;
  apply_signs(t, signs);
}

// -------------------------------------------------------------- scale bytes
// E4M3 (OCP FN variant: bias 7, max 448, no infinities) of r >= 0, round to
// nearest even, saturating at 448.  Below 2^-6 the format is subnormal with
// step 2^-9, so the code is rint(r * 512); above, the binary32 mantissa is
// rounded to 3 bits and rebiased.  Branch-free.
__device__ __forceinline__ uint32_t e4m3_encode(float r) {
  const uint32_t sub = (uint32_t)__builtin_rintf(fminf(r, 0.015625f) * 512.0f);
  uint32_t b = __float_as_uint(r);
  b += 0x7FFFFu + ((b >> 20) & 1u);
  const uint32_t nor = (b >> 20) - (120u << 3);
  const uint32_t s = r < 0.015625f ? sub : nor;
  return r < 448.0f ? s : 0x7Eu;
}

// e4m3_encode(r) of the binary32 quotient r = a / den, given rden, the
// binary32 reciprocal of den (0 when it is not a normal number).  The
// product q = a * rden is within 2.5 units in the last place of r (two
// roundings of relative size 2^-24 each, against r's half unit), so where
// no rounding midpoint of the E4M3 grid lies within 4 binary32 patterns of
// q, and q is in the normal E4M3 range, q and r round to the same code
// (r is then no midpoint either, so no tie is decided differently); the
// midpoints there are the patterns with low 20 bits 0x80000.  Elsewhere
// (rare: near a midpoint, subnormal E4M3 codes, saturation, non-finite
// values) the quotient is divided out.  The result is e4m3_encode(a / den)
// in every case; one multiply replaces a correctly rounded division.
__device__ __forceinline__ uint32_t e4m3_encode_quotient(float a, float den, float rden) {
  const float q = a * rden;
  const uint32_t b = __float_as_uint(q);
  const bool near = ((b & 0xFFFFFu) - 0x7FFFCu) <= 8u;
  if (q >= 0x1.0001p-6f && q < 448.0f && !near)
    return ((b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20) - (120u << 3);
  return e4m3_encode(a / den);
}

__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t e = c >> 3, m = c & 7u;
  const float sub = (float)m * 0.001953125f;  // m * 2^-9
  const float nor = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return e == 0 ? sub : nor;
}

// HiF4's E6M2 block scale ([HIF] 2. Metodologia; reading: unsigned, exponent
// bias 31, subnormal step 2^-32, every byte finite) of r >= 0, round to
// nearest even, saturating at byte 0xFF = 1.75 * 2^32.  Below 2^-30 the
// format is subnormal: code rint(r * 2^32) (4 is the smallest normal, so
// the carry lands right); above, the binary32 significand is rounded to 2
// bits and the exponent rebiased (127 - 31 = 96, times 4 for the mantissa
// bits); past the top the code exceeds 255 and clamps.  Branch-free.
__device__ __forceinline__ uint32_t e6m2_encode(float r) {
  const uint32_t sub = (uint32_t)__builtin_rintf(fminf(r, 0x1p-30f) * 0x1p32f);
  uint32_t b = __float_as_uint(r);
  b += 0xFFFFFu + ((b >> 21) & 1u);
  const uint32_t nor = (b >> 21) - (96u << 2);
  const uint32_t s = r < 0x1p-30f ? sub : nor;
  return s < 255u ? s : 255u;
}

__device__ __forceinline__ float e6m2_decode(uint32_t c) {
  const uint32_t e = c >> 2, m = c & 3u;
  const float sub = (float)m * 0x1p-32f;
  const float nor = __uint_as_float(((e + 96u) << 23) | (m << 21));
  return e == 0 ? sub : nor;
}

// MX scale exponent ([MXFP4] 2: power-of-two E8M0 scale): floor(log2 amax)
// minus E2M1's top exponent 2, clamped to [-127, 127]; zero or subnormal
// amax lands on -127.  amax >= 0.
__device__ __forceinline__ int e8m0_exponent(float amax) {
  const int ex = (int)(__float_as_uint(amax) >> 23);
  const int e = ex - 129;
  return (ex == 0 || e < -127) ? -127 : e;
}

// x >= 0 finite, rounded to 8 fraction bits (9 significant bits from its
// leading one), ties to even.  Normal: the low 15 significand bits go, with
// the carry running into the exponent.  Subnormal: the bits below the
// leading one's ninth go (none when it has at most nine).
__device__ __forceinline__ float round8(float x) {
  uint32_t u = __float_as_uint(x);
  if (u >= 0x00800000u) {
    u = (u + 0x3FFFu + ((u >> 15) & 1u)) & 0xFFFF8000u;
  } else if (u != 0u) {
    const int drop = (31 - __builtin_clz(u)) - 8;
    if (drop > 0) {
      const uint32_t lsb = (u >> drop) & 1u;
      u = (u + (1u << (drop - 1)) - 1u + lsb) & ~((1u << drop) - 1u);
    }
  }
  return __uint_as_float(u);
}

// MBS-Static macro scale ([MXFP4] 2.B, computed directly from the macro
// block's maximum): round8(amax / 6), so the maximum lands on E2M1's 6.
__device__ __forceinline__ float mbs_macro_scale(float amax) { return round8(amax / 6.0f); }

// Overflow-aware MX exponent ([MXFP4] 2.A): amax / 2^e in (3.5, 7].  From
// the standard e, amax / 2^e = 4 * 1.f lies in [4, 8); it exceeds 7 exactly
// when the significand 1.f exceeds 1.75 (fraction bits above 0x600000), and
// then e grows by one.  Zero and subnormal amax land on -127.
__device__ __forceinline__ int e8m0_exponent_oas(float amax) {
  const uint32_t b = __float_as_uint(amax);
  const int ex = (int)(b >> 23);
  const int e = ex - 129 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return (ex == 0 || e < -127) ? -127 : e;
}

// ---------------------------------------------------------- element grids
// E2M1 levels 0, .5, 1, 1.5, 2, 3, 4, 6 ([UFP4] Problema; [TJ2] Riepilogo 1;
// [MXFP4] 2.A limit 6).  Uniform levels 0..7 ([UFP4] Metodologia 2).
__device__ __forceinline__ float e2m1_level(uint32_t k) {
  const float big = __uint_as_float((((k >> 1) + 126u) << 23) | ((k & 1u) << 22));
  return k < 2u ? (k ? 0.5f : 0.0f) : big;
}

template <int FMT>
__device__ __forceinline__ float grid_level(uint32_t k) {
  if constexpr (FMT == kUFP4) return (float)k;
  else return e2m1_level(k);
}

// Magnitude code of m >= 0 (or +inf), round to nearest even code.
// E2M1: inside each binade the levels are equally spaced (0.5 below 2, 1 in
// [2,4), 2 above 4) and the even code is the even multiple of the spacing,
// so rint(m / spacing) decides; values past 6 saturate.
// Uniform: rint(m), saturating at 7.
// The cut E2M1 saturates at code 4 (magnitude 2).
template <int FMT>
__device__ __forceinline__ uint32_t round_rtne_sw(float m) {
  if constexpr (FMT == kUFP4) {
    return (uint32_t)fminf(__builtin_rintf(m), 7.0f);
  } else {
    const bool lo = m < 2.0f, mid = m < 4.0f;
    const float q = lo ? m * 2.0f : (mid ? m : m * 0.5f);
    const float off = lo ? 0.0f : (mid ? 2.0f : 4.0f);
    return (uint32_t)fminf(__builtin_rintf(q) + off, FMT == kCAP2 ? 4.0f : 7.0f);
  }
}

// Stochastic rounding ([TJ2] 2.A; [UFP4] Metodologia 2): with L[k] <= m <
// L[k+1], round up iff p * 2^22 >= 64 * u16 + 1, p = (m - L[k]) /
// (L[k+1] - L[k]), which is the (exact) fractional part of m / spacing;
// both sides of the comparison are exact in binary32.
template <int FMT>
__device__ __forceinline__ uint32_t round_sr_sw(float m, uint32_t u16) {
  float q, off;
  if constexpr (FMT == kUFP4) {
    q = m;
    off = 0.0f;
  } else {
    const bool lo = m < 2.0f, mid = m < 4.0f;
    q = lo ? m * 2.0f : (mid ? m : m * 0.5f);
    off = lo ? 0.0f : (mid ? 2.0f : 4.0f);
  }
  const float fl = __builtin_floorf(q);
  const float up = (q - fl) * 4194304.0f >= (float)(u16 * 64u + 1u) ? 1.0f : 0.0f;
  return (uint32_t)fminf(fl + off + up, FMT == kCAP2 ? 4.0f : 7.0f);
}

// G, the largest level, in the two-level tensor scale amax / (G * 448).
template <int FMT>
__device__ __forceinline__ float grid_max() {
  return FMT == kUFP4 ? 7.0f : (FMT == kCAP2 ? 2.0f : 6.0f);
}

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Max over aligned groups of N consecutive lanes (N = 1, 2, 4 or 8); every
// lane of a group gets the group's max.  DPP moves inside quads (lane xor 1,
// lane xor 2) and half rows (mirror of 8 lanes), no LDS round trip.  All
// lanes of a group must be active.
template <int N>
__device__ __forceinline__ float group_max(float v) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8, "group of 1, 2, 4 or 8 lanes");
  auto move = [](float x, auto ctrl) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value, 0xF, 0xF, false));
  };
  if constexpr (N >= 2) v = fmaxf(v, move(v, std::integral_constant<int, 0xB1>{}));  // [1,0,3,2]
  if constexpr (N >= 4) v = fmaxf(v, move(v, std::integral_constant<int, 0x4E>{}));  // [2,3,0,1]
  if constexpr (N >= 8) v = fmaxf(v, move(v, std::integral_constant<int, 0x141>{})); // half mirror
  return v;
}

// Max over the 8 lanes of one parity inside each aligned group of 16 lanes
// (a DPP row): lane xor 2 inside quads, then rotations of the row by 4 and
// by 8, which keep the parity.  All 16 lanes must be active.
__device__ __forceinline__ float parity_max16(float v) {
  auto move = [](float x, auto ctrl) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value, 0xF, 0xF, false));
  };
  v = fmaxf(v, move(v, std::integral_constant<int, 0x4E>{}));   // quad [2,3,0,1]
  v = fmaxf(v, move(v, std::integral_constant<int, 0x124>{}));  // row_ror:4
  v = fmaxf(v, move(v, std::integral_constant<int, 0x128>{}));  // row_ror:8
  return v;
}

// Swap a 32-bit word with the neighbouring lane (lane xor 1).
__device__ __forceinline__ uint32_t swap_lane_pair(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
}

// Block-wide max over a workgroup of NT threads (a multiple of 64, at most
// 1024); every thread gets the result.
template <int NT>
__device__ __forceinline__ float block_max(float v) {
  static_assert(NT % 64 == 0 && NT <= 1024, "whole waves, at most 16");
  constexpr int kWaves = NT / 64;
  __shared__ float red[kWaves];
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) m = fmaxf(m, red[i]);
  __syncthreads();
  return m;
}

__device__ __forceinline__ float block_max_256(float v) { return block_max<256>(v); }

}  // namespace fp4dev
