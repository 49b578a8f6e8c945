// fp4_kernels.hip -- gfx950 kernels of the FP4 codec and their launchers.
//
// Terms: x is the caller's rows x cols tensor (row-major, leading dimension
// ld).  The logical operand A is x (row axis) or x^T (column axis); W is the
// length of A's rows, B the block size (16 or 32).  Codes are A-row-major,
// two per byte (even column in the low nibble); scales are one byte per
// block, A-row-major.  SR draws are keyed on the logical A coordinate, so
// any tiling gives the same bytes.
//
// Work decomposition: a "unit" is one block of one A-row.  Units are
// enumerated minor-index-fastest, where the minor index is the block within
// the A-row for the row axis (lanes read consecutive 32-byte pieces of a
// row) and the A-row for the column axis (lanes read consecutive columns of
// x, so each 2-byte load of a wave is one contiguous 128-byte segment).
// Workgroups stride over units; each lane keeps its (major, minor) position
// incrementally, with no integer division in the loop.
#include "fp4_device.h"
#include "fp4_launch.h"

using namespace fp4dev;

namespace {

constexpr int kThreads = 256;

// ------------------------------------------------------------------ loads
// Load 16 consecutive elements of a row (16-byte aligned) and widen.
__device__ __forceinline__ void load16_row(const uint16_t* p, float (&t)[16]) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
  const uint4 a = q[0], b = q[1];
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    t[2 * i] = bf16_lo(w[i]);
    t[2 * i + 1] = bf16_hi(w[i]);
  }
}
__device__ __forceinline__ void load16_row(const float* p, float (&t)[16]) {
  const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 v = q[i];
    t[4 * i] = v.x; t[4 * i + 1] = v.y; t[4 * i + 2] = v.z; t[4 * i + 3] = v.w;
  }
}

// Load 16 elements down a column (stride ld) and widen.
__device__ __forceinline__ void load16_col(const uint16_t* p, int64_t ld, float (&t)[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) t[i] = __uint_as_float((uint32_t)p[(int64_t)i * ld] << 16);
}
__device__ __forceinline__ void load16_col(const float* p, int64_t ld, float (&t)[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) t[i] = p[(int64_t)i * ld];
}

// Group g (16 elements) of unit (major, minor) in A's frame.
template <int AXIS, typename T>
__device__ __forceinline__ void load_group(const T* x, int64_t ld, int64_t ra, int64_t col0,
                                           float (&t)[16]) {
  if (AXIS == 0) load16_row(x + ra * ld + col0, t);
  else load16_col(x + col0 * ld + ra, ld, t);
}

// Incremental (major, minor) walk over units for a grid stride.
struct Walk {
  int64_t major, minor;
  __device__ __forceinline__ void init(int64_t u, int64_t M) {
    major = u / M;
    minor = u - major * M;
  }
  __device__ __forceinline__ void advance(int64_t sq, int64_t sr, int64_t M) {
    minor += sr;
    major += sq;
    if (minor >= M) { minor -= M; major += 1; }
  }
};

// ------------------------------------------------------------ tensor amax
// Partial maxima of |A| or, with the RHT, of |H16 D a| (before the exact
// scaling by 1/4, which is monotone and is applied once to the total).
// One float per workgroup; the max is order-independent.
template <int AXIS, bool RHT, typename T>
__global__ __launch_bounds__(kThreads) void amax_partials_kernel(
    const T* __restrict__ x, int64_t ld, int64_t n_major, int64_t M, int64_t sq, int64_t sr,
    uint32_t signs, float* __restrict__ partials) {
  // units are 16-element groups here
  Walk w;
  w.init((int64_t)blockIdx.x * kThreads + threadIdx.x, M);
  float m = 0.0f;
  while (w.major < n_major) {
    float t[16];
    const int64_t ra = AXIS == 0 ? w.major : w.minor;
    const int64_t g = AXIS == 0 ? w.minor : w.major;
    load_group<AXIS>(x, ld, ra, g * 16, t);
    if (RHT) {
      apply_signs(t, signs);
      fwht16(t);
    }
#pragma unroll
    for (int j = 0; j < 16; j += 2) m = fmaxf(m, fmaxf(fabsf(t[j]), fabsf(t[j + 1])));
    w.advance(sq, sr, M);
  }
  m = block_max_256(m);
  if (threadIdx.x == 0) partials[blockIdx.x] = RHT ? m * 0.25f : m;
}

// ------------------------------------------------------------- quantize
struct QuantArgs {
  int64_t ld, W;
  int64_t n_major, M, sq, sr;  // unit walk
  uint8_t* codes;
  uint8_t* scales;
  const float* ts_in;      // given tensor scale (GIVEN mode)
  float* ts_out;           // computed tensor scale (COMPUTE mode)
  const float* partials;   // amax partials (COMPUTE mode)
  int npartials;
  uint32_t signs;
  uint32_t sr_k0, sr_k1;
};

// Encode 8 values v[0..8) (already multiplied by the reciprocal block
// scale, all finite) into one 32-bit word of 4-bit codes.
template <int FMT, bool SR>
__device__ __forceinline__ uint32_t encode8_fast(const float* v, const uint32_t (&r)[4]) {
  uint32_t word = 0;
  if constexpr (FMT != kUFP4 && !SR) {
    // E2M1 round-to-nearest-even in hardware: two values per instruction,
    // sign and saturation included (scale operand 1.0: no rescaling).
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, v[0], v[1], 1.0f, 0);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, v[2], v[3], 1.0f, 1);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, v[4], v[5], 1.0f, 2);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, v[6], v[7], 1.0f, 3);
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

// Per-element path for blocks whose reciprocal scale (or the product with
// the block amax) is not finite: codes of zero elements are signed zeros,
// everything else follows v = y * inv exactly as in the scalar definition.
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

template <int FMT, bool SR, bool RHT, int AXIS, bool GIVEN, typename T>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const T* __restrict__ x, QuantArgs a) {
  constexpr int B = FMT == kMXFP4 ? 32 : 16;
  constexpr bool kBf16 = sizeof(T) == 2;
  // With BF16 input every RHT partial sum is a multiple of 2^-133, so
  // t * 0.25 is exact and the 1/4 can join the reciprocal block scale.
  constexpr bool kFoldQuarter = RHT && kBf16;

  // Reciprocal of every decoded block scale, once per workgroup:
  // inv[S] = 1 / (s_t * decode(S)), 0 where the decode scale is 0.
  __shared__ float inv_tab[128];
  float s_t = 0.0f, den = 0.0f;
  if constexpr (FMT != kMXFP4) {
    if (GIVEN) {
      s_t = a.ts_in[0];
    } else {
      float m = 0.0f;
      for (int i = threadIdx.x; i < a.npartials; i += kThreads) m = fmaxf(m, a.partials[i]);
      m = block_max_256(m);
      s_t = m / (grid_max<FMT>() * 448.0f);
      if (blockIdx.x == 0 && threadIdx.x == 0) a.ts_out[0] = s_t;
    }
    den = s_t * grid_max<FMT>();
    if (threadIdx.x < 128) {
      const uint32_t S = threadIdx.x;
      const float d = S ? s_t * e4m3_decode(S < 127u ? S : 126u) : 0.0f;
      inv_tab[S] = d != 0.0f ? 1.0f / d : 0.0f;
    }
    __syncthreads();
  }

  Walk w;
  w.init((int64_t)blockIdx.x * kThreads + threadIdx.x, a.M);
  while (w.major < a.n_major) {
    const int64_t ra = AXIS == 0 ? w.major : w.minor;
    const int64_t b = AXIS == 0 ? w.minor : w.major;
    // load, rotate (without the 1/4), block amax of the rotated values
    float t[B];
    float amax_t = 0.0f;
#pragma unroll
    for (int h = 0; h < B / 16; ++h) {
      float g[16];
      load_group<AXIS>(x, a.ld, ra, b * B + h * 16, g);
      if (RHT) {
        apply_signs(g, a.signs);
        fwht16(g);
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        t[h * 16 + j] = g[j];
        amax_t = fmaxf(amax_t, fabsf(g[j]));
      }
    }
    // block amax of y = t / 4 (monotone, exact) and the block scale
    const float amax_b = RHT ? amax_t * 0.25f : amax_t;
    uint32_t sbyte;
    float inv;
    if constexpr (FMT == kMXFP4) {
      const int e = e8m0_exponent(amax_b);
      sbyte = (uint32_t)(e + 127);
      inv = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, exact
    } else {
      sbyte = (s_t != 0.0f && amax_b != 0.0f) ? e4m3_encode(amax_b / den) : 0u;
      inv = inv_tab[sbyte];
    }
    // Element multiplier: with the 1/4 folded in (exact while inv >= 2^-124),
    // or inv itself.  Blocks where that fails, or where the largest scaled
    // value is not finite, take the per-element careful path.
    float mul;
    bool fast;
    if constexpr (kFoldQuarter) {
      mul = inv * 0.25f;
      fast = inv >= 4.70197740328915e-38f && amax_t * mul < __builtin_inff();
    } else {
      mul = inv;
      fast = amax_b * inv < __builtin_inff();
    }

    // SR draws: one Philox call per 8 consecutive elements of the A-row
    const uint64_t n0 = (uint64_t)ra * (uint64_t)a.W + (uint64_t)(b * B);
    uint32_t packed[B / 8];
#pragma unroll
    for (int q = 0; q < B / 8; ++q) {
      uint32_t r[4] = {0u, 0u, 0u, 0u};
      if constexpr (SR) {
        const uint64_t g = (n0 >> 3) + (uint64_t)q;
        const u32x4 o = philox4x32_10(a.sr_k0, a.sr_k1, (uint32_t)g, (uint32_t)(g >> 32), 0u, 0u);
        r[0] = o.x; r[1] = o.y; r[2] = o.z; r[3] = o.w;
      }
      float* tq = t + 8 * q;
      if (fast) {
        float v[8];
#pragma unroll
        for (int l = 0; l < 8; ++l) {
          const float y = (RHT && !kFoldQuarter) ? tq[l] * 0.25f : tq[l];
          v[l] = y * mul;
        }
        packed[q] = encode8_fast<FMT, SR>(v, r);
      } else {
        float y[8];
#pragma unroll
        for (int l = 0; l < 8; ++l) y[l] = RHT ? tq[l] * 0.25f : tq[l];
        packed[q] = encode8_careful<FMT, SR>(y, inv, r);
      }
    }
    uint8_t* cp = a.codes + ra * (a.W / 2) + b * (B / 2);
    if constexpr (B == 16) *reinterpret_cast<uint2*>(cp) = make_uint2(packed[0], packed[1]);
    else *reinterpret_cast<uint4*>(cp) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    a.scales[ra * (a.W / B) + b] = (uint8_t)sbyte;
    w.advance(a.sq, a.sr, a.M);
  }
}

__global__ void write_scalar_kernel(float* p, float v) {
  if (threadIdx.x == 0 && blockIdx.x == 0) p[0] = v;
}

// ----------------------------------------------------------- dequantize
struct DequantArgs {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* ts;
  int64_t ld_out, W;
  int64_t n_major, M, sq, sr;
  uint32_t signs;
};

__device__ __forceinline__ void store_elem(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_elem(uint16_t* p, float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) {
    *p = (uint16_t)((u >> 16) | 0x0040u);
    return;
  }
  u += 0x7FFFu + ((u >> 16) & 1u);
  *p = (uint16_t)(u >> 16);
}

template <int FMT, bool INV, int AXIS, typename T>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(T* __restrict__ out, DequantArgs a) {
  constexpr int B = FMT == kMXFP4 ? 32 : 16;
  const float s_t = FMT == kMXFP4 ? 0.0f : a.ts[0];
  Walk w;
  w.init((int64_t)blockIdx.x * kThreads + threadIdx.x, a.M);
  while (w.major < a.n_major) {
    const int64_t ra = AXIS == 0 ? w.major : w.minor;
    const int64_t b = AXIS == 0 ? w.minor : w.major;
    const uint32_t S = a.scales[ra * (a.W / B) + b];
    float d;
    if constexpr (FMT == kMXFP4) d = S ? __uint_as_float(S << 23) : 5.877471754111438e-39f;
    else d = S ? s_t * e4m3_decode(S) : 0.0f;
    const uint8_t* cp = a.codes + ra * (a.W / 2) + b * (B / 2);
    uint32_t words[B / 8];
    if constexpr (B == 16) {
      const uint2 v = *reinterpret_cast<const uint2*>(cp);
      words[0] = v.x; words[1] = v.y;
    } else {
      const uint4 v = *reinterpret_cast<const uint4*>(cp);
      words[0] = v.x; words[1] = v.y; words[2] = v.z; words[3] = v.w;
    }
#pragma unroll
    for (int h = 0; h < B / 16; ++h) {
      float t[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t c = (words[(h * 16 + j) >> 3] >> (4 * (j & 7))) & 15u;
        const float mag = grid_level<FMT>(c & 7u) * d;
        t[j] = (c & 8u) ? -mag : mag;
      }
      if (INV) rht16_inverse(t, a.signs);
      const int64_t j0 = b * B + h * 16;
      if (AXIS == 0 && sizeof(T) == 4) {
        float4* o = reinterpret_cast<float4*>(out + ra * a.ld_out + j0);
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = make_float4(t[4 * i], t[4 * i + 1], t[4 * i + 2], t[4 * i + 3]);
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          T* p = AXIS == 0 ? out + ra * a.ld_out + j0 + j : out + (j0 + j) * a.ld_out + ra;
          store_elem(p, t[j]);
        }
      }
    }
    w.advance(a.sq, a.sr, a.M);
  }
}

// ------------------------------------------------------------ standalone RHT
template <bool INV, int AXIS, typename T>
__global__ __launch_bounds__(kThreads) void rht_kernel(const T* __restrict__ x, int64_t ld,
                                                       int64_t cols, int64_t n_major, int64_t M,
                                                       int64_t sq, int64_t sr, uint32_t signs,
                                                       float* __restrict__ y) {
  Walk w;
  w.init((int64_t)blockIdx.x * kThreads + threadIdx.x, M);
  while (w.major < n_major) {
    const int64_t ra = AXIS == 0 ? w.major : w.minor;
    const int64_t g = AXIS == 0 ? w.minor : w.major;
    float t[16];
    load_group<AXIS>(x, ld, ra, g * 16, t);
    if (INV) rht16_inverse(t, signs);
    else rht16_forward(t, signs);
    if (AXIS == 0) {
      float4* o = reinterpret_cast<float4*>(y + ra * cols + g * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = make_float4(t[4 * i], t[4 * i + 1], t[4 * i + 2], t[4 * i + 3]);
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) y[(g * 16 + j) * cols + ra] = t[j];
    }
    w.advance(sq, sr, M);
  }
}

// ------------------------------------------------------------ dispatch
constexpr int64_t kMaxGrid = 8192;

// Grid size and unit-walk parameters for n_major x M units.
struct WalkPlan {
  unsigned grid;
  int64_t sq, sr;
};
inline WalkPlan plan_walk(int64_t n_major, int64_t M, int64_t cap) {
  const int64_t units = n_major * M;
  int64_t g = (units + kThreads - 1) / kThreads;
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  const int64_t stride = g * kThreads;
  return {(unsigned)g, stride / M, stride % M};
}

template <int FMT, bool SR, bool RHT, int AXIS, bool GIVEN, typename T>
hipError_t launch_quantize_t(const QuantLaunch& q, hipStream_t s) {
  constexpr int B = FMT == kMXFP4 ? 32 : 16;
  const int64_t W = AXIS == 0 ? q.cols : q.rows;
  const int64_t RA = AXIS == 0 ? q.rows : q.cols;
  const T* x = static_cast<const T*>(q.x);
  if (FMT != kMXFP4 && !GIVEN) {
    // 16-element groups: row axis (ra major, group minor); column (group major, ra minor)
    const int64_t nmaj = AXIS == 0 ? RA : W / 16;
    const int64_t M = AXIS == 0 ? W / 16 : RA;
    // exactly kAmaxPartials workgroups: the quantize kernel reduces that many floats
    const int64_t stride = (int64_t)kAmaxPartials * kThreads;
    hipLaunchKernelGGL((amax_partials_kernel<AXIS, RHT, T>), dim3(kAmaxPartials), dim3(kThreads),
                       0, s, x, q.ld, nmaj, M, stride / M, stride % M, q.signs, q.workspace);
  }
  const int64_t nmaj = AXIS == 0 ? RA : W / B;
  const int64_t M = AXIS == 0 ? W / B : RA;
  const WalkPlan wp = plan_walk(nmaj, M, kMaxGrid);
  QuantArgs a{q.ld, W, nmaj, M, wp.sq, wp.sr, q.codes, q.scales, q.tensor_scale,
              q.tensor_scale, q.workspace, kAmaxPartials, q.signs, q.sr_k0, q.sr_k1};
  hipLaunchKernelGGL((quantize_kernel<FMT, SR, RHT, AXIS, GIVEN, T>), dim3(wp.grid),
                     dim3(kThreads), 0, s, x, a);
  return hipGetLastError();
}

template <int FMT, bool SR, bool RHT, int AXIS, bool GIVEN>
hipError_t pick_dtype(const QuantLaunch& q, hipStream_t s) {
  return q.in_dtype == 0 ? launch_quantize_t<FMT, SR, RHT, AXIS, GIVEN, uint16_t>(q, s)
                         : launch_quantize_t<FMT, SR, RHT, AXIS, GIVEN, float>(q, s);
}
template <int FMT, bool SR, bool RHT, int AXIS>
hipError_t pick_given(const QuantLaunch& q, hipStream_t s) {
  return q.ts_given ? pick_dtype<FMT, SR, RHT, AXIS, true>(q, s)
                    : pick_dtype<FMT, SR, RHT, AXIS, false>(q, s);
}
template <int FMT, bool SR, bool RHT>
hipError_t pick_axis(const QuantLaunch& q, hipStream_t s) {
  return q.axis == 0 ? pick_given<FMT, SR, RHT, 0>(q, s) : pick_given<FMT, SR, RHT, 1>(q, s);
}
template <int FMT, bool SR>
hipError_t pick_rht(const QuantLaunch& q, hipStream_t s) {
  return q.rht ? pick_axis<FMT, SR, true>(q, s) : pick_axis<FMT, SR, false>(q, s);
}
template <int FMT>
hipError_t pick_sr(const QuantLaunch& q, hipStream_t s) {
  return q.sr ? pick_rht<FMT, true>(q, s) : pick_rht<FMT, false>(q, s);
}

template <int FMT, bool INV, int AXIS, typename T>
hipError_t launch_dequant_t(const DequantLaunch& q, hipStream_t s) {
  constexpr int B = FMT == kMXFP4 ? 32 : 16;
  const int64_t W = AXIS == 0 ? q.cols : q.rows;
  const int64_t RA = AXIS == 0 ? q.rows : q.cols;
  const int64_t nmaj = AXIS == 0 ? RA : W / B;
  const int64_t M = AXIS == 0 ? W / B : RA;
  const WalkPlan wp = plan_walk(nmaj, M, kMaxGrid);
  DequantArgs a{q.codes, q.scales, q.tensor_scale, q.ld_out, W, nmaj, M, wp.sq, wp.sr, q.signs};
  hipLaunchKernelGGL((dequantize_kernel<FMT, INV, AXIS, T>), dim3(wp.grid), dim3(kThreads), 0, s,
                     static_cast<T*>(q.out), a);
  return hipGetLastError();
}
template <int FMT, bool INV, int AXIS>
hipError_t dq_dtype(const DequantLaunch& q, hipStream_t s) {
  return q.out_dtype == 0 ? launch_dequant_t<FMT, INV, AXIS, uint16_t>(q, s)
                          : launch_dequant_t<FMT, INV, AXIS, float>(q, s);
}
template <int FMT, bool INV>
hipError_t dq_axis(const DequantLaunch& q, hipStream_t s) {
  return q.axis == 0 ? dq_dtype<FMT, INV, 0>(q, s) : dq_dtype<FMT, INV, 1>(q, s);
}
template <int FMT>
hipError_t dq_inv(const DequantLaunch& q, hipStream_t s) {
  return q.inverse_rht ? dq_axis<FMT, true>(q, s) : dq_axis<FMT, false>(q, s);
}

template <bool INV, int AXIS, typename T>
hipError_t launch_rht_t(const RhtLaunch& q, hipStream_t s) {
  const int64_t W = AXIS == 0 ? q.cols : q.rows;
  const int64_t RA = AXIS == 0 ? q.rows : q.cols;
  const int64_t nmaj = AXIS == 0 ? RA : W / 16;
  const int64_t M = AXIS == 0 ? W / 16 : RA;
  const WalkPlan wp = plan_walk(nmaj, M, kMaxGrid);
  hipLaunchKernelGGL((rht_kernel<INV, AXIS, T>), dim3(wp.grid), dim3(kThreads), 0, s,
                     static_cast<const T*>(q.x), q.ld, q.cols, nmaj, M, wp.sq, wp.sr, q.signs,
                     q.y);
  return hipGetLastError();
}
template <bool INV, int AXIS>
hipError_t rht_dtype(const RhtLaunch& q, hipStream_t s) {
  return q.in_dtype == 0 ? launch_rht_t<INV, AXIS, uint16_t>(q, s)
                         : launch_rht_t<INV, AXIS, float>(q, s);
}
template <bool INV>
hipError_t rht_axis(const RhtLaunch& q, hipStream_t s) {
  return q.axis == 0 ? rht_dtype<INV, 0>(q, s) : rht_dtype<INV, 1>(q, s);
}

}  // namespace

hipError_t fp4_launch_quantize(const QuantLaunch& q, hipStream_t s) {
  switch (q.format) {
    case kNVFP4: return pick_sr<kNVFP4>(q, s);
    case kMXFP4: return pick_sr<kMXFP4>(q, s);
    default: return pick_sr<kUFP4>(q, s);
  }
}

hipError_t fp4_launch_dequantize(const DequantLaunch& q, hipStream_t s) {
  switch (q.format) {
    case kNVFP4: return dq_inv<kNVFP4>(q, s);
    case kMXFP4: return dq_inv<kMXFP4>(q, s);
    default: return dq_inv<kUFP4>(q, s);
  }
}

hipError_t fp4_launch_rht(const RhtLaunch& q, hipStream_t s) {
  return q.inverse ? rht_axis<true>(q, s) : rht_axis<false>(q, s);
}

hipError_t fp4_launch_write_scalar(float* p, float v, hipStream_t s) {
  hipLaunchKernelGGL(write_scalar_kernel, dim3(1), dim3(64), 0, s, p, v);
  return hipGetLastError();
}
