// fp4_dequant.hip -- gfx950 kernels of the dequantize and standalone-RHT
// paths and their launchers.
//
// Dequantize rebuilds each element as sign * L[k] * d with d the decoded
// block scale (one binary32 product), optionally undoes the RHT in
// registers, and writes x's layout (row axis: the A-row is a row of x;
// column axis: lanes on consecutive columns, so each store of a wave is one
// contiguous segment of a row).
#include "fp4_device.h"
#include "fp4_launch.h"
#include "fp4_tiles.h"

using namespace fp4dev;

namespace {

// Group g (16 elements) of A-row ra: row axis reads 16 contiguous elements,
// column axis 16 rows of one column.
template <int AXIS, typename T>
__device__ __forceinline__ void load_group(const T* x, int64_t ld, int64_t ra, int64_t col0,
                                           float (&t)[16]) {
  if (AXIS == 0) {
    RowRaw<T, 16> r;
    r.load(x + ra * ld + col0);
    r.template group<false>(0, t, 0u);
  } else {
    ColRaw<T, 1> c;
    c.load(x + col0 * ld + ra, ld);
    c.column(0, t);
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

// Row-axis output staging.  A lane's unit is WORDS contiguous 32-bit words
// of output, and consecutive lanes hold consecutive units; writing them
// straight out would make every store instruction touch 64 separate
// 16-byte pieces.  Instead each lane parks its words in LDS, and the
// workgroup then stores 16-byte chunks so that consecutive lanes write
// consecutive chunks (whole 64-byte segments and more per instruction).
template <int WORDS>
struct RowStage {
  static constexpr int P = WORDS + 4;  // word pitch: 16-byte aligned, banks spread
  static constexpr int kChunks = WORDS / 4;
  uint32_t* buf;  // [kThreads][P]
  uint32_t** dst;  // [kThreads] destination of each lane's unit (null: none)
  __device__ __forceinline__ void put(const uint32_t (&v)[WORDS], uint32_t* to) const {
#pragma unroll
    for (int q = 0; q < kChunks; ++q)
      *reinterpret_cast<uint4*>(buf + threadIdx.x * P + 4 * q) =
          make_uint4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    dst[threadIdx.x] = to;
  }
  // after a barrier: chunk k = i * kThreads + lane of the workgroup's units
  __device__ __forceinline__ void flush() const {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int k = i * kThreads + threadIdx.x;
      const int u = k / kChunks, part = k % kChunks;
      uint32_t* to = dst[u];
      if (to) {
        const uint4 v = *reinterpret_cast<const uint4*>(buf + u * P + 4 * part);
        store16<false>(to + 4 * part, v.x, v.y, v.z, v.w);
      }
    }
  }
};

__device__ __forceinline__ void pack_f32(const float* t, uint32_t* w, int n) {
  for (int j = 0; j < n; ++j) w[j] = __float_as_uint(t[j]);
}

// sign * L[k] of the two E2M1 codes in byte `sel` of w (low nibble first),
// exactly: the hardware pair convert with scale 1.0.
typedef float f2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f2 e2m1_pair(uint32_t w, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  }
}

// Output words of block (ra, b): sign * L[k] * d (one binary32 product),
// optionally through the inverse RHT a = D (1/4) H16 y, packed as T (two
// BF16 values per word, or one FP32 value).  B * sizeof(T) / 4 words.
//
// E2M1 codes decode in hardware: the FP4 -> FP32 pair convert with scale
// 1.0 gives sign * L[k] exactly (-0 for code 8), and (sign * L) * d equals
// sign * (L * d) in IEEE arithmetic.  BF16 packing uses the packed RNE
// convert (same bits as round-to-nearest-even, NaN kept quiet).  With the
// inverse RHT the 1/4 moves into d when 2^-100 <= d <= 2^100: then every
// y = L * d/4 is exactly y/4 rounded as y was, every butterfly sum is a
// multiple of 2^-126 (no bits lost to the subnormal range) and no sum nears
// overflow, so the butterfly of y/4 is the butterfly of y times 1/4 exactly;
// other blocks multiply by 1/4 after the butterfly, as written.  The D sign
// flips act on the packed words (negation commutes with rounding).
template <int FMT, bool OUTER, bool INV, typename T>
__device__ __forceinline__ void dequant_block(const DequantArgs& a, float s_t, int64_t ra,
                                              int64_t b, uint32_t* out) {
  constexpr int B = block_of<FMT>();
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const uint32_t S = a.scales[ra * (a.W / B) + b];
  float d;
  if constexpr (is_mx(FMT)) {
    d = S ? __uint_as_float(S << 23) : 5.877471754111438e-39f;
  } else {
    // outer scales: the 128-piece of the A-row that holds block b
    const float so = OUTER ? a.ts[ra * (a.W / kOuter) + b * B / kOuter] : s_t;
    d = S ? so * e4m3_decode(S) : 0.0f;
  }
  const uint8_t* cp = a.codes + ra * (a.W / 2) + b * (B / 2);
  uint32_t words[B / 8];
  if constexpr (B == 16) {
    const uint2 v = *reinterpret_cast<const uint2*>(cp);
    words[0] = v.x; words[1] = v.y;
  } else {
    const uint4 v = *reinterpret_cast<const uint4*>(cp);
    words[0] = v.x; words[1] = v.y; words[2] = v.z; words[3] = v.w;
  }
  const bool fold = INV && d >= 0x1p-100f && d <= 0x1p100f;
  const float dm = fold ? d * 0.25f : d;
#pragma unroll
  for (int h = 0; h < B / 16; ++h) {
    float g[16];
    if constexpr (FMT == kUFP4) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t c = (words[(h * 16 + j) >> 3] >> (4 * (j & 7))) & 15u;
        const float mag = (float)(c & 7u) * dm;
        g[j] = (c & 8u) ? -mag : mag;
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) {  // byte k of the group: elements 2k, 2k + 1
        const f2 l = e2m1_pair(words[2 * h + (k >> 2)], k & 3);
        g[2 * k] = l.x * dm;
        g[2 * k + 1] = l.y * dm;
      }
    }
    if constexpr (INV) {
      fwht16(g);
      if (!fold) {
#pragma unroll
        for (int j = 0; j < 16; ++j) g[j] = g[j] * 0.25f;
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t m = INV ? pair_sign_mask(a.signs, k) : 0u;  // bits 15 and 31
      if constexpr (sizeof(T) == 2) {
        f2 v;
        v.x = g[2 * k];
        v.y = g[2 * k + 1];
        out[8 * h + k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2)) ^ m;
      } else {
        out[16 * h + 2 * k] = __float_as_uint(g[2 * k]) ^ (m << 16);
        out[16 * h + 2 * k + 1] = __float_as_uint(g[2 * k + 1]) ^ (m & 0x80000000u);
      }
    }
  }
}

template <int FMT, bool OUTER, bool INV, int AXIS, typename T>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(T* __restrict__ out, DequantArgs a) {
  constexpr int B = block_of<FMT>();
  const float s_t = (is_mx(FMT) || OUTER) ? 0.0f : a.ts[0];
  Walk w;
  w.init((int64_t)blockIdx.x * kThreads + threadIdx.x, a.M);
  if constexpr (AXIS == 0 && sizeof(T) == 2) {
    // BF16 rows: 2 bytes per value, a lane's 16-value group is two 16-byte
    // stores (staging measured slower here)
    while (w.major < a.n_major) {
      uint32_t v[B / 2];
      dequant_block<FMT, OUTER, INV, T>(a, s_t, w.major, w.minor, v);
      uint32_t* to = reinterpret_cast<uint32_t*>(out + w.major * a.ld_out + w.minor * B);
#pragma unroll
      for (int q = 0; q < B / 8; ++q) store16<false>(to + 4 * q, v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
      w.advance(a.sq, a.sr, a.M);
    }
  } else if constexpr (AXIS == 0) {
    // FP32 rows: units (A-row, block), block fastest; the whole workgroup
    // steps together so that it can stage its outputs
    constexpr int WORDS = B * (int)sizeof(T) / 4;
    using Stage = RowStage<WORDS>;
    __shared__ __align__(16) uint32_t sbuf[kThreads * Stage::P];
    __shared__ uint32_t* sdst[kThreads];
    const Stage st{sbuf, sdst};
    const int64_t units = a.n_major * a.M;
    for (int64_t base = (int64_t)blockIdx.x * kThreads; base < units;
         base += (int64_t)gridDim.x * kThreads) {
      uint32_t v[WORDS];
      uint32_t* to = nullptr;
      if (w.major < a.n_major) {
        dequant_block<FMT, OUTER, INV, T>(a, s_t, w.major, w.minor, v);
        to = reinterpret_cast<uint32_t*>(out + w.major * a.ld_out + w.minor * B);
      } else {
#pragma unroll
        for (int j = 0; j < WORDS; ++j) v[j] = 0u;
      }
      st.put(v, to);
      __syncthreads();
      st.flush();
      __syncthreads();
      w.advance(a.sq, a.sr, a.M);
    }
  } else {
    while (w.major < a.n_major) {
      const int64_t ra = w.minor, b = w.major;
      constexpr int WORDS = B * (int)sizeof(T) / 4;
      uint32_t v[WORDS];
      dequant_block<FMT, OUTER, INV, T>(a, s_t, ra, b, v);
#pragma unroll
      for (int j = 0; j < B; ++j) {
        T* p = out + (b * B + j) * a.ld_out + ra;
        if constexpr (sizeof(T) == 2) *p = (T)(v[j / 2] >> (16 * (j & 1)));
        else *p = __uint_as_float(v[j]);
      }
      w.advance(a.sq, a.sr, a.M);
    }
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
  if constexpr (AXIS == 0) {
    using Stage = RowStage<16>;
    __shared__ __align__(16) uint32_t sbuf[kThreads * Stage::P];
    __shared__ uint32_t* sdst[kThreads];
    const Stage st{sbuf, sdst};
    const int64_t units = n_major * M;
    for (int64_t base = (int64_t)blockIdx.x * kThreads; base < units;
         base += (int64_t)gridDim.x * kThreads) {
      uint32_t v[16];
      uint32_t* to = nullptr;
      if (w.major < n_major) {
        float t[16];
        load_group<0>(x, ld, w.major, w.minor * 16, t);
        if (INV) rht16_inverse(t, signs);
        else rht16_forward(t, signs);
        pack_f32(t, v, 16);
        to = reinterpret_cast<uint32_t*>(y + w.major * cols + w.minor * 16);
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = 0u;
      }
      st.put(v, to);
      __syncthreads();
      st.flush();
      __syncthreads();
      w.advance(sq, sr, M);
    }
  } else {
    while (w.major < n_major) {
      const int64_t ra = w.minor, g = w.major;
      float t[16];
      load_group<1>(x, ld, ra, g * 16, t);
      if (INV) rht16_inverse(t, signs);
      else rht16_forward(t, signs);
#pragma unroll
      for (int j = 0; j < 16; ++j) y[(g * 16 + j) * cols + ra] = t[j];
      w.advance(sq, sr, M);
    }
  }
}

// ------------------------------------------------------------ dispatch
constexpr int64_t kMaxGrid = 8192;

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

template <int FMT, bool OUTER, bool INV, int AXIS, typename T>
hipError_t launch_dequant_t(const DequantLaunch& q, hipStream_t s) {
  constexpr int B = block_of<FMT>();
  const int64_t W = AXIS == 0 ? q.cols : q.rows;
  const int64_t RA = AXIS == 0 ? q.rows : q.cols;
  const int64_t nmaj = AXIS == 0 ? RA : W / B;
  const int64_t M = AXIS == 0 ? W / B : RA;
  const WalkPlan wp = plan_walk(nmaj, M, kMaxGrid);
  DequantArgs a{q.codes, q.scales, q.tensor_scale, q.ld_out, W, nmaj, M, wp.sq, wp.sr, q.signs};
  hipLaunchKernelGGL((dequantize_kernel<FMT, OUTER, INV, AXIS, T>), dim3(wp.grid),
                     dim3(kThreads), 0, s, static_cast<T*>(q.out), a);
  return hipGetLastError();
}
template <int FMT, bool OUTER, bool INV, int AXIS>
hipError_t dq_dtype(const DequantLaunch& q, hipStream_t s) {
  return q.out_dtype == 0 ? launch_dequant_t<FMT, OUTER, INV, AXIS, uint16_t>(q, s)
                          : launch_dequant_t<FMT, OUTER, INV, AXIS, float>(q, s);
}
template <int FMT, bool OUTER, bool INV>
hipError_t dq_axis(const DequantLaunch& q, hipStream_t s) {
  return q.axis == 0 ? dq_dtype<FMT, OUTER, INV, 0>(q, s) : dq_dtype<FMT, OUTER, INV, 1>(q, s);
}
template <int FMT, bool OUTER>
hipError_t dq_inv(const DequantLaunch& q, hipStream_t s) {
  return q.inverse_rht ? dq_axis<FMT, OUTER, true>(q, s) : dq_axis<FMT, OUTER, false>(q, s);
}
template <int FMT>
hipError_t dq_outer(const DequantLaunch& q, hipStream_t s) {
  if constexpr (is_mx(FMT)) return dq_inv<FMT, false>(q, s);
  else return q.outer ? dq_inv<FMT, true>(q, s) : dq_inv<FMT, false>(q, s);
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

hipError_t fp4_launch_dequantize(const DequantLaunch& q, hipStream_t s) {
  switch (q.format) {
    case kNVFP4: return dq_outer<kNVFP4>(q, s);
    case kMXFP4: return dq_outer<kMXFP4>(q, s);
    case kUFP4: return dq_outer<kUFP4>(q, s);
    default: return dq_outer<kMXOAS>(q, s);
  }
}

hipError_t fp4_launch_rht(const RhtLaunch& q, hipStream_t s) {
  return q.inverse ? rht_axis<true>(q, s) : rht_axis<false>(q, s);
}

hipError_t fp4_launch_write_scalar(float* p, float v, hipStream_t s) {
  hipLaunchKernelGGL(write_scalar_kernel, dim3(1), dim3(64), 0, s, p, v);
  return hipGetLastError();
}
