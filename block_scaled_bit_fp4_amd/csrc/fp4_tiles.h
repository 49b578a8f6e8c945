// fp4_tiles.h -- memory-side helpers shared by the gfx950 kernels: vector
// loads and widening of BF16/FP32 rows and columns, and the incremental
// walk of a workgroup grid over units of work.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fp4_device.h"

namespace fp4dev {

constexpr int kThreads = 256;

// 16- and 8-byte stores of outputs the kernel does not read again.  NT:
// with the nontemporal hint, measured faster for the code bytes of the
// quantize kernels and much slower (about 2x) for the FP32 outputs of the
// dequantize and RHT kernels, which therefore use plain stores.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
template <bool NT>
__device__ __forceinline__ void store16(void* p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const u32x4_t v = {a, b, c, d};
  if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
  else *reinterpret_cast<u32x4_t*>(p) = v;
}
template <bool NT>
__device__ __forceinline__ void store8(void* p, uint32_t a, uint32_t b) {
  const u32x2_t v = {a, b};
  if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<u32x2_t*>(p));
  else *reinterpret_cast<u32x2_t*>(p) = v;
}

// ---------------------------------------------------------------- rows
// Raw bytes of N consecutive elements of a row (16-byte aligned).
template <typename T, int N>
struct RowRaw {
  static constexpr int kVec = N * (int)sizeof(T) / 16;
  uint4 q[kVec];
  __device__ __forceinline__ void load(const T* p) {
    const uint4* s = reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int i = 0; i < kVec; ++i) q[i] = s[i];
  }
  // widen elements [16h, 16h + 16) to fp32; SIGN applies the RHT's sign
  // flips (bit j of signs: element j negated)
  template <bool SIGN>
  __device__ __forceinline__ void group(int h, float (&t)[16], uint32_t signs) const {
    if constexpr (sizeof(T) == 2) {
      const uint4 a = q[2 * h], b = q[2 * h + 1];
      const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      widen_bf16_group<SIGN>(w, signs, t);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v = q[4 * h + i];
        t[4 * i] = __uint_as_float(v.x); t[4 * i + 1] = __uint_as_float(v.y);
        t[4 * i + 2] = __uint_as_float(v.z); t[4 * i + 3] = __uint_as_float(v.w);
      }
      if (SIGN) apply_signs(t, signs);
    }
  }
};

// ------------------------------------------------------------- columns
// C adjacent columns of 16 consecutive rows: one load of C * sizeof(T)
// bytes (2 to 16) per row, so a wave of lanes on consecutive column groups
// reads one contiguous segment per row.
template <typename T, int C>
struct ColRaw {
  static constexpr int kBytes = C * (int)sizeof(T);
  static constexpr int NW = kBytes < 4 ? 1 : kBytes / 4;  // 32-bit words per row
  static_assert(kBytes == 2 || kBytes == 4 || kBytes == 8 || kBytes == 16, "row piece");
  uint32_t w[16][NW];
  __device__ __forceinline__ void load(const T* p, int64_t ld) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const T* r = p + (int64_t)i * ld;
      if constexpr (kBytes == 2) {
        w[i][0] = *reinterpret_cast<const uint16_t*>(r);
      } else if constexpr (kBytes == 4) {
        w[i][0] = *reinterpret_cast<const uint32_t*>(r);
      } else if constexpr (kBytes == 8) {
        const uint2 v = *reinterpret_cast<const uint2*>(r);
        w[i][0] = v.x; w[i][1] = v.y;
      } else {
        const uint4 v = *reinterpret_cast<const uint4*>(r);
        w[i][0] = v.x; w[i][1] = v.y; w[i][2] = v.z; w[i][3] = v.w;
      }
    }
  }
  // the RHT's sign flips down the columns: row i negated where bit i of
  // signs is set (one xor per 32-bit word)
  __device__ __forceinline__ void flip_rows(uint32_t signs) {
    constexpr uint32_t kSign =
        sizeof(T) == 2 ? (kBytes == 2 ? 0x8000u : 0x80008000u) : 0x80000000u;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t m = ((signs >> i) & 1u) ? kSign : 0u;
#pragma unroll
      for (int k = 0; k < NW; ++k) w[i][k] ^= m;
    }
  }
  // widen column k (0 <= k < C) of the 16 rows
  __device__ __forceinline__ void column(int k, float (&t)[16]) const {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if constexpr (sizeof(T) == 2) {
        const uint32_t v = w[i][k / 2];
        t[i] = (k & 1) ? bf16_hi(v) : bf16_lo(v);
      } else {
        t[i] = __uint_as_float(w[i][k]);
      }
    }
  }
};

// Incremental (major, minor) walk over n_major x M units for a grid stride
// sq * M + sr: no integer division inside loops.
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

// Column-axis tiles of TR x-rows by TC x-columns (TC * sizeof(T) = 128
// bytes), held in LDS transposed: A-row-major (an A-row is a column of x),
// packed row pairs for BF16.  The quantize tiles write this layout from
// row loads and read whole blocks from it; the dequantize tiles write
// whole blocks into it and read it back as rows.
template <typename T>
struct ColTile {
  static constexpr int TR = 256;                        // rows per tile
  static constexpr int TC = 128 / (int)sizeof(T);       // columns per tile
  static constexpr int EPW = 4 / (int)sizeof(T);        // elements per LDS word
  // Words per A-row.  BF16: 128 words (row pairs) plus 4 of padding, so
  // every A-row starts 16-byte aligned and a block reads as 128-bit words;
  // FP32: an odd pitch.
  static constexpr int P = sizeof(T) == 2 ? TR / 2 + 4 : TR + 1;
  static constexpr int kWords = TC * P;
  // LDS word of (A-row col, position pr).  BF16 positions are XOR-swizzled
  // in 4-word units, by bits 3-5 of col (the transposing stores of one
  // instruction then reach 32 distinct banks per half wave) and by bit 5 of
  // pr (the eight 128-bit reads of lanes on consecutive blocks then reach
  // distinct 4-bank groups); aligned 4-word groups stay whole.
  __device__ static __forceinline__ int at(int col, int pr) {
    if constexpr (sizeof(T) == 2)
      return col * P + (pr ^ (((col >> 3) & 7) << 2) ^ (((pr >> 5) & 1) << 2));
    else
      return col * P + pr;
  }
};

}  // namespace fp4dev
