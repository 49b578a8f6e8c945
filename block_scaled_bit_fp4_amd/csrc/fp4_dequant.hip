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

#ifndef FP4_DEQ_WAVE_ROWS
#define FP4_DEQ_WAVE_ROWS 1
#endif

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
  int64_t blk0, col0;  // column axis: first block down the rows, first column
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
// The inputs of block (ra, b): its scale byte, its outer scale (double
// block) and its code words.  Loaded one block ahead of the decode so the
// loads fly while the previous block is decoded and stored.
template <int FMT, bool OUTER>
struct BlockIn {
  uint32_t S;  // scale byte (HiF4: the 4-byte scale word)
  float so;
  uint32_t words[block_of<FMT>() / 8];
};

template <int FMT, bool OUTER>
__device__ __forceinline__ BlockIn<FMT, OUTER> load_block(const DequantArgs& a, int64_t ra,
                                                          int64_t b) {
  constexpr int B = block_of<FMT>();
  BlockIn<FMT, OUTER> in;
  if constexpr (FMT == kHIF4)
    in.S = *reinterpret_cast<const uint32_t*>(a.scales + ra * (a.W / B * 4) + b * 4);
  else
    in.S = a.scales[ra * (a.W / B) + b];
  // outer scales: the 128-piece of the A-row that holds block b
  in.so = OUTER ? a.ts[ra * (a.W / kOuter) + b * B / kOuter] : 0.0f;
  const uint8_t* cp = a.codes + ra * (a.W / 2) + b * (B / 2);
  if constexpr (B == 16) {
    const uint2 v = *reinterpret_cast<const uint2*>(cp);
    in.words[0] = v.x; in.words[1] = v.y;
  } else {
#pragma unroll
    for (int q = 0; q < B / 32; ++q) {
      const uint4 v = *reinterpret_cast<const uint4*>(cp + 16 * q);
      in.words[4 * q] = v.x; in.words[4 * q + 1] = v.y; in.words[4 * q + 2] = v.z;
      in.words[4 * q + 3] = v.w;
    }
  }
  return in;
}

template <int FMT, bool OUTER, bool INV, typename T>
__device__ __forceinline__ void dequant_block(const DequantArgs& a, float s_t,
                                              const BlockIn<FMT, OUTER>& in, uint32_t* out) {
  constexpr int B = block_of<FMT>();
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const uint32_t S = in.S;
  float d;
  if constexpr (FMT == kHIF4) {
    d = e6m2_decode(S & 0xFFu);  // the block scale; each micro-block's step below
  } else if constexpr (is_mx(FMT)) {
    d = S ? __uint_as_float(S << 23) : 5.877471754111438e-39f;
  } else if constexpr (FMT == kMBS) {
    d = __builtin_ldexpf(in.so, (int)S - 127);  // macro scale times 2^e_b
  } else {
    d = S ? (OUTER ? in.so : s_t) * e4m3_decode(S) : 0.0f;
  }
  const uint32_t (&words)[B / 8] = in.words;
  // (HiF4: every step d * f8 * f4 / 4 is within [2^-38, 2^31] when d != 0)
  const bool fold = INV && d >= 0x1p-100f && d <= 0x1p100f;
  const float dm = fold ? d * 0.25f : d;
#pragma unroll
  for (int h = 0; h < B / 16; ++h) {
    float g[16];
    if constexpr (FMT == kHIF4) {
      // micro-block u = 4h + j/4 of sub-block u/2: step d * f8 * f4 / 4,
      // value k * step (exact: 3-bit k times a 3-bit significand)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int u = 4 * h + q;
        const float f8 = ((S >> (8 + u / 2)) & 1u) ? 1.0f : 0.5f;
        const float f4 = ((S >> (16 + u)) & 1u) ? 1.0f : 0.5f;
        const float step = dm * f8 * f4 * 0.25f;
#pragma unroll
        for (int l = 0; l < 4; ++l) {
          const int j = 4 * q + l;
          const uint32_t c = (words[(h * 16 + j) >> 3] >> (4 * (j & 7))) & 15u;
          const float mag = (float)(c & 7u) * step;
          g[j] = (c & 8u) ? -mag : mag;
        }
      }
    } else if constexpr (FMT == kUFP4) {
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
  const float s_t = (!has_tensor_scale(FMT) || OUTER) ? 0.0f : a.ts[0];
  Walk w;
  w.init((int64_t)blockIdx.x * kThreads + threadIdx.x, a.M);
  if constexpr (AXIS == 2) {
    // BF16 rows with a multiple of 64 blocks per A-row: the 64 lanes of a
    // wave decode 64 consecutive blocks of one A-row (2 KB of output), then
    // trade halves across lanes (ds_bpermute, no LDS memory) so that each of
    // the two 16-byte store instructions writes one contiguous 1 KB: lane l
    // stores half l % 2 of block l / 2, then of block 32 + l / 2.  Every lane
    // of a wave takes the same A-row, so a wave is active or done as a whole.
    static_assert(B == 16 && sizeof(T) == 2, "16-element blocks, BF16 rows");
    const int l = threadIdx.x & 63;
    const int src1 = 4 * (l >> 1), src2 = 4 * (32 + (l >> 1));
    const bool odd = l & 1;
    while (w.major < a.n_major) {
      uint32_t v[8];
      dequant_block<FMT, OUTER, INV, T>(a, s_t, load_block<FMT, OUTER>(a, w.major, w.minor), v);
      uint32_t p[4], q[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t a1 = (uint32_t)__builtin_amdgcn_ds_bpermute(src1, (int)v[k]);
        const uint32_t b1 = (uint32_t)__builtin_amdgcn_ds_bpermute(src1, (int)v[4 + k]);
        const uint32_t a2 = (uint32_t)__builtin_amdgcn_ds_bpermute(src2, (int)v[k]);
        const uint32_t b2 = (uint32_t)__builtin_amdgcn_ds_bpermute(src2, (int)v[4 + k]);
        p[k] = odd ? b1 : a1;
        q[k] = odd ? b2 : a2;
      }
      // the wave's first block is this lane's block minus l
      uint32_t* to = reinterpret_cast<uint32_t*>(out + w.major * a.ld_out + (w.minor - l) * B);
      store16<false>(to + 4 * l, p[0], p[1], p[2], p[3]);
      store16<false>(to + 256 + 4 * l, q[0], q[1], q[2], q[3]);
      w.advance(a.sq, a.sr, a.M);
    }
  } else if constexpr (AXIS == 0 && sizeof(T) == 2) {
    // BF16 rows: 2 bytes per value, a lane's 16-value group is two 16-byte
    // stores (staging measured slower here)
    // (loading the next block ahead measured slower here)
    while (w.major < a.n_major) {
      uint32_t v[B / 2];
      dequant_block<FMT, OUTER, INV, T>(a, s_t, load_block<FMT, OUTER>(a, w.major, w.minor),
                                        v);
      uint32_t* to = reinterpret_cast<uint32_t*>(out + w.major * a.ld_out + w.minor * B);
#pragma unroll
      for (int q = 0; q < B / 8; ++q)
        store16<false>(to + 4 * q, v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
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
    bool have = w.major < a.n_major;
    BlockIn<FMT, OUTER> cur{};
    if (have) cur = load_block<FMT, OUTER>(a, w.major, w.minor);
    for (int64_t base = (int64_t)blockIdx.x * kThreads; base < units;
         base += (int64_t)gridDim.x * kThreads) {
      Walk nw = w;
      nw.advance(a.sq, a.sr, a.M);
      const bool have_next = nw.major < a.n_major;
      BlockIn<FMT, OUTER> nxt{};
      if (have_next) nxt = load_block<FMT, OUTER>(a, nw.major, nw.minor);
      uint32_t v[WORDS];
      uint32_t* to = nullptr;
      if (have) {
        dequant_block<FMT, OUTER, INV, T>(a, s_t, cur, v);
        to = reinterpret_cast<uint32_t*>(out + w.major * a.ld_out + w.minor * B);
      } else {
#pragma unroll
        for (int j = 0; j < WORDS; ++j) v[j] = 0u;
      }
      st.put(v, to);
      __syncthreads();
      st.flush();
      __syncthreads();
      cur = nxt;
      w = nw;
      have = have_next;
    }
  } else {
    // edge strips of the tiled interior: units (block, column), column
    // fastest, offset by (blk0, col0)
    bool have = w.major < a.n_major;
    BlockIn<FMT, OUTER> cur{};
    if (have) cur = load_block<FMT, OUTER>(a, a.col0 + w.minor, a.blk0 + w.major);
    while (have) {
      Walk nw = w;
      nw.advance(a.sq, a.sr, a.M);
      const bool have_next = nw.major < a.n_major;
      BlockIn<FMT, OUTER> nxt{};
      if (have_next) nxt = load_block<FMT, OUTER>(a, a.col0 + nw.minor, a.blk0 + nw.major);
      const int64_t ra = a.col0 + w.minor, b = a.blk0 + w.major;
      constexpr int WORDS = B * (int)sizeof(T) / 4;
      uint32_t v[WORDS];
      dequant_block<FMT, OUTER, INV, T>(a, s_t, cur, v);
#pragma unroll
      for (int j = 0; j < B; ++j) {
        T* p = out + (b * B + j) * a.ld_out + ra;
        if constexpr (sizeof(T) == 2) *p = (T)(v[j / 2] >> (16 * (j & 1)));
        else *p = __uint_as_float(v[j]);
      }
      cur = nxt;
      w = nw;
      have = have_next;
    }
  }
}

// Column axis, interior tiles (the mirror of the quantize column tiles):
// each lane decodes whole blocks of A-rows (columns of x) into LDS in the
// tile's transposed layout, then the workgroup writes the tile out by rows,
// 16 bytes per lane with 8 lanes on one 128-byte row segment.
template <int FMT, bool OUTER, bool INV, typename T>
__global__ __launch_bounds__(kThreads) void dequantize_col_tile_kernel(T* __restrict__ out,
                                                                       DequantArgs a,
                                                                       int64_t n_rt,
                                                                       int64_t n_ct) {
  using Tile = ColTile<T>;
  constexpr int B = block_of<FMT>();
  constexpr int TR = Tile::TR, TC = Tile::TC;
  constexpr int kStores = TR * TC * (int)sizeof(T) / 16 / kThreads;  // 16-byte stores per lane
  constexpr int kUnits = TC * (TR / B) / kThreads;                   // blocks per lane
  constexpr int LPR = TR / B;                // lanes per A-row of a tile
  constexpr int kRowStep = kThreads / LPR;   // A-rows between a lane's units
  constexpr int WORDS = B * (int)sizeof(T) / 4;
  __shared__ __align__(16) uint32_t lds[Tile::kWords];
  const float s_t = (!has_tensor_scale(FMT) || OUTER) ? 0.0f : a.ts[0];
  const int64_t ntile = n_rt * n_ct;
  const int lane_ra = threadIdx.x / LPR, j = threadIdx.x % LPR;
  const int seg = threadIdx.x & 7;
  // (row tile, column tile) walk with a grid stride, no division in the loop
  const int64_t step_r = gridDim.x / n_ct, step_c = gridDim.x - step_r * n_ct;
  int64_t tr = blockIdx.x / n_ct, tc = blockIdx.x - tr * n_ct;
  for (int64_t tile = blockIdx.x; tile < ntile; tile += gridDim.x) {
    const int64_t r0 = tr * TR, c0 = tc * TC;
    BlockIn<FMT, OUTER> in[kUnits];
#pragma unroll
    for (int i = 0; i < kUnits; ++i)
      in[i] = load_block<FMT, OUTER>(a, c0 + lane_ra + kRowStep * i, r0 / B + j);
    __syncthreads();  // the previous tile's rows are read out
    // ---- decode unit i (A-row lane_ra + kRowStep * i, block j) into LDS
#pragma unroll
    for (int i = 0; i < kUnits; ++i) {
      const int cl = lane_ra + kRowStep * i;
      uint32_t v[WORDS];
      dequant_block<FMT, OUTER, INV, T>(a, s_t, in[i], v);
      if constexpr (sizeof(T) == 2) {
        // row pairs j*B/2 .. : whole aligned 4-word groups
#pragma unroll
        for (int q = 0; q < WORDS / 4; ++q)
          *reinterpret_cast<uint4*>(lds + Tile::at(cl, j * B / 2 + 4 * q)) =
              make_uint4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
      } else {
#pragma unroll
        for (int e = 0; e < B; ++e) lds[Tile::at(cl, j * B + e)] = v[e];
      }
    }
    __syncthreads();
    // ---- rows out: 16-byte pieces, 8 lanes per row segment
    T* base = out + r0 * a.ld_out + c0;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int i = 0; i < kStores / 2; ++i) {
        const int pr = (threadIdx.x >> 3) + 32 * i;  // row pair
        uint32_t ev[4], od[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int col = seg * 8 + 2 * k;
          const uint32_t w0 = lds[Tile::at(col, pr)], w1 = lds[Tile::at(col + 1, pr)];
          ev[k] = __builtin_amdgcn_perm(w1, w0, 0x05040100u);  // row 2pr, columns col, col+1
          od[k] = __builtin_amdgcn_perm(w1, w0, 0x07060302u);  // row 2pr + 1
        }
        T* p = base + (int64_t)(2 * pr) * a.ld_out + seg * 8;
        store16<false>(p, ev[0], ev[1], ev[2], ev[3]);
        store16<false>(p + a.ld_out, od[0], od[1], od[2], od[3]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kStores; ++i) {
        const int row = (threadIdx.x >> 3) + 32 * i;
        uint32_t v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = lds[Tile::at(seg * 4 + k, row)];
        store16<false>(base + (int64_t)row * a.ld_out + seg * 4, v[0], v[1], v[2], v[3]);
      }
    }
    tr += step_r;
    tc += step_c;
    if (tc >= n_ct) { tc -= n_ct; tr += 1; }
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

constexpr int64_t kTileGrid = 4096;  // workgroups of the column tiles (cap)

template <int FMT, bool OUTER, bool INV, int AXIS, typename T>
hipError_t launch_dequant_t(const DequantLaunch& q, hipStream_t s) {
  constexpr int B = block_of<FMT>();
  T* out = static_cast<T*>(q.out);
  if (AXIS == 0) {
    const int64_t W = q.cols, nmaj = q.rows, M = W / B;
    const WalkPlan wp = plan_walk(nmaj, M, kMaxGrid);
    DequantArgs a{q.codes, q.scales, q.tensor_scale, q.ld_out, W, nmaj, M, wp.sq, wp.sr,
                  q.signs, 0, 0};
    if constexpr (B == 16 && sizeof(T) == 2) {
      // whole waves on one A-row: 64 | blocks per row (the walk's stride is
      // a multiple of 64 lanes, so every wave starts on a multiple of 64)
      if (FP4_DEQ_WAVE_ROWS && M % 64 == 0) {
        hipLaunchKernelGGL((dequantize_kernel<FMT, OUTER, INV, 2, T>), dim3(wp.grid),
                           dim3(kThreads), 0, s, out, a);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((dequantize_kernel<FMT, OUTER, INV, 0, T>), dim3(wp.grid),
                       dim3(kThreads), 0, s, out, a);
    return hipGetLastError();
  }
  // column axis: whole tiles through LDS (16-byte row stores), the right and
  // bottom strips per element
  using Tile = ColTile<T>;
  const int64_t W = q.rows;
  // (a HiF4 FP32 tile holds fewer blocks than lanes: strips only)
  const bool tiles = (q.ld_out * (int64_t)sizeof(T)) % 16 == 0 && !(FMT == kHIF4 && sizeof(T) == 4);
  const int64_t nrt = tiles ? q.rows / Tile::TR : 0, nct = tiles ? q.cols / Tile::TC : 0;
  const int64_t rows_main = nct > 0 ? nrt * Tile::TR : 0;
  const int64_t cols_main = nrt > 0 ? nct * Tile::TC : 0;
  DequantArgs a{q.codes, q.scales, q.tensor_scale, q.ld_out, W, 0, 0, 0, 0, q.signs, 0, 0};
  if constexpr (!(FMT == kHIF4 && sizeof(T) == 4)) {
    if (rows_main > 0 && cols_main > 0) {
      const int64_t ntile = nrt * nct;
      hipLaunchKernelGGL((dequantize_col_tile_kernel<FMT, OUTER, INV, T>),
                         dim3((unsigned)(ntile < kTileGrid ? ntile : kTileGrid)),
                         dim3(kThreads), 0, s, out, a, nrt, nct);
    }
  }
  auto strip = [&](int64_t blk_begin, int64_t blk_end, int64_t col_begin, int64_t col_end) {
    if (blk_end <= blk_begin || col_end <= col_begin) return;
    DequantArgs e = a;
    e.blk0 = blk_begin;
    e.col0 = col_begin;
    e.n_major = blk_end - blk_begin;
    e.M = col_end - col_begin;
    const WalkPlan wp = plan_walk(e.n_major, e.M, kMaxGrid);
    e.sq = wp.sq;
    e.sr = wp.sr;
    hipLaunchKernelGGL((dequantize_kernel<FMT, OUTER, INV, 1, T>), dim3(wp.grid),
                       dim3(kThreads), 0, s, out, e);
  };
  strip(0, rows_main / B, cols_main, q.cols);    // right of the tiles
  strip(rows_main / B, W / B, 0, q.cols);        // below them
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
  if constexpr (is_mx(FMT) || FMT == kHIF4) return dq_inv<FMT, false>(q, s);
  else if constexpr (FMT == kMBS) return dq_inv<FMT, true>(q, s);  // macro scales only
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
    case kCAP2: return dq_outer<kNVFP4>(q, s);  // E2M1 codes, E4M3 scales: decoded as NVFP4
    case kMBS: return dq_outer<kMBS>(q, s);
    case kMXOAS16: return dq_outer<kMXOAS16>(q, s);
    case kHIF4: return dq_outer<kHIF4>(q, s);
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
