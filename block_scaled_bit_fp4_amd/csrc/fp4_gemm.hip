// fp4_gemm.hip -- GEMM consumer of MXFP4 operands on gfx950 scaled MFMA.
//
// C = A · Bᵀ with A (M x K) and B (N x K) quantized along K (the row axis)
// in MXFP4 (E2M1 codes, one E8M0 scale per 32 elements): exactly the code
// and scale layout fp4_quantize writes for axis ROW, so the forward GEMM of
// a linear layer takes X and W as quantized.  An RHT applied to both
// operands along K cancels in the product (the 16-point transform ¼·H16·D
// is orthogonal), so rotated operands need no inverse here.
//
// The instruction is v_mfma_scale_f32_16x16x128_f8f6f4 with both operands
// FP4: lane l holds 32 codes (16 bytes) of row l % 16 at K block l / 16 and
// that block's E8M0 scale byte; the block scales are applied inside the
// instruction; lane l receives C[(l / 16) * 4 + i][l % 16], i = 0..3
// (layout confirmed by an exhaustive probe against a host model).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4_launch.h"

namespace {

constexpr int kThreads = 256;
constexpr int kBM = 128, kBN = 128;   // workgroup tile of C
constexpr int kBK = 128;              // K elements per step (one MFMA deep)
constexpr int kRowBytes = kBK / 2;    // code bytes of one row per step
constexpr int kPitch = kRowBytes + 16;  // LDS row pitch: 16 lanes' 16-byte
                                        // fragment reads hit distinct banks

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 b2 __attribute__((ext_vector_type(2)));

struct GemmArgs {
  const uint8_t* a;   // [M][K/2] codes
  const uint8_t* as;  // [M][K/32] E8M0 scales
  const uint8_t* b;   // [N][K/2]
  const uint8_t* bs;  // [N][K/32]
  void* c;
  int64_t M, N, K, ldc;
  int64_t n_tn;       // column tiles
};

// One K step of a workgroup's operands, global -> registers: 512 16-byte
// pieces of A and of B (two each per lane) and one 4-byte word of scales
// (the step's 4 blocks) per row of A (lanes 0-127) or B (lanes 128-255).
struct Stage {
  uint4 a[2], b[2];
  uint32_t s;
};

__device__ __forceinline__ Stage load_stage(const GemmArgs& g, int64_t m0, int64_t n0,
                                            int64_t ks) {
  Stage st;
  const int64_t rb = g.K / 2, sb = g.K / 32;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int p = threadIdx.x + kThreads * j;
    const int row = p >> 2, seg = p & 3;
    st.a[j] = *reinterpret_cast<const uint4*>(g.a + (m0 + row) * rb + ks * kRowBytes + seg * 16);
    st.b[j] = *reinterpret_cast<const uint4*>(g.b + (n0 + row) * rb + ks * kRowBytes + seg * 16);
  }
  const int r = threadIdx.x & 127;
  const uint8_t* sp = threadIdx.x < 128 ? g.as + (m0 + r) * sb : g.bs + (n0 + r) * sb;
  st.s = *reinterpret_cast<const uint32_t*>(sp + ks * (kBK / 32));
  return st;
}

__device__ __forceinline__ void store_stage(const Stage& st, uint8_t* la, uint8_t* lb,
                                            uint32_t* lsa, uint32_t* lsb) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int p = threadIdx.x + kThreads * j;
    const int row = p >> 2, seg = p & 3;
    *reinterpret_cast<uint4*>(la + row * kPitch + seg * 16) = st.a[j];
    *reinterpret_cast<uint4*>(lb + row * kPitch + seg * 16) = st.b[j];
  }
  if (threadIdx.x < 128) lsa[threadIdx.x] = st.s;
  else lsb[threadIdx.x - 128] = st.s;
}

__device__ __forceinline__ void store_c(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_c(uint16_t* p, float v) {
  f2 w;
  w.x = v;
  w.y = 0.0f;
  *p = (uint16_t)__builtin_bit_cast(uint32_t, __builtin_convertvector(w, b2));
}

// Workgroup: 4 waves in 2 x 2, each computing a 64 x 64 block of C as 4 x 4
// MFMA tiles; K steps double-buffered through LDS.
template <typename TC>
__global__ __launch_bounds__(kThreads) void gemm_mx_kernel(GemmArgs g) {
  __shared__ __align__(16) uint8_t la[2][kBM * kPitch];
  __shared__ __align__(16) uint8_t lb[2][kBN * kPitch];
  __shared__ uint32_t lsa[2][kBM], lsb[2][kBN];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t tm = blockIdx.x / g.n_tn, tn = blockIdx.x - tm * g.n_tn;
  const int64_t m0 = tm * kBM, n0 = tn * kBN;
  const int64_t nk = g.K / kBK;

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  {
    const Stage st = load_stage(g, m0, n0, 0);
    store_stage(st, la[0], lb[0], lsa[0], lsb[0]);
  }
  __syncthreads();
  const int fr = lane & 15, fk = lane >> 4;  // fragment row, K block
  for (int64_t ks = 0; ks < nk; ++ks) {
    const int buf = (int)(ks & 1);
    const bool more = ks + 1 < nk;
    Stage nxt;
    if (more) nxt = load_stage(g, m0, n0, ks + 1);  // in flight during the MFMAs
    i32x8 af[4], bf[4];
    int sa[4], sb[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int ra = wm * 64 + t * 16 + fr, rbw = wn * 64 + t * 16 + fr;
      const uint4 va = *reinterpret_cast<const uint4*>(&la[buf][ra * kPitch + fk * 16]);
      const uint4 vb = *reinterpret_cast<const uint4*>(&lb[buf][rbw * kPitch + fk * 16]);
      af[t] = i32x8{(int)va.x, (int)va.y, (int)va.z, (int)va.w, 0, 0, 0, 0};
      bf[t] = i32x8{(int)vb.x, (int)vb.y, (int)vb.z, (int)vb.w, 0, 0, 0, 0};
      // the instruction reads its scale from byte 0
      sa[t] = (int)((lsa[buf][ra] >> (8 * fk)) & 0xFFu);
      sb[t] = (int)((lsb[buf][rbw] >> (8 * fk)) & 0xFFu);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bf[j], acc[i][j], 4,
                                                                     4, 0, sa[i], 0, sb[j]);
    if (more) store_stage(nxt, la[buf ^ 1], lb[buf ^ 1], lsa[buf ^ 1], lsb[buf ^ 1]);
    __syncthreads();
  }

  TC* c = static_cast<TC*>(g.c);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t m = m0 + wm * 64 + i * 16 + fk * 4 + e;
        const int64_t n = n0 + wn * 64 + j * 16 + fr;
        store_c(c + m * g.ldc + n, acc[i][j][e]);
      }
}

}  // namespace

hipError_t fp4_launch_gemm_mx(const GemmLaunch& q, hipStream_t s) {
  GemmArgs g{q.a_codes, q.a_scales, q.b_codes, q.b_scales, q.c, q.M, q.N, q.K, q.ldc,
             q.N / kBN};
  const int64_t tiles = (q.M / kBM) * (q.N / kBN);
  if (q.c_dtype == 0)
    hipLaunchKernelGGL(gemm_mx_kernel<uint16_t>, dim3((unsigned)tiles), dim3(kThreads), 0, s, g);
  else
    hipLaunchKernelGGL(gemm_mx_kernel<float>, dim3((unsigned)tiles), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}
