// fp4_gemm.hip -- GEMM consumer of MXFP4 operands on gfx950 scaled MFMA.
//
// C = A · Bᵀ with A (M x K) and B (N x K) quantized along K (the row axis)
// in MXFP4 (E2M1 codes, one E8M0 scale per 32 elements): exactly the code
// and scale layout fp4_quantize writes for axis ROW, so the forward GEMM of
// a linear layer takes X and W as quantized.  An RHT applied to both
// operands along K cancels in the product (the 16-point transform ¼·H16·D
// is orthogonal), so rotated operands need no inverse here.
//
// The instruction is v_mfma_scale_f32_32x32x64_f8f6f4 with both operands
// FP4: lane l holds 32 codes (16 bytes) of row l % 32 at K block l / 32 and
// that block's E8M0 scale byte; the block scales are applied inside the
// instruction; lane l receives C[(i / 4) * 8 + (l / 32) * 4 + i % 4][l % 32],
// i = 0..15 (layout confirmed by a probe against a host model).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4_launch.h"

namespace {

constexpr int kThreads = 256;
constexpr int kBM = 256, kBN = 256;  // workgroup tile of C (4 waves of 128 x 128)
constexpr int kBK = 128;             // K elements per step: two MFMAs deep
constexpr int kRowBytes = kBK / 2;   // code bytes of one row per step
constexpr int kPitch = kRowBytes + 16;  // LDS row pitch: the 16 lanes of a
                                        // 16-byte read phase hit distinct banks
constexpr int kStageBytes = (kBM + kBN) * kPitch;

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
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

// One K step of a workgroup's operands, global -> registers: 1024 16-byte
// row pieces of A and of B (four each per lane), and the step's four scale
// bytes of one row of A and one of B per lane.  Native vector types (not
// HIP's uint4 wrapper), so they stay in registers.
struct Stage {
  u32x4 a[4], b[4];
  uint32_t sa, sb;
};

__device__ __forceinline__ void load_stage(const GemmArgs& g, int64_t m0, int64_t n0,
                                           int64_t ks, Stage& st) {
  // rows past M or N (the last tile when M or N is an odd multiple of 128)
  // read the last row instead; their results are not stored
  const int64_t rb = g.K / 2, sb = g.K / 32;
  const int seg = threadIdx.x & 3;
  const int64_t off = ks * kRowBytes + seg * 16;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = (threadIdx.x >> 2) + 64 * j;
    st.a[j] = *reinterpret_cast<const u32x4*>(g.a + min(m0 + row, g.M - 1) * rb + off);
    st.b[j] = *reinterpret_cast<const u32x4*>(g.b + min(n0 + row, g.N - 1) * rb + off);
  }
  const int64_t ra = min(m0 + (int64_t)threadIdx.x, g.M - 1);
  const int64_t rbw = min(n0 + (int64_t)threadIdx.x, g.N - 1);
  st.sa = *reinterpret_cast<const uint32_t*>(g.as + ra * sb + ks * 4);
  st.sb = *reinterpret_cast<const uint32_t*>(g.bs + rbw * sb + ks * 4);
}

// LDS stage: A rows [0, 256), then B rows, kPitch bytes each; then the
// scale words of A and of B (the step's four blocks of a row).
__device__ __forceinline__ void store_stage(const Stage& st, uint8_t* lds, uint32_t* lsc) {
  const int seg = threadIdx.x & 3;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = (threadIdx.x >> 2) + 64 * j;
    *reinterpret_cast<u32x4*>(lds + row * kPitch + seg * 16) = st.a[j];
    *reinterpret_cast<u32x4*>(lds + (kBM + row) * kPitch + seg * 16) = st.b[j];
  }
  lsc[threadIdx.x] = st.sa;
  lsc[kBM + threadIdx.x] = st.sb;
}

__device__ __forceinline__ void store_c(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_c(uint16_t* p, float v) {
  f2 w;
  w.x = v;
  w.y = 0.0f;
  *p = (uint16_t)__builtin_bit_cast(uint32_t, __builtin_convertvector(w, b2));
}

// One K step of a wave from an LDS buffer: two sub-steps of 4 x 4 MFMAs of
// 32 x 32 x 64.
__device__ __forceinline__ void mma_step(const uint8_t* lds, const uint32_t* lsc,
                                         f32x16 (&acc)[4][4], int wm, int wn, int fr, int fk) {
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    i32x8 af[4], bf[4];
    int sa[4], sb[4];
    const int kb = sub * 2 + fk;  // the lane's 32-element block within the step
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int ra = wm * 128 + t * 32 + fr, rbw = wn * 128 + t * 32 + fr;
      const u32x4 va = *reinterpret_cast<const u32x4*>(lds + ra * kPitch + kb * 16);
      const u32x4 vb = *reinterpret_cast<const u32x4*>(lds + (kBM + rbw) * kPitch + kb * 16);
      af[t] = i32x8{(int)va.x, (int)va.y, (int)va.z, (int)va.w, 0, 0, 0, 0};
      bf[t] = i32x8{(int)vb.x, (int)vb.y, (int)vb.z, (int)vb.w, 0, 0, 0, 0};
      // the instruction reads its scale from byte 0
      sa[t] = (int)((lsc[ra] >> (8 * kb)) & 0xFFu);
      sb[t] = (int)((lsc[kBM + rbw] >> (8 * kb)) & 0xFFu);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], 4,
                                                                    4, 0, sa[i], 0, sb[j]);
  }
}

// Workgroup: 4 waves in 2 x 2, each computing a 128 x 128 block of C as
// 4 x 4 MFMA tiles of 32 x 32; K steps double-buffered through LDS, the
// next step's global loads in flight during the current step's MFMAs.
template <typename TC>
__global__ __launch_bounds__(kThreads, 1) void gemm_mx_kernel(GemmArgs g) {
  __shared__ __align__(16) uint8_t lds[2][kStageBytes];
  __shared__ uint32_t lsc[2][kBM + kBN];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t tm = blockIdx.x / g.n_tn, tn = blockIdx.x - tm * g.n_tn;
  const int64_t m0 = tm * kBM, n0 = tn * kBN;
  const int64_t nk = g.K / kBK;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  const int fr = lane & 31, fk = lane >> 5;  // fragment row, K block
  // The next step's global loads fly during this step's MFMAs (the last
  // step reloads itself into the idle buffer: in bounds, never used).
  Stage st;
  load_stage(g, m0, n0, 0, st);
  store_stage(st, lds[0], lsc[0]);
  __syncthreads();
  for (int64_t ks = 0; ks < nk; ++ks) {
    const int buf = (int)(ks & 1);
    load_stage(g, m0, n0, min(ks + 1, nk - 1), st);
    mma_step(lds[buf], lsc[buf], acc, wm, wn, fr, fk);
    store_stage(st, lds[buf ^ 1], lsc[buf ^ 1]);
    __syncthreads();
  }

  // M and N are multiples of 128, so a wave's 128 x 128 block lies wholly
  // inside C or wholly past its edge
  if (m0 + wm * 128 >= g.M || n0 + wn * 128 >= g.N) return;
  TC* c = static_cast<TC*>(g.c) + (m0 + wm * 128 + fk * 4) * g.ldc + n0 + wn * 128 + fr;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        store_c(c + (int64_t)(i * 32 + (e / 4) * 8 + e % 4) * g.ldc + j * 32, acc[i][j][e]);
}

}  // namespace

hipError_t fp4_launch_gemm_mx(const GemmLaunch& q, hipStream_t s) {
  const int64_t n_tm = (q.M + kBM - 1) / kBM, n_tn = (q.N + kBN - 1) / kBN;
  GemmArgs g{q.a_codes, q.a_scales, q.b_codes, q.b_scales, q.c, q.M, q.N, q.K, q.ldc, n_tn};
  const int64_t tiles = n_tm * n_tn;
  if (q.c_dtype == 0)
    hipLaunchKernelGGL(gemm_mx_kernel<uint16_t>, dim3((unsigned)tiles), dim3(kThreads), 0, s, g);
  else
    hipLaunchKernelGGL(gemm_mx_kernel<float>, dim3((unsigned)tiles), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}
