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

// Direct global -> LDS loads (the buffer instructions' LDS form): each lane
// of a wave deposits its 16 (or 4) bytes at the wave's LDS base + lane *
// size, so a wave instruction fills 1 KB (256 B) contiguously and no
// staging registers are needed, which leaves room for a three-deep pipeline.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ void buffer_load_lds(i32x4 rsrc, __attribute__((address_space(3))) void* lds,
                                int size, int voffset, int soffset, int offset,
                                int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

// Buffer descriptor (base, byte range, gfx9 data format word), wave-uniform.
__device__ __forceinline__ i32x4 make_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  r.z = __builtin_amdgcn_readfirstlane((int)bytes);
  r.w = 0x00020000;
  return r;
}

constexpr int kStages = 3;                 // K steps in LDS at once
constexpr int kTileBytes = kBM * kRowBytes;  // one operand's codes per step (16 KB)
constexpr int kScaleOff = 2 * kTileBytes;    // then A's and B's scale words
constexpr int kStageSize = kScaleOff + (kBM + kBN) * 4;

// Position of (row, 16-byte segment s) of a step's operand tile: rows of 64
// bytes, segments XOR-swizzled by bits 2-3 of the row, so the 16 lanes of a
// 16-byte fragment-read phase (16 consecutive rows, one segment) reach 16
// distinct 4-bank groups.
__device__ __forceinline__ int tile_at(int row, int s) {
  return row * kRowBytes + ((s ^ ((row >> 2) & 3)) << 4);
}

// One K step of the workgroup's operands into LDS stage `st`: wave w loads
// rows 64w .. 64w + 63 of A and of B (4 instructions each, 16 rows of 64
// bytes per instruction) and the step's scale words of those rows.  Rows
// past M or N read the last row (never stored).
__device__ __forceinline__ void issue_stage(const GemmArgs& g, i32x4 ra, i32x4 rbs, i32x4 rsa,
                                            i32x4 rsb, int64_t m0, int64_t n0, int64_t ks,
                                            uint8_t* st) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t rb = g.K / 2, sb = g.K / 32;
  const int seg_phys = lane & 3;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r0 = wave * 64 + q * 16;       // first row of this instruction
    const int r = r0 + (lane >> 2);
    const int s = seg_phys ^ ((r >> 2) & 3);  // the global segment this lane fetches
    const int va = (int)(min(m0 + r, g.M - 1) * rb + ks * kRowBytes + s * 16);
    const int vb = (int)(min(n0 + r, g.N - 1) * rb + ks * kRowBytes + s * 16);
    buffer_load_lds(ra, (__attribute__((address_space(3))) void*)(st + r0 * kRowBytes), 16, va,
                    0, 0, 0);
    buffer_load_lds(rbs,
                    (__attribute__((address_space(3))) void*)(st + kTileBytes + r0 * kRowBytes),
                    16, vb, 0, 0, 0);
  }
  const int r = wave * 64 + lane;
  const int vsa = (int)(min(m0 + r, g.M - 1) * sb + ks * 4);
  const int vsb = (int)(min(n0 + r, g.N - 1) * sb + ks * 4);
  buffer_load_lds(rsa, (__attribute__((address_space(3))) void*)(st + kScaleOff + wave * 256), 4,
                  vsa, 0, 0, 0);
  buffer_load_lds(rsb,
                  (__attribute__((address_space(3))) void*)(st + kScaleOff + kBM * 4 + wave * 256),
                  4, vsb, 0, 0, 0);
}

__device__ __forceinline__ void store_c(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_c(uint16_t* p, float v) {
  f2 w;
  w.x = v;
  w.y = 0.0f;
  *p = (uint16_t)__builtin_bit_cast(uint32_t, __builtin_convertvector(w, b2));
}

// One K step of a wave from an LDS stage: two sub-steps of 4 x 4 MFMAs of
// 32 x 32 x 64.
__device__ __forceinline__ void mma_step(const uint8_t* st, f32x16 (&acc)[4][4], int wm, int wn,
                                         int fr, int fk) {
  const uint32_t* sca = reinterpret_cast<const uint32_t*>(st + kScaleOff);
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    i32x8 af[4], bf[4];
    int sa[4], sb[4];
    const int kb = sub * 2 + fk;  // the lane's 32-element block within the step
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int ra = wm * 128 + t * 32 + fr, rbw = wn * 128 + t * 32 + fr;
      const u32x4 va = *reinterpret_cast<const u32x4*>(st + tile_at(ra, kb));
      const u32x4 vb = *reinterpret_cast<const u32x4*>(st + kTileBytes + tile_at(rbw, kb));
      af[t] = i32x8{(int)va.x, (int)va.y, (int)va.z, (int)va.w, 0, 0, 0, 0};
      bf[t] = i32x8{(int)vb.x, (int)vb.y, (int)vb.z, (int)vb.w, 0, 0, 0, 0};
      // the instruction reads its scale from byte 0
      sa[t] = (int)((sca[ra] >> (8 * kb)) & 0xFFu);
      sb[t] = (int)((sca[kBM + rbw] >> (8 * kb)) & 0xFFu);
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
// 4 x 4 MFMA tiles of 32 x 32; K steps of 128 in a three-stage LDS ring
// filled by direct loads two steps ahead.
template <typename TC>
__global__ __launch_bounds__(kThreads, 1) void gemm_mx_kernel(GemmArgs g) {
  __shared__ __align__(16) uint8_t lds[kStages * kStageSize];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t tm = blockIdx.x / g.n_tn, tn = blockIdx.x - tm * g.n_tn;
  const int64_t m0 = tm * kBM, n0 = tn * kBN;
  const int64_t nk = g.K / kBK;
  const i32x4 ra = make_rsrc(g.a, (uint32_t)(g.M * (g.K / 2)));
  const i32x4 rbs = make_rsrc(g.b, (uint32_t)(g.N * (g.K / 2)));
  const i32x4 rsa = make_rsrc(g.as, (uint32_t)(g.M * (g.K / 32)));
  const i32x4 rsb = make_rsrc(g.bs, (uint32_t)(g.N * (g.K / 32)));

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  const int fr = lane & 31, fk = lane >> 5;  // fragment row, K block
  issue_stage(g, ra, rbs, rsa, rsb, m0, n0, 0, lds);
  issue_stage(g, ra, rbs, rsa, rsb, m0, n0, min((int64_t)1, nk - 1), lds + kStageSize);
  for (int64_t ks = 0; ks < nk; ++ks) {
    // this wave's loads of step ks are done before the barrier (the
    // compiler waits for all of this wave's outstanding loads here: it
    // cannot tell the stages apart); the barrier makes every wave's share
    // visible and frees the stage read in step ks - 1
    __builtin_amdgcn_s_waitcnt((10 & 0xF) | (0x7 << 4) | (0xF << 8));
    __syncthreads();
    issue_stage(g, ra, rbs, rsa, rsb, m0, n0, min(ks + 2, nk - 1),
                lds + ((ks + 2) % kStages) * kStageSize);
    mma_step(lds + (ks % kStages) * kStageSize, acc, wm, wn, fr, fk);
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
