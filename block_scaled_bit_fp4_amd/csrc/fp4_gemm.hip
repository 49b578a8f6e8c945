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
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
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
  int64_t n_tm, n_tn;  // row and column tiles
  int xcd;             // place tiles by XCD (see tile_of)
  int group_m;         // tile rows per raster group
};

// The C tile of workgroup b.  Workgroups are dealt to the eight XCDs in
// turn (b mod 8), and each XCD has its own L2.  With xcd set, XCD x takes
// a contiguous eighth of the tiles (in dispatch order) instead of every
// eighth tile; within that range tiles run in groups of group_m tile rows,
// column by column, so that the workgroups an XCD runs together share A
// rows and B rows in its L2.  A bijection of [0, tiles).
__device__ __forceinline__ void tile_of(const GemmArgs& g, int64_t b, int64_t& tm, int64_t& tn) {
  const int64_t tiles = g.n_tm * g.n_tn;
  int64_t l = b;
  if (g.xcd) {
    const int64_t full = tiles - tiles % 8;
    if (b < full) l = (b % 8) * (full / 8) + b / 8;
  }
  const int64_t gsize = (int64_t)g.group_m * g.n_tn;
  const int64_t grp = l / gsize, first = grp * g.group_m;
  const int64_t rows = g.n_tm - first < g.group_m ? g.n_tm - first : g.group_m;
  const int64_t in = l - grp * gsize;
  tm = first + in % rows;
  tn = in / rows;
}

// LDS: two stages of codes (A tile then B tile, 256 rows x 64 bytes each)
// and two buffers of scales, each holding a group of 16 K steps: the step's
// E8M0 word (four K blocks) of each row, step-major -- word (step s, row r)
// at s * 1 KB + 4 r, A then B -- so the words a wave reads for one step
// (32 consecutive rows) are consecutive.
constexpr int kTileBytes = kBM * kRowBytes;            // 16 KB
constexpr int kStageBytes = 2 * kTileBytes;            // 32 KB
constexpr int kGroupSteps = 16;                        // K steps per scale group
constexpr int kScaleOpBytes = kGroupSteps * kBM * 4;   // 16 KB per operand
constexpr int kScaleBufBytes = 2 * kScaleOpBytes;      // 32 KB
constexpr int kScaleBase = 2 * kStageBytes;
constexpr int kLdsBytes = kScaleBase + 2 * kScaleBufBytes;  // 128 KB

// Position of (row, 16-byte segment s) of a stage's operand tile: rows of 64
// bytes, segments XOR-swizzled by bits 2-3 of the row, so the 16 lanes of a
// 16-byte fragment-read phase (16 consecutive rows, one segment) and of a
// 16-byte store phase (4 rows, 4 segments) reach 16 distinct 4-bank groups.
__device__ __forceinline__ int tile_at(int row, int s) {
  return row * kRowBytes + ((s ^ ((row >> 2) & 3)) << 4);
}

// Global fetches.  Wave w fetches rows 64w .. 64w + 63 of A and of B, four
// loads each per K step: 16 rows per load, four lanes per row reading the
// row's 64 code bytes in address order (64-byte row pieces are what the L2
// serves at full rate; narrower per-row pieces run several times slower).
// Scales come the same way, 64 bytes per row = a group of 16 steps: group
// g + 1 is fetched as eight loads per wave during steps 16g + 8 .. 16g + 15
// (loads 0-3 for A's rows, 4-7 for B's), into the buffer group g - 1 used.
struct Fetch {
  __amdgpu_buffer_rsrc_t ra, rb, rsa, rsb;
  int code_a[4], code_b[4];  // lane byte offsets of its four rows' codes (step 0)
  int row_a, row_b;          // the lane's first row in A and in B (q = 0)
  int last_a, last_b;        // M - 1, N - 1
  uint32_t sb;               // scale bytes per row, K / 32
};

// Byte offset of the lane's 16-byte scale piece of (clamped) row `row` in
// group `grp`: the row's words of steps 16 grp + 4p .. 16 grp + 4p + 3.
__device__ __forceinline__ uint32_t scale_off(const Fetch& f, int row, int grp) {
  return (uint32_t)row * f.sb + 16u * (threadIdx.x & 3) + (uint32_t)grp * (kGroupSteps * 4);
}

// Step j's code loads of one operand (four per wave); past the last step a
// harmless re-read of it.
__device__ __forceinline__ void fetch_codes(__amdgpu_buffer_rsrc_t r, const int (&off)[4], int j,
                                            int nk, u32x4 (&c)[4]) {
  const int js = min(j, nk - 1);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    c[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off[q] + js * kRowBytes, 0, 0));
}

// The scale piece step j carries (steps 16g + 8 .. 16g + 15 carry group
// g + 1: piece i = j mod 16 - 8, A's rows for i < 4, B's for the rest).
// Pieces past the row's last group read the next row (or nothing, past the
// buffer) into a buffer no step reads.
__device__ __forceinline__ bool has_piece(int j) {
  return (j & (kGroupSteps - 1)) >= kGroupSteps / 2;
}

__device__ __forceinline__ void fetch_scale(const Fetch& f, int j, u32x4& sc) {
  const int i = (j & (kGroupSteps - 1)) - kGroupSteps / 2, q = i & 3;
  const bool is_a = i < 4;
  const int row = is_a ? min(f.row_a + 16 * q, f.last_a) : min(f.row_b + 16 * q, f.last_b);
  sc = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                     is_a ? f.rsa : f.rsb, (int)scale_off(f, row, (j >> 4) + 1), 0, 0));
}

// A scale row piece (16 bytes: the row's words of steps 4p .. 4p + 3 of
// its group) into the group's buffer, operand `op`, row `r`.
__device__ __forceinline__ void store_scale_piece(uint8_t* lds, int group, int op, int r,
                                                  const u32x4& sc) {
  const int p = threadIdx.x & 3;
  uint8_t* base = lds + kScaleBase + (group & 1) * kScaleBufBytes + op * kScaleOpBytes +
                  (4 * p) * (kBM * 4) + r * 4;
  *reinterpret_cast<uint32_t*>(base) = sc.x;
  *reinterpret_cast<uint32_t*>(base + kBM * 4) = sc.y;
  *reinterpret_cast<uint32_t*>(base + 2 * kBM * 4) = sc.z;
  *reinterpret_cast<uint32_t*>(base + 3 * kBM * 4) = sc.w;
}

// Store a fetched step's codes into its LDS stage.
__device__ __forceinline__ void store_codes(uint8_t* lds, int j, const int (&st_off)[4],
                                            const u32x4 (&ca)[4], const u32x4 (&cb)[4]) {
  uint8_t* st = lds + (j & 1) * kStageBytes;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    *reinterpret_cast<u32x4*>(st + st_off[q]) = ca[q];
    *reinterpret_cast<u32x4*>(st + kTileBytes + st_off[q]) = cb[q];
  }
}

// Store step j's scale piece (has_piece(j)) into its group's buffer.
__device__ __forceinline__ void store_scale(uint8_t* lds, int j, const u32x4& sc) {
  const int i = (j & (kGroupSteps - 1)) - kGroupSteps / 2;
  const int r = (threadIdx.x >> 6) * 64 + (i & 3) * 16 + ((threadIdx.x & 63) >> 2);
  store_scale_piece(lds, (j >> 4) + 1, i >> 2, r, sc);
}

__device__ __forceinline__ void store_c(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_c(uint16_t* p, float v) {
  f2 w;
  w.x = v;
  w.y = 0.0f;
  *p = (uint16_t)__builtin_bit_cast(uint32_t, __builtin_convertvector(w, b2));
}

// Fragment reads of one half step (64 of the 128 K elements) for a wave:
// A rows wm * 128 + t * 32 + fr and B rows wn * 128 + t * 32 + fr, t = 0..3,
// 16 bytes each at the lane's segment; `oa` and `ob` are the lane's byte
// offsets of its t = 0 rows (swizzled segment included).
__device__ __forceinline__ void load_frags(const uint8_t* st, int oa, int ob, u32x4 (&a)[4],
                                           u32x4 (&b)[4]) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    a[t] = *reinterpret_cast<const u32x4*>(st + oa + t * 32 * kRowBytes);
    b[t] = *reinterpret_cast<const u32x4*>(st + kTileBytes + ob + t * 32 * kRowBytes);
  }
}

// Step j's scale words of the lane's rows (byte i = K block i of the step).
__device__ __forceinline__ void load_scales(const uint8_t* lds, int j, int ra, int rb,
                                            uint32_t (&wa)[4], uint32_t (&wb)[4]) {
  const uint8_t* plane = lds + kScaleBase + ((j >> 4) & 1) * kScaleBufBytes +
                         (j & (kGroupSteps - 1)) * (kBM * 4);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    wa[t] = *reinterpret_cast<const uint32_t*>(plane + (ra + t * 32) * 4);
    wb[t] = *reinterpret_cast<const uint32_t*>(plane + kScaleOpBytes + (rb + t * 32) * 4);
  }
}

// 4 x 4 MFMAs of 32 x 32 x 64 on one half step; `sh` selects the lane's
// scale byte (its K block) in the step's scale words.
__device__ __forceinline__ void mma_half(const u32x4 (&a)[4], const u32x4 (&b)[4],
                                         const uint32_t (&wa)[4], const uint32_t (&wb)[4], int sh,
                                         f32x16 (&acc)[4][4]) {
  i32x8 af[4], bf[4];
  int sa[4], sb[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    af[t] = i32x8{(int)a[t].x, (int)a[t].y, (int)a[t].z, (int)a[t].w, 0, 0, 0, 0};
    bf[t] = i32x8{(int)b[t].x, (int)b[t].y, (int)b[t].z, (int)b[t].w, 0, 0, 0, 0};
    // the instruction reads its scale from byte 0
    sa[t] = (int)((wa[t] >> sh) & 0xFFu);
    sb[t] = (int)((wb[t] >> sh) & 0xFFu);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], 4, 4, 0,
                                                                  sa[i], 0, sb[j]);
}

// An empty statement that reads one register of every accumulator: the
// half step's MFMAs (pure operations, which instruction selection may
// otherwise sink past the scheduling barrier into the next half step) are
// issued before it.
__device__ __forceinline__ void pin_acc(f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) asm volatile("" ::"a"(acc[i][j][0]));
}

// Interleave a half step's 16 MFMAs with the memory instructions issued
// beside them: `READS` LDS reads and `LOADS` global loads, one after each
// MFMA, loads every other MFMA.  The MFMA stream keeps the matrix pipe busy
// while the reads' latency hides behind it, and the loads trickle into the
// address unit (about 16 clocks per 1 KB wave load) instead of blocking all
// four waves' instruction streams at once.
template <int READS, int LOADS>
__device__ __forceinline__ void interleave_half() {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // one MFMA
    if (i < READS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i < LOADS) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one global load
    if (READS > 8 && i < READS - 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_barrier(0);  // nothing crosses the half-step boundary
}

// One K step ks.  The register set holds step ks + 1, fetched about two
// steps earlier (two sets alternate).  Start: store it to LDS (the stage
// step ks - 1 used, which every wave finished reading before the previous
// barrier) and refill the set's scale piece.  First half: MFMAs on the
// first fragments, while this step's second-half fragments are read and
// A's codes of step ks + 3 are fetched into the set.  One barrier publishes
// step ks + 1.  Second half: MFMAs on the second fragments, while step
// ks + 1's first fragments and scale words are read and B's codes of step
// ks + 3 are fetched.
__device__ __forceinline__ void k_step(const Fetch& f, uint8_t* lds, int ks, int nk,
                                       const int (&st_off)[4], int rowa, int rowb, int oa0,
                                       int ob0, int oa1, int ob1, int sh0, int sh1,
                                       u32x4 (&a0)[4], u32x4 (&b0)[4], u32x4 (&a1)[4],
                                       u32x4 (&b1)[4], uint32_t (&wa)[4], uint32_t (&wb)[4],
                                       u32x4 (&ca)[4], u32x4 (&cb)[4], u32x4& sc,
                                       f32x16 (&acc)[4][4]) {
  const uint8_t* st = lds + (ks & 1) * kStageBytes;
  store_codes(lds, ks + 1, st_off, ca, cb);
  if (has_piece(ks + 1)) store_scale(lds, ks + 1, sc);
  if (has_piece(ks + 3)) fetch_scale(f, ks + 3, sc);
  __builtin_amdgcn_sched_barrier(0);

  load_frags(st, oa1, ob1, a1, b1);
  fetch_codes(f.ra, f.code_a, ks + 3, nk, ca);
  mma_half(a0, b0, wa, wb, sh0, acc);
  pin_acc(acc);
  interleave_half<8, 4>();

  // LDS traffic done (the loads in flight stay in flight), then a plain
  // s_barrier: the workgroup fence of __syncthreads would make the
  // compiler wait for every outstanding load.
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  // the next step's first fragments and scale words (a clamped, unused
  // read after the last step)
  const uint8_t* sn = lds + ((ks + 1) & 1) * kStageBytes;
  uint32_t wan[4], wbn[4];
  load_scales(lds, ks + 1, rowa, rowb, wan, wbn);
  load_frags(sn, oa0, ob0, a0, b0);
  fetch_codes(f.rb, f.code_b, ks + 3, nk, cb);
  mma_half(a1, b1, wa, wb, sh1, acc);
  pin_acc(acc);
  interleave_half<12, 4>();
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    wa[t] = wan[t];
    wb[t] = wbn[t];
  }
}

// Workgroup: 4 waves in 2 x 2, each computing a 128 x 128 block of C as
// 4 x 4 MFMA tiles of 32 x 32; K steps of 128.  Software pipeline per step
// ks: the first half's MFMAs run on fragments read earlier while the second
// half's fragments are read; at mid step the registers fetched for step
// ks + 1 go to LDS (the stage step ks - 1 used), one barrier publishes them,
// step ks + 2 is fetched, and the second half's MFMAs run while step
// ks + 1's first fragments and scale words are read.
template <typename TC>
__global__ __launch_bounds__(kThreads, 1) void gemm_mx_kernel(GemmArgs g) {
  __shared__ __align__(16) uint8_t lds[kLdsBytes];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int64_t tm, tn;
  tile_of(g, blockIdx.x, tm, tn);
  const int64_t m0 = tm * kBM, n0 = tn * kBN;
  const int nk = (int)(g.K / kBK);
  const int64_t rb = g.K / 2, sb = g.K / 32;

  Fetch f;
  f.ra = __builtin_amdgcn_make_buffer_rsrc((void*)g.a, (short)0, (int)(uint32_t)(g.M * rb), 0x00020000);
  f.rb = __builtin_amdgcn_make_buffer_rsrc((void*)g.b, (short)0, (int)(uint32_t)(g.N * rb), 0x00020000);
  f.rsa = __builtin_amdgcn_make_buffer_rsrc((void*)g.as, (short)0, (int)(uint32_t)(g.M * sb), 0x00020000);
  f.rsb = __builtin_amdgcn_make_buffer_rsrc((void*)g.bs, (short)0, (int)(uint32_t)(g.N * sb), 0x00020000);
  int st_off[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = wave * 64 + q * 16 + (lane >> 2), p = lane & 3;
    // rows past M or N read the last row (never stored)
    f.code_a[q] = (int)(min(m0 + r, g.M - 1) * rb) + p * 16;
    f.code_b[q] = (int)(min(n0 + r, g.N - 1) * rb) + p * 16;
    st_off[q] = tile_at(r, p);
  }
  f.row_a = (int)m0 + wave * 64 + (lane >> 2);
  f.row_b = (int)n0 + wave * 64 + (lane >> 2);
  f.last_a = (int)g.M - 1;
  f.last_b = (int)g.N - 1;
  f.sb = (uint32_t)sb;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  const int fr = lane & 31, fk = lane >> 5;  // fragment row, K block
  const int rowa = wm * 128 + fr, rowb = wn * 128 + fr;
  // tile_at() of the lane's t = 0 rows for the two half steps (the swizzle
  // depends on bits 2-3 of the row, which t * 32 does not change)
  const int oa0 = tile_at(rowa, fk), oa1 = tile_at(rowa, 2 + fk);
  const int ob0 = tile_at(rowb, fk), ob1 = tile_at(rowb, 2 + fk);
  const int sh0 = 8 * fk, sh1 = 8 * (2 + fk);

  // Prologue: scale group 0 (all eight pieces) and step 0 stored; steps 1
  // and 2 in flight in the two register sets.
  u32x4 ca0[4], cb0[4], sc0 = {}, ca1[4], cb1[4], sc1 = {};
  {
    u32x4 s0[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      s0[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            f.rsa, (int)scale_off(f, min(f.row_a + 16 * q, f.last_a), 0), 0, 0));
      s0[4 + q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                f.rsb, (int)scale_off(f, min(f.row_b + 16 * q, f.last_b), 0), 0, 0));
    }
    fetch_codes(f.ra, f.code_a, 0, nk, ca0);
    fetch_codes(f.rb, f.code_b, 0, nk, cb0);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      store_scale_piece(lds, 0, i >> 2, wave * 64 + (i & 3) * 16 + (lane >> 2), s0[i]);
    store_codes(lds, 0, st_off, ca0, cb0);
  }
  // steps 0 .. 2 carry no scale piece
  fetch_codes(f.ra, f.code_a, 1, nk, ca1);
  fetch_codes(f.rb, f.code_b, 1, nk, cb1);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // step 0's stores done before set 0 is refilled
  fetch_codes(f.ra, f.code_a, 2, nk, ca0);
  fetch_codes(f.rb, f.code_b, 2, nk, cb0);
  __syncthreads();

  u32x4 a0[4], b0[4], a1[4], b1[4];  // first- and second-half fragments
  uint32_t wa[4], wb[4];             // the step's scale words
  load_scales(lds, 0, rowa, rowb, wa, wb);
  load_frags(lds, oa0, ob0, a0, b0);
  // steps in pairs (step ks stores set 1 = step ks + 1, step ks + 1 set 0),
  // an odd last step after the loop
  int ks = 0;
  for (; ks + 1 < nk; ks += 2) {
    k_step(f, lds, ks, nk, st_off, rowa, rowb, oa0, ob0, oa1, ob1, sh0, sh1, a0, b0, a1, b1, wa,
           wb, ca1, cb1, sc1, acc);
    k_step(f, lds, ks + 1, nk, st_off, rowa, rowb, oa0, ob0, oa1, ob1, sh0, sh1, a0, b0, a1, b1,
           wa, wb, ca0, cb0, sc0, acc);
  }
  if (ks < nk)
    k_step(f, lds, ks, nk, st_off, rowa, rowb, oa0, ob0, oa1, ob1, sh0, sh1, a0, b0, a1, b1, wa,
           wb, ca1, cb1, sc1, acc);
  __builtin_amdgcn_s_waitcnt(0);

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
  // Tiles by XCD in groups of 4 tile rows: L2 fetches of the linear-layer
  // GEMMs measured 25-35% lower than in row-major dispatch order.  Groups of
  // 1, 2, 4, 8, 16 and 32 tile rows, and no XCD placement, measured side by
  // side: 4 is fastest (forward GEMM 561 us against 585 with 8, 627 with
  // 32, 588 without placement).
  GemmArgs g{q.a_codes, q.a_scales, q.b_codes, q.b_scales, q.c, q.M, q.N, q.K, q.ldc, n_tm, n_tn,
             1, 4};
  const int64_t tiles = n_tm * n_tn;
  if (q.c_dtype == 0)
    hipLaunchKernelGGL(gemm_mx_kernel<uint16_t>, dim3((unsigned)tiles), dim3(kThreads), 0, s, g);
  else
    hipLaunchKernelGGL(gemm_mx_kernel<float>, dim3((unsigned)tiles), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}
