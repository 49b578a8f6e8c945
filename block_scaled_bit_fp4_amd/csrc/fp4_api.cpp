// fp4_api.cpp -- the C ABI declared in include/fp4.h: host-side validation
// (no HIP call happens before every argument has been checked) and dispatch
// to the gfx950 kernels.
#include <hip/hip_runtime.h>

#include <atomic>
#include <chrono>
#include <cstdint>
#include <cstdlib>
#include <mutex>
#include <random>

#include "fp4.h"
#include "fp4_launch.h"

namespace {

// Host Philox4x32-10 (Salmon et al., SC'11) for the RHT sign mask.
void philox10_host(uint32_t k0, uint32_t k1, uint32_t c[4]) {
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = (uint32_t)p1;
    c[2] = n2;
    c[3] = (uint32_t)p0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

bool debug_sync() {
  static const bool on = [] {
    const char* e = std::getenv("FP4_DEBUG_SYNC");
    return e && e[0] == '1';
  }();
  return on;
}

fp4_status finish(hipError_t e, hipStream_t s) {
  if (e != hipSuccess) return FP4_ERR_DEVICE;
  if (debug_sync()) {
    if (hipStreamSynchronize(s) != hipSuccess) return FP4_ERR_DEVICE;
    if (hipGetLastError() != hipSuccess) return FP4_ERR_DEVICE;
  }
  return FP4_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_size(int32_t dt) { return dt == FP4_BF16 ? 2 : 4; }

bool is_mx(int32_t format) {
  return format == FP4_MXFP4 || format == FP4_MXFP4_OAS || format == FP4_MXFP4_OAS16;
}

// Block size of each format: 16, but 32 for MXFP4 and MXFP4_OAS, 64 for HiF4.
int32_t block_of(int32_t format) {
  if (format == FP4_HIF4) return 64;
  return (format == FP4_MXFP4 || format == FP4_MXFP4_OAS) ? 32 : 16;
}

// Formats with a tensor scale (computed or given) or outer scales; the MX
// formats and HiF4 carry every scale per block.
bool two_level(const fp4_params* p) { return !is_mx(p->format) && p->format != FP4_HIF4; }

bool outer_scales(const fp4_params* p) {
  return two_level(p) && p->ts_mode == FP4_TS_OUTER128;
}

fp4_status check_params(const fp4_params* p) {
  if (!p) return FP4_ERR_NULL;
  if (p->format != FP4_NVFP4 && p->format != FP4_MXFP4 && p->format != FP4_UFP4 &&
      p->format != FP4_MXFP4_OAS && p->format != FP4_E2M1_CAP2 && p->format != FP4_MXFP4_MBS &&
      p->format != FP4_MXFP4_OAS16 && p->format != FP4_HIF4)
    return FP4_ERR_FORMAT;
  if (p->format == FP4_MXFP4_MBS && p->ts_mode != FP4_TS_OUTER128) return FP4_ERR_FORMAT;
  if (p->block != block_of(p->format)) return FP4_ERR_FORMAT;
  if (p->axis != FP4_AXIS_ROW && p->axis != FP4_AXIS_COL) return FP4_ERR_FORMAT;
  if (p->rounding != FP4_RTNE && p->rounding != FP4_SR) return FP4_ERR_FORMAT;
  if (p->rht != 0 && p->rht != 1) return FP4_ERR_FORMAT;
  if (two_level(p) && p->ts_mode != FP4_TS_COMPUTE && p->ts_mode != FP4_TS_GIVEN &&
      p->ts_mode != FP4_TS_OUTER128)
    return FP4_ERR_FORMAT;
  return FP4_OK;
}

fp4_status check_shape(const fp4_params* p, int64_t rows, int64_t cols, int64_t ld) {
  if (rows < 0 || cols < 0 || ld < cols || ld < 0) return FP4_ERR_SHAPE;
  const int64_t W = p->axis == FP4_AXIS_ROW ? cols : rows;
  if (W % p->block) return FP4_ERR_SHAPE;
  if (p->rht && (W % 16)) return FP4_ERR_SHAPE;
  if (outer_scales(p) && (W % 128)) return FP4_ERR_SHAPE;
  return FP4_OK;
}

bool needs_workspace(const fp4_params* p) {
  return two_level(p) && p->ts_mode == FP4_TS_COMPUTE;
}

// Tag of one quantize call: unique within the process (a counter) and,
// from a random start, unlike the tags of other processes that may have
// used the same device memory.  Never 0.
uint64_t next_call_tag() {
  static std::atomic<uint64_t> next{[] {
    uint64_t v = (uint64_t)(uintptr_t)&next;
    try {
      std::random_device rd;  // may throw where no entropy source exists
      v ^= ((uint64_t)rd() << 32) ^ rd();
    } catch (...) {
    }
    v ^= (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count() * 0x9E3779B97F4A7C15ull;
    return v;
  }()};
  uint64_t t;
  while ((t = next.fetch_add(1, std::memory_order_relaxed)) == 0) {
  }
  return t;
}

// Microseconds workgroup 0 of the single-pass row kernel waits for the
// other workgroups' partial maxima before computing the missing ones
// itself: FP4_AMAX_WAIT_US if set (0 makes every wait end at once), else
// 10 us plus the time to read the operand at 2.5 TB/s, several times what
// the loads take when the whole grid is resident (about 6 us for a
// 4096 x 4096 BF16 operand).
uint32_t amax_wait_us(int64_t operand_bytes) {
  const char* e = std::getenv("FP4_AMAX_WAIT_US");
  if (!e || !*e) return 10u + (uint32_t)(operand_bytes / 2500000);
  const long v = std::strtol(e, nullptr, 10);
  return v < 0 ? 0u : (v > 1000000 ? 1000000u : (uint32_t)v);
}

// Every argument check of fp4_quantize but the workspace's.
fp4_status check_quantize_args(const void* x, int32_t in_dtype, int64_t rows, int64_t cols,
                               int64_t ld, const fp4_params* p, const uint8_t* codes,
                               const uint8_t* scales, const float* tensor_scale) {
  fp4_status st = check_params(p);
  if (st != FP4_OK) return st;
  if (in_dtype != FP4_BF16 && in_dtype != FP4_F32) return FP4_ERR_DTYPE;
  if ((st = check_shape(p, rows, cols, ld)) != FP4_OK) return st;
  const bool empty = rows == 0 || cols == 0;
  if (two_level(p) && !tensor_scale) return FP4_ERR_NULL;
  if (!empty) {
    if (!x || !codes || !scales) return FP4_ERR_NULL;
    if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return FP4_ERR_ALIGN;
    if ((ld * (int64_t)elem_size(in_dtype)) % 16) return FP4_ERR_ALIGN;
  }
  return FP4_OK;
}

// The allocation-free entry point's workspace: a fixed array in the
// library's device memory (each device holds its own copy until the process
// ends).  Host code never passes `scratch` itself to a kernel -- on the host
// that name is a stand-in, not a device address -- but the address
// hipGetSymbolAddress returns for the current device, looked up once per
// device on its first call.
static __device__ __align__(256) unsigned char scratch[FP4_NOALLOC_SCRATCH_BYTES];
static_assert(FP4_NOALLOC_SCRATCH_BYTES >= kSinglePassWsBytes,
              "the scratch holds the single-pass exchange records");
static_assert(FP4_NOALLOC_SCRATCH_BYTES >= sizeof(float) * (size_t)kAmaxPartials,
              "the scratch holds the two-pass partial maxima");

void* scratch_address() {
  static std::mutex mu;
  static void* ptr[64] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    ptr[dev] = p;
  }
  return ptr[dev];
}

}  // namespace

extern "C" {

size_t fp4_workspace_bytes(int64_t rows, int64_t cols, const fp4_params* p) {
  (void)rows;
  (void)cols;
  if (check_params(p) != FP4_OK) return 0;
  return needs_workspace(p) ? kSinglePassWsBytes : 0;
}

uint16_t fp4_rht_signs(uint64_t rht_seed) {
  uint32_t c[4] = {0u, 0u, 1u, 0u};
  philox10_host((uint32_t)rht_seed, (uint32_t)(rht_seed >> 32), c);
  return (uint16_t)(c[0] & 0xFFFFu);
}

fp4_status fp4_quantize(const void* x, int32_t in_dtype, int64_t rows, int64_t cols,
                        int64_t ld, const fp4_params* p, uint8_t* codes, uint8_t* scales,
                        float* tensor_scale, void* workspace, size_t ws_bytes,
                        void* stream) {
  fp4_status st = check_quantize_args(x, in_dtype, rows, cols, ld, p, codes, scales,
                                      tensor_scale);
  if (st != FP4_OK) return st;
  const bool empty = rows == 0 || cols == 0;
  if (needs_workspace(p)) {
    if (!workspace) return FP4_ERR_WORKSPACE;
    if (ws_bytes < sizeof(float) * (size_t)kAmaxPartials) return FP4_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FP4_ERR_ALIGN;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (empty) {
    if (needs_workspace(p)) return finish(fp4_launch_write_scalar(tensor_scale, 0.0f, s), s);
    return FP4_OK;
  }
  QuantLaunch q{};
  q.x = x;
  q.in_dtype = in_dtype;
  q.rows = rows;
  q.cols = cols;
  q.ld = ld;
  q.format = p->format;
  q.axis = p->axis;
  q.sr = p->rounding == FP4_SR;
  q.rht = p->rht;
  q.ts_mode = two_level(p) ? p->ts_mode : FP4_TS_COMPUTE;
  q.signs = p->rht ? fp4_rht_signs(p->rht_seed) : 0u;
  q.sr_k0 = (uint32_t)p->sr_seed;
  q.sr_k1 = (uint32_t)(p->sr_seed >> 32);
  q.codes = codes;
  q.scales = scales;
  q.tensor_scale = tensor_scale;
  q.workspace = static_cast<float*>(workspace);
  q.ws_bytes = workspace ? ws_bytes : 0;
  // A launch captured into a graph replays with the tag it was captured
  // with, so a replay would read the previous replay's records as its own:
  // under capture the two-pass path is taken (tag 0 disables the single
  // pass).
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  bool capturing = cap != hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cap) != hipSuccess) {
    (void)hipGetLastError();  // not left for the launch check to report
    capturing = true;
  } else {
    capturing = cap != hipStreamCaptureStatusNone;
  }
  q.call_tag = capturing ? 0 : next_call_tag();
  q.wait_us = amax_wait_us(rows * cols * (int64_t)elem_size(in_dtype));
  return finish(fp4_launch_quantize(q, s), s);
}

fp4_status fp4_quantize_input_bytes(int32_t in_dtype, int64_t rows, int64_t cols, int64_t ld,
                                    const fp4_params* p, size_t ws_bytes, int64_t* bytes) {
  if (!bytes) return FP4_ERR_NULL;
  fp4_status st = check_params(p);
  if (st != FP4_OK) return st;
  if (in_dtype != FP4_BF16 && in_dtype != FP4_F32) return FP4_ERR_DTYPE;
  if ((st = check_shape(p, rows, cols, ld)) != FP4_OK) return st;
  if (needs_workspace(p) && ws_bytes < sizeof(float) * (size_t)kAmaxPartials)
    return FP4_ERR_WORKSPACE;
  *bytes = 0;
  if (rows == 0 || cols == 0) return FP4_OK;
  int64_t elems = 0;
  QuantLaunch q{};
  q.in_dtype = in_dtype;
  q.rows = rows;
  q.cols = cols;
  q.ld = ld;
  q.format = p->format;
  q.axis = p->axis;
  q.sr = p->rounding == FP4_SR;
  q.rht = p->rht;
  q.ts_mode = two_level(p) ? p->ts_mode : FP4_TS_COMPUTE;
  q.ws_bytes = ws_bytes;
  q.call_tag = 1;  // as a call outside graph capture
  q.plan_reads = &elems;
  if (fp4_launch_quantize(q, nullptr) != hipSuccess) return FP4_ERR_DEVICE;
  *bytes = elems * (int64_t)elem_size(in_dtype);
  return FP4_OK;
}

fp4_status fp4_quantize_noalloc(const void* x, int32_t in_dtype, int64_t rows, int64_t cols,
                                int64_t ld, const fp4_params* p, uint8_t* codes,
                                uint8_t* scales, float* tensor_scale, void* stream) {
  fp4_status st = check_quantize_args(x, in_dtype, rows, cols, ld, p, codes, scales,
                                      tensor_scale);
  if (st != FP4_OK) return st;
  const size_t need = fp4_workspace_bytes(rows, cols, p);
  if (need > FP4_NOALLOC_SCRATCH_BYTES) return FP4_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need) {
    ws = scratch_address();
    if (!ws) return FP4_ERR_DEVICE;
  }
  return fp4_quantize(x, in_dtype, rows, cols, ld, p, codes, scales, tensor_scale, ws,
                      ws ? (size_t)FP4_NOALLOC_SCRATCH_BYTES : 0, stream);
}

size_t fp4_workspace_bytes_dual(int64_t rows, int64_t cols, const fp4_params* p) {
  (void)rows;
  (void)cols;
  if (check_params(p) != FP4_OK) return 0;
  if (!needs_workspace(p)) return 0;
  const size_t dual = 2 * sizeof(float) * (size_t)kAmaxPartials;
  return dual > kSinglePassWsBytes ? dual : kSinglePassWsBytes;
}

fp4_status fp4_quantize_dual(const void* x, int32_t in_dtype, int64_t rows, int64_t cols,
                             int64_t ld, const fp4_params* p, uint8_t* codes_row,
                             uint8_t* scales_row, float* ts_row, uint8_t* codes_col,
                             uint8_t* scales_col, float* ts_col, void* workspace,
                             size_t ws_bytes, void* stream) {
  fp4_status st = check_params(p);
  if (st != FP4_OK) return st;
  if (in_dtype != FP4_BF16 && in_dtype != FP4_F32) return FP4_ERR_DTYPE;
  fp4_params pr = *p, pc = *p;
  pr.axis = FP4_AXIS_ROW;
  pc.axis = FP4_AXIS_COL;
  if ((st = check_shape(&pr, rows, cols, ld)) != FP4_OK) return st;
  if ((st = check_shape(&pc, rows, cols, ld)) != FP4_OK) return st;
  const bool empty = rows == 0 || cols == 0;
  if (two_level(p) && (!ts_row || !ts_col)) return FP4_ERR_NULL;
  if (!empty) {
    if (!x || !codes_row || !scales_row || !codes_col || !scales_col) return FP4_ERR_NULL;
    if (!aligned16(x) || !aligned16(codes_row) || !aligned16(scales_row) ||
        !aligned16(codes_col) || !aligned16(scales_col))
      return FP4_ERR_ALIGN;
    if ((ld * (int64_t)elem_size(in_dtype)) % 16) return FP4_ERR_ALIGN;
  }
  if (needs_workspace(p)) {
    if (!workspace) return FP4_ERR_WORKSPACE;
    if (ws_bytes < 2 * sizeof(float) * (size_t)kAmaxPartials) return FP4_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FP4_ERR_ALIGN;
  }
  // fused tiles: BF16, whole 128 x 128 tiles, a tile's byte extent below 2^31
  const bool fused = !empty && in_dtype == FP4_BF16 && two_level(p) && rows % 128 == 0 &&
                     cols % 128 == 0 && ld * 2 * 128 < ((int64_t)1 << 31);
  if (!fused) {
    // the two single-axis calls, one after the other on the stream
    st = fp4_quantize(x, in_dtype, rows, cols, ld, &pr, codes_row, scales_row, ts_row,
                      workspace, ws_bytes, stream);
    if (st != FP4_OK) return st;
    return fp4_quantize(x, in_dtype, rows, cols, ld, &pc, codes_col, scales_col, ts_col,
                        workspace, ws_bytes, stream);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  DualLaunch q{};
  q.x = x;
  q.rows = rows;
  q.cols = cols;
  q.ld = ld;
  q.format = p->format;
  q.sr = p->rounding == FP4_SR;
  q.rht = p->rht;
  q.ts_mode = p->ts_mode;
  q.signs = p->rht ? fp4_rht_signs(p->rht_seed) : 0u;
  q.sr_k0 = (uint32_t)p->sr_seed;
  q.sr_k1 = (uint32_t)(p->sr_seed >> 32);
  q.codes_row = codes_row;
  q.scales_row = scales_row;
  q.ts_row = ts_row;
  q.codes_col = codes_col;
  q.scales_col = scales_col;
  q.ts_col = ts_col;
  q.workspace = static_cast<float*>(workspace);
  const hipError_t e = p->format == FP4_NVFP4        ? fp4_launch_quantize_dual_nvfp4(q, s)
                       : p->format == FP4_UFP4      ? fp4_launch_quantize_dual_ufp4(q, s)
                       : p->format == FP4_E2M1_CAP2 ? fp4_launch_quantize_dual_e2m1_cap2(q, s)
                                                    : fp4_launch_quantize_dual_mxfp4_mbs(q, s);
  return finish(e, s);
}

fp4_status fp4_dequantize(const uint8_t* codes, const uint8_t* scales,
                          const float* tensor_scale, int64_t rows, int64_t cols,
                          const fp4_params* p, int32_t inverse_rht, void* out,
                          int32_t out_dtype, int64_t ld_out, void* stream) {
  fp4_status st = check_params(p);
  if (st != FP4_OK) return st;
  if (out_dtype != FP4_BF16 && out_dtype != FP4_F32) return FP4_ERR_DTYPE;
  if (inverse_rht != 0 && inverse_rht != 1) return FP4_ERR_FORMAT;
  if (inverse_rht && !p->rht) return FP4_ERR_FORMAT;
  if ((st = check_shape(p, rows, cols, ld_out)) != FP4_OK) return st;
  if (rows == 0 || cols == 0) return FP4_OK;
  if (!codes || !scales || !out) return FP4_ERR_NULL;
  if (two_level(p) && !tensor_scale) return FP4_ERR_NULL;
  if (!aligned16(codes) || !aligned16(out)) return FP4_ERR_ALIGN;
  if ((ld_out * (int64_t)elem_size(out_dtype)) % 16) return FP4_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  DequantLaunch q{};
  q.codes = codes;
  q.scales = scales;
  q.tensor_scale = tensor_scale;
  q.rows = rows;
  q.cols = cols;
  q.format = p->format;
  q.axis = p->axis;
  q.inverse_rht = inverse_rht;
  q.outer = outer_scales(p);
  q.signs = p->rht ? fp4_rht_signs(p->rht_seed) : 0u;
  q.out = out;
  q.out_dtype = out_dtype;
  q.ld_out = ld_out;
  return finish(fp4_launch_dequantize(q, s), s);
}

fp4_status fp4_rht(const void* x, int32_t in_dtype, int64_t rows, int64_t cols, int64_t ld,
                   int32_t axis, uint64_t rht_seed, int32_t inverse, float* y, void* stream) {
  if (in_dtype != FP4_BF16 && in_dtype != FP4_F32) return FP4_ERR_DTYPE;
  if (axis != FP4_AXIS_ROW && axis != FP4_AXIS_COL) return FP4_ERR_FORMAT;
  if (inverse != 0 && inverse != 1) return FP4_ERR_FORMAT;
  if (rows < 0 || cols < 0 || ld < cols) return FP4_ERR_SHAPE;
  const int64_t W = axis == FP4_AXIS_ROW ? cols : rows;
  if (W % 16) return FP4_ERR_SHAPE;
  if (rows == 0 || cols == 0) return FP4_OK;
  if (!x || !y) return FP4_ERR_NULL;
  if (!aligned16(x) || !aligned16(y)) return FP4_ERR_ALIGN;
  if ((ld * (int64_t)elem_size(in_dtype)) % 16 || (cols * 4) % 16) return FP4_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  RhtLaunch q{};
  q.x = x;
  q.in_dtype = in_dtype;
  q.rows = rows;
  q.cols = cols;
  q.ld = ld;
  q.axis = axis;
  q.inverse = inverse;
  q.signs = fp4_rht_signs(rht_seed);
  q.y = y;
  return finish(fp4_launch_rht(q, s), s);
}

fp4_status fp4_gemm_mx(const uint8_t* a_codes, const uint8_t* a_scales,
                       const uint8_t* b_codes, const uint8_t* b_scales, int64_t M, int64_t N,
                       int64_t K, void* c, int32_t c_dtype, int64_t ldc, void* stream) {
  if (c_dtype != FP4_BF16 && c_dtype != FP4_F32) return FP4_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 0 || ldc < N) return FP4_ERR_SHAPE;
  if (M % 128 || N % 128 || K % 128 || K == 0) return FP4_ERR_SHAPE;
  // each operand's codes are addressed with 32-bit byte offsets
  if (M * (K / 2) > 0xFFFFFFFFll || N * (K / 2) > 0xFFFFFFFFll) return FP4_ERR_SHAPE;
  if (M == 0 || N == 0) return FP4_OK;
  if (!a_codes || !a_scales || !b_codes || !b_scales || !c) return FP4_ERR_NULL;
  if (!aligned16(a_codes) || !aligned16(b_codes) || !aligned16(c)) return FP4_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(a_scales) | reinterpret_cast<uintptr_t>(b_scales)) % 4)
    return FP4_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  GemmLaunch q{};
  q.a_codes = a_codes;
  q.a_scales = a_scales;
  q.b_codes = b_codes;
  q.b_scales = b_scales;
  q.M = M;
  q.N = N;
  q.K = K;
  q.c = c;
  q.c_dtype = c_dtype;
  q.ldc = ldc;
  return finish(fp4_launch_gemm_mx(q, s), s);
}

}  // extern "C"

hipError_t fp4_launch_quantize(const QuantLaunch& q, hipStream_t s) {
  switch (q.format) {
    case FP4_NVFP4: return fp4_launch_quantize_nvfp4(q, s);
    case FP4_MXFP4: return fp4_launch_quantize_mxfp4(q, s);
    case FP4_UFP4: return fp4_launch_quantize_ufp4(q, s);
    case FP4_E2M1_CAP2: return fp4_launch_quantize_e2m1_cap2(q, s);
    case FP4_MXFP4_MBS: return fp4_launch_quantize_mxfp4_mbs(q, s);
    case FP4_MXFP4_OAS16: return fp4_launch_quantize_mxfp4_oas16(q, s);
    case FP4_HIF4: return fp4_launch_quantize_hif4(q, s);
    default: return fp4_launch_quantize_mxfp4_oas(q, s);
  }
}

extern "C" {

const char* fp4_status_str(fp4_status s) {
  switch (s) {
    case FP4_OK: return "ok";
    case FP4_ERR_NULL: return "a required pointer is NULL";
    case FP4_ERR_FORMAT: return "invalid format, block, axis, rounding or mode";
    case FP4_ERR_SHAPE: return "invalid shape or leading dimension";
    case FP4_ERR_ALIGN: return "pointer or leading dimension not 16-byte aligned";
    case FP4_ERR_DTYPE: return "unknown element type";
    case FP4_ERR_WORKSPACE: return "workspace missing or too small";
    case FP4_ERR_DEVICE: return "HIP launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
