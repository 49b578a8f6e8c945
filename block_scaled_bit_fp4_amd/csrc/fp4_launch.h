// fp4_launch.h -- internal interface between the C-ABI layer and the kernels.
// Arguments here are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Number of per-workgroup partial maxima of the tensor-amax pass; the
// workspace of a two-level quantize in computed-scale mode holds this many
// floats.
constexpr int kAmaxPartials = 1024;
// The single-pass row kernel's exchange: kAmaxPartials slots and one result
// slot of 16 bytes each (two words, each half of a 64-bit call tag above
// the binary32 maximum XOR-ed with the other half).
constexpr int kAmaxSlotBytes = 16;
constexpr size_t kSinglePassWsBytes = (size_t)(kAmaxPartials + 1) * kAmaxSlotBytes;

struct QuantLaunch {
  const void* x;
  int in_dtype;  // 0 bf16, 1 f32
  int64_t rows, cols, ld;
  int format, axis, sr, rht;
  int ts_mode;  // two-level formats: 0 computed, 1 given, 2 outer scales per 128
  uint32_t signs;
  uint32_t sr_k0, sr_k1;
  uint8_t* codes;
  uint8_t* scales;
  float* tensor_scale;
  float* workspace;
  size_t ws_bytes;
  uint64_t call_tag;  // unique per call (single-pass exchange); 0: two-pass only
  uint32_t wait_us;   // single-pass: workgroup 0's wait before it computes what is missing
  int64_t* plan_reads;  // non-null: launch nothing, store the input elements the path reads
};

// Row-axis and column-axis quantization of one BF16 x in one pass
// (16-element-block formats; rows and cols multiples of 128).
struct DualLaunch {
  const void* x;
  int64_t rows, cols, ld;
  int format, sr, rht, ts_mode;
  uint32_t signs;
  uint32_t sr_k0, sr_k1;
  uint8_t* codes_row;
  uint8_t* scales_row;
  float* ts_row;
  uint8_t* codes_col;
  uint8_t* scales_col;
  float* ts_col;
  float* workspace;  // 2 * kAmaxPartials floats (computed tensor scales)
};

struct DequantLaunch {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* tensor_scale;
  int64_t rows, cols;
  int format, axis, inverse_rht;
  int outer;  // tensor_scale holds one outer scale per 128 elements of an A-row
  uint32_t signs;
  void* out;
  int out_dtype;  // 0 bf16, 1 f32
  int64_t ld_out;
};

struct RhtLaunch {
  const void* x;
  int in_dtype;
  int64_t rows, cols, ld;
  int axis, inverse;
  uint32_t signs;
  float* y;
};

// C = A · Bᵀ of MXFP4 operands quantized along K (M, N, K multiples of 128).
struct GemmLaunch {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const uint8_t* b_codes;
  const uint8_t* b_scales;
  int64_t M, N, K;
  void* c;
  int c_dtype;  // 0 bf16, 1 f32
  int64_t ldc;
};

hipError_t fp4_launch_quantize(const QuantLaunch& q, hipStream_t s);
// per-format instantiations (fp4_quantize_<format>.hip)
hipError_t fp4_launch_quantize_nvfp4(const QuantLaunch& q, hipStream_t s);
hipError_t fp4_launch_quantize_mxfp4(const QuantLaunch& q, hipStream_t s);
hipError_t fp4_launch_quantize_ufp4(const QuantLaunch& q, hipStream_t s);
hipError_t fp4_launch_quantize_mxfp4_oas(const QuantLaunch& q, hipStream_t s);
hipError_t fp4_launch_quantize_e2m1_cap2(const QuantLaunch& q, hipStream_t s);
hipError_t fp4_launch_quantize_mxfp4_mbs(const QuantLaunch& q, hipStream_t s);
hipError_t fp4_launch_quantize_mxfp4_oas16(const QuantLaunch& q, hipStream_t s);
hipError_t fp4_launch_quantize_hif4(const QuantLaunch& q, hipStream_t s);
hipError_t fp4_launch_quantize_dual_nvfp4(const DualLaunch& q, hipStream_t s);
hipError_t fp4_launch_quantize_dual_ufp4(const DualLaunch& q, hipStream_t s);
hipError_t fp4_launch_quantize_dual_e2m1_cap2(const DualLaunch& q, hipStream_t s);
hipError_t fp4_launch_quantize_dual_mxfp4_mbs(const DualLaunch& q, hipStream_t s);
hipError_t fp4_launch_dequantize(const DequantLaunch& q, hipStream_t s);
hipError_t fp4_launch_rht(const RhtLaunch& q, hipStream_t s);
hipError_t fp4_launch_gemm_mx(const GemmLaunch& q, hipStream_t s);
hipError_t fp4_launch_write_scalar(float* p, float v, hipStream_t s);
