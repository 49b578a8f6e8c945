// fp4_quantize_nvfp4.hip -- quantize kernels and launcher for one format (the
// formats build as separate translation units, in parallel).
#include "fp4_quantize.h"

hipError_t fp4_launch_quantize_nvfp4(const QuantLaunch& q, hipStream_t s) {
  return quantize_format<kNVFP4>(q, s);
}

hipError_t fp4_launch_quantize_dual_nvfp4(const DualLaunch& q, hipStream_t s) {
  return quantize_dual_format<kNVFP4>(q, s);
}
