// fp4_quantize_mxfp4_mbs.hip -- quantize kernels and launcher for MXFP4 with
// static macro-block scaling (the formats build as separate translation
// units, in parallel).
#include "fp4_quantize.h"

hipError_t fp4_launch_quantize_mxfp4_mbs(const QuantLaunch& q, hipStream_t s) {
  return quantize_format<kMBS>(q, s);
}

hipError_t fp4_launch_quantize_dual_mxfp4_mbs(const DualLaunch& q, hipStream_t s) {
  return quantize_dual_format<kMBS>(q, s);
}
