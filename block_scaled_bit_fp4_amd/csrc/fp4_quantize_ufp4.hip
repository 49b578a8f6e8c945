// fp4_quantize_ufp4.hip -- quantize kernels and launcher for one format (the
// formats build as separate translation units, in parallel).
#include "fp4_quantize.h"

hipError_t fp4_launch_quantize_ufp4(const QuantLaunch& q, hipStream_t s) {
  return quantize_format<kUFP4>(q, s);
}

hipError_t fp4_launch_quantize_dual_ufp4(const DualLaunch& q, hipStream_t s) {
  return quantize_dual_format<kUFP4>(q, s);
}
