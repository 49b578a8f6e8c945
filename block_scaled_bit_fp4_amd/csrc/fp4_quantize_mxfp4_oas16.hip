// fp4_quantize_mxfp4_oas16.hip -- quantize kernels and launcher for one format (the
// formats build as separate translation units, in parallel).
#include "fp4_quantize.h"

hipError_t fp4_launch_quantize_mxfp4_oas16(const QuantLaunch& q, hipStream_t s) {
  return quantize_format<kMXOAS16>(q, s);
}
