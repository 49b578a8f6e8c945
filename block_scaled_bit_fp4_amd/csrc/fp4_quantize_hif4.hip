// fp4_quantize_hif4.hip -- quantize kernels and launcher for one format (the
// formats build as separate translation units, in parallel).
#include "fp4_quantize.h"

hipError_t fp4_launch_quantize_hif4(const QuantLaunch& q, hipStream_t s) {
  return quantize_format<kHIF4>(q, s);
}
