// fp4_quantize_e2m1_cap2.hip -- quantize kernels and launcher for the E2M1
// grid cut at 2 (the formats build as separate translation units, in
// parallel).
#include "fp4_quantize.h"

hipError_t fp4_launch_quantize_e2m1_cap2(const QuantLaunch& q, hipStream_t s) {
  return quantize_format<kCAP2>(q, s);
}

hipError_t fp4_launch_quantize_dual_e2m1_cap2(const DualLaunch& q, hipStream_t s) {
  return quantize_dual_format<kCAP2>(q, s);
}
