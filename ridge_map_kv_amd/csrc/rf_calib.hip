// One-pass calibration statistics (placeholder until the kernels land).
#include "rf_common.h"
#include "rf_internal.h"

namespace rf {

CalibLayout calib_layout(int d, int n_layers) {
  CalibLayout L;
  L.header = 0;
  L.sum_S = 256;
  L.sum_l = L.sum_S + align256((size_t)d * 8);
  L.G = L.sum_l + align256((size_t)n_layers * d * 8);
  L.YX = L.G + align256((size_t)d * d * 4);
  L.total = L.YX + (size_t)n_layers * d * d * 4;
  return L;
}

hipError_t launch_calib_reset(void*, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_calibrate(void*, int, int, const uint16_t*, const uint16_t* const*, int64_t,
                            hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace rf
