// Ridge solve (placeholder until the kernels land).
#include "rf_common.h"
#include "rf_internal.h"

namespace rf {

SolveLayout solve_layout(int d, int n_layers) {
  SolveLayout L = {};
  L.total = 256 + (size_t)d * d * 8 * 4 + (size_t)(n_layers + 2) * d * 8;
  return L;
}

hipError_t launch_solve(const void*, int, int, double, float*, float*, uint16_t*, void*,
                        hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace rf
