// Internal interface between the C ABI (ridgefill.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rf {

constexpr int kMaxGroup = 32;   // layers sharing one fill launch
constexpr int kTile = 256;      // fill/calibration tile edge (rows and features)
constexpr size_t kStatusBytes = 256;
// Device status bits kept in the first word of a fill or solve workspace.
constexpr unsigned kStatusRowsBit = 1u;
constexpr unsigned kStatusNotSpdBit = 2u;

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct FillLayerPtrs {
  const uint16_t* A;
  const float* b;
  const uint16_t* w;
  const uint16_t* WK;
  const uint16_t* WV;
  uint16_t* kp;
  uint16_t* vp;
};

struct FillPlan {
  int d, n_kv, hd, kv;
  float eps;
  double theta;
  const uint16_t* xS;
  int64_t x_stride;
  int64_t N, P;                 // prompt rows, prefix rows
  const int32_t* idx;
  int n_filled;
  int mpad;                     // n_filled rounded up to kTile
  const int32_t* block_table;
  int64_t n_logical;
  int page_size, num_pages;
  // workspace carve-up
  unsigned* status;
  float* rope_cos;              // [mpad / 32][hd / 8][32][4]: (row, j) at
  float* rope_sin;              //   ((row / 32) * hd / 8 + j / 4) * 128 + (row % 32) * 4 + j % 4
  int64_t* row_slot;            // [mpad] element offset of the row in a page pool, or -1
  uint16_t* hbuf;               // per layer: [mpad][d] bf16, [d/128][mpad] fp32, [mpad] fp32
  int group;                    // layers per launch
};

// Workspace layout of a fill call (bytes from the start of ws).
struct FillWsLayout {
  size_t rope_cos, rope_sin, row_slot, hbuf, per_layer_h, per_layer_ssq, per_layer_rstd, fixed,
      per_layer;
};
FillWsLayout fill_ws_layout(int d, int hd, int64_t n_filled);

hipError_t launch_fill(const FillPlan& plan, const FillLayerPtrs* layers, int n_layers,
                       hipStream_t stream);

// Calibration -------------------------------------------------------------------
struct CalibLayout {
  size_t header, sum_S, sum_l, G, YX, total;
};
CalibLayout calib_layout(int d, int n_layers);
constexpr uint32_t kCalibMagic = 0x52464331u;   // "RFC1"

hipError_t launch_calib_reset(void* state, int d, int n_layers, hipStream_t stream);
hipError_t launch_calibrate(void* state, int d, int n_layers, const uint16_t* xS,
                            const uint16_t* const* xl, int64_t n_rows, hipStream_t stream);

// Solve ---------------------------------------------------------------------------
struct SolveLayout {
  size_t scalars, mu, C, W, M64, M32, linv, v, total;
};
SolveLayout solve_layout(int d, int n_layers);
hipError_t launch_solve(const void* state, int d, int n_layers, double lambda, float* A_out,
                        float* b_out, uint16_t* A_bf16, void* ws, hipStream_t stream);

hipError_t launch_clear_status(unsigned* status, hipStream_t stream);

}  // namespace rf
