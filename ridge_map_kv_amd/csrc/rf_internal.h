// Internal interface between the C ABI (ridgefill.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rf {

constexpr int kMaxGroup = 32;   // layers sharing one fill launch
constexpr int kMaxFoldGroup = 64;   // layers folded side by side
constexpr int kTile = 256;      // fill/calibration tile edge (rows and features)
constexpr size_t kStatusBytes = 256;
// Device status bits kept in the first word of a fill or solve workspace.
constexpr unsigned kStatusRowsBit = 1u;
constexpr unsigned kStatusNotSpdBit = 2u;
constexpr unsigned kStatusScoreBit = 4u;     // a selection score was NaN
constexpr unsigned kStatusStateBit = 8u;     // the calibration state did not match the sizes

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// One layer of a fill launch.  Plain maps use A, b, w, WK, WV.  A folded layer (kWsFolded)
// puts its unit-diagonal triangular factor R1 [d_in][d_in] in A, r1 [d_in] in b, diag(R)
// [d_in] in fg, the K and V halves of P in WK and WV (rows of d_in), c [2 kv] in fc and
// kappa in kap; w is unused.
struct FillLayerPtrs {
  const uint16_t* A;            // bf16 map (null for an int8 map, which the GEMM reads as codes)
  const float* b;
  const uint16_t* w;
  const uint16_t* WK;
  const uint16_t* WV;
  uint16_t* kp;
  uint16_t* vp;
  const uint16_t* kn;           // per-head key-norm weight [hd] or null
  const float* vs;              // value-rescale factors [n_kv] or null
  const int8_t* Aq;             // int8 map codes or null
  const float* As;              // int8 map row scales
  const float* fc;              // folded: c
  const float* kap;             // folded: kappa
  const float* fg;              // folded: diag(R)
};

// Workspace variants of a fill call.
constexpr unsigned kWsInt8 = 1u;       // int8 maps (codes read by the map GEMM itself)
constexpr unsigned kWsStreamed = 2u;   // host maps: two landing slots per layer
constexpr unsigned kWsFolded = 4u;     // folded layers: no predicted-input buffer

// Folded form of one layer in its caller-owned buffer (byte offsets): P bf16 [2 kv][d_in],
// R1 bf16 [d_in][d_in] (unit upper triangle, zeros below), c fp32 [2 kv], r1 fp32 [d_in],
// g = diag(R) fp32 [d_in], kappa fp32.
struct FoldLayout {
  size_t P, R, c, r, g, kappa, total;
};
FoldLayout fold_layout(int d_in, int kv);

// Workspace of the fold: the status word, then up to kFoldGemmSlots operand slots rebuilt
// for each layer ([A^T | A^T] and [W_hi | W_lo] in bf16), then one block per layer of a
// group folded side by side: A^T A in fp64 (the Cholesky works in place), the
// diagonal-block inverses, A^T b and r in fp64, |b|^2.  Block offsets are from the block's
// start; `total` covers n_par blocks.  An int8 map takes two [A^T | A^T]-sized slots: its
// codes [Aq^T | Aq^T] and [C_hi | C_lo] with C[j][k] = s_k^2 Aq[k][j], so that
// A^T A = Aq^T diag(s^2) Aq is one product over 2 d; its layers then share a launch two at
// a time.
constexpr int kFoldGemmSlots = 4;   // layers whose fold GEMMs share one launch
struct FoldWsLayout {
  int slots;                          // layers per GEMM launch ([W_hi | W_lo] slots)
  int int8;                           // 1: two [A^T | A^T]-sized slots per layer
  size_t At, at_bytes, Wx, wx_bytes, blocks;
  size_t H64, linv, g, r, scal, per_layer;
  size_t total;
};
FoldWsLayout fold_ws_layout(int d, int d_in, int kv, int n_par, bool int8 = false);
// One layer's plain fields: A bf16 [d][d_in] or Aq int8 [d][d_in] with As fp32 [d] (the map
// Aq[o][i] As[o]), b fp32 [d], w bf16 [d], W_K / W_V bf16 [kv][d].
struct FoldLayerIn {
  const uint16_t* A;
  const float* b;
  const uint16_t* w;
  const uint16_t* WK;
  const uint16_t* WV;
  const int8_t* Aq;
  const float* As;
};
// Folds G layers (G <= the n_par of W) into their buffers out[0 .. G-1]: the GEMMs layer by
// layer, then one batched Cholesky and substitution for the G layers.  A non-positive pivot
// of some A^T A sets kStatusNotSpdBit.
hipError_t launch_fold(int d, int d_in, int kv, const FoldLayerIn* layers, int G,
                       void* const* out, void* ws, const FoldWsLayout& W, hipStream_t stream);

// Workspace layout of a fill call (bytes from the start of ws; per-layer offsets from the
// start of that layer's block).
struct FillWsLayout {
  size_t rope_cos, rope_sin, row_slot, hbuf, fixed;
  size_t per_layer_h, per_layer_ssq, per_layer_rstd, land, land_slot, per_layer;
};
FillWsLayout fill_ws_layout(int d, int d_in, int hd, int kv, int64_t n_filled, unsigned flags);

struct FillPlan {
  int d, d_in, n_kv, hd, kv;
  unsigned flags;               // kWsInt8 | kWsStreamed | kWsFolded
  int has_knorm;
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
  FillWsLayout L;
};

hipError_t launch_fill(const FillPlan& plan, const FillLayerPtrs* layers, int n_layers,
                       hipStream_t stream);

// The fixed scratch array of ridgefill_fill_noalloc (in rf_fill.hip): its device address on
// the current device, looked up there on the first call.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_fill_streamed(const FillPlan& plan, const FillLayerPtrs* layers, int n_layers,
                                hipStream_t stream, hipStream_t copy_stream);

// Value-rescale pass: the plan describes c tail rows as its "filled" rows (idx points at
// an int32 [mpad] scratch list the pass fills with 0 .. mpad-1); predicted rows use the
// plan's per-layer blocks, exact rows the blocks at `exact`.
// Value-rescale workspace: status, row indices, value norms [2][group][cpad][n_kv]
// (predicted, then exact rows), a layer-pointer table of 2 group entries, then 2 group
// per-layer blocks (the predicted rows' staged inputs and norms, then the exact rows').
constexpr int kVsMaxGroup = 64;  // layers sharing the value-scale launches
struct VsLayout {
  size_t idx, vn_off, table_off, blocks, total_fixed;
  float* vn;
  FillLayerPtrs* table;
};
// The predicted rows use `layers` (plain or folded, as plan.flags says); the exact rows
// always go through the layers' own W_V, exact_wv[l].
hipError_t launch_value_scale(const FillPlan& plan, const FillLayerPtrs* layers,
                              const uint16_t* const* x_exact, const uint16_t* const* exact_wv,
                              int n_layers, float* out, const VsLayout& V, hipStream_t stream);

// Calibration -------------------------------------------------------------------
// State: header, fp64 sums, fp32 moments of the shifted x_S, the shift, and a scratch area
// where each call stages its shifted x_S rows (bf16, up to kCalibStageRows rows at a time).
struct CalibLayout {
  size_t header, sum_S, sum_l, G, YX, shift, stage, total;
};
CalibLayout calib_layout(int d_in, int d_out, int n_layers);
constexpr uint32_t kCalibMagic = 0x52464332u;   // "RFC2"
constexpr int kCalibStageRows = 16384;
// Header words (int32 index into the 256-byte header).
constexpr int kHdrDOut = 2, kHdrLayers = 3, kHdrMagic = 4, kHdrDIn = 5;
constexpr int kHdrShiftSet = 6;   // 1 once the shift is fixed (by the first call with rows)
constexpr int kHdrBad = 7;        // 1 once a call's sizes disagreed with the reset's
constexpr int kHdrDeciding = 8;   // 1 while the current call computes the shift

hipError_t launch_calib_reset(void* state, int d_in, int d_out, int n_layers, hipStream_t stream);
hipError_t launch_calibrate(void* state, int d_in, int d_out, int n_layers, const uint16_t* xS,
                            const uint16_t* const* xl, int64_t n_rows, hipStream_t stream);

// Solve ---------------------------------------------------------------------------
constexpr int kSolveGroup = 4;   // layers per split-map GEMM launch of the solve
// In a solve workspace: fp64 kappa_F at kSolveInfoOff, then int32 parts.
constexpr int kSolveInfoOff = 32, kSolveInfoBytes = 12;
struct SolveLayout {
  size_t scalars, mu, mut, C, W, M64, Mx, Cx, norms, linv, v, total;
  int group;
};
SolveLayout solve_layout(int d_in, int d_out, int n_layers);
hipError_t launch_solve(const void* state, int d_in, int d_out, int n_layers, double lambda,
                        float* A_out, float* b_out, uint16_t* A_bf16, void* ws,
                        hipStream_t stream);

// Blocked fp64 Cholesky of the lower triangle of C [d][d] (d a multiple of 64), in place:
// C's lower triangle becomes L (C = L L^T) and linv [d/64][64][64] the inverses of L's
// 64 x 64 diagonal blocks.  A non-positive pivot sets kStatusNotSpdBit in *status.  A batch
// of nbatch such matrices is factored side by side: matrix b at C + b sC with its
// inverses at linv + b sL (strides in doubles).  With U (nbatch 1 only) the same launches
// also write U = L^-T [d][d] (upper triangle; U is cleared first).
hipError_t launch_cholesky(double* C, int d, double* linv, unsigned* status, hipStream_t stream,
                           int nbatch, size_t sC, size_t sL, double* U = nullptr);

hipError_t launch_clear_status(unsigned* status, hipStream_t stream);

// Exact-row selection ------------------------------------------------------------
struct SelLayout {
  size_t state, hist, blocks, total;
};
SelLayout select_layout(int64_t P);
hipError_t launch_select(const float* scores, int64_t P, int64_t k, uint8_t* exact,
                         int32_t* filled, void* ws, hipStream_t stream);
hipError_t launch_quantize(const float* A, int64_t rows, int64_t cols, int8_t* q, float* scale,
                           hipStream_t stream);

}  // namespace rf
