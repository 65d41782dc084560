// 256x256 bf16 matrix-core tile shared by the fill and calibration GEMMs (gfx950).
//
// LDS holds each operand as 256 rows of one 64-element (128-byte) reduction slice,
// 16-byte chunks swizzled by lds_off128.  Four waves split the tile 2 x 2; each wave
// owns 128 F-rows x 128 T-rows as 4 x 4 blocks of v_mfma_f32_32x32x16_bf16.  In the
// result block (m, n) lane l holds T-row n*32 + (l & 31) and F-rows
// m*32 + 8*(r/4) + 4*(l/32) + (r%4) in register r.
#pragma once

#include "rf_common.h"

namespace rf {
namespace {

constexpr int BK = 64;                          // reduction slice per LDS stage
constexpr int kThreads = 256;                   // 4 waves: 2 (features) x 2 (tokens)
constexpr int kOperandStage = kTile * BK * 2;   // 32 KB: 256 rows x 64 bf16
constexpr int kStageBytes = 2 * kOperandStage;  // F and T operands
constexpr int kLdsBytes = 2 * kStageBytes;      // double buffered: 128 KB
constexpr int kTokGroup = 4;                    // T tiles walked together in tile order

// One BK slice of the 256x256 tile: each wave multiplies its 128 features x 128 tokens.
__device__ __forceinline__ void mma_slice(f32x16 (&acc)[4][4], const unsigned char* Fs,
                                          const unsigned char* Ts, int wf, int wt, int lane) {
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) {
    const int c = kk * 2 + (lane >> 5);
    bf16x8 a[4], b[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
      a[m] = *reinterpret_cast<const bf16x8*>(Fs + lds_off128(wf * 128 + m * 32 + (lane & 31), c));
#pragma unroll
    for (int n = 0; n < 4; ++n)
      b[n] = *reinterpret_cast<const bf16x8*>(Ts + lds_off128(wt * 128 + n * 32 + (lane & 31), c));
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int n = 0; n < 4; ++n)
        acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m], b[n], acc[m][n], 0, 0, 0);
  }
}

}  // namespace
}  // namespace rf
