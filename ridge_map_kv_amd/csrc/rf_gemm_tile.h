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


// ---------------------------------------------------------------------------------
// Direct-to-LDS pipeline (used by the fill GEMMs).
//
// A stage holds a 32-element (64-byte) reduction slice of both 256-row operands: 32 KB.
// Four stages rotate through 128 KB of LDS; the slice kt + 4 is loaded (global_load_lds,
// one 1 KB block of 16 rows per wave instruction) as soon as every wave has read slice kt,
// so loads run three slices ahead of the MFMAs.  Within a slice, the fragments of the second
// 16-wide half are read while the first half's MFMAs run, and the next slice's first-half
// fragments are read (after the barrier) while the second half's MFMAs run.
//
// The LDS loads are issued from inline assembly: the compiler does not track them, so the
// waits for them are explicit (vmcnt counts 8 loads per stage per thread), and it does not
// place a full vmcnt(0) before every LDS read as it does for loads it cannot tell apart
// from the data being read.
constexpr int kBK2 = 32;                      // bf16 per reduction slice
constexpr int kRow2 = kBK2 * 2;               // 64-byte LDS rows
constexpr int kOp2 = kTile * kRow2;           // 16 KB per operand per stage
constexpr int kStage2 = 2 * kOp2;             // 32 KB per stage
constexpr int kNStage = 4;
constexpr int kLds2 = kNStage * kStage2;      // 128 KB

// Chunk swizzle for 64-byte rows (4 chunks): rows of one parity within an aligned group
// of 8, and rows of one residue mod 4 within an aligned group of 16, get distinct chunk
// positions, so fragment reads are free of bank conflicts for 32 and 64 banks alike.
__device__ __forceinline__ int swz64(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }
__device__ __forceinline__ int lds_off64(int r, int c) { return r * kRow2 + ((c ^ swz64(r)) << 4); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One 16-byte global -> LDS load per lane; lane l lands at lds + 16 l.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

__device__ __forceinline__ void wait_vm_stages(int later) {
  if (later >= 2)
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else if (later == 1)
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// This thread's global row pointers: rows 64 p + 16 wave + (lane >> 2), p = 0..3, of each
// operand, already offset to the 16-byte chunk the lane fetches (its LDS position
// lane & 3 holds logical chunk (lane & 3) ^ swz64(row)).
struct DmaRows {
  const uint16_t* f[4];
  const uint16_t* t[4];
};

__device__ __forceinline__ int dma_row(int p, int wave, int lane) { return 64 * p + 16 * wave + (lane >> 2); }
__device__ __forceinline__ int dma_chunk_elems(int row, int lane) { return (((lane & 3) ^ swz64(row)) * 8); }

__device__ __forceinline__ void issue_stage(const DmaRows& rs, int k0, uint32_t stage, int wave) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int j = p * 4 + wave;               // 1 KB block = rows 16 j .. 16 j + 15
    dma16(rs.f[p] + k0, stage + j * 1024);
    dma16(rs.t[p] + k0, stage + kOp2 + j * 1024);
  }
}

__device__ __forceinline__ void read_frags(bf16x8 (&a)[4], bf16x8 (&b)[4], const unsigned char* st,
                                           int half, int wf, int wt, int lane) {
  const int c = half * 2 + (lane >> 5);
#pragma unroll
  for (int m = 0; m < 4; ++m)
    a[m] = *reinterpret_cast<const bf16x8*>(st + lds_off64(wf * 128 + m * 32 + (lane & 31), c));
#pragma unroll
  for (int n = 0; n < 4; ++n)
    b[n] = *reinterpret_cast<const bf16x8*>(st + kOp2 + lds_off64(wt * 128 + n * 32 + (lane & 31), c));
}

__device__ __forceinline__ void mma16(f32x16 (&acc)[4][4], const bf16x8 (&a)[4], const bf16x8 (&b)[4]) {
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n)
      acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m], b[n], acc[m][n], 0, 0, 0);
}

// acc = F[256 x K] * T[256 x K]^T with the pipeline above; K a multiple of 32.  Leaves LDS
// free for the epilogue (ends with a barrier).
__device__ __forceinline__ void gemm_pipeline(f32x16 (&acc)[4][4], const DmaRows& rs, int K,
                                              unsigned char* smem) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wf = wave >> 1, wt = wave & 1;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[m][n][r] = 0.f;

  const int nk = K / kBK2;
  const uint32_t base = lds_addr(smem);
  const int pro = nk < kNStage ? nk : kNStage;
  for (int s = 0; s < pro; ++s) issue_stage(rs, s * kBK2, base + s * kStage2, wave);
  wait_vm_stages(pro - 1);
  __syncthreads();
  bf16x8 a0[4], b0[4], a1[4], b1[4];
  read_frags(a0, b0, smem, 0, wf, wt, lane);
  // all slices but the last: the last one has no successor to wait for or prefetch, and is
  // peeled so the loop body has a single path (no conservative waits at a merge point)
  // sched_barrier(0) keeps each batch of fragment reads ahead of the 16 MFMAs that hide it
  for (int kt = 0; kt < nk - 1; ++kt) {
    const unsigned char* cur = smem + (kt % kNStage) * kStage2;
    read_frags(a1, b1, cur, 1, wf, wt, lane);
    __builtin_amdgcn_sched_barrier(0);
    mma16(acc, a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    const int issued = (nk < kt + kNStage) ? nk : kt + kNStage;
    wait_vm_stages(issued - (kt + 2));
    __syncthreads();                         // slice kt + 1 landed; slice kt fully read
    if (kt + kNStage < nk)
      issue_stage(rs, (kt + kNStage) * kBK2, base + (kt % kNStage) * kStage2, wave);
    read_frags(a0, b0, smem + ((kt + 1) % kNStage) * kStage2, 0, wf, wt, lane);
    __builtin_amdgcn_sched_barrier(0);
    mma16(acc, a1, b1);
    __builtin_amdgcn_sched_barrier(0);
  }
  read_frags(a1, b1, smem + ((nk - 1) % kNStage) * kStage2, 1, wf, wt, lane);
  mma16(acc, a0, b0);
  mma16(acc, a1, b1);
  __syncthreads();
}

}  // namespace
}  // namespace rf
