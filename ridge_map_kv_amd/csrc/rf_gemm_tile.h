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
// A stage holds a 64-element (128-byte) reduction slice of both 256-row operands: 64 KB;
// two stages fill 128 KB of LDS.  Each wave instruction global_load_lds_dwordx4 moves one
// 1 KB block (8 rows x 128 bytes) straight from memory into LDS.  Slice kt + 2 is loaded
// while slice kt + 1 is multiplied (one slice of ~2048 MFMA cycles ahead suffices), with a
// single barrier per slice.  Every load and every fragment read is issued between two
// MFMAs: a wave issues in order, and these instructions then go out in the shadow of an
// MFMA that is executing, instead of holding up the next one.
//
// The LDS loads are issued from inline assembly: the compiler does not track them, so the
// waits for them are explicit, and it does not place a full vmcnt(0) in front of every
// LDS read as it does for LDS loads it cannot tell apart from the data being read.
constexpr int kPipeBK = 64;                   // bf16 per reduction slice
constexpr int kPipeOp = kTile * 128;          // 32 KB per operand per stage
constexpr int kPipeStage = 2 * kPipeOp;       // 64 KB per stage
constexpr int kPipeLds = 2 * kPipeStage;      // 128 KB

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One 16-byte load per lane from sbase + voff (sbase wave-uniform); lane l lands at
// lds + 16 l.  The LDS destination goes through M0.  A scalar write of M0 followed by an
// LDS DMA needs one wait state on this architecture family, which the compiler cannot
// insert inside an asm string: the s_nop provides it.  M0 is declared clobbered, so the
// compiler keeps none of its own values there across the load (none of the kernels built
// on this helper uses M0 otherwise: their gfx950 assembly is the same with and without the
// clobber).
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}

// This lane's index in its wave, read from the hardware's lane counters in a way the
// compiler cannot trace back to the work-item id: a value derived from that id, used in every
// iteration of a persistent loop, keeps the id itself live across the loop's main loops,
// where it is spilled, and its reload at a tile's first slice waits for every slice load in
// flight.
__device__ __forceinline__ int lane_id_opaque() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// Block j = 4 p + wave (p = 0..7) of an operand stage: LDS rows 8 j .. 8 j + 7.  Lane l
// lands on row 8 j + (l >> 3) at chunk position l & 7, which holds logical chunk
// (l & 7) ^ swz(row).  base[p]: wave-uniform byte pointer, off[p]: this lane's byte offset
// from it (row and chunk), both for reduction index 0.
struct DmaOperand {
  const unsigned char* base[8];
  uint32_t off[8];
};

__device__ __forceinline__ int dma_block_row(int p, int wave) { return 8 * (4 * p + wave); }
__device__ __forceinline__ int dma_lane_row(int lane) { return lane >> 3; }
__device__ __forceinline__ int dma_chunk_elems(int row, int lane) { return ((lane & 7) ^ swz(row)) * 8; }

__device__ __forceinline__ void dma_block(const DmaOperand& o, int p, int kbytes, uint32_t lds_op,
                                          int wave) {
  dma16(o.base[p] + kbytes, o.off[p], lds_op + (4 * p + wave) * 1024);
}

// ---- int8 F operand (FQ = 1): maps stored as int8 codes are read as they are and turned
// into bf16 numbers between LDS and the MFMA (|q| <= 127 is exact in bf16).  A stage's F
// operand is then 256 rows of 64 bytes (16 KB); 1 KB DMA block j holds rows 16 j .. 16 j + 15,
// lane l of the block landing on row 16 j + (l >> 2) at 16-byte position l & 3, which holds
// logical chunk (l & 3) ^ ((l >> 4) & 3), i.e. chunk q of row r sits at q ^ ((r >> 2) & 3).
// One 16-wide step reads chunk s of each row, 8 bytes per lane: the 32 rows of a half-wave
// then spread over all 16 (row & 3, position) bank groups twice, the least a 64-byte row
// pitch allows.
__device__ __forceinline__ int i8_off(int r, int q) {
  return (r >> 4) * 1024 + ((r & 15) * 4 + (q ^ ((r >> 2) & 3))) * 16;
}

// Eight int8 codes -> eight bf16 numbers (exact).
__device__ __forceinline__ bf16x8 i8_to_bf16x8(u32x2 q) {
  u32x4 o;
  o.x = pack_bf16x2((float)(int8_t)(q.x & 0xff), (float)(int8_t)((q.x >> 8) & 0xff));
  o.y = pack_bf16x2((float)(int8_t)((q.x >> 16) & 0xff), (float)(int8_t)(q.x >> 24));
  o.z = pack_bf16x2((float)(int8_t)(q.y & 0xff), (float)(int8_t)((q.y >> 8) & 0xff));
  o.w = pack_bf16x2((float)(int8_t)((q.y >> 16) & 0xff), (float)(int8_t)(q.y >> 24));
  return __builtin_bit_cast(bf16x8, o);
}

// Per-lane LDS offsets of the fragment reads.  Row R0 + (lane & 31) (R0 a multiple of 32)
// at chunk c = 2 s + (lane >> 5) sits at R0 * 128 + (lane & 31) * 128 + ((c ^ swz) << 4)
// with swz = (lane & 7) ^ ((lane >> 3) & 3) ^ 4 ((R0 / 32) & 1) -- lds_off128 written out:
// eight per-lane values, for the four 16-wide steps of a slice and the parity of the 32-row
// block, computed once per tile; a read then adds the block's R0 * 128 as an immediate.
// (A loop probe of the fill's operands: 1,317-1,325 against 1,300-1,305 TFLOP/s with the
// offsets computed per read, and 20 fewer registers.)
struct FragOff {
  uint32_t o[4][2];
  uint32_t a[4];        // TRI: this wave half's F-read offsets, o[s][wf] + 4096 wf
};
__device__ __forceinline__ FragOff frag_off(int lane) {
  FragOff f;
  const uint32_t lrow = (lane & 31) * 128;
  const int sw = (lane & 7) ^ ((lane >> 3) & 3);
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int q = 0; q < 2; ++q) f.o[s][q] = lrow + ((((2 * s + (lane >> 5)) ^ sw ^ (4 * q)) & 7) << 4);
  return f;
}

// TRI: the F blocks of wave half wf are 2 m + wf, of parity wf: o[s][wf] = o[s][0] ^ 64 wf (the
// chunk term's bit 2), plus the block's odd 4096 bytes.
__device__ __forceinline__ void frag_off_tri(FragOff& f, int wf) {
#pragma unroll
  for (int s = 0; s < 4; ++s) f.a[s] = (f.o[s][0] ^ (64u * wf)) + 4096u * wf;
}

// Fragment i (0..3: F rows, 4..7: T rows) of 16-wide step s of a stage.  TRI: wave half wf
// owns the F blocks 2 m + wf (m = 0..3) instead of 4 wf + m, rows interleaved by 32.
template <int FQ = 0, bool TRI = false>
__device__ __forceinline__ void read_frag(bf16x8 (&a)[4], bf16x8 (&b)[4], const unsigned char* st,
                                          int i, int s, int wf, int wt, int lane, const FragOff& fo) {
  // Read order a0 b0 b1 b2 b3 a1 a2 a3: the next step's MFMAs (m-major: a0 with b0..b3,
  // then a1 ...) need the reads in this order, so each MFMA waits on a read issued at least
  // five slots before it, instead of the first four MFMAs waiting on the last four reads.
  i = i == 0 ? 0 : i <= 4 ? i + 3 : i - 4;
  if (TRI && i < 4) {
    a[i] = *reinterpret_cast<const bf16x8*>(st + fo.a[s] + 2 * i * 4096);
  } else if (i < 4) {
    const int blk = wf * 4 + i;
    if (FQ)
      a[i] = i8_to_bf16x8(*reinterpret_cast<const u32x2*>(st + i8_off(blk * 32 + (lane & 31), s) +
                                                           (lane >> 5) * 8));
    else
      a[i] = *reinterpret_cast<const bf16x8*>(st + fo.o[s][blk & 1] + blk * 4096);
  } else {
    const int blk = wt * 4 + (i - 4);
    b[i - 4] = *reinterpret_cast<const bf16x8*>(st + kPipeOp + fo.o[s][blk & 1] + blk * 4096);
  }
}

__device__ __forceinline__ void mfma_i(f32x16 (&acc)[4][4], const bf16x8 (&a)[4], const bf16x8 (&b)[4],
                                       int i) {
  acc[i >> 2][i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i >> 2], b[i & 3], acc[i >> 2][i & 3], 0, 0, 0);
}

// Load issue j of a slice.  bf16 F (16 issues): even j -> F block j / 2, odd j -> T block
// j / 2.  int8 F (12 issues, F blocks hold 16 rows and advance half as many bytes per slice):
// j % 3 == 2 -> F block j / 3, else T block 2 (j / 3) + j % 3.
template <int FQ = 0>
__device__ __forceinline__ void dma_issue(const DmaOperand& F, const DmaOperand& T, int j, int kb,
                                          uint32_t dst, int wave) {
  if (FQ) {
    if (j % 3 == 2)
      dma_block(F, j / 3, kb >> 1, dst, wave);
    else
      dma_block(T, 2 * (j / 3) + j % 3, kb, dst + kPipeOp, wave);
  } else if (j & 1) {
    dma_block(T, j >> 1, kb, dst + kPipeOp, wave);
  } else {
    dma_block(F, j >> 1, kb, dst, wave);
  }
}
template <int FQ> constexpr int kIssues = FQ ? 12 : 16;   // load issues per wave and slice

// 16 MFMAs on (a, b); after each of the first 8, one fragment of step s of stage st is
// read into (na, nb).  With `dma`, the second half of the slice's load issues (j0 onwards)
// at byte offset kb go out after the even-numbered MFMAs, into the stage at LDS address dst.
// MACT < 4: only the MFMAs of F blocks m < MACT are issued (the others would multiply zeros).
template <int FQ = 0, bool TRI = false, int MACT = 4>
__device__ __forceinline__ void mfma16_read(f32x16 (&acc)[4][4], const bf16x8 (&a)[4],
                                            const bf16x8 (&b)[4], bf16x8 (&na)[4], bf16x8 (&nb)[4],
                                            const unsigned char* st, int s, int wf, int wt, int lane,
                                            const FragOff& fo, bool dma, const DmaOperand& F,
                                            const DmaOperand& T, int kb, uint32_t dst, int j0,
                                            int wave) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if ((i >> 2) < MACT) mfma_i(acc, a, b, i);
    if (dma && !(i & 1) && (i >> 1) < kIssues<FQ> / 2) dma_issue<FQ>(F, T, j0 + (i >> 1), kb, dst, wave);
    if (i < 8) read_frag<FQ, TRI>(na, nb, st, i, s, wf, wt, lane, fo);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// acc = F[256 x K] * T[256 x K]^T, K a multiple of 64, in two parts: gemm_prologue issues
// the first loads, gemm_mainloop does the rest and ends with a barrier, leaving the 128 KB
// of LDS to the epilogue.  With REV the slices are taken from the last to the first: the
// operands' base pointers then point at the last slice (reduction index K - 64), and each
// further slice lies 128 bytes before the previous one.
//
// Two 64 KB stages.  The 16 load issues per wave that refill a stage are split: the first 8
// follow the barrier that frees the stage (one after every other MFMA of the last 16-wide
// step), the other 8 go out during the first step of the next slice, so the CU's address
// unit never has all 64 of a slice queued inside one 16-MFMA window.
//
// gemm_prologue: the loads of slices 0 and 1 (32 per wave), into the two stages.  The LDS
// must be free of readers (after a barrier).
template <bool REV = false, int FQ = 0>
__device__ __forceinline__ void gemm_prologue(const DmaOperand& F, const DmaOperand& T, int K,
                                              unsigned char* smem) {
  constexpr int kStep = REV ? -kPipeBK * 2 : kPipeBK * 2;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nk = K / kPipeBK;
  const uint32_t base = lds_addr(smem);
  for (int s = 0; s < 2 && s < nk; ++s) {
#pragma unroll
    for (int j = 0; j < kIssues<FQ>; ++j) dma_issue<FQ>(F, T, j, s * kStep, base + s * kPipeStage, wave);
  }
}

// Slice kt of the main loop (kt + 1 < nk): steps 1 to 3 of slice kt, the barrier that
// frees its stage, step 0 of slice kt + 1.  PEND: the second half of slice kt + 1's loads
// goes out in step 1 (kt >= 1; slices 0 and 1 came whole with the prologue).  MORE: slice
// kt + 2 exists and the first half of its loads goes out in step 0.  With both flags fixed at
// compile time the steady-state body carries no load conditions, which measurably shortens
// the issue of the 64 MFMAs of a slice.
template <bool REV, bool PEND, bool MORE, int FQ = 0, bool TRI = false, int MACT = 4>
__device__ __forceinline__ void gemm_slice(f32x16 (&acc)[4][4], bf16x8 (&a0)[4], bf16x8 (&b0)[4],
                                           bf16x8 (&a1)[4], bf16x8 (&b1)[4], const DmaOperand& F,
                                           const DmaOperand& T, unsigned char* smem, uint32_t base,
                                           int kt, int wf, int wt, int lane, const FragOff& fo,
                                           int wave) {
  constexpr int kStep = REV ? -kPipeBK * 2 : kPipeBK * 2;    // bytes from one slice to the next
  const unsigned char* cur = smem + (kt & 1) * kPipeStage;
  const int kbp = (kt + 1) * kStep;
  const uint32_t dstp = base + ((kt + 1) & 1) * kPipeStage;
  mfma16_read<FQ, TRI, MACT>(acc, a0, b0, a1, b1, cur, 1, wf, wt, lane, fo, PEND, F, T, kbp, dstp,
                             kIssues<FQ> / 2, wave);
  mfma16_read<FQ, TRI, MACT>(acc, a1, b1, a0, b0, cur, 2, wf, wt, lane, fo, false, F, T, 0, 0, 0, wave);
  mfma16_read<FQ, TRI, MACT>(acc, a0, b0, a1, b1, cur, 3, wf, wt, lane, fo, false, F, T, 0, 0, 0, wave);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");     // slice kt + 1, the only one in flight
  __syncthreads();                                       // ... landed for every wave; slice kt read
  const unsigned char* nxt = smem + ((kt + 1) & 1) * kPipeStage;
  const uint32_t dst = base + (kt & 1) * kPipeStage;
  const int kb = (kt + 2) * kStep;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if ((i >> 2) < MACT) mfma_i(acc, a1, b1, i);
    if (MORE && !(i & 1) && (i >> 1) < kIssues<FQ> / 2) dma_issue<FQ>(F, T, i >> 1, kb, dst, wave);
    if (i >= 8) read_frag<FQ, TRI>(a0, b0, nxt, i - 8, 0, wf, wt, lane, fo);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The rest of the pipeline, once gemm_prologue's loads are issued.  The wait for slice 0
// counts on loads completing in order: while any load of slice 0 is pending, all 16 of
// slice 1 are too, so at most 16 outstanding operations (stores issued after the
// prologue included) means slice 0 has landed.
template <bool REV = false, int FQ = 0>
__device__ __forceinline__ void gemm_mainloop(f32x16 (&acc)[4][4], const DmaOperand& F,
                                              const DmaOperand& T, int K, unsigned char* smem) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wf = wave >> 1, wt = wave & 1;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[m][n][r] = 0.f;

  const int nk = K / kPipeBK;
  const uint32_t base = lds_addr(smem);
  if (nk > 1) {                                          // slice 0 landed: at most slice 1's
    if (FQ)                                              // loads are outstanding
      asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();

  const FragOff fo = frag_off(lane);
  bf16x8 a0[4], b0[4], a1[4], b1[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) read_frag<FQ>(a0, b0, smem, i, 0, wf, wt, lane, fo);
  // slices 0 .. nk - 2: the first has nothing pending, the last starts no further slice
  if (nk == 2) {
    gemm_slice<REV, false, false, FQ>(acc, a0, b0, a1, b1, F, T, smem, base, 0, wf, wt, lane, fo,
                                      wave);
  } else if (nk > 2) {
    gemm_slice<REV, false, true, FQ>(acc, a0, b0, a1, b1, F, T, smem, base, 0, wf, wt, lane, fo,
                                     wave);
    for (int kt = 1; kt < nk - 2; ++kt)
      gemm_slice<REV, true, true, FQ>(acc, a0, b0, a1, b1, F, T, smem, base, kt, wf, wt, lane, fo,
                                      wave);
    gemm_slice<REV, true, false, FQ>(acc, a0, b0, a1, b1, F, T, smem, base, nk - 2, wf, wt, lane,
                                     fo, wave);
  }
  {
    const unsigned char* cur = smem + ((nk - 1) & 1) * kPipeStage;
    mfma16_read<FQ>(acc, a0, b0, a1, b1, cur, 1, wf, wt, lane, fo, false, F, T, 0, 0, 0, wave);
    mfma16_read<FQ>(acc, a1, b1, a0, b0, cur, 2, wf, wt, lane, fo, false, F, T, 0, 0, 0, wave);
    mfma16_read<FQ>(acc, a0, b0, a1, b1, cur, 3, wf, wt, lane, fo, false, F, T, 0, 0, 0, wave);
#pragma unroll
    for (int i = 0; i < 16; ++i) mfma_i(acc, a1, b1, i);
  }
  __syncthreads();
}

// The main loop of an upper-triangular F operand (the folded layers' norm GEMM): F rows
// f0 .. f0 + 255 are zero left of their diagonal, and the tile's reduction starts (or, with
// REV, ends) at column f0.  The first four slices from column f0 then hold the triangle's
// diagonal block: in its slice s (columns f0 + 64 s ..), 32-row block b is zero for
// b > 2 s + 1.  With the F blocks of the two wave halves interleaved (TRI: blocks 2 m + wf),
// both halves need exactly the blocks m <= s there, so each diagonal slice issues only the
// MFMAs of m < s + 1 and the halves stay balanced: 96 of a tile's MFMAs are skipped, 6 of
// every 16 in the diagonal block (whose zeros would otherwise be multiplied).  The result
// is that of the full loop (the skipped products are of zero blocks).  K >= 256.
template <bool REV>
__device__ __forceinline__ void gemm_mainloop_tri(f32x16 (&acc)[4][4], const DmaOperand& F,
                                                  const DmaOperand& T, int K, unsigned char* smem) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wf = wave >> 1, wt = wave & 1;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[m][n][r] = 0.f;

  const int nk = K / kPipeBK;
  const uint32_t base = lds_addr(smem);
  asm volatile("s_waitcnt vmcnt(16)" ::: "memory");     // slice 0 landed: slice 1 may be pending
  __syncthreads();

  // the offsets are formed anew for every tile: in a persistent caller, hoisted out of its
  // loop they would live across the epilogue, where they were spilled and then reloaded
  // inside the first slices (a reload waits for every load in flight, the slices' too)
  FragOff fo = frag_off(lane_id_opaque());
  frag_off_tri(fo, wf);
  bf16x8 a0[4], b0[4], a1[4], b1[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) read_frag<0, true>(a0, b0, smem, i, 0, wf, wt, lane, fo);
  if (!REV) {            // diagonal slices first: MACT 1, 2, 3, then 4
    gemm_slice<REV, false, true, 0, true, 1>(acc, a0, b0, a1, b1, F, T, smem, base, 0, wf, wt, lane, fo, wave);
    gemm_slice<REV, true, true, 0, true, 2>(acc, a0, b0, a1, b1, F, T, smem, base, 1, wf, wt, lane, fo, wave);
    if (nk == 4) {
      gemm_slice<REV, true, false, 0, true, 3>(acc, a0, b0, a1, b1, F, T, smem, base, 2, wf, wt, lane, fo, wave);
    } else {
      gemm_slice<REV, true, true, 0, true, 3>(acc, a0, b0, a1, b1, F, T, smem, base, 2, wf, wt, lane, fo, wave);
      for (int kt = 3; kt < nk - 2; ++kt)
        gemm_slice<REV, true, true, 0, true, 4>(acc, a0, b0, a1, b1, F, T, smem, base, kt, wf, wt, lane, fo, wave);
      gemm_slice<REV, true, false, 0, true, 4>(acc, a0, b0, a1, b1, F, T, smem, base, nk - 2, wf, wt, lane, fo, wave);
    }
  } else {               // diagonal slices last: MACT 4, ..., then 3, 2 and (the last slice) 1
    gemm_slice<REV, false, true, 0, true, 4>(acc, a0, b0, a1, b1, F, T, smem, base, 0, wf, wt, lane, fo, wave);
    for (int kt = 1; kt < nk - 3; ++kt)
      gemm_slice<REV, true, true, 0, true, 4>(acc, a0, b0, a1, b1, F, T, smem, base, kt, wf, wt, lane, fo, wave);
    gemm_slice<REV, true, true, 0, true, 3>(acc, a0, b0, a1, b1, F, T, smem, base, nk - 3, wf, wt, lane, fo, wave);
    gemm_slice<REV, true, false, 0, true, 2>(acc, a0, b0, a1, b1, F, T, smem, base, nk - 2, wf, wt, lane, fo, wave);
  }
  {
    constexpr int kLast = REV ? 1 : 4;
    const unsigned char* cur = smem + ((nk - 1) & 1) * kPipeStage;
    mfma16_read<0, true, kLast>(acc, a0, b0, a1, b1, cur, 1, wf, wt, lane, fo, false, F, T, 0, 0, 0, wave);
    mfma16_read<0, true, kLast>(acc, a1, b1, a0, b0, cur, 2, wf, wt, lane, fo, false, F, T, 0, 0, 0, wave);
    mfma16_read<0, true, kLast>(acc, a0, b0, a1, b1, cur, 3, wf, wt, lane, fo, false, F, T, 0, 0, 0, wave);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if ((i >> 2) < kLast) mfma_i(acc, a1, b1, i);
  }
  __syncthreads();
}

// acc = F[256 x K] * T[256 x K]^T: gemm_prologue then gemm_mainloop.
template <bool REV = false, int FQ = 0>
__device__ __forceinline__ void gemm_pipeline(f32x16 (&acc)[4][4], const DmaOperand& F,
                                              const DmaOperand& T, int K, unsigned char* smem) {
  gemm_prologue<REV, FQ>(F, T, K, smem);
  gemm_mainloop<REV, FQ>(acc, F, T, K, smem);
}

}  // namespace
}  // namespace rf
