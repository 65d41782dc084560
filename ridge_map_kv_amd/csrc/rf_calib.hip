// One-pass calibration statistics on gfx950.
//
// Source: English RidgeFill review (jaehun.me), section "Ridge map: predict the input,
// and the original projection runs unchanged" -- calibration gathers X^T X, X^T Y_l
// and both means while the unmodified model runs once over the calibration rows; another
// lambda is then just another solve.  Raw sums and raw second moments are kept; the solve centres them.
//
// Per call (n rows of x_S, bf16 [n][d_in], and of every x_l, bf16 [n][d_out]):
//   shift  x_S is accumulated about a per-feature shift s, fixed by the first call that
//          adds rows: s_i = bf16(mean of x_S[:, i] over that call) where the mean exceeds
//          twice the standard deviation of those rows, else 0.  Each call stages
//          x'_S = bf16(x_S - s) in the state's scratch area.  Where a feature's values lie
//          within [s/2, 2s] the difference is exact (Sterbenz), so a feature whose mean
//          dwarfs its spread is accumulated without the cancellation that raw fp32
//          moments suffer when centred: sum x x^T ~ n mu mu^T would swamp the centred part.
//   sums   fp64 s_S += sum_t x'_S[t], s_l += sum_t x_l[t]; header n += rows
//   moments one launch over the lower-triangle tiles of G += x'_S^T x'_S and all tiles of
//           every YX_l += x_l^T x'_S (row = output feature of x_l, column = feature of x_S).
//           Centring is invariant to the shift (x'_S - mean(x'_S) = x_S - mean(x_S)), and
//           the solve adds s back to mean(x'_S) where the offset b needs the true mean.
// The moments kernel reduces over rows: each thread loads an 8-row x 8-feature block
// (eight 16-byte loads), transposes it in registers and writes eight feature-major
// 16-byte chunks, so the LDS tiles have the same [feature][row] layout the fill's
// [row][reduction] tiles have, and the same MFMA slice code runs on them.
#include "rf_common.h"
#include "rf_gemm_tile.h"
#include "rf_internal.h"
#include "rf_profile.h"
#include "ridgefill.h"

namespace rf {

CalibLayout calib_layout(int d_in, int d_out, int n_layers) {
  CalibLayout L;
  L.header = 0;
  L.sum_S = 256;
  L.sum_l = L.sum_S + align256((size_t)d_in * 8);
  L.G = L.sum_l + align256((size_t)n_layers * d_out * 8);
  L.YX = L.G + align256((size_t)d_in * d_in * 4);
  L.shift = L.YX + align256((size_t)n_layers * d_out * d_in * 4);
  L.stage = L.shift + align256((size_t)d_in * 4);
  L.total = L.stage + (size_t)kCalibStageRows * d_in * 2;
  return L;
}

namespace {

constexpr int kMaxCalibLayers = 64;

struct CalibArgs {
  const unsigned char* hdr;      // the state's header: no work once it is marked bad
  const uint16_t* xS;
  const uint16_t* xl[kMaxCalibLayers];
  int row0;                      // first row this launch covers
  int n_rows, d_in, d_out, n_layers;   // rows covered (from row0)
  int nt_in, nt_out;             // 256-wide tiles of d_in and of d_out
  int ngram;                     // lower-triangle tiles of G
  float* G;
  float* YX;
};

// Clears the sums, moments and shift (the scratch area after them is left alone) and
// writes the header.
__global__ void calib_reset_kernel(unsigned char* state, size_t bytes, int d_in, int d_out,
                                   int n_layers) {
  const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  u32x4* p = reinterpret_cast<u32x4*>(state + 256);
  const size_t n16 = (bytes - 256) / 16;
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (size_t i = tid; i < n16; i += stride) p[i] = z;
  if (tid == 0) {
    int32_t* h = reinterpret_cast<int32_t*>(state);
    *reinterpret_cast<int64_t*>(state) = 0;
    h[kHdrDOut] = d_out;
    h[kHdrLayers] = n_layers;
    reinterpret_cast<uint32_t*>(state)[kHdrMagic] = kCalibMagic;
    h[kHdrDIn] = d_in;
    h[kHdrShiftSet] = 0;
    h[kHdrBad] = 0;
    h[kHdrDeciding] = 0;
  }
}

__device__ __forceinline__ float lo16f(uint32_t x) { return bf16_to_f32(x & 0xffffu); }
__device__ __forceinline__ float hi16f(uint32_t x) { return bf16_to_f32(x >> 16); }

__device__ __forceinline__ bool state_bad(const unsigned char* state) {
  return reinterpret_cast<const volatile int32_t*>(state)[kHdrBad] != 0;
}

// First step of every call (one thread): a header that disagrees with the call's sizes
// marks the state bad (every later step of this and later calls then does nothing, and a
// solve reports it).  On a state whose shift is not yet fixed, this call fixes it: from its
// own rows when it has at least 64 (kHdrDeciding tells the next two kernels to compute
// it), as zero otherwise.
__global__ void calib_check_kernel(unsigned char* state, int d_in, int d_out, int n_layers,
                                   int n_rows) {
  int32_t* h = reinterpret_cast<int32_t*>(state);
  if (reinterpret_cast<uint32_t*>(state)[kHdrMagic] != kCalibMagic || h[kHdrDIn] != d_in ||
      h[kHdrDOut] != d_out || h[kHdrLayers] != n_layers)
    h[kHdrBad] = 1;
  h[kHdrDeciding] = 0;
  if (h[kHdrBad] || h[kHdrShiftSet]) return;
  h[kHdrDeciding] = n_rows >= 64 ? 1 : 0;
  h[kHdrShiftSet] = 1;
}

// Shift statistics, part 1: block (column block cb, row part p of kShiftParts) sums x_S
// and x_S^2 over rows p, p + kShiftParts, ... in fp64; partials [2][kShiftParts][d_in].
constexpr int kShiftParts = 64;
__global__ __launch_bounds__(256) void shift_partials_kernel(const unsigned char* state,
                                                             const uint16_t* xS, int n_rows,
                                                             int d_in, double* part) {
  if (reinterpret_cast<const int32_t*>(state)[kHdrDeciding] == 0) return;
  const int col = blockIdx.x * 256 + threadIdx.x, p = blockIdx.y;
  double s1 = 0.0, s2 = 0.0;
  for (int t = p; t < n_rows; t += kShiftParts) {
    const double v = (double)bf16_to_f32(xS[(size_t)t * d_in + col]);
    s1 += v;
    s2 += v * v;
  }
  part[(size_t)p * d_in + col] = s1;
  part[((size_t)kShiftParts + p) * d_in + col] = s2;
}

// Part 2: per column, the partials in a fixed order; s = bf16(mean) where |mean| > 2 sd.
__global__ __launch_bounds__(256) void shift_decide_kernel(unsigned char* state, int n_rows,
                                                           int d_in, const double* part,
                                                           float* shift) {
  if (reinterpret_cast<const int32_t*>(state)[kHdrDeciding] == 0) return;
  const int col = blockIdx.x * 256 + threadIdx.x;
  double s1 = 0.0, s2 = 0.0;
  for (int p = 0; p < kShiftParts; ++p) {
    s1 += part[(size_t)p * d_in + col];
    s2 += part[((size_t)kShiftParts + p) * d_in + col];
  }
  const double mean = s1 / n_rows;
  const double var = s2 / n_rows - mean * mean;
  const double sd = var > 0.0 ? sqrt(var) : 0.0;
  shift[col] = fabs(mean) > 2.0 * sd ? bf16_to_f32(f32_to_bf16((float)mean)) : 0.0f;
}

// x'_S = bf16(x_S - s) for rows [0, n_rows) of x_S into the stage; 8 features per thread.
__global__ __launch_bounds__(256) void shift_stage_kernel(const unsigned char* state,
                                                          const uint16_t* xS, int n_rows, int d_in,
                                                          const float* shift, uint16_t* stage) {
  if (state_bad(state)) return;
  for (int row = blockIdx.x; row < n_rows; row += gridDim.x)
  for (int c8 = threadIdx.x * 8; c8 < d_in; c8 += 256 * 8) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(xS + (size_t)row * d_in + c8);
    const f32x4 s0 = *reinterpret_cast<const f32x4*>(shift + c8);
    const f32x4 s1 = *reinterpret_cast<const f32x4*>(shift + c8 + 4);
    u32x4 o;
    o[0] = pack_bf16x2(lo16f(v[0]) - s0[0], hi16f(v[0]) - s0[1]);
    o[1] = pack_bf16x2(lo16f(v[1]) - s0[2], hi16f(v[1]) - s0[3]);
    o[2] = pack_bf16x2(lo16f(v[2]) - s1[0], hi16f(v[2]) - s1[1]);
    o[3] = pack_bf16x2(lo16f(v[3]) - s1[2], hi16f(v[3]) - s1[3]);
    *reinterpret_cast<u32x4*>(stage + (size_t)row * d_in + c8) = o;
  }
}

// Column sums: block (column block cb of 256, matrix m: 0 = x_S, 1 + l = x_l).  Thread
// (slice s = tid / 32, group q = tid % 32) sums rows s, s + 8, ... of columns 8q..8q+7 in
// fp32; the 8 slices are then added in order in fp64 and folded into the state.
struct SumArgs {
  const unsigned char* hdr;
  const uint16_t* x[kMaxCalibLayers + 1];
  int n_rows, d_in, d_out;
  int ncb;               // column blocks of the wider of d_in and d_out
  double* sums;          // sum_S [d_in], then sum_l [n_layers][d_out], contiguous
  int64_t* count;
};

// Column block cb of matrix m; part: 8 KB of LDS.
__device__ __forceinline__ void sums_block(const SumArgs& a, int cb, int m, float (*part)[256]) {
  const int width = m == 0 ? a.d_in : a.d_out;
  if (cb * 256 >= width) return;                 // the grid covers the wider of the two
  const int tid = threadIdx.x, s = tid >> 5, q = tid & 31;
  const uint16_t* base = a.x[m] + cb * 256 + q * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int t = s; t < a.n_rows; t += 8) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(base + (size_t)t * width);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += bf16_to_f32(v[e] & 0xffffu);
      acc[2 * e + 1] += bf16_to_f32(v[e] >> 16);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[s][q * 8 + e] = acc[e];
  __syncthreads();
  double tot = 0.0;
#pragma unroll
  for (int k = 0; k < 8; ++k) tot += (double)part[k][tid];
  double* dst = a.sums + (m == 0 ? 0 : (size_t)a.d_in + (size_t)(m - 1) * a.d_out) + cb * 256 + tid;
  *dst += tot;
  if (cb == 0 && m == 0 && tid == 0) *a.count += a.n_rows;
}

__global__ __launch_bounds__(256) void calib_sums_kernel(SumArgs a) {
  __shared__ float part[8][256];
  if (state_bad(a.hdr)) return;
  sums_block(a, blockIdx.x, blockIdx.y, part);
}

// Loads rows t0 + 8*rg .. +7, features f0 + 8*fg .. +7 of a row-major [n][d] bf16 matrix
// (rows past n read as zero).
__device__ __forceinline__ void load_block(u32x4 (&v)[8], const uint16_t* x, int d, int n_rows,
                                           int t0, int rg, int f0, int fg) {
  const uint16_t* p = x + (size_t)(t0 + rg * 8) * d + f0 + fg * 8;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (t0 + rg * 8 + e < n_rows) {
      v[e] = *reinterpret_cast<const u32x4*>(p + (size_t)e * d);
    } else {
      v[e] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

// Transposes the 8x8 bf16 block and writes feature row 8*fg + q, chunk rg.
__device__ __forceinline__ void store_block_t(unsigned char* buf, const u32x4 (&v)[8], int rg,
                                              int fg) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    u32x4 o;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t a = v[2 * m][q >> 1], b = v[2 * m + 1][q >> 1];
      o[m] = (q & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
    *reinterpret_cast<u32x4*>(buf + lds_off128(fg * 8 + q, rg)) = o;
  }
}

// Lower-triangle tile k of G -> (ti <= tj): tj = largest j with j (j + 1) / 2 <= k.
__device__ __forceinline__ void gram_tile(int k, int& ti, int& tj) {
  int j = (int)((sqrtf(8.0f * k + 1.0f) - 1.0f) * 0.5f);
  while ((j + 1) * (j + 2) / 2 <= k) ++j;
  while (j * (j + 1) / 2 > k) --j;
  tj = j;
  ti = k - j * (j + 1) / 2;
}

// Tile k of one launch: lower-triangle tiles of G first, then every layer's cross tiles in
// groups of kTokGroup output-row tiles against all column tiles.  X = x_S (output
// columns), Y = x_S or x_l (output rows).
struct CalibTile {
  const uint16_t* X;
  const uint16_t* Y;
  float* out;
  int f0, o0;
  int dy;                        // row stride of Y (d_in for G, d_out for a layer)
};

__device__ __forceinline__ CalibTile calib_tile(const CalibArgs& a, int tile) {
  CalibTile t;
  int fi, tj;
  t.X = a.xS;
  if (tile < a.ngram) {
    gram_tile(tile, fi, tj);     // rows tj >= columns fi
    t.Y = a.xS;
    t.out = a.G;
    t.dy = a.d_in;
  } else {
    const int k = tile - a.ngram;
    const int per = a.nt_out * a.nt_in;
    const int l = k / per;
    const int r = k - l * per;
    const int tg = r / (kTokGroup * a.nt_in);
    const int within = r - tg * kTokGroup * a.nt_in;
    const int left = a.nt_out - tg * kTokGroup;
    const int gsz = left < kTokGroup ? left : kTokGroup;
    fi = within / gsz;
    tj = tg * kTokGroup + (within - fi * gsz);
    t.Y = a.xl[l];
    t.out = a.YX + (size_t)l * a.d_out * a.d_in;
    t.dy = a.d_out;
  }
  t.f0 = fi * kTile;
  t.o0 = tj * kTile;
  return t;
}

// out[o][i .. i+3] += the lane's four consecutive M-entries (M = x_S feature i, N = o).
__device__ __forceinline__ void calib_store(const f32x16 (&acc)[4][4], const CalibTile& t, int d) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wf = wave >> 1, wt = wave & 1, h = lane >> 5;
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int o = t.o0 + wt * 128 + n * 32 + (lane & 31);
    float* row = t.out + (size_t)o * d;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = t.f0 + wf * 128 + m * 32 + q * 8 + h * 4;
        f32x4 v = *reinterpret_cast<const f32x4*>(row + i);
        v[0] += acc[m][n][q * 4 + 0];
        v[1] += acc[m][n][q * 4 + 1];
        v[2] += acc[m][n][q * 4 + 2];
        v[3] += acc[m][n][q * 4 + 3];
        *reinterpret_cast<f32x4*>(row + i) = v;
      }
  }
}

// The moments of a tile added to the state row by row (the DMA kernel's epilogue): each
// half of the tile (128 rows of 256 fp32 columns, 128 KB) is parked in the LDS the main
// loop has left, then every wave adds whole 1 KB row segments to the state, one 16-byte
// piece per lane, and writes them back as full cache lines, non-temporally: the next call
// reads them only after every tile of this one.  The same fp32 addition as calib_store, so
// the same results.  16-byte piece k of LDS row r sits at position k ^ (r & 63).
__device__ __forceinline__ void calib_store_rows(const f32x16 (&acc)[4][4], const CalibTile& t,
                                                 int d, unsigned char* smem) {
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wf = wave >> 1, wt = wave & 1, h = lane >> 5;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    __syncthreads();                      // the LDS is free (the main loop's, or the last half's)
    if (wt == hh) {
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int r = n * 32 + (lane & 31);
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int k = wf * 32 + m * 8 + q * 2 + h;        // 16-byte piece of the row
            const f32x4 v = {acc[m][n][q * 4 + 0], acc[m][n][q * 4 + 1], acc[m][n][q * 4 + 2],
                             acc[m][n][q * 4 + 3]};
            *reinterpret_cast<f32x4*>(smem + r * 1024 + ((k ^ (r & 63)) << 4)) = v;
          }
      }
    }
    __syncthreads();
    // rows wave, wave + 4, ..., wave + 124 of this half: all 32 reads in flight at once
    f32x4 old[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int r = wave + 4 * i;
      old[i] = *reinterpret_cast<const f32x4*>(t.out + (size_t)(t.o0 + hh * 128 + r) * d + t.f0 +
                                              lane * 4);
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int r = wave + 4 * i;
      const f32x4 v = *reinterpret_cast<const f32x4*>(smem + r * 1024 + ((lane ^ (r & 63)) << 4));
      f32x4 o = old[i];
      o[0] += v[0];
      o[1] += v[1];
      o[2] += v[2];
      o[3] += v[3];
      __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(t.out + (size_t)(t.o0 + hh * 128 + r) * d +
                                                          t.f0 + lane * 4));
    }
  }
}

// Rows row0 .. row0 + n_rows - 1 (any count; rows past the end read as zero), register-
// staged with the transpose done in registers.  Used for the ragged row tail.
__global__ __launch_bounds__(kThreads, 1) void calib_moments_kernel(CalibArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kLdsBytes];
  if (state_bad(a.hdr)) return;
  const CalibTile t = calib_tile(a, xcd_remap(blockIdx.x, gridDim.x));
  const uint16_t* X = t.X + (size_t)a.row0 * a.d_in;
  const uint16_t* Y = t.Y + (size_t)a.row0 * t.dy;
  const int f0 = t.f0, o0 = t.o0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wf = wave >> 1, wt = wave & 1, rg = tid >> 5, fg = tid & 31;

  f32x16 acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[m][n][r] = 0.f;

  u32x4 vx[8], vy[8];
  load_block(vx, X, a.d_in, a.n_rows, 0, rg, f0, fg);
  load_block(vy, Y, t.dy, a.n_rows, 0, rg, o0, fg);
  store_block_t(smem, vx, rg, fg);
  store_block_t(smem + kOperandStage, vy, rg, fg);
  __syncthreads();
  const int nk = (a.n_rows + BK - 1) / BK;
  for (int kt = 0; kt < nk; ++kt) {
    const unsigned char* cur = smem + (kt & 1) * kStageBytes;
    const bool more = kt + 1 < nk;
    if (more) {
      load_block(vx, X, a.d_in, a.n_rows, (kt + 1) * BK, rg, f0, fg);
      load_block(vy, Y, t.dy, a.n_rows, (kt + 1) * BK, rg, o0, fg);
    }
    mma_slice(acc, cur, cur + kOperandStage, wf, wt, lane);
    if (more) {
      unsigned char* nxt = smem + ((kt + 1) & 1) * kStageBytes;
      store_block_t(nxt, vx, rg, fg);
      store_block_t(nxt + kOperandStage, vy, rg, fg);
    }
    __syncthreads();
  }
  calib_store(acc, t, a.d_in);
}

// ---------------------------------------------------------------- full 64-row slices
// The fill's pipeline (two 64 KB stages, loads straight into LDS one slice ahead, loads
// and fragment reads between MFMAs), with LDS holding each operand's 64 rows x 256
// features untransposed: 512 bytes per row.  The fragments come out transposed through
// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i % 4 of the
// 8-byte pieces named by lanes i/4, i/4 + 4, i/4 + 8, i/4 + 12.  With lane p of the group
// naming reduction row (p >> 2) and feature 4 (p & 3), lane i receives feature i at four
// consecutive rows; two such reads give the eight consecutive reduction indices of a
// v_mfma_f32_32x32x16_bf16 operand.
//
// Placement of 16-byte chunk c of row r: position t(c) ^ ((r & 3) << 1), where t flips bit 3
// of c when bit 1 is set.  One read's four 16-lane groups take rows r0 .. r0 + 3 (groups 0,
// 1) and r0 + 8 .. r0 + 11 (groups 2, 3), groups 0 and 2 chunks c0, c0 + 1, groups 1 and 3
// chunks c0 + 2, c0 + 3 (c0 a multiple of 4).  The row term spreads a group's four rows
// over eight chunk positions (32 banks); t moves groups 1 and 3 to the other eight
// positions of the 256-byte bank window, so each half-wave (groups 0, 1 or 2, 3) reads all
// 64 banks once.  Without t the four groups met in the same 32 banks: two extra cycles per
// read.  t is an involution, so position p holds chunk t(p ^ ((r & 3) << 1)).
typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int tr_flip(int c) { return c ^ (((c >> 1) & 1) << 3); }
__device__ __forceinline__ int tr_pos(int c, int r) { return tr_flip(c) ^ ((r & 3) << 1); }

__device__ __forceinline__ int tr_off(int r, int col) {
  return r * 512 + ((tr_pos(col >> 3, r) << 4) | ((col & 7) << 1));
}

// A transposed fragment of step s at columns col0 .. col0 + 31 (col0 = 128 W + 32 i) of an
// operand: lane (g = (lane >> 4) & 3, p = lane & 15) reads rows r = 16 s + 8 (g >> 1) + (p >> 2)
// and r + 4 at column col0 + 16 (g & 1) + 4 (p & 3).  tr_off of those splits into s * 8192, W *
// 256 (the bits tr_pos leaves alone), + 2048 for the second row, and a per-lane term of i
// alone: the eight per-lane terms (F with wf, T with wt and the operand's stage offset) are
// computed once per tile, and the rest are immediates.
struct TrOff {
  uint32_t f[4], t[4];
};
__device__ __forceinline__ TrOff tr_offsets(int lane, int wf, int wt) {
  const int g = (lane >> 4) & 3, p = lane & 15;
  TrOff o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = 4 * i + 2 * (g & 1) + ((p & 3) >> 1);
    const uint32_t v = (8 * (g >> 1) + (p >> 2)) * 512 +
                       ((tr_pos(c, p >> 2) << 4) | (((4 * (p & 3)) & 7) << 1));
    o.f[i] = v + wf * 256;
    o.t[i] = v + wt * 256 + kPipeOp;
  }
  return o;
}

__device__ __forceinline__ bf16x8 tr_frag(const unsigned char* at) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(const __attribute__((address_space(3))) unsigned char*)(at));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(const __attribute__((address_space(3))) unsigned char*)(at + 2048));
  struct Pair { s16x4 a, b; } pr = {lo, hi};
  return __builtin_bit_cast(bf16x8, pr);
}

__device__ __forceinline__ void read_frag_tr(bf16x8 (&a)[4], bf16x8 (&b)[4], const unsigned char* st,
                                             int i, int s, const TrOff& to) {
  if (i < 4)
    a[i] = tr_frag(st + to.f[i] + s * 8192);
  else
    b[i - 4] = tr_frag(st + to.t[i - 4] + s * 8192);
}

// As mfma16_read, with transposed fragment reads; with `dma`, load issues 8 .. 15 of the
// slice the operand pointers hold go out after the even-numbered MFMAs, into stage dst.
__device__ __forceinline__ void mfma16_read_tr(f32x16 (&acc)[4][4], const bf16x8 (&a)[4],
                                               const bf16x8 (&b)[4], bf16x8 (&na)[4], bf16x8 (&nb)[4],
                                               const unsigned char* st, int s, const TrOff& to,
                                               bool dma, const DmaOperand& F, const DmaOperand& T,
                                               uint32_t dst, int wave) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    mfma_i(acc, a, b, i);
    if (dma && !(i & 1)) dma_issue(F, T, 8 + (i >> 1), 0, dst, wave);
    if (i < 8) read_frag_tr(na, nb, st, i, s, to);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Slice kt of the moments loop (kt + 1 < nk): steps 1 to 3 of slice kt, the barrier that
// frees its stage, step 0 of slice kt + 1.  PEND: the second half of slice kt + 1's loads
// goes out in step 1 (kt >= 1; slices 0 and 1 came whole before the loop).  MORE: slice
// kt + 2 exists and the first half of its loads goes out in step 0.  Each block pointer moves
// on by one slice once its load has gone out.
template <bool PEND, bool MORE>
__device__ __forceinline__ void calib_slice(f32x16 (&acc)[4][4], bf16x8 (&a0)[4], bf16x8 (&b0)[4],
                                            bf16x8 (&a1)[4], bf16x8 (&b1)[4], DmaOperand& F,
                                            DmaOperand& T, unsigned char* smem, uint32_t base,
                                            int kt, const TrOff& to, int64_t fslice,
                                            int64_t tslice, int wave) {
  const unsigned char* cur = smem + (kt & 1) * kPipeStage;
  mfma16_read_tr(acc, a0, b0, a1, b1, cur, 1, to, PEND, F, T,
                 base + ((kt + 1) & 1) * kPipeStage, wave);
  if (PEND) {
#pragma unroll
    for (int p = 4; p < 8; ++p) {
      F.base[p] += fslice;
      T.base[p] += tslice;
    }
  }
  mfma16_read_tr(acc, a1, b1, a0, b0, cur, 2, to, false, F, T, 0, wave);
  mfma16_read_tr(acc, a0, b0, a1, b1, cur, 3, to, false, F, T, 0, wave);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  const unsigned char* nxt = smem + ((kt + 1) & 1) * kPipeStage;
  const uint32_t dst = base + (kt & 1) * kPipeStage;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    mfma_i(acc, a1, b1, i);
    if (MORE && !(i & 1)) dma_issue(F, T, i >> 1, 0, dst, wave);
    if (i >= 8) read_frag_tr(a0, b0, nxt, i - 8, 0, to);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (MORE) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      F.base[p] += fslice;
      T.base[p] += tslice;
    }
  }
}

// DMA block j = 4 p + wave (p = 0..7) of an operand stage: rows 2 j, 2 j + 1 (1 KB).  Lane
// l lands on row 2 j + (l >> 5), chunk position l & 31, which holds logical chunk
// tr_flip((l & 31) ^ ((row & 3) << 1)).
__device__ __forceinline__ void calib_operand(DmaOperand& o, const uint16_t* x, int d, int col0,
                                              int wave, int lane) {
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int r0 = 2 * (4 * p + wave), r = r0 + (lane >> 5);
    const int c = tr_flip((lane & 31) ^ ((r & 3) << 1));
    o.base[p] = reinterpret_cast<const unsigned char*>(x + (size_t)r0 * d + col0);
    o.off[p] = (uint32_t)((((lane >> 5) * d) + c * 8) * 2);
  }
}

// The column sums ride in the same launch: workgroups from the tile count on each take one
// column block.  They are dispatched after every tile, into the launch's last round, where
// the tiles (5,256 at d = 4096 with 20 layers: 20.5 rounds of 256) leave CUs idle; the
// sums read the same rows again, from HBM, while the last tiles multiply.
__global__ __launch_bounds__(kThreads, 1) void calib_moments_dma_kernel(CalibArgs a, SumArgs s) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kPipeLds];
  if (state_bad(a.hdr)) return;
  const int ntiles = a.ngram + a.n_layers * a.nt_out * a.nt_in;
  if ((int)blockIdx.x >= ntiles) {
    const int b = blockIdx.x - ntiles;
    sums_block(s, b % s.ncb, b / s.ncb, reinterpret_cast<float (*)[256]>(smem));
    return;
  }
  const CalibTile t = calib_tile(a, xcd_remap(blockIdx.x, ntiles));
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wf = wave >> 1, wt = wave & 1;
  DmaOperand F, T;
  calib_operand(F, t.X + (size_t)a.row0 * a.d_in, a.d_in, t.f0, wave, lane);
  calib_operand(T, t.Y + (size_t)a.row0 * t.dy, t.dy, t.o0, wave, lane);

  f32x16 acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[m][n][r] = 0.f;

  const int nk = a.n_rows / kPipeBK;                 // a multiple of 64 rows
  const int64_t fslice = (int64_t)kPipeBK * a.d_in * 2;   // bytes between consecutive slices
  const int64_t tslice = (int64_t)kPipeBK * t.dy * 2;
  const uint32_t base = lds_addr(smem);
  for (int s = 0; s < 2 && s < nk; ++s) {
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      dma_block(F, p, (int)0, base + s * kPipeStage, wave);
      dma_block(T, p, (int)0, base + s * kPipeStage + kPipeOp, wave);
    }
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      F.base[p] += fslice;
      T.base[p] += tslice;
    }
  }
  if (nk > 1)
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  const TrOff to = tr_offsets(lane, wf, wt);
  bf16x8 a0[4], b0[4], a1[4], b1[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) read_frag_tr(a0, b0, smem, i, 0, to);
  // Loads split as in the fill pipeline: blocks 0..3 of each operand right after the
  // barrier that frees a stage, blocks 4..7 during the next slice's first step.  The first
  // slice has no pending half, the last starts no further slice; the steady slices between
  // carry no load conditions.
  if (nk == 2) {
    calib_slice<false, false>(acc, a0, b0, a1, b1, F, T, smem, base, 0, to, fslice, tslice, wave);
  } else if (nk > 2) {
    calib_slice<false, true>(acc, a0, b0, a1, b1, F, T, smem, base, 0, to, fslice, tslice, wave);
    for (int kt = 1; kt < nk - 2; ++kt)
      calib_slice<true, true>(acc, a0, b0, a1, b1, F, T, smem, base, kt, to, fslice, tslice, wave);
    calib_slice<true, false>(acc, a0, b0, a1, b1, F, T, smem, base, nk - 2, to, fslice, tslice,
                             wave);
  }
  {
    const unsigned char* cur = smem + ((nk - 1) & 1) * kPipeStage;
    mfma16_read_tr(acc, a0, b0, a1, b1, cur, 1, to, false, F, T, 0, wave);
    mfma16_read_tr(acc, a1, b1, a0, b0, cur, 2, to, false, F, T, 0, wave);
    mfma16_read_tr(acc, a0, b0, a1, b1, cur, 3, to, false, F, T, 0, wave);
#pragma unroll
    for (int i = 0; i < 16; ++i) mfma_i(acc, a1, b1, i);
  }
  calib_store_rows(acc, t, a.d_in, smem);
}

}  // namespace

hipError_t launch_calib_reset(void* state, int d_in, int d_out, int n_layers, hipStream_t stream) {
  const CalibLayout L = calib_layout(d_in, d_out, n_layers);
  hipLaunchKernelGGL(calib_reset_kernel, dim3(2048), dim3(256), 0, stream,
                     static_cast<unsigned char*>(state), L.stage, d_in, d_out, n_layers);
  return hipGetLastError();
}

// One call: the header check and (first call) the shift, then per piece of at most
// kCalibStageRows rows the staging of x'_S and the moments and sums of that piece.
hipError_t launch_calibrate(void* state, int d_in, int d_out, int n_layers, const uint16_t* xS,
                            const uint16_t* const* xl, int64_t n_rows, hipStream_t stream) {
  if (n_layers > kMaxCalibLayers) return hipErrorInvalidValue;
  const CalibLayout L = calib_layout(d_in, d_out, n_layers);
  unsigned char* st = static_cast<unsigned char*>(state);
  float* shift = reinterpret_cast<float*>(st + L.shift);
  uint16_t* stage = reinterpret_cast<uint16_t*>(st + L.stage);

  hipLaunchKernelGGL(calib_check_kernel, dim3(1), dim3(1), 0, stream, st, d_in, d_out, n_layers,
                     (int)n_rows);
  // the shift statistics use the stage as scratch (2 x 64 x d_in doubles) before any staging
  static_assert(2 * kShiftParts * 8 <= kCalibStageRows * 2, "partials fit in the stage");
  double* part = reinterpret_cast<double*>(stage);
  hipLaunchKernelGGL(shift_partials_kernel, dim3(d_in / 256, kShiftParts), dim3(256), 0, stream,
                     st, xS, (int)n_rows, d_in, part);
  hipLaunchKernelGGL(shift_decide_kernel, dim3(d_in / 256), dim3(256), 0, stream, st,
                     (int)n_rows, d_in, part, shift);

  for (int64_t r0 = 0; r0 < n_rows; r0 += kCalibStageRows) {
    const int rows = (int)(n_rows - r0 < kCalibStageRows ? n_rows - r0 : kCalibStageRows);
    const uint16_t* xs_piece = xS + r0 * d_in;
    hipLaunchKernelGGL(shift_stage_kernel, dim3(2048), dim3(256), 0, stream, st, xs_piece, rows,
                       d_in, shift, stage);

    SumArgs s = {};
    s.hdr = st;
    s.x[0] = stage;
    for (int l = 0; l < n_layers; ++l) s.x[1 + l] = xl[l] + r0 * d_out;
    s.n_rows = rows;
    s.d_in = d_in;
    s.d_out = d_out;
    s.sums = reinterpret_cast<double*>(st + L.sum_S);
    s.count = reinterpret_cast<int64_t*>(st);
    s.ncb = (d_in > d_out ? d_in : d_out) / 256;
    const int nsums = s.ncb * (1 + n_layers);
    // sum_l follows sum_S contiguously: d_in * 8 is a multiple of 256 (d_in % 256 == 0).

    CalibArgs a = {};
    a.hdr = st;
    a.xS = stage;
    for (int l = 0; l < n_layers; ++l) a.xl[l] = xl[l] + r0 * d_out;
    a.d_in = d_in;
    a.d_out = d_out;
    a.n_layers = n_layers;
    a.nt_in = d_in / kTile;
    a.nt_out = d_out / kTile;
    a.ngram = a.nt_in * (a.nt_in + 1) / 2;
    a.G = reinterpret_cast<float*>(st + L.G);
    a.YX = reinterpret_cast<float*>(st + L.YX);
    const int tiles = a.ngram + n_layers * a.nt_out * a.nt_in;
    const int bulk = rows / kPipeBK * kPipeBK;
    if (bulk > 0) {                 // the moments of whole 64-row slices, and the sums
      a.row0 = 0;
      a.n_rows = bulk;
      ProfileScope ps(RF_KERNEL_CALIB_MOMENTS, stream);
      hipLaunchKernelGGL(calib_moments_dma_kernel, dim3(tiles + nsums), dim3(kThreads), 0, stream,
                         a, s);
    } else {                        // fewer than 64 rows: the sums alone
      ProfileScope ps(RF_KERNEL_CALIB_SUMS, stream);
      hipLaunchKernelGGL(calib_sums_kernel, dim3(s.ncb, 1 + n_layers), dim3(256), 0, stream, s);
    }
    if (rows > bulk) {
      a.row0 = bulk;
      a.n_rows = rows - bulk;
      hipLaunchKernelGGL(calib_moments_kernel, dim3(tiles), dim3(kThreads), 0, stream, a);
    }
  }
  return hipGetLastError();
}

}  // namespace rf
