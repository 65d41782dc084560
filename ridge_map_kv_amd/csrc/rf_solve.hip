// Closed-form ridge solve on gfx950, from the one-pass calibration state.
//
// Source: English RidgeFill review (jaehun.me), section "Ridge map: predict the input,
// and the original projection runs unchanged" -- after subtracting the means,
// A_l = Y_l^T X (X^T X + alpha I)^-1, b_l = mu_l - A_l mu_S, alpha = lambda tr(X^T X)/d_in.
//
// Per call (one lambda):
//   means    mu = sums / n                                              fp64
//            (the state holds the moments of x'_S = x_S - s, s the calibration's shift;
//            mu_S below is the mean of x'_S, the centring being invariant to the shift)
//   centre   C = G - n mu_S mu_S^T (G mirrored from its lower triangle);
//            alpha = lambda tr(C) / d; C += alpha I                      fp64
//   Cholesky blocked, 64-wide blocks: diagonal block factor + its inverse, block
//            column L_ik = A_ik L_kk^-T, update of the rest of its 256-wide panel;
//            after each panel one trailing update A_ij -= L_ik L_jk^T over the
//            panel's 256 columns (fp64 matrix cores)                    fp64
//   inverse  U = L^-T built in the Cholesky's own launches (U L^T = I, column by
//            column as L's block columns become final); M = (C + alpha I)^-1 = U U^T  fp64
//   maps     A_l = C_l M with C_l = YX_l - n mu_l mu_S^T centred in fp64.  Each fp64
//            operand x is split into bf16 parts x_hi = bf16(x), x_lo = bf16(x - x_hi),
//            which hold it to about 2^-17; then
//              A_l ~ C_hi M_hi + C_hi M_lo + C_lo M_hi
//            is one bf16 matrix-core GEMM with the reduction axis tripled:
//            [C_hi | C_hi | C_lo] (d x 3d) times [M_hi | M_lo | M_hi]^T (M symmetric),
//            fp32 accumulation, on the fill's 256 x 256 tile pipeline.  Layers go in
//            groups sized by the workspace.
//   offsets  b_l = mu_l - A_l (mu_S + s) = mu_l - YX_l v + n mu_l (v . mu_S), with
//            v = M (mu_S + s)                                           fp64 accumulate
// Every launch is on the caller's stream; nothing is synchronised.
#include "rf_common.h"
#include "rf_gemm_tile.h"
#include "rf_internal.h"
#include "rf_profile.h"
#include "ridgefill.h"

namespace rf {

namespace {
constexpr int NB = 64;        // Cholesky / substitution block
constexpr int kCholPanel = 4; // 64-blocks per Cholesky panel: one trailing update per panel
constexpr int LDT = NB + 1;   // padded LDS row (fp64)
constexpr int kSplitMax = 6;  // bf16 parts per operand row of the map GEMM (3 or 6 used)
constexpr int kNormParts = 1024;   // partial sums of |C + alpha I|_F^2
}  // namespace

SolveLayout solve_layout(int d_in, int d_out, int n_layers) {
  SolveLayout L;
  const size_t dd = (size_t)d_in * d_in;
  L.scalars = 0;
  L.mu = 256;
  L.mut = L.mu + align256(((size_t)d_in + (size_t)n_layers * d_out) * 8);
  L.v = L.mut + align256((size_t)d_in * 8);
  L.linv = L.v + align256((size_t)d_in * 8);
  L.C = L.linv + align256((size_t)(d_in / NB) * NB * NB * 8);
  L.W = L.C + align256(dd * 8);
  L.M64 = L.W + align256(dd * 8);
  L.Mx = L.M64 + align256(dd * 8);
  L.group = n_layers < kSolveGroup ? n_layers : kSolveGroup;
  L.Cx = L.Mx + align256(dd * 2 * kSplitMax);
  L.norms = L.Cx + align256((size_t)L.group * d_out * d_in * 2 * kSplitMax);
  const int nbk = d_in / NB;
  L.total = L.norms + align256(((size_t)kNormParts + (size_t)nbk * (nbk + 1) / 2) * 8);
  return L;
}

namespace {

// scalars block: [0] status word (unsigned), then doubles at byte offsets below, and the
// int32 number of bf16 parts the map GEMM uses
constexpr int kAlphaOff = 8, kNOff = 16, kVMuOff = 24, kKappaOff = kSolveInfoOff,
              kPartsOff = kSolveInfoOff + 8;

__device__ __forceinline__ double* scal(unsigned char* s, int off) {
  return reinterpret_cast<double*>(s + off);
}

// mu = sums / n for mu_S [d_in] and every mu_l [d_out] (count = d_in + n_layers d_out).
// The sums of x_S are those of the shifted rows x_S - s: mu[0 .. d_in) is the shifted mean
// (all the centring needs), mut = mu + s the true mean of x_S (the offsets need it).  A
// state whose header disagrees with the call's sizes, or that a calibrate call marked,
// sets the state bit of the status.
__global__ void means_kernel(const unsigned char* state, int count, size_t sum_off,
                             size_t shift_off, int d_in, int d_out, int n_layers, double* mu,
                             double* mut, unsigned char* scalars) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const double n = (double)*reinterpret_cast<const int64_t*>(state);
  const double* sums = reinterpret_cast<const double*>(state + sum_off);
  const float* shift = reinterpret_cast<const float*>(state + shift_off);
  const double m = i < count && n > 0 ? sums[i] / n : 0.0;
  if (i < count) mu[i] = m;
  if (i < d_in) mut[i] = m + (double)shift[i];
  if (i == 0) {
    *scal(scalars, kNOff) = n;
    const int32_t* h = reinterpret_cast<const int32_t*>(state);
    if (reinterpret_cast<const uint32_t*>(state)[kHdrMagic] != kCalibMagic || h[kHdrDIn] != d_in ||
        h[kHdrDOut] != d_out || h[kHdrLayers] != n_layers || h[kHdrBad] != 0)
      atomicOr(reinterpret_cast<unsigned*>(scalars), kStatusStateBit);
  }
}

// C[r][c] = G[max][min] - n mu_r mu_c (full symmetric, fp64).
// C = G - n mu mu^T on and below the diagonal, one row per workgroup row (coalesced).  The
// Cholesky reads nothing above the diagonal (the diagonal blocks' upper entries only under
// masks, and it writes them as zeros), so the upper triangle is left as it is.
__global__ void centre_kernel(const float* G, const double* mu, const unsigned char* scalars,
                              int d, double* C) {
  const double n = *reinterpret_cast<const double*>(scalars + kNOff);
  for (int r = blockIdx.y; r < d; r += gridDim.y) {
    const double nr = n * mu[r];
    for (int c = blockIdx.x * blockDim.x + threadIdx.x; c <= r; c += gridDim.x * blockDim.x)
      C[(size_t)r * d + c] = (double)G[(size_t)r * d + c] - nr * mu[c];
  }
}

// alpha = lambda tr(C) / d in a fixed order; then C += alpha I.
__global__ __launch_bounds__(1024) void alpha_kernel(double* C, int d, double lambda,
                                                     unsigned char* scalars) {
  __shared__ double part[1024];
  const int t = threadIdx.x;
  double s = 0.0;
  for (int i = t; i < d; i += 1024) s += C[(size_t)i * d + i];
  part[t] = s;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (t < w) part[t] += part[t + w];
    __syncthreads();
  }
  const double alpha = lambda * part[0] / d;
  for (int i = t; i < d; i += 1024) C[(size_t)i * d + i] += alpha;
  if (t == 0) *scal(scalars, kAlphaOff) = alpha;
}

// Fixed-order sum of 256 per-thread values of a block (tree in LDS); valid in thread 0.
__device__ __forceinline__ double block_sum256(double v, double* red) {
  const int t = threadIdx.x;
  red[t] = v;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w) red[t] += red[t + w];
    __syncthreads();
  }
  return red[0];
}

// |C + alpha I|_F^2 from its lower triangle (entries below the diagonal twice), as
// kNormParts partial sums: block b takes rows b, b + kNormParts, ...
__global__ __launch_bounds__(256) void cnorm_kernel(const double* C, int d, double* part) {
  __shared__ double red[256];
  double s = 0.0;
  for (int r = blockIdx.x; r < d; r += gridDim.x)
    for (int c = threadIdx.x; c <= r; c += 256) {
      const double v = C[(size_t)r * d + c];
      s += (c == r ? 1.0 : 2.0) * v * v;
    }
  const double tot = block_sum256(s, red);
  if (threadIdx.x == 0) part[blockIdx.x] = tot;
}

// kappa_F = |C + alpha I|_F |M|_F from the partial sums (fixed order), and the number of
// bf16 parts per operand of the map product: with two parts (hi + lo, three products) the
// relative error of A grows about as 5e-6 kappa_F / d, with three parts (hi + mid + lo,
// six products) about as 1e-7 kappa_F / d (measured on rotated spectra spread over up to
// six decades).  Three parts are taken once two would pass about 1e-4.
constexpr double kSplit6Kappa = 16.0;
__global__ __launch_bounds__(1024) void kappa_kernel(const double* cpart, const double* mpart,
                                                     int nm, int d, unsigned char* scalars) {
  __shared__ double red[1024];
  const int t = threadIdx.x;
  double s = t < kNormParts ? cpart[t] : 0.0;
  red[t] = s;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (t < w) red[t] += red[t + w];
    __syncthreads();
  }
  const double cn = red[0];
  __syncthreads();
  double m = 0.0;
  for (int i = t; i < nm; i += 1024) m += mpart[i];
  red[t] = m;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (t < w) red[t] += red[t + w];
    __syncthreads();
  }
  if (t == 0) {
    const double kap = sqrt(cn) * sqrt(red[0]);
    *scal(scalars, kKappaOff) = kap;
    *reinterpret_cast<int*>(scalars + kPartsOff) = kap > kSplit6Kappa * d ? 6 : 3;
  }
}

// ---------------------------------------------------------------- 64x64 fp64 tiles

// LDS tile [64][65]; load rows r of src (leading dimension ld), or its transpose.
__device__ __forceinline__ void load64(double* t, const double* src, size_t ld, bool trans) {
  for (int e = threadIdx.x; e < NB * NB; e += blockDim.x) {
    const int r = e >> 6, c = e & 63;
    if (trans)
      t[c * LDT + r] = src[(size_t)r * ld + c];
    else
      t[r * LDT + c] = src[(size_t)r * ld + c];
  }
}

// 64 x 64 fp64 accumulator on the fp64 matrix cores: wave w of a 256-thread block owns rows
// 32 (w >> 1) .. and columns 32 (w & 1) .. as 2 x 2 blocks of v_mfma_f64_16x16x4_f64.  That
// instruction takes A[m][k] from lane 16 k + m, B[k][n] from lane 16 k + n, and leaves
// D[i + 4 j][n] in register j of lane 16 i + n (measured on gfx950).
typedef double f64x4 __attribute__((ext_vector_type(4)));
struct Acc64 {
  f64x4 v[2][2];
};

__device__ __forceinline__ void zero44(Acc64& acc) {
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) acc.v[bi][bj] = f64x4{0.0, 0.0, 0.0, 0.0};
}

// acc += A * Bt^T for the LDS tiles A, Bt [64][LDT]: acc[r][c] += sum_q A[r][q] Bt[c][q].
__device__ __forceinline__ void mac64(Acc64& acc, const double* A, const double* Bt) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r0 = (w >> 1) * 32 + (lane & 15), c0 = (w & 1) * 32 + (lane & 15), kq = lane >> 4;
#pragma unroll 4
  for (int k = 0; k < NB; k += 4) {
    const double a0 = A[r0 * LDT + k + kq], a1 = A[(r0 + 16) * LDT + k + kq];
    const double b0 = Bt[c0 * LDT + k + kq], b1 = Bt[(c0 + 16) * LDT + k + kq];
    acc.v[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, acc.v[0][0], 0, 0, 0);
    acc.v[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b1, acc.v[0][1], 0, 0, 0);
    acc.v[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b0, acc.v[1][0], 0, 0, 0);
    acc.v[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, acc.v[1][1], 0, 0, 0);
  }
}

// Element (row, col) of the tile held in register j of block (bi, bj) of this lane.
__device__ __forceinline__ int acc_row(int bi, int j) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  return (w >> 1) * 32 + bi * 16 + (lane >> 4) + 4 * j;
}
__device__ __forceinline__ int acc_col(int bj) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  return (w & 1) * 32 + bj * 16 + (lane & 15);
}

// dst[r][c] = s * acc + (add ? dst : 0)
__device__ __forceinline__ void store44(double* dst, size_t ld, const Acc64& acc, double s,
                                        bool add) {
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        double* p = dst + (size_t)acc_row(bi, j) * ld + acc_col(bj);
        *p = s * acc.v[bi][bj][j] + (add ? *p : 0.0);
      }
}

// 1/p from the hardware reciprocal and two Newton steps (each doubles the correct bits):
// within an ulp or two of the correctly rounded quotient, at a fraction of its cost.
__device__ __forceinline__ double recip(double p) {
  double r = __builtin_amdgcn_rcp(p);
  double e = fma(-p, r, 1.0);
  r = fma(r, e, r);
  e = fma(-p, r, 1.0);
  return fma(r, e, r);
}

// Factor diagonal block k in place (lower) and store its inverse in linv[k].  1024 threads;
// thread t owns row t / 16 and the 4 columns 4 (t % 16) .. + 3, and keeps its segment of
// the block and of Y in registers for the whole sweep.  (The column steps are sequential;
// with 4 columns per thread each is a few instructions, measured 2.5x faster than 16
// columns per thread on 256 threads.)
//
// Column j is eliminated with its pivot d_j left unscaled: every row below subtracts
// (a_ij / d_j) times column j from its columns j+1 .. i, which leaves a_ij = L_ij sqrt(d_j).
// The inverse is built in the same sweep on Y = diag(L) L^-1: row i of Y (i > j) subtracts
// (a_ij / d_j) times row j of Y, since L_ij / L_jj = a_ij / d_j.
//
// Columns go two per barrier.  Step (j, j+1) reads column j and row j of Y as left by the
// columns before j (final for column j), and column j+1 and row j+1 of Y as left by the
// columns before j (one elimination short).  Every thread applies that missing
// elimination itself where it needs column j+1: with g = a_(j+1)j / d_j,
//   column j+1 at row x:  a_x(j+1) - a_xj g,   pivot d_(j+1) = a_(j+1)(j+1) - a_(j+1)j g,
//   row j+1 of Y:         Y_(j+1) - g Y_j,
// then eliminates column j from its entries in columns j+1 .. i and column j+1 from those
// in columns j+2 .. i.  The owners of columns j+2, j+3 and of rows j+2, j+3 of Y then
// publish them to LDS (double-buffered by step parity): one barrier per two columns.  At
// the end L_ij = a_ij / sqrt(d_j), L_jj = sqrt(d_j) and (L^-1)_i = Y_i / sqrt(d_i).  A
// non-positive or non-finite pivot sets the NOT_SPD bit and is taken as 1.
constexpr int kDiagThreads = 1024, kDiagW = 4;
__global__ __launch_bounds__(kDiagThreads) void chol_diag_kernel(double* C, int d, int k,
                                                                 double* linv, unsigned* status,
                                                                 size_t sC, size_t sL) {
  // columns j, j+1 and rows j, j+1 of Y, by step parity
  __shared__ __attribute__((aligned(16))) double colA[2][NB], colB[2][NB];
  __shared__ __attribute__((aligned(16))) double yA[2][NB], yB[2][NB];
  __shared__ double piv[NB];          // pivots d_j (after the NOT_SPD replacement)
  C += blockIdx.y * sC;               // matrix blockIdx.y of a batch
  linv += blockIdx.y * sL;
  double* blk = C + (size_t)k * NB * d + (size_t)k * NB;
  const int t = threadIdx.x;
  constexpr int TPR = NB / kDiagW;
  const int row = t / TPR, c0 = (t % TPR) * kDiagW;
  double ar[kDiagW], yr[kDiagW];
#pragma unroll
  for (int cc = 0; cc < kDiagW; ++cc) {
    ar[cc] = blk[(size_t)row * d + c0 + cc];
    yr[cc] = row == c0 + cc ? 1.0 : 0.0;
  }
  // publish columns 0, 1 and rows 0, 1 of Y
  if (c0 == 0) {
    colA[0][row] = ar[0];
    colB[0][row] = ar[1];
  }
  if (row < 2) {
#pragma unroll
    for (int cc = 0; cc < kDiagW; ++cc) (row == 0 ? yA : yB)[0][c0 + cc] = yr[cc];
  }
  __syncthreads();
  for (int j = 0; j < NB; j += 2) {
    const int b = (j >> 1) & 1;
    // rows up to j have nothing left to eliminate: their waves skip the step, the pivot
    // arithmetic included (every row below works it out for itself; row j + 1 records it)
    if (row > j) {
      double p0 = colA[b][j];
      const bool bad0 = !(p0 > 0.0) || !isfinite(p0);
      if (bad0) p0 = 1.0;
      const double r0 = recip(p0);
      const double a10 = colA[b][j + 1];
      const double g = a10 * r0;
      double p1 = colB[b][j + 1] - a10 * g;
      const bool bad1 = !(p1 > 0.0) || !isfinite(p1);
      if (bad1) p1 = 1.0;
      if (row == j + 1 && c0 == 0) {
        piv[j] = p0;
        piv[j + 1] = p1;
        if (bad0 || bad1) atomicOr(status, kStatusNotSpdBit);
      }
      const double xa = colA[b][row];
      const double m0 = xa * r0;
      // column j+1 of this row, after column j's elimination, and its multiplier
      const double m1 = row > j + 1 ? (colB[b][row] - xa * g) * recip(p1) : 0.0;
      const double2* av = reinterpret_cast<const double2*>(&colA[b][c0]);
      const double2* bv = reinterpret_cast<const double2*>(&colB[b][c0]);
      const double2* ya = reinterpret_cast<const double2*>(&yA[b][c0]);
      const double2* yb = reinterpret_cast<const double2*>(&yB[b][c0]);
#pragma unroll
      for (int q = 0; q < kDiagW / 2; ++q) {
        const double2 aq = av[q], bq = bv[q], yaq = ya[q], ybq = yb[q];
        const double ca[2] = {aq.x, aq.y}, cb[2] = {bq.x - aq.x * g, bq.y - aq.y * g};
        const double ua[2] = {yaq.x, yaq.y}, ub[2] = {ybq.x - yaq.x * g, ybq.y - yaq.y * g};
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int cc = 2 * q + e, c = c0 + cc;
          if (c > j && c <= row) ar[cc] -= m0 * ca[e];
          if (c > j + 1 && c <= row) ar[cc] -= m1 * cb[e];
          yr[cc] -= m0 * ua[e] + m1 * ub[e];
        }
      }
    }
    // columns j+2, j+3 and rows j+2, j+3 of Y are now as the next step expects them
    if (j + 2 < NB) {
      if (c0 == ((j + 2) & ~(kDiagW - 1))) {       // j+2 and j+3 fall in one 4-column group
        colA[b ^ 1][row] = ar[(j + 2) & (kDiagW - 1)];
        colB[b ^ 1][row] = ar[(j + 3) & (kDiagW - 1)];
      }
      if (row == j + 2 || row == j + 3) {
#pragma unroll
        for (int cc = 0; cc < kDiagW; ++cc) (row == j + 2 ? yA : yB)[b ^ 1][c0 + cc] = yr[cc];
      }
    }
    __syncthreads();
  }
  // 1 / sqrt(d_j): own columns and own row
  double* li = linv + (size_t)k * NB * NB;
  const double rrow = 1.0 / sqrt(piv[row]);
#pragma unroll
  for (int cc = 0; cc < kDiagW; ++cc) {
    const int c = c0 + cc;
    double lv = 0.0;
    if (c < row) lv = ar[cc] / sqrt(piv[c]);
    else if (c == row) lv = sqrt(piv[row]);
    blk[(size_t)row * d + c] = lv;
    li[row * NB + c] = c <= row ? yr[cc] * rrow : 0.0;
  }
}

// The solve also needs the inverse factor.  It builds U = L^-T (upper triangular, 64-blocks
// U[a][b], a <= b) inside the Cholesky's own launches, from U L^T = I:
//   U[b][b] = Linv_bb^T,   U[a][b] = -(sum_{a <= k < b} U[a][k] L[b][k]^T) Linv_bb^T  (a < b).
// U's storage at [a][b] accumulates the sum's negative as the columns k < b become final
// (right-looking, like the trailing updates), and column b is finished once L's block
// column b is: the sums need only L's rows, which the factorization has then produced.
// U must start at zero.

// Block row i = k + 1 + blockIdx.x (blockIdx.x < below):  L_ik = A_ik * Linv_kk^T (matrix
// blockIdx.y).  With U, the blocks after those finish U's column k: block row
// a = blockIdx.x - below (0 .. k) gets U[a][k] = S[a][k] Linv_kk^T, U[k][k] = Linv_kk^T.
__global__ __launch_bounds__(256) void chol_panel_kernel(double* C, int d, int k,
                                                         const double* linv, size_t sC,
                                                         size_t sL, double* U) {
  __shared__ double a[NB * LDT];
  __shared__ double li[NB * LDT];
  C += blockIdx.y * sC;
  linv += blockIdx.y * sL;
  const int below = d / NB - k - 1;
  double* blk;
  if ((int)blockIdx.x < below) {
    blk = C + (size_t)(k + 1 + blockIdx.x) * NB * d + (size_t)k * NB;
  } else {
    const int ar = blockIdx.x - below;
    blk = U + (size_t)ar * NB * d + (size_t)k * NB;
    if (ar == k) {                                  // the diagonal block: Linv_kk transposed
      const double* lk = linv + (size_t)k * NB * NB;
      for (int e = threadIdx.x; e < NB * NB; e += blockDim.x) {
        const int r = e >> 6, c = e & 63;
        blk[(size_t)r * d + c] = lk[c * NB + r];
      }
      return;
    }
  }
  load64(a, blk, d, false);
  load64(li, linv + (size_t)k * NB * NB, NB, false);
  __syncthreads();
  Acc64 acc;
  zero44(acc);
  mac64(acc, a, li);
  __syncthreads();
  store44(blk, d, acc, 1.0, false);
}

// Blocks (i, j) of the current panel's remaining columns, k < j < j_end, j <= i < d / 64:
// A_ij -= L_ik L_jk^T (matrix blockIdx.y); blockIdx.x < nchol counts them column by column.
// With U, the blocks after those update U's accumulators in the same columns:
// U[ar][j] -= U[ar][k] L[j][k]^T for block rows ar <= k.
__global__ __launch_bounds__(256) void chol_update_kernel(double* C, int d, int k, int j_end,
                                                          size_t sC, int nchol, double* U) {
  __shared__ double a[NB * LDT];
  __shared__ double b[NB * LDT];
  C += blockIdx.y * sC;
  const int nbk = d / NB;
  const double *sa, *sb;
  double* out;
  if ((int)blockIdx.x < nchol) {
    int j = k + 1, e = blockIdx.x;
    while (j < j_end - 1 && e >= nbk - j) {
      e -= nbk - j;
      ++j;
    }
    const int i = j + e;
    sa = C + (size_t)i * NB * d + (size_t)k * NB;
    sb = C + (size_t)j * NB * d + (size_t)k * NB;
    out = C + (size_t)i * NB * d + (size_t)j * NB;
  } else {
    const int e = blockIdx.x - nchol;
    const int ar = e % (k + 1), j = k + 1 + e / (k + 1);
    sa = U + (size_t)ar * NB * d + (size_t)k * NB;
    sb = C + (size_t)j * NB * d + (size_t)k * NB;
    out = U + (size_t)ar * NB * d + (size_t)j * NB;
  }
  load64(a, sa, d, false);
  load64(b, sb, d, false);
  __syncthreads();
  Acc64 acc;
  zero44(acc);
  mac64(acc, a, b);
  store44(out, d, acc, -1.0, true);
}

// Trailing update after the panel of block columns [k0, k1): for the 64-blocks
// k1 <= j <= i, A_ij -= sum_{k0 <= k < k1} L_ik L_jk^T (matrix blockIdx.y).  The trailing
// matrix (rows and columns from 64 k1 on) is cut into 128 x 128 tiles (I, J), J <= I; when
// its size is an odd number of 64-blocks the last tile row and column are half outside the
// matrix.  With U, the blocks from ntri on take U's accumulators of the columns after the
// panel, rows before its end, as 128 x 128 tiles of a rectangle:
// U[a][b] -= sum_{k0 <= k < k1} U[a][k] L[b][k]^T, a < k1 <= b.
// Each wave owns one 64 x 64 block of a tile as 4 x 4 fp64 MFMA blocks (the block above
// the diagonal of a diagonal tile, and blocks outside the region, are neither computed
// nor stored).  The reduction runs over 16-wide slices through two LDS stages: slice s + 1
// is fetched into registers while slice s is multiplied.
constexpr int kTrT = 128, kTrK = 16, kTrLd = kTrK + 2;   // padded rows stay 16-byte aligned
__global__ __launch_bounds__(256, 2) void chol_trail_kernel(double* C, int d, int k0, int k1,
                                                            size_t sC, int ntri, double* U) {
  __shared__ __attribute__((aligned(16))) double sa[2][kTrT * kTrLd];
  __shared__ __attribute__((aligned(16))) double sb[2][kTrT * kTrLd];
  C += blockIdx.y * sC;
  const int e = blockIdx.x;
  const double *A, *B;
  double* O;
  int r0, c0, rend;
  bool diag;
  if (e < ntri) {
    int I = (int)((sqrt(8.0 * e + 1.0) - 1.0) * 0.5);
    while ((I + 1) * (I + 2) / 2 <= e) ++I;
    while (I * (I + 1) / 2 > e) --I;
    const int J = e - I * (I + 1) / 2;
    A = B = O = C;
    r0 = k1 * NB + I * kTrT;
    c0 = k1 * NB + J * kTrT;
    rend = d;
    diag = I == J;
  } else {
    const int nI = (k1 * NB + kTrT - 1) / kTrT, u = e - ntri;
    A = O = U;
    B = C;
    r0 = (u % nI) * kTrT;
    c0 = k1 * NB + (u / nI) * kTrT;
    rend = k1 * NB;
    diag = false;
  }
  const int kc0 = k0 * NB, nks = (k1 - k0) * NB / kTrK;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // loader: row tid / 2 of each operand, 8 doubles from column 8 (tid % 2) of the slice
  const int lrow = tid >> 1, lcol = (tid & 1) * 8;
  const bool va = r0 + lrow < rend, vb = c0 + lrow < d;
  const double* ga = A + (size_t)(va ? r0 + lrow : 0) * d + kc0 + lcol;
  const double* gb = B + (size_t)(vb ? c0 + lrow : 0) * d + kc0 + lcol;
  double2 ra[4], rb[4];
  auto fetch = [&](int ks) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ra[q] = va ? *reinterpret_cast<const double2*>(ga + ks + 2 * q) : double2{0.0, 0.0};
      rb[q] = vb ? *reinterpret_cast<const double2*>(gb + ks + 2 * q) : double2{0.0, 0.0};
    }
  };
  auto park = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      *reinterpret_cast<double2*>(&sa[buf][lrow * kTrLd + lcol + 2 * q]) = ra[q];
      *reinterpret_cast<double2*>(&sb[buf][lrow * kTrLd + lcol + 2 * q]) = rb[q];
    }
  };
  // this wave's 64 x 64 block of the tile
  const int wr = (w >> 1) * 64, wc = (w & 1) * 64;
  const bool active = r0 + wr < rend && c0 + wc < d && !(diag && wc > wr);
  f64x4 acc[4][4];
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) acc[bi][bj] = f64x4{0.0, 0.0, 0.0, 0.0};

  fetch(0);
  park(0);
  __syncthreads();
  for (int s = 0; s < nks; ++s) {
    if (s + 1 < nks) fetch((s + 1) * kTrK);
    if (active) {
      const double* As = sa[s & 1];
      const double* Bs = sb[s & 1];
      const int m = lane & 15, kq = lane >> 4;
#pragma unroll
      for (int kk = 0; kk < kTrK; kk += 4) {
        double a[4], b[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          a[q] = As[(wr + 16 * q + m) * kTrLd + kk + kq];
          b[q] = Bs[(wc + 16 * q + m) * kTrLd + kk + kq];
        }
#pragma unroll
        for (int bi = 0; bi < 4; ++bi)
#pragma unroll
          for (int bj = 0; bj < 4; ++bj)
            acc[bi][bj] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[bi], b[bj], acc[bi][bj], 0, 0, 0);
      }
    }
    if (s + 1 < nks) park((s + 1) & 1);   // the other stage: last read before the previous barrier
    __syncthreads();
  }
  if (!active) return;
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < 4; ++bj)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        double* p = O + (size_t)(r0 + wr + 16 * bi + (lane >> 4) + 4 * j) * d + c0 + wc +
                    16 * bj + (lane & 15);
        *p -= acc[bi][bj][j];
      }
}

__global__ void zero_kernel(double* W, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    W[i] = 0.0;
}

// M = U U^T for lower tiles (ab >= bb), mirrored: M[a][b] = sum_k U[a][k] U[b][k], k >= ab.
// bf16 parts of an fp64 value: hi = bf16(x), mid = bf16(x - hi), lo = bf16(x - hi - mid);
// |x - hi - mid| <= ~2^-17 |x| and |x - hi - mid - lo| <= ~2^-25 |x|.
__device__ __forceinline__ void split_bf16(double x, uint16_t& hi, uint16_t& mid) {
  hi = f32_to_bf16((float)x);
  mid = f32_to_bf16((float)(x - (double)bf16_to_f32(hi)));
}
__device__ __forceinline__ void split3_bf16(double x, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
  split_bf16(x, hi, mid);
  lo = f32_to_bf16((float)(x - (double)bf16_to_f32(hi) - (double)bf16_to_f32(mid)));
}

// M = U U^T (= W^T W with W = L^-1) for one lower tile pair, written to both triangles in
// fp64 and as the first three parts of the GEMM operand Mx [d][6d] = [M_hi | M_mid | M_hi |
// M_lo | M_hi | M_mid] (bf16; the last three only when the product takes six parts,
// mx_more_kernel).  mpart[e]: the tile's share of |M|_F^2.
constexpr int kWk = 32, kWld = kWk + 2;     // reduction slice; padded LDS rows (16-byte aligned)
__global__ __launch_bounds__(256) void wtw_kernel(const double* U, int d, double* M64, uint16_t* Mx,
                                                  double* mpart) {
  __shared__ __attribute__((aligned(16))) double wa[2][NB * kWld];
  __shared__ __attribute__((aligned(16))) double wb[2][NB * kWld];
  const int e = blockIdx.x;
  int ab = (int)((sqrt(8.0 * e + 1.0) - 1.0) * 0.5);
  while ((ab + 1) * (ab + 2) / 2 <= e) ++ab;
  while (ab * (ab + 1) / 2 > e) --ab;
  const int bb = e - ab * (ab + 1) / 2;
  // k from 64 ab (U is zero before its diagonal) in 32-wide slices through two LDS stages;
  // slice s + 1 is fetched into registers while slice s is multiplied
  const int tid = threadIdx.x, lrow = tid >> 2, lcol = (tid & 3) * (kWk / 4);
  const double* ga = U + (size_t)(ab * NB + lrow) * d + lcol;
  const double* gb = U + (size_t)(bb * NB + lrow) * d + lcol;
  const int k0 = ab * NB, nks = (d - k0) / kWk;
  constexpr int kV = kWk / 8;                 // double2 per thread and operand
  // the next slice in registers: written out as plain code (through lambdas capturing these
  // arrays, the compiler kept them in scratch memory and waited for every load right away)
  static_assert(kV == 4, "four 16-byte pieces per thread and operand");
  double2 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;
#define WTW_FETCH(k)                                                        \
  {                                                                         \
    const double2* pa = reinterpret_cast<const double2*>(ga + (k));         \
    const double2* pb = reinterpret_cast<const double2*>(gb + (k));         \
    ra0 = pa[0]; ra1 = pa[1]; ra2 = pa[2]; ra3 = pa[3];                     \
    rb0 = pb[0]; rb1 = pb[1]; rb2 = pb[2]; rb3 = pb[3];                     \
  }
#define WTW_PARK(buf)                                                       \
  {                                                                         \
    double2* qa = reinterpret_cast<double2*>(&wa[buf][lrow * kWld + lcol]); \
    double2* qb = reinterpret_cast<double2*>(&wb[buf][lrow * kWld + lcol]); \
    qa[0] = ra0; qa[1] = ra1; qa[2] = ra2; qa[3] = ra3;                     \
    qb[0] = rb0; qb[1] = rb1; qb[2] = rb2; qb[3] = rb3;                     \
  }
  const int lane = tid & 63, w = tid >> 6;
  const int r0 = (w >> 1) * 32 + (lane & 15), c0 = (w & 1) * 32 + (lane & 15), kq = lane >> 4;
  Acc64 acc;
  zero44(acc);
  WTW_FETCH(k0)
  WTW_PARK(0)
  __syncthreads();
  for (int s = 0; s < nks; ++s) {
    if (s + 1 < nks) { WTW_FETCH(k0 + (s + 1) * kWk) }
    const double* A = wa[s & 1];
    const double* B = wb[s & 1];
#pragma unroll
    for (int k = 0; k < kWk; k += 4) {
      const double a0 = A[r0 * kWld + k + kq], a1 = A[(r0 + 16) * kWld + k + kq];
      const double b0 = B[c0 * kWld + k + kq], b1 = B[(c0 + 16) * kWld + k + kq];
      acc.v[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, acc.v[0][0], 0, 0, 0);
      acc.v[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b1, acc.v[0][1], 0, 0, 0);
      acc.v[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b0, acc.v[1][0], 0, 0, 0);
      acc.v[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, acc.v[1][1], 0, 0, 0);
    }
    if (s + 1 < nks) { WTW_PARK((s + 1) & 1) }   // the other stage: last read before the previous barrier
    __syncthreads();
  }
#undef WTW_FETCH
#undef WTW_PARK
  // the tile through LDS, so that it and its mirror image leave as row segments; a
  // diagonal tile takes its lower triangle for both halves (exactly symmetric)
  constexpr int kT = NB + 1;
  static_assert(NB * kT <= 2 * NB * kWld, "tile fits in the first operand's two stages");
  double* t = &wa[0][0];
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int j = 0; j < 4; ++j) t[acc_row(bi, j) * kT + acc_col(bj)] = acc.v[bi][bj][j];
  __syncthreads();
  const size_t d6 = (size_t)kSplitMax * d;
  double sq = 0.0;
  for (int e = tid; e < NB * NB; e += blockDim.x) {
    const int r = e >> 6, c = e & 63;
    for (int side = 0; side < (ab == bb ? 1 : 2); ++side) {
      const int rt = side == 0 ? ab : bb, ct = side == 0 ? bb : ab;
      double v;
      if (side == 1) v = t[c * kT + r];                       // the mirror image
      else if (ab == bb && r < c) v = t[c * kT + r];          // a diagonal tile's lower triangle
      else v = t[r * kT + c];
      sq += v * v;
      const size_t a = (size_t)rt * NB + r, b = (size_t)ct * NB + c;
      M64[a * d + b] = v;
      uint16_t hi, mid;
      split_bf16(v, hi, mid);
      Mx[a * d6 + b] = hi;
      Mx[a * d6 + d + b] = mid;
      Mx[a * d6 + 2 * d + b] = hi;
    }
  }
  __shared__ double red[256];
  const double tot = block_sum256(sq, red);
  if (tid == 0) mpart[e] = tot;
}

// The last three parts of Mx, [M_lo | M_hi | M_mid], when the product takes six.
__global__ __launch_bounds__(256) void mx_more_kernel(const double* M64, int d,
                                                      const unsigned char* scalars, uint16_t* Mx) {
  if (*reinterpret_cast<const int*>(scalars + kPartsOff) != 6) return;
  const size_t d6 = (size_t)kSplitMax * d;
  for (int a = blockIdx.x; a < d; a += gridDim.x)
    for (int b = threadIdx.x; b < d; b += 256) {
      uint16_t hi, mid, lo;
      split3_bf16(M64[(size_t)a * d + b], hi, mid, lo);
      uint16_t* row = Mx + (size_t)a * d6;
      row[3 * d + b] = lo;
      row[4 * d + b] = hi;
      row[5 * d + b] = mid;
    }
}

// v = M mu_S (one wave per row, fixed-order reduction); then v . mu_S.
__global__ __launch_bounds__(256) void mv_kernel(const double* M64, const double* mu, int d,
                                                 double* v) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= d) return;
  double s = 0.0;
  for (int k = lane; k < d; k += 64) s += M64[(size_t)row * d + k] * mu[k];
  for (int w = 32; w > 0; w >>= 1) s += __shfl_xor(s, w);
  if (lane == 0) v[row] = s;
}

__global__ __launch_bounds__(1024) void dot_kernel(const double* v, const double* mu, int d,
                                                   unsigned char* scalars) {
  __shared__ double part[1024];
  const int t = threadIdx.x;
  double s = 0.0;
  for (int i = t; i < d; i += 1024) s += v[i] * mu[i];
  part[t] = s;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (t < w) part[t] += part[t + w];
    __syncthreads();
  }
  if (t == 0) *scal(scalars, kVMuOff) = part[0];
}

// b_l[o] = mu_l[o] - sum_k YX_l[o][k] v[k] + n mu_l[o] (v . mu_S); one wave per (l, o).
__global__ __launch_bounds__(256) void bias_kernel(const float* YX, const double* mu,
                                                   const double* v, const unsigned char* scalars,
                                                   int d_in, int d_out, int n_layers, float* b_out) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= n_layers * d_out) return;
  const float* y = YX + (size_t)row * d_in;
  double s = 0.0;
  // 16-byte loads (d_in % 64 == 0), unrolled so that several steps' loads are in flight
  // together instead of each step waiting for its own
#pragma unroll 4
  for (int k = lane * 4; k < d_in; k += 256) {
    const f32x4 q = *reinterpret_cast<const f32x4*>(y + k);
    const double2 v01 = *reinterpret_cast<const double2*>(v + k);
    const double2 v23 = *reinterpret_cast<const double2*>(v + k + 2);
    s += (double)q[0] * v01.x + (double)q[1] * v01.y + (double)q[2] * v23.x +
         (double)q[3] * v23.y;
  }
  for (int w = 32; w > 0; w >>= 1) s += __shfl_xor(s, w);
  if (lane == 0) {
    const double n = *reinterpret_cast<const double*>(scalars + kNOff);
    const double vmu = *reinterpret_cast<const double*>(scalars + kVMuOff);
    const double m = mu[(size_t)d_in + row];
    b_out[row] = (float)(m - s + n * m * vmu);
  }
}

// ---------------------------------------------------------------- split bf16 map GEMM
// Cx[g][o] = [C_hi | C_hi | C_mid] of row o of C_l = YX_l - n mu_l mu_S^T (l = l0 + g;
// o < d_out, columns k < d_in), the centring in fp64, followed by [C_hi | C_lo | C_mid]
// when the product takes six parts: the six products C_hi M_hi, C_hi M_mid, C_mid M_hi,
// C_hi M_lo, C_lo M_hi and C_mid M_mid.  One row per blockIdx.y (g d_out + o), four
// consecutive k per thread.
__global__ void split_c_kernel(const float* YX, const double* mu, const unsigned char* scalars,
                               int d_in, int d_out, int l0, int rows, uint16_t* Cx) {
  const double n = *reinterpret_cast<const double*>(scalars + kNOff);
  const int parts = *reinterpret_cast<const int*>(scalars + kPartsOff);
  const size_t d = (size_t)d_in;
  for (int row = blockIdx.y; row < rows; row += gridDim.y)
  for (int k = (blockIdx.x * blockDim.x + threadIdx.x) * 4; k < d_in;
       k += gridDim.x * blockDim.x * 4) {
    const int g = row / d_out, o = row - g * d_out, l = l0 + g;
    const float* src = YX + ((size_t)l * d_out + o) * d_in;
    const double nm = n * mu[(size_t)d_in + (size_t)l * d_out + o];
    uint16_t* dst = Cx + (size_t)row * (kSplitMax * d);
    const f32x4 y = *reinterpret_cast<const f32x4*>(src + k);
    // mu_S[k .. k + 3] as two 16-byte loads issued with y's (one at a time, each waited for
    // inside the split, they were four dependent round trips)
    const double2 m01 = *reinterpret_cast<const double2*>(mu + k);
    const double2 m23 = *reinterpret_cast<const double2*>(mu + k + 2);
    const double ms[4] = {m01.x, m01.y, m23.x, m23.y};
    uint16_t hi[4], mid[4], lo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) split3_bf16((double)y[j] - nm * ms[j], hi[j], mid[j], lo[j]);
    u32x2 h2, m2, l2;
    h2.x = hi[0] | (uint32_t)hi[1] << 16;
    h2.y = hi[2] | (uint32_t)hi[3] << 16;
    m2.x = mid[0] | (uint32_t)mid[1] << 16;
    m2.y = mid[2] | (uint32_t)mid[3] << 16;
    l2.x = lo[0] | (uint32_t)lo[1] << 16;
    l2.y = lo[2] | (uint32_t)lo[3] << 16;
    *reinterpret_cast<u32x2*>(dst + k) = h2;
    *reinterpret_cast<u32x2*>(dst + d + k) = h2;
    *reinterpret_cast<u32x2*>(dst + 2 * d + k) = m2;
    if (parts == 6) {
      *reinterpret_cast<u32x2*>(dst + 3 * d + k) = h2;
      *reinterpret_cast<u32x2*>(dst + 4 * d + k) = l2;
      *reinterpret_cast<u32x2*>(dst + 5 * d + k) = m2;
    }
  }
}

struct SolveGemmArgs {
  const uint16_t* Cx;       // [G][d_out][6 d_in]
  const uint16_t* Mx;       // [d_in][6 d_in]
  const unsigned char* scalars;   // the number of parts in use (3 or 6)
  float* A_out;             // [n_layers][d_out][d_in] or null
  uint16_t* A_bf16;         // [n_layers][d_out][d_in] or null
  int d_in, d_out, l0, nt_in, nt_out;
};

// A_l[o][i] for one 256 x 256 tile: F = rows o of Cx, T = rows i of Mx, K = 3 d_in or
// 6 d_in (the parts in use; rows are 6 d_in apart either way).  In the
// MFMA result each lane holds one i and runs of four o, so for each o a half-wave writes
// 32 consecutive i.
__global__ __launch_bounds__(kThreads, 1) void solve_gemm_kernel(SolveGemmArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kPipeLds];
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int per = a.nt_out * a.nt_in;
  const int g = tile / per;
  const int r = tile - g * per;
  // groups of 4 o-tiles against all i-tiles (o-tiles share the Cx rows across i)
  const int fg = r / (4 * a.nt_in), within = r - fg * 4 * a.nt_in;
  const int left = a.nt_out - fg * 4, gsz = left < 4 ? left : 4;
  const int it = within / gsz, ot = fg * 4 + (within - it * gsz);
  const int o0 = ot * kTile, i0 = it * kTile;
  const size_t d3 = (size_t)kSplitMax * a.d_in;
  const int parts = *reinterpret_cast<const int*>(a.scalars + kPartsOff);
  const int tid = threadIdx.x;
  DmaOperand Fo, To;
  {
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int r0 = dma_block_row(p, wave), rr = r0 + dma_lane_row(lane);
      const int ce = dma_chunk_elems(rr, lane);
      Fo.base[p] = reinterpret_cast<const unsigned char*>(a.Cx + ((size_t)g * a.d_out + o0 + r0) * d3);
      Fo.off[p] = (uint32_t)((dma_lane_row(lane) * d3 + ce) * 2);
      To.base[p] = reinterpret_cast<const unsigned char*>(a.Mx + (size_t)(i0 + r0) * d3);
      To.off[p] = Fo.off[p];
    }
  }
  f32x16 acc[4][4];
  gemm_pipeline(acc, Fo, To, parts * a.d_in, smem);

  const int lane = tid & 63, wave = tid >> 6, wf = wave >> 1, wt = wave & 1, h = lane >> 5;
  const int l = a.l0 + g;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int i = i0 + wt * 128 + n * 32 + (lane & 31);
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int o = o0 + wf * 128 + m * 32 + q * 8 + h * 4 + e;
          const size_t idx = ((size_t)l * a.d_out + o) * a.d_in + i;
          const float v = acc[m][n][q * 4 + e];
          if (a.A_out) a.A_out[idx] = v;
          if (a.A_bf16) a.A_bf16[idx] = f32_to_bf16(v);
        }
    }
}

}  // namespace

hipError_t launch_cholesky(double* C, int d, double* linv, unsigned* status, hipStream_t stream,
                           int nbatch, size_t sC, size_t sL, double* U) {
  const int nbk = d / NB;
  if (U) {
    if (nbatch != 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(zero_kernel, dim3(2048), dim3(256), 0, stream, U, (size_t)d * d);
  }
  for (int k0 = 0; k0 < nbk; k0 += kCholPanel) {
    const int k1 = k0 + kCholPanel < nbk ? k0 + kCholPanel : nbk;
    for (int k = k0; k < k1; ++k) {
      hipLaunchKernelGGL(chol_diag_kernel, dim3(1, nbatch), dim3(kDiagThreads), 0, stream, C, d,
                         k, linv, status, sC, sL);
      const int below = nbk - k - 1;
      const int npanel = below + (U ? k + 1 : 0);
      if (npanel > 0)
        hipLaunchKernelGGL(chol_panel_kernel, dim3(npanel, nbatch), dim3(256), 0, stream, C, d, k,
                           linv, sC, sL, U);
      int thin = 0;
      for (int j = k + 1; j < k1; ++j) thin += nbk - j;
      const int nthin = thin + (U ? (k + 1) * (k1 - 1 - k) : 0);
      if (nthin > 0)
        hipLaunchKernelGGL(chol_update_kernel, dim3(nthin, nbatch), dim3(256), 0, stream, C, d, k,
                           k1, sC, thin, U);
    }
    if (k1 < nbk) {
      const int m = (d - k1 * NB + kTrT - 1) / kTrT;
      const int ntri = m * (m + 1) / 2;
      const int nrect = U ? ((k1 * NB + kTrT - 1) / kTrT) * m : 0;
      hipLaunchKernelGGL(chol_trail_kernel, dim3(ntri + nrect, nbatch), dim3(256), 0, stream, C,
                         d, k0, k1, sC, ntri, U);
    }
  }
  return hipGetLastError();
}

hipError_t launch_solve(const void* state, int d_in, int d_out, int n_layers, double lambda,
                        float* A_out, float* b_out, uint16_t* A_bf16, void* ws,
                        hipStream_t stream) {
  const CalibLayout CL = calib_layout(d_in, d_out, n_layers);
  const SolveLayout L = solve_layout(d_in, d_out, n_layers);
  const int d = d_in;            // the Cholesky, inverse and M live on the d_in x d_in side
  const unsigned char* st = static_cast<const unsigned char*>(state);
  unsigned char* w = static_cast<unsigned char*>(ws);
  unsigned* status = reinterpret_cast<unsigned*>(w);
  double* mu = reinterpret_cast<double*>(w + L.mu);
  double* mut = reinterpret_cast<double*>(w + L.mut);
  double* v = reinterpret_cast<double*>(w + L.v);
  double* linv = reinterpret_cast<double*>(w + L.linv);
  double* C = reinterpret_cast<double*>(w + L.C);
  double* W = reinterpret_cast<double*>(w + L.W);
  double* M64 = reinterpret_cast<double*>(w + L.M64);
  uint16_t* Mx = reinterpret_cast<uint16_t*>(w + L.Mx);
  uint16_t* Cx = reinterpret_cast<uint16_t*>(w + L.Cx);
  const float* G = reinterpret_cast<const float*>(st + CL.G);
  const float* YX = reinterpret_cast<const float*>(st + CL.YX);
  const int nbk = d / NB;

  hipError_t e = launch_clear_status(status, stream);
  if (e != hipSuccess) return e;
  const int nmu = d_in + n_layers * d_out;
  hipLaunchKernelGGL(means_kernel, dim3((nmu + 255) / 256), dim3(256), 0, stream, st, nmu,
                     CL.sum_S, CL.shift, d_in, d_out, n_layers, mu, mut, w);
  hipLaunchKernelGGL(centre_kernel, dim3((d + 255) / 256, d < 65535 ? d : 65535), dim3(256), 0,
                     stream, G, mu, w, d, C);
  hipLaunchKernelGGL(alpha_kernel, dim3(1), dim3(1024), 0, stream, C, d, lambda, w);
  double* cpart = reinterpret_cast<double*>(w + L.norms);
  double* mpart = cpart + kNormParts;
  hipLaunchKernelGGL(cnorm_kernel, dim3(kNormParts), dim3(256), 0, stream, C, d, cpart);
  // L and U = L^-T together, then M = U U^T
  if ((e = launch_cholesky(C, d, linv, status, stream, 1, 0, 0, W)) != hipSuccess) return e;
  const int ntri = nbk * (nbk + 1) / 2;
  hipLaunchKernelGGL(wtw_kernel, dim3(ntri), dim3(256), 0, stream, W, d, M64, Mx, mpart);
  hipLaunchKernelGGL(kappa_kernel, dim3(1), dim3(1024), 0, stream, cpart, mpart, ntri, d, w);
  hipLaunchKernelGGL(mx_more_kernel, dim3(d < 4096 ? d : 4096), dim3(256), 0, stream, M64, d, w,
                     Mx);
  // v = M (mu' + s) with the true mean; v . mu' with the shifted one (the centring's)
  hipLaunchKernelGGL(mv_kernel, dim3((d + 3) / 4), dim3(256), 0, stream, M64, mut, d, v);
  hipLaunchKernelGGL(dot_kernel, dim3(1), dim3(1024), 0, stream, v, mu, d, w);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  for (int l0 = 0; l0 < n_layers; l0 += L.group) {
    const int G = (n_layers - l0) < L.group ? (n_layers - l0) : L.group;
    const int rows = G * d_out;
    hipLaunchKernelGGL(split_c_kernel, dim3((d_in + 1023) / 1024, rows < 65535 ? rows : 65535),
                       dim3(256), 0, stream, YX, mu, w, d_in, d_out, l0, rows, Cx);
    SolveGemmArgs a = {Cx, Mx, w, A_out, A_bf16, d_in, d_out, l0, d_in / kTile, d_out / kTile};
    ProfileScope ps(RF_KERNEL_SOLVE_MAP, stream);
    hipLaunchKernelGGL(solve_gemm_kernel, dim3(G * a.nt_out * a.nt_in), dim3(kThreads), 0, stream,
                       a);
  }
  hipLaunchKernelGGL(bias_kernel, dim3((n_layers * d_out + 3) / 4), dim3(256), 0, stream, YX, mu,
                     v, w, d_in, d_out, n_layers, b_out);
  return hipGetLastError();
}

}  // namespace rf
