// Folded form of an upper layer on gfx950.
//
// Source of the arithmetic: English RidgeFill review (jaehun.me), section "Ridge map:
// predict the input, and the original projection runs unchanged": x_hat = A x_S + b, then
// the layer's own RMSNorm (weight w) and its K/V projections (Fig. 2).  The weight and
// the projections are linear, so they multiply into the map; the only non-linear
// quantity is the scalar |x_hat|^2, and with R the upper-triangular factor of A^T A
//     |A x + b|^2 = |R x + r|^2 + kappa,  r = R^-T A^T b,  kappa = |b|^2 - |r|^2
// (expand |R x + r|^2).  R x costs half of A x.  R is stored with unit diagonal,
// R = diag(g) R1 (g = diag(R) in fp32, R1 in bf16 with its diagonal exactly 1), and r as
// r1 = r / g, so |R x + r|^2 = sum_i g_i^2 (R1_i x + r1_i)^2: the diagonal term, which
// carries a feature whose magnitude dwarfs the others' alone through row 0 when it is
// feature 0, takes no bf16 rounding.  Per layer:
//   At  = [A^T | A^T]              bf16 [d_in][2d], a transpose (exact)
//   Wx  = [W_hi | W_lo]            W = [W_K; W_V] diag(w), each product exact in fp32,
//                                  split hi = bf16(W), lo = bf16(W - hi) (~2^-17 of W)
//   P   = Wx At^T = W_hi A + W_lo A   bf16 MFMA, fp32 accumulation, one bf16 rounding
//   H   = A^T A (lower tiles)      bf16 MFMA: exact products, fp32 accumulation, kept fp64
//   L   = Cholesky(H)              fp64, the solve's blocked kernels;  R1 = bf16 of the rows
//                                  of L^T over their diagonal entries, g = diag(L)
//   g   = A^T b,  c = W b,  |b|^2  fp64 accumulation in a fixed order
//   r   = L^-1 g                   blocked forward substitution (right-looking), fp64
//   kappa = |b|^2 - |r|^2          fp64;  r1 = r / g
// An int8 map A = diag(s) Aq (section "Ridge map ...", map-size paragraph) folds with its
// codes, which bf16 holds exactly: W diag(w) A = W diag(w s) Aq, so Wx splits W diag(w s)
// (each product formed in fp64) and At holds [Aq^T | Aq^T]; A^T A = Aq^T diag(s^2) Aq is
// At times [C_hi | C_lo]^T, C[j][k] = s_k^2 Aq[k][j] split into two bf16 parts (~2^-17),
// over 2 d; A^T b = Aq^T (s b).
// Layers go in groups as large as the workspace holds: the GEMMs layer by layer, then the
// group's Cholesky factorizations and substitutions side by side.  Every launch is on the
// caller's stream.
#include "rf_common.h"
#include "rf_gemm_tile.h"
#include "rf_internal.h"
#include "ridgefill.h"

namespace rf {

FoldLayout fold_layout(int d_in, int kv) {
  FoldLayout F;
  F.P = 0;
  F.R = align256((size_t)2 * kv * d_in * 2);
  F.c = F.R + align256((size_t)d_in * d_in * 2);
  F.r = F.c + align256((size_t)2 * kv * 4);
  F.g = F.r + align256((size_t)d_in * 4);
  F.kappa = F.g + align256((size_t)d_in * 4);
  F.total = F.kappa + 256;
  return F;
}

FoldWsLayout fold_ws_layout(int d, int d_in, int kv, int n_par, bool int8) {
  FoldWsLayout W;
  const int most = int8 ? kFoldGemmSlots / 2 : kFoldGemmSlots;
  W.slots = n_par < most ? n_par : most;
  W.int8 = int8 ? 1 : 0;
  W.At = kStatusBytes;
  W.at_bytes = align256((size_t)d_in * 2 * d * 2);
  W.Wx = W.At + (size_t)W.slots * (int8 ? 2 : 1) * W.at_bytes;
  W.wx_bytes = align256((size_t)2 * kv * 2 * d * 2);
  W.blocks = W.Wx + (size_t)W.slots * W.wx_bytes;
  W.H64 = 0;
  W.linv = W.H64 + align256((size_t)d_in * d_in * 8);
  W.g = W.linv + align256((size_t)d_in * 64 * 8);
  W.r = W.g + align256((size_t)d_in * 8);
  W.scal = W.r + align256((size_t)d_in * 8);
  W.per_layer = W.scal + 256;
  W.total = W.blocks + (size_t)n_par * W.per_layer;
  return W;
}

namespace {

constexpr int FB = 64;   // substitution block (the Cholesky's diagonal block)

// At[i][k] = At[i][d + k] = A[k][i] through a 64 x 64 LDS tile.
__global__ __launch_bounds__(256) void fold_transpose_kernel(const uint16_t* A, int d, int d_in,
                                                             uint16_t* At) {
  __shared__ uint16_t t[64][66];
  const int i0 = blockIdx.x * 64, k0 = blockIdx.y * 64;
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int r = e >> 6, c = e & 63;
    t[r][c] = A[(size_t)(k0 + r) * d_in + i0 + c];
  }
  __syncthreads();
  const size_t ld = (size_t)2 * d;
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int r = e >> 6, c = e & 63;   // r: i within the tile, c: k within the tile
    const uint16_t v = t[c][r];
    At[(size_t)(i0 + r) * ld + k0 + c] = v;
    At[(size_t)(i0 + r) * ld + d + k0 + c] = v;
  }
}

// int8 map: At[i][k] = At[i][d + k] = Aq[k][i] (exact in bf16) and Ct[i] = [hi | lo] of
// s_k^2 Aq[k][i], through a 64 x 64 LDS tile.
__global__ __launch_bounds__(256) void fold_transpose_q_kernel(const int8_t* Aq, const float* As,
                                                               int d, int d_in, uint16_t* At,
                                                               uint16_t* Ct) {
  __shared__ int8_t t[64][68];
  __shared__ double s2[64];
  const int i0 = blockIdx.x * 64, k0 = blockIdx.y * 64;
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int r = e >> 6, c = e & 63;
    t[r][c] = Aq[(size_t)(k0 + r) * d_in + i0 + c];
  }
  if (threadIdx.x < 64) {
    const double sk = (double)As[k0 + threadIdx.x];
    s2[threadIdx.x] = sk * sk;
  }
  __syncthreads();
  const size_t ld = (size_t)2 * d;
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int r = e >> 6, c = e & 63;   // r: i within the tile, c: k within the tile
    const int q = t[c][r];
    const uint16_t v = (uint16_t)f32_to_bf16((float)q);
    const size_t o = (size_t)(i0 + r) * ld + k0 + c;
    At[o] = v;
    At[o + d] = v;
    const double cv = s2[c] * (double)q;
    const uint32_t hi = f32_to_bf16((float)cv);
    Ct[o] = (uint16_t)hi;
    Ct[o + d] = (uint16_t)f32_to_bf16((float)(cv - (double)bf16_to_f32(hi)));
  }
}

// Wx[i] = [hi | lo] of row i of [W_K; W_V] diag(w) (int8 map: diag(w As)).
__global__ void fold_wsplit_kernel(const uint16_t* WK, const uint16_t* WV, const uint16_t* w,
                                   const float* As, int kv, int d, uint16_t* Wx) {
  const size_t n = (size_t)2 * kv * d;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (size_t)gridDim.x * blockDim.x) {
    const int i = (int)(e / d), k = (int)(e - (size_t)i * d);
    const uint16_t wb = i < kv ? WK[(size_t)i * d + k] : WV[(size_t)(i - kv) * d + k];
    const float v = bf16_to_f32(wb) * bf16_to_f32(w[k]);          // exact: 8 x 8 bits
    uint32_t hi, lo;
    if (As) {
      const double vs = (double)v * (double)As[k];
      hi = f32_to_bf16((float)vs);
      lo = f32_to_bf16((float)(vs - (double)bf16_to_f32(hi)));
    } else {
      hi = f32_to_bf16(v);
      lo = f32_to_bf16(v - bf16_to_f32(hi));                     // v - hi exact in fp32
    }
    Wx[(size_t)i * 2 * d + k] = (uint16_t)hi;
    Wx[(size_t)i * 2 * d + d + k] = (uint16_t)lo;
  }
}

// out_l[m][n] = sum_k F_l[m][k] T_l[n][k] for 256 x 256 tiles of the layers l of one launch
// (F_l, T_l bf16 rows at a fixed element stride from layer to layer, K a multiple of 64);
// bf16 (mode 0) or fp64 (mode 1) output.  With `lower`, only tiles n <= m.
//
// The fp64 output is A^T A, accumulated in fp32 (the products are exact).  Its rounding
// error E is about 1e-6 of the diagonal in the Jacobi-scaled sense (|E_ij| ~ 1e-6
// sqrt(H_ii H_jj) at d_in = 4096), which is larger than the smallest eigenvalue of
// diag(H)^-1/2 H diag(H)^-1/2 once A's condition number passes a few thousand: the
// Cholesky would then meet a non-positive pivot at random.  The diagonal is therefore
// lifted by a relative 2^-16, H + 2^-16 diag(H), which keeps the factorization positive
// for any A without a zero column, at the price of an exactly known bias in the folded
// norm: |R x + r|^2 + kappa = |A x + b|^2 + 2^-16 sum_i |A_i|^2 x_i^2, about 1.5e-5 of
// |x_hat|^2 for rows where the columns do not cancel.  A zero column still gives a zero
// pivot (RF_E_NOT_SPD).
constexpr double kGramDiagLift = 1.0 + 1.0 / 65536.0;
struct NtGemmArgs {
  const uint16_t* F;
  const uint16_t* T;
  int64_t sF, sT;                 // elements from one layer's operand to the next
  void* out[kFoldGemmSlots];
  int64_t ldf, ldt, ldo;
  int K, ntm, ntn, mode, lower;
};

__global__ __launch_bounds__(kThreads, 1) void fold_gemm_kernel(NtGemmArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kPipeLds];
  const int per = a.ntm * a.ntn;
  const int l = blockIdx.x / per, tile = blockIdx.x - l * per;
  const int mt = tile / a.ntn, nt = tile - mt * a.ntn;
  if (a.lower && nt > mt) return;                 // whole block, before any barrier
  const uint16_t* Fl = a.F + l * a.sF;
  const uint16_t* Tl = a.T + l * a.sT;
  void* out = a.out[l];
  const int m0 = mt * kTile, n0 = nt * kTile;
  const int tid = threadIdx.x;
  DmaOperand Fo, To;
  {
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int r0 = dma_block_row(p, wave), rr = r0 + dma_lane_row(lane);
      const int ce = dma_chunk_elems(rr, lane);
      Fo.base[p] = reinterpret_cast<const unsigned char*>(Fl + (size_t)(m0 + r0) * a.ldf);
      Fo.off[p] = (uint32_t)((dma_lane_row(lane) * a.ldf + ce) * 2);
      To.base[p] = reinterpret_cast<const unsigned char*>(Tl + (size_t)(n0 + r0) * a.ldt);
      To.off[p] = (uint32_t)((dma_lane_row(lane) * a.ldt + ce) * 2);
    }
  }
  f32x16 acc[4][4];
  gemm_pipeline(acc, Fo, To, a.K, smem);
  const int lane = tid & 63, wave = tid >> 6, wf = wave >> 1, wt = wave & 1, h = lane >> 5;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const size_t col = (size_t)n0 + wt * 128 + n * 32 + (lane & 31);
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const size_t row = (size_t)m0 + wf * 128 + m * 32 + q * 8 + h * 4 + e;
          const float v = acc[m][n][q * 4 + e];
          if (a.mode == 0)
            reinterpret_cast<uint16_t*>(out)[row * a.ldo + col] = (uint16_t)f32_to_bf16(v);
          else
            reinterpret_cast<double*>(out)[row * a.ldo + col] =
                row == col ? (double)v * kGramDiagLift : (double)v;
        }
    }
}

// One wave per output: rows 0 .. d_in-1 give g[i] = sum_k A[k][i] b[k] (from At; an int8
// map's At holds the codes, and the scale multiplies b), rows d_in .. d_in + 2kv - 1 give
// c[j] = sum_k W[j][k] w[k] b[k]; lane-strided fp64 partial sums, then a fixed xor tree.
__global__ __launch_bounds__(256) void fold_gemv_kernel(const uint16_t* At, const float* As,
                                                        const uint16_t* WK, const uint16_t* WV,
                                                        const uint16_t* w, const float* b, int d,
                                                        int d_in, int kv, double* g, float* c) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= d_in + 2 * kv) return;
  double s = 0.0;
  if (row < d_in) {
    const uint16_t* a = At + (size_t)row * 2 * d;
    if (As)
      for (int k = lane; k < d; k += 64)
        s += (double)bf16_to_f32(a[k]) * ((double)As[k] * (double)b[k]);
    else
      for (int k = lane; k < d; k += 64) s += (double)bf16_to_f32(a[k]) * (double)b[k];
  } else {
    const int j = row - d_in;
    const uint16_t* wr = j < kv ? WK + (size_t)j * d : WV + (size_t)(j - kv) * d;
    for (int k = lane; k < d; k += 64)
      s += (double)(bf16_to_f32(wr[k]) * bf16_to_f32(w[k])) * (double)b[k];
  }
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) {
    if (row < d_in) g[row] = s;
    else c[row - d_in] = (float)s;
  }
}

// scal[0] = |b|^2 (fixed-order tree).
__global__ __launch_bounds__(1024) void fold_bb_kernel(const float* b, int d, double* scal) {
  __shared__ double part[1024];
  const int t = threadIdx.x;
  double s = 0.0;
  for (int i = t; i < d; i += 1024) s += (double)b[i] * (double)b[i];
  part[t] = s;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if (t < o) part[t] += part[t + o];
    __syncthreads();
  }
  if (t == 0) scal[0] = part[0];
}

// Step i of L r = g, right-looking: g_i is final (the steps before subtracted every earlier
// block from it), so every workgroup of the launch forms r_i = Linv_ii g_i itself (a 64 x 64
// triangular product); workgroup 0 stores it, workgroup m >= 1 subtracts L[i+m][i] r_i from
// g_{i+m} (four threads per row, combined in a fixed order).  No workgroup writes what
// another of the same launch reads.
__global__ __launch_bounds__(256) void fold_fsub_kernel(const double* L, int d, int i,
                                                        const double* linv, double* g,
                                                        double* r, size_t sP) {
  __shared__ double ri[FB];
  const size_t off = blockIdx.y * sP;             // layer blockIdx.y of the group
  L += off;
  linv += off;
  g += off;
  r += off;
  const int t = threadIdx.x;
  if (t < FB) {
    const double* li = linv + (size_t)i * FB * FB + (size_t)t * FB;
    const double* gi = g + (size_t)i * FB;
    double v = 0.0;
    for (int j = 0; j <= t; ++j) v += li[j] * gi[j];
    ri[t] = v;
  }
  __syncthreads();
  const int m = blockIdx.x;
  if (m == 0) {
    if (t < FB) r[(size_t)i * FB + t] = ri[t];
    return;
  }
  const int row = t >> 2, q = t & 3;
  const double* Lr = L + (size_t)((i + m) * FB + row) * d + (size_t)i * FB;
  double s = 0.0;
  for (int j = q; j < FB; j += 4) s += Lr[j] * ri[j];
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);
  if (q == 0) g[(size_t)(i + m) * FB + row] -= s;
}

// r1 = r / g and g = diag(L) to fp32, kappa = |b|^2 - |r|^2 (fixed-order tree).
__global__ __launch_bounds__(1024) void fold_finish_kernel(const double* r, const double* scal,
                                                           const double* L, int d_in,
                                                           float* r_out, float* g_out,
                                                           float* kappa_out) {
  __shared__ double part[1024];
  const int t = threadIdx.x;
  double s = 0.0;
  for (int i = t; i < d_in; i += 1024) {
    const double gi = L[(size_t)i * d_in + i];
    s += r[i] * r[i];
    r_out[i] = (float)(r[i] / gi);
    g_out[i] = (float)gi;
  }
  part[t] = s;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if (t < o) part[t] += part[t + o];
    __syncthreads();
  }
  if (t == 0) *kappa_out = (float)(scal[0] - part[0]);
}

// R1[f][k] = bf16(L[k][f] / L[f][f]) for k > f, exactly 1 for k = f, 0 below the diagonal,
// through a 64 x 64 LDS tile.
__global__ __launch_bounds__(256) void fold_rt_kernel(const double* L, int d_in, uint16_t* R) {
  __shared__ double t[64][65];
  __shared__ double gd[64];
  const int f0 = blockIdx.x * 64, k0 = blockIdx.y * 64;
  const bool zero = k0 < f0;                      // the whole tile is below the diagonal
  if (!zero) {
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
      const int r = e >> 6, c = e & 63;           // r: k, c: f
      t[r][c] = L[(size_t)(k0 + r) * d_in + f0 + c];
    }
    if (threadIdx.x < 64) gd[threadIdx.x] = L[(size_t)(f0 + threadIdx.x) * (d_in + 1)];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int r = e >> 6, c = e & 63;             // r: f, c: k
    const int f = f0 + r, k = k0 + c;
    uint16_t v = 0;
    if (!zero && k == f) v = 0x3f80u;             // bf16 1.0
    else if (!zero && k > f) v = (uint16_t)f32_to_bf16((float)(t[c][r] / gd[r]));
    R[(size_t)f * d_in + k] = v;
  }
}

}  // namespace

hipError_t launch_fold(int d, int d_in, int kv, const FoldLayerIn* layers, int G,
                       void* const* out, void* ws, const FoldWsLayout& W, hipStream_t stream) {
  const FoldLayout F = fold_layout(d_in, kv);
  unsigned char* s = static_cast<unsigned char*>(ws);
  unsigned* status = reinterpret_cast<unsigned*>(s);
  uint16_t* At0 = reinterpret_cast<uint16_t*>(s + W.At);
  uint16_t* Wx0 = reinterpret_cast<uint16_t*>(s + W.Wx);
  auto blk = [&](int l) { return s + W.blocks + (size_t)l * W.per_layer; };
  hipError_t e;
  // the GEMMs of up to W.slots layers per launch, each layer with its own operand slot
  // int8: layer j's codes in At slot 2 j, its [C_hi | C_lo] in slot 2 j + 1; A^T A over 2 d
  const int aslots = W.int8 ? 2 : 1;
  const int64_t sA = (int64_t)(aslots * W.at_bytes / 2);       // elements per layer
  const uint16_t* Ct0 = W.int8 ? At0 + W.at_bytes / 2 : At0;
  for (int l0 = 0; l0 < G; l0 += W.slots) {
    const int ns = G - l0 < W.slots ? G - l0 : W.slots;
    NtGemmArgs pa = {Wx0, At0, (int64_t)(W.wx_bytes / 2), sA, {},
                     2 * (int64_t)d, 2 * (int64_t)d, d_in, 2 * d, 2 * kv / kTile, d_in / kTile,
                     0, 0};
    NtGemmArgs ha = {At0, Ct0, sA, sA, {}, 2 * (int64_t)d, 2 * (int64_t)d, d_in,
                     W.int8 ? 2 * d : d, d_in / kTile, d_in / kTile, 1, 1};
    for (int j = 0; j < ns; ++j) {
      const int l = l0 + j;
      const FoldLayerIn& in = layers[l];
      unsigned char* o = static_cast<unsigned char*>(out[l]);
      uint16_t* At = reinterpret_cast<uint16_t*>(s + W.At + (size_t)j * aslots * W.at_bytes);
      uint16_t* Wx = reinterpret_cast<uint16_t*>(s + W.Wx + (size_t)j * W.wx_bytes);
      if (W.int8)
        hipLaunchKernelGGL(fold_transpose_q_kernel, dim3(d_in / 64, d / 64), dim3(256), 0, stream,
                           in.Aq, in.As, d, d_in, At, At + W.at_bytes / 2);
      else
        hipLaunchKernelGGL(fold_transpose_kernel, dim3(d_in / 64, d / 64), dim3(256), 0, stream,
                           in.A, d, d_in, At);
      const float* As = W.int8 ? in.As : nullptr;
      hipLaunchKernelGGL(fold_wsplit_kernel, dim3(2048), dim3(256), 0, stream, in.WK, in.WV, in.w,
                         As, kv, d, Wx);
      hipLaunchKernelGGL(fold_gemv_kernel, dim3((d_in + 2 * kv + 3) / 4), dim3(256), 0, stream,
                         At, As, in.WK, in.WV, in.w, in.b, d, d_in, kv,
                         reinterpret_cast<double*>(blk(l) + W.g), reinterpret_cast<float*>(o + F.c));
      hipLaunchKernelGGL(fold_bb_kernel, dim3(1), dim3(1024), 0, stream, in.b, d,
                         reinterpret_cast<double*>(blk(l) + W.scal));
      pa.out[j] = o + F.P;
      ha.out[j] = blk(l) + W.H64;
    }
    hipLaunchKernelGGL(fold_gemm_kernel, dim3(ns * pa.ntm * pa.ntn), dim3(kThreads), 0, stream, pa);
    hipLaunchKernelGGL(fold_gemm_kernel, dim3(ns * ha.ntm * ha.ntn), dim3(kThreads), 0, stream, ha);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // the G factorizations and substitutions side by side (strides in doubles)
  const size_t sP = W.per_layer / 8;
  double* H0 = reinterpret_cast<double*>(blk(0) + W.H64);
  double* linv0 = reinterpret_cast<double*>(blk(0) + W.linv);
  if ((e = launch_cholesky(H0, d_in, linv0, status, stream, G, sP, sP)) != hipSuccess) return e;
  const int nb = d_in / FB;
  for (int i = 0; i < nb; ++i)
    hipLaunchKernelGGL(fold_fsub_kernel, dim3(nb - i, G), dim3(256), 0, stream, H0, d_in, i,
                       linv0, reinterpret_cast<double*>(blk(0) + W.g),
                       reinterpret_cast<double*>(blk(0) + W.r), sP);
  for (int l = 0; l < G; ++l) {
    unsigned char* o = static_cast<unsigned char*>(out[l]);
    const double* H = reinterpret_cast<const double*>(blk(l) + W.H64);
    hipLaunchKernelGGL(fold_finish_kernel, dim3(1), dim3(1024), 0, stream,
                       reinterpret_cast<const double*>(blk(l) + W.r),
                       reinterpret_cast<const double*>(blk(l) + W.scal), H, d_in,
                       reinterpret_cast<float*>(o + F.r), reinterpret_cast<float*>(o + F.g),
                       reinterpret_cast<float*>(o + F.kappa));
    hipLaunchKernelGGL(fold_rt_kernel, dim3(d_in / 64, d_in / 64), dim3(256), 0, stream, H, d_in,
                       reinterpret_cast<uint16_t*>(o + F.R));
  }
  return hipGetLastError();
}

}  // namespace rf
