// RidgeFill upper-layer KV fill on gfx950.
//
// Source of the computation: English RidgeFill review (jaehun.me), section "Ridge map:
// predict the input, and the original projection runs unchanged" -- the prediction
// equation x_hat = A x_S + b, and the predicted input passing through the layer's own
// normalisation and key/value projections (Fig. 2).  Exact rows and the tail are not
// given to these kernels ("Two numbers set the skip range").
//
// Two bf16 matrix-core GEMMs per upper layer, both "NT" (both operands contiguous along
// the reduction axis):
//   map   [token][feature]  x_hat = x_S[filled] * A^T + b   (M=features of A, N=tokens)
//         epilogue: + b, per-row sum of squares over each 128-feature chunk (fp32,
//         written to a small partials buffer), bf16(x_hat * norm_w) to the workspace.
//   kv    [token][2*kv]     (x_hat*w) * [W_K; W_V]^T
//         epilogue: * 1/sqrt(mean(x_hat^2)+eps) (reduced from the partials by a small
//         kernel between the two), RoPE on the key half in registers, bf16 store into
//         the paged cache.
// The weight rows sit on the MFMA M axis and the token rows on N, so in the 32x32 MFMA
// result each lane holds one token and runs of four consecutive features: the row
// reduction needs one cross-lane add, RoPE's pair (j, j + hd/2) sits in the same lane
// and register of two MFMA blocks, and stores are 8-byte vectors.
#include <atomic>

#include "rf_common.h"
#include "rf_gemm_tile.h"
#include "rf_internal.h"
#include "rf_profile.h"
#include "ridgefill.h"

namespace rf {

namespace {

struct FillKArgs {
  FillLayerPtrs L[kMaxGroup];
  const FillLayerPtrs* Ltab;    // or null; else layer g's pointers are Ltab[g] (device memory)
  const uint16_t* xS;
  int64_t x_stride;
  const int32_t* idx;
  int64_t P;                    // rows with index >= P are not read (tail / out of range)
  int n_filled;
  int d, d_in, kv, hd, n_kv;
  float eps;
  int mpad, nchunk;             // nchunk = d / 128 sum-of-squares partials per row
  unsigned char* layer_ws;      // per layer: hbuf [mpad][d] bf16, ssq [nchunk][mpad], rstd [mpad]
  size_t per_layer, per_layer_h, per_layer_ssq;
  const float* rcos;
  const float* rsin;
  const int64_t* row_slot;
  float* vnorm;                 // norms mode: |v| per row and head, [group][mpad][n_kv]
  int ntt, nft;                 // token tiles, feature tiles of this launch
  int f_base;                   // first feature tile (norms mode: the V half)
  int has_scale, has_knorm;     // int8 map row scales; per-head key norm
  int folded;                   // folded layers: kv operands P [2 kv][d_in] and gathered x_S
  int kdim;                     // reduction length of the kv GEMM: d, or d_in when folded
  int n_items;                  // tiles (or tile pairs) of the launch
};
static_assert(sizeof(FillKArgs) <= 4096, "kernel arguments must fit in 4 KB");

// Layer g's pointers: from the kernel arguments (up to kMaxGroup layers), or from a table in
// the workspace when a launch covers more layers than the arguments hold.
// (A table entry comes in through a vector load; each pointer is made wave-uniform again,
// since the direct-to-LDS loads take their base addresses in scalar registers.)
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<T*>((uint64_t)hi << 32 | lo);
}

__device__ __forceinline__ FillLayerPtrs layer_ptrs(const FillKArgs& a, int g) {
  if (!a.Ltab) return a.L[g];
  FillLayerPtrs t = a.Ltab[g];
  t.A = uniform_ptr(t.A);
  t.b = uniform_ptr(t.b);
  t.w = uniform_ptr(t.w);
  t.WK = uniform_ptr(t.WK);
  t.WV = uniform_ptr(t.WV);
  t.kp = uniform_ptr(t.kp);
  t.vp = uniform_ptr(t.vp);
  t.kn = uniform_ptr(t.kn);
  t.vs = uniform_ptr(t.vs);
  t.Aq = uniform_ptr(t.Aq);
  t.As = uniform_ptr(t.As);
  t.fc = uniform_ptr(t.fc);
  t.kap = uniform_ptr(t.kap);
  t.fg = uniform_ptr(t.fg);
  return t;
}

// Tile order: layer, then groups of kFeatGroup feature tiles (weight rows) swept against
// every token tile.  Combined with xcd_remap, an XCD's 32 concurrent tiles are a block of
// 8 token tiles x 4 feature tiles, and the group's 4 weight tiles stay hot in its L2
// while the token tiles go by (measured faster than token-major orders on MI355X).
constexpr int kFeatGroup = 4;
__device__ __forceinline__ void decode_tile(int tile, int ntt, int nft, int& g, int& tt, int& ft) {
  const int per_layer = ntt * nft;
  g = tile / per_layer;
  const int r = tile - g * per_layer;
  const int fg = r / (kFeatGroup * ntt);
  const int within = r - fg * kFeatGroup * ntt;
  const int left = nft - fg * kFeatGroup;
  const int gsz = left < kFeatGroup ? left : kFeatGroup;
  tt = within / gsz;
  ft = fg * kFeatGroup + (within - tt * gsz);
}

// Map kernel output staging: after the main loop the 128 KB of LDS hold one 256 (rows) x
// 256 (features) bf16 tile, 512 bytes per row, 16-byte chunk c of row r stored at chunk
// c ^ (r & 31).  Lanes write their runs of four features (8 bytes); the tile then leaves
// as 16-byte vectors, 32 lanes per 512-byte row segment.
__device__ __forceinline__ int stage_off(int r, int f) {
  return r * 512 + ((((f >> 3) ^ (r & 31)) << 4) | ((f & 7) << 1));
}

__device__ __forceinline__ void stage_put4(unsigned char* smem, int r, int f, float v0, float v1,
                                           float v2, float v3) {
  u32x2 o;
  o.x = pack_bf16x2(v0, v1);
  o.y = pack_bf16x2(v2, v3);
  *reinterpret_cast<u32x2*>(smem + stage_off(r, f)) = o;
}

// The kv kernel's outputs go from the accumulators straight to their page slots (through
// the LDS, as in the map kernel, was 1% slower).  In an MFMA result block, half-wave h
// holds features 8 q + 4 h .. 8 q + 4 h + 3 of its row (lane & 31), q = 0..3.  For a pair
// q = 2 p, 2 p + 1, swapping half 0's q = 2 p + 1 run with half 1's q = 2 p run
// (v_permlane32_swap, which exchanges lanes 32..63 of its first operand with lanes 0..31 of
// its second) leaves half 0 with features 16 p .. 16 p + 7 and half 1 with 16 p + 8 ..
// 16 p + 15 of the same row: one 16-byte store per lane, 32 contiguous bytes per row.
// x0, x1: the q = 2 p run as bf16 pairs, y0, y1: the q = 2 p + 1 run; row: the row's feature
// 16 p (bf16 elements).  The page pools are global memory and the store is issued as such
// (through the generic layer-table pointer it would be a flat store, which also counts
// against the LDS reads' wait counter; measured the same).
typedef __attribute__((address_space(1))) u32x4 global_u32x4;
__device__ __forceinline__ void store_run_pair(uint16_t* row, int h, uint32_t x0, uint32_t x1,
                                               uint32_t y0, uint32_t y1, bool valid) {
  const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
  const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
  const u32x4 v = {s0[0], s1[0], s0[1], s1[1]};
  if (valid) *(global_u32x4*)(row + 8 * h) = v;
}

__device__ __forceinline__ float lo16(uint32_t x) { return bf16_to_f32(x & 0xffffu); }
__device__ __forceinline__ float hi16(uint32_t x) { return bf16_to_f32(x >> 16); }

// FQ = 1: int8 map codes, read by the GEMM as they are (the F operand's LDS layout of
// i8_off) and scaled per output row in the epilogue.
// A load through a layer-table pointer, issued as a global-memory load.  The table's pointers
// are generic, and a generic (flat) load also counts against the LDS wait counter: pending
// across a main loop, it turned every fragment-read wait there into a wait for all of them.
template <typename T>
__device__ __forceinline__ T gload(const T* p) {
  return *(const __attribute__((address_space(1))) T*)p;
}

// x_S rows behind the 8 DMA blocks of a tile's gathered operand (token tile t0): lane
// (lane >> 3) of block p is filled-list entry t0 + 8 (4 p + wave) + (lane >> 3).  The eight
// index loads go out together and are waited for once: each reads an entry of the list (a
// position past its end reads the last one), and positions past the end or invalid entries
// then take row 0 (padding rows, never stored).  Loaded one at a time under a condition, they
// were eight dependent round trips at the start of every tile.
__device__ __forceinline__ void gathered_rows(const FillKArgs& a, int t0, int wave, int lane,
                                              int (&row)[8]) {
  const int last = a.n_filled > 0 ? a.n_filled - 1 : 0;
  int x[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int tok = t0 + dma_block_row(p, wave) + dma_lane_row(lane);
    x[p] = a.n_filled > 0 ? a.idx[tok < last ? tok : last] : 0;
  }
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int tok = t0 + dma_block_row(p, wave) + dma_lane_row(lane);
    row[p] = (tok < a.n_filled && x[p] >= 0 && x[p] < a.P) ? x[p] : 0;
  }
}

template <int FQ>
__device__ __forceinline__ void fill_map_tile(const FillKArgs& a, int tile) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kPipeLds];
  int g, tt, ft;
  decode_tile(tile, a.ntt, a.nft, g, tt, ft);
  const FillLayerPtrs Lp = layer_ptrs(a, g);
  const int t0 = tt * kTile, f0 = ft * kTile;
  const int tid = threadIdx.x;

  DmaOperand Fo, To;
  {
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (FQ) {                    // 1 KB block j = 4 p + wave: rows 16 j .. 16 j + 15 of 64 bytes
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int r0 = 16 * (4 * p + wave);
        Fo.base[p] = reinterpret_cast<const unsigned char*>(Lp.Aq + (size_t)(f0 + r0) * a.d_in);
        Fo.off[p] = (uint32_t)((lane >> 2) * a.d_in + 16 * ((lane & 3) ^ ((lane >> 4) & 3)));
      }
    }
    int row[8];
    gathered_rows(a, t0, wave, lane, row);
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int r0 = dma_block_row(p, wave), r = r0 + dma_lane_row(lane);
      const int ce = dma_chunk_elems(r, lane);
      if (!FQ) {
        Fo.base[p] = reinterpret_cast<const unsigned char*>(Lp.A + (size_t)(f0 + r0) * a.d_in);
        Fo.off[p] = (uint32_t)((dma_lane_row(lane) * a.d_in + ce) * 2);
      }
      To.base[p] = reinterpret_cast<const unsigned char*>(a.xS);
      To.off[p] = (uint32_t)(((size_t)row[p] * a.x_stride + ce) * 2);
    }
  }

  // bias, norm weight (and int8 row scale) of feature f0 + tid, fetched under the main loop
  // and parked in LDS for the epilogue
  __shared__ __attribute__((aligned(16))) float sbias[kTile];
  __shared__ __attribute__((aligned(16))) float swt[kTile];
  __shared__ __attribute__((aligned(16))) float ssc[kTile];
  const float my_b = gload(Lp.b + f0 + tid);
  const uint16_t my_w = gload(Lp.w + f0 + tid);
  const float my_s = a.has_scale ? gload(Lp.As + f0 + tid) : 1.0f;

  f32x16 acc[4][4];
  gemm_pipeline<false, FQ>(acc, Fo, To, a.d_in, smem);

  sbias[tid] = my_b;
  swt[tid] = bf16_to_f32(my_w);
  ssc[tid] = my_s;
  __syncthreads();
  const int lane = tid & 63, wave = tid >> 6, wf = wave >> 1, wt = wave & 1, h = lane >> 5;
  uint16_t* hb = reinterpret_cast<uint16_t*>(a.layer_ws + g * a.per_layer);
  float* ssq = reinterpret_cast<float*>(a.layer_ws + g * a.per_layer + a.per_layer_h);
  float ss[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < 4; ++m) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int fl = wf * 128 + m * 32 + q * 8 + h * 4;      // feature within the tile
      const f32x4 bias = *reinterpret_cast<const f32x4*>(sbias + fl);
      const f32x4 wv = *reinterpret_cast<const f32x4*>(swt + fl);
      const float w0 = wv.x, w1 = wv.y, w2 = wv.z, w3 = wv.w;
      f32x4 sc = {1.f, 1.f, 1.f, 1.f};
      if (a.has_scale) sc = *reinterpret_cast<const f32x4*>(ssc + fl);
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int tl = wt * 128 + n * 32 + (lane & 31);
        const float v0 = acc[m][n][q * 4 + 0] * sc.x + bias.x;
        const float v1 = acc[m][n][q * 4 + 1] * sc.y + bias.y;
        const float v2 = acc[m][n][q * 4 + 2] * sc.z + bias.z;
        const float v3 = acc[m][n][q * 4 + 3] * sc.w + bias.w;
        ss[n] += v0 * v0 + v1 * v1 + v2 * v2 + v3 * v3;
        stage_put4(smem, tl, fl, v0 * w0, v1 * w1, v2 * w2, v3 * w3);
      }
    }
  }
#pragma unroll
  for (int n = 0; n < 4; ++n) ss[n] += __shfl_xor(ss[n], 32);
  if (h == 0) {
    const int chunk = (f0 + wf * 128) >> 7;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int tok = t0 + wt * 128 + n * 32 + (lane & 31);
      ssq[(size_t)chunk * a.mpad + tok] = ss[n];        // chunk-major: coalesced
    }
  }
  __syncthreads();
  // rows t0 .. t0 + 255 of the staging buffer (rows past n_filled are padding, in bounds),
  // whole 512-byte row segments as full cache lines, non-temporal: the K/V kernel reads them
  // only after the whole launch, long after any cache could have kept them (stored normally,
  // they displace the operand slices the next tiles read: map kernel 13.84-13.87 against
  // 13.47-13.57 ms, same box)
  const int c = tid & 31;
#pragma unroll 8
  for (int i = 0; i < 32; ++i) {
    const int r = (tid >> 5) + 8 * i;
    const u32x4 v = *reinterpret_cast<const u32x4*>(smem + r * 512 + ((c ^ (r & 31)) << 4));
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(hb + (size_t)(t0 + r) * a.d + f0 + c * 8));
  }
}

template <int FQ>
__global__ __launch_bounds__(kThreads, 1) void fill_map_kernel(FillKArgs a) {
  fill_map_tile<FQ>(a, xcd_remap(blockIdx.x, gridDim.x));
}

// Folded layers: per row, the sum of squares of (R x_S + r) over 256-feature tiles of the
// upper-triangular factor R (A^T A = R^T R), written as 128-feature partials.  R is held
// as R1 = diag(g)^-1 R with unit diagonal (bf16) and r as r1 = r / g: feature f of the
// output is g_f (R1_f x_S + r1_f).  Row f of R
// is zero before column f, so tile ft reduces over columns 256 ft .. d_in - 1 only, and in
// its first 256 columns skips the MFMAs of the 32-row blocks that are zero there
// (gemm_mainloop_tri; the wave halves own interleaved blocks, so each 128-feature chunk's
// sum of squares is the sum of both halves' shares).  A
// workgroup takes the pair of tiles ft and nft - 1 - ft (the longer first): every pair
// then reduces over d_in + 256 columns, so the workgroups are of equal length and the
// short tiles share the fixed cost of a tile with long ones.  With nft odd the middle
// tile is a pair of its own.  a.nft counts pairs.  The first tile of a pair reduces from
// the last column down to its first, the second from its first column up to the last:
// the first tiles of all pairs then start together at column d_in - 64, and, every pair
// being of the same length, the second tiles all end together at column d_in - 1.  So the
// workgroups of one token tile (with different pairs, side by side on an XCD) read each
// slice of its x_S rows in the same step, in both halves, and share it in L2.  (Both
// halves top-down had the second halves of different pairs a few slices apart: 88% of
// their x_S reads missed L2 in a slice-level model of one XCD, 20 GB of fetch per
// 20-layer launch against 15 GB with this order.)
//
// One tile of the norm kernel: item `item` of the launch, half 0 (tile pp) or half 1 (tile
// nft - 1 - pp).
struct NormTile {
  int g, tt, ft;
};

__device__ __forceinline__ NormTile norm_tile(const FillKArgs& a, int item, int half) {
  NormTile t;
  int pp;
  decode_tile(xcd_remap(item, a.n_items), a.ntt, a.nft, t.g, t.tt, pp);
  t.ft = half == 0 ? pp : a.d_in / kTile - 1 - pp;
  return t;
}

// DMA operands of a norm tile: rows f0 .. f0 + 255 of R over columns f0 .. d_in - 1, and
// the tile's gathered x_S rows (the same rows for both tiles of an item).  Half 0 runs from
// the last column down (the bases point at column d_in - 64), half 1 from column f0 up.
__device__ __forceinline__ void norm_operands(const FillKArgs& a, const NormTile& t, int half,
                                              int lane, DmaOperand& Fo, DmaOperand& To) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int f0 = t.ft * kTile, t0 = t.tt * kTile;
  const int col = half == 0 ? a.d_in - kPipeBK : f0;
  const uint16_t* R = layer_ptrs(a, t.g).A;
  int row[8];
  gathered_rows(a, t0, wave, lane, row);
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int r0 = dma_block_row(p, wave), r = r0 + dma_lane_row(lane);
    const int ce = dma_chunk_elems(r, lane);
    Fo.base[p] = reinterpret_cast<const unsigned char*>(R + (size_t)(f0 + r0) * a.d_in + col);
    Fo.off[p] = (uint32_t)((dma_lane_row(lane) * a.d_in + ce) * 2);
    To.base[p] = reinterpret_cast<const unsigned char*>(a.xS + col);
    To.off[p] = (uint32_t)(((size_t)row[p] * a.x_stride + ce) * 2);
  }
}

// The first loads of a norm tile, in its half's direction.
__device__ __forceinline__ void norm_prologue(const DmaOperand& Fo, const DmaOperand& To, int K,
                                              int half, unsigned char* smem) {
  if (half == 0)
    gemm_prologue<true>(Fo, To, K, smem);
  else
    gemm_prologue<false>(Fo, To, K, smem);
}

// The norm kernel is persistent: one workgroup per CU (each holds 128 KB of LDS) takes
// items blockIdx.x, blockIdx.x + gridDim.x, ..., each one or two tiles.  The loads of a
// tile's first two slices are issued as soon as the previous tile's main loop has left
// the LDS, before that tile's epilogue, so the epilogue arithmetic and stores overlap
// them.  (The map kernel stages its outputs through that LDS and the kv kernel its RoPE
// tables, so both stay one tile per workgroup; a kv kernel in such a loop, without the
// tables in LDS, measured no faster: its epilogue's own loads then wait behind the next
// tile's slice loads, which complete first.)
// gridDim.x is a multiple of 8 or equal to n_items, so item i runs on XCD i % 8 and
// xcd_remap's tile ranges hold.
__global__ __launch_bounds__(kThreads, 1) void fill_norm_kernel(FillKArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kPipeLds];
  __shared__ __attribute__((aligned(16))) float sr[kTile];
  __shared__ __attribute__((aligned(16))) float sg[kTile];
  __shared__ float2 xch[2][4][32];      // the wf = 1 halves' chunk sums, per token
  const int nft = a.d_in / kTile;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wf = wave >> 1, wt = wave & 1, h = lane >> 5;

  int item = blockIdx.x, half = 0;
  if (item >= a.n_items) return;
  NormTile cur = norm_tile(a, item, 0);
  DmaOperand Fo, To;
  norm_operands(a, cur, 0, lane, Fo, To);
  norm_prologue(Fo, To, a.d_in - cur.ft * kTile, 0, smem);
  for (;;) {
    const int f0 = cur.ft * kTile, t0 = cur.tt * kTile;
    f32x16 acc[4][4];
    if (half == 0)                                              // each ends with a barrier:
      gemm_mainloop_tri<true>(acc, Fo, To, a.d_in - f0, smem);  // the LDS is free
    else
      gemm_mainloop_tri<false>(acc, Fo, To, a.d_in - f0, smem);

    // Per-lane values of the rest of the iteration are formed from a thread index the
    // compiler cannot trace back to the work-item id: hoisted out of the loop, they lived
    // across it and were spilled, and their reloads in the epilogue waited for the next tile's
    // slice loads issued just before.
    int ltid = (wave << 6) | lane_id_opaque();
    const int llane = ltid & 63, lh = llane >> 5;
    // this tile's r1 and g, loaded now with the next tile's index loads (loaded before the
    // main loop, they were spilled across it)
    const FillLayerPtrs Lc = layer_ptrs(a, cur.g);
    const float my_r = gload(Lc.b + f0 + ltid);
    const float my_g = gload(Lc.fg + f0 + ltid);
    // the next tile: the other half of this item (unless it is the middle tile of an odd
    // nft), else the first half of the next item
    int nitem = item, nhalf = half + 1;
    if (nhalf == 2 || nft - 1 - cur.ft == cur.ft) {
      nitem = item + gridDim.x;
      nhalf = 0;
    }
    const bool more = nitem < a.n_items;
    NormTile nxt = cur;
    if (more) {
      nxt = norm_tile(a, nitem, nhalf);
      norm_operands(a, nxt, nhalf, llane, Fo, To);
      norm_prologue(Fo, To, a.d_in - nxt.ft * kTile, nhalf, smem);
    }

    float* ssq = reinterpret_cast<float*>(a.layer_ws + cur.g * a.per_layer + a.per_layer_h);
    ltid = (wave << 6) | lane_id_opaque();          // again, now that the loads are out
    const int elane = ltid & 63, eh = elane >> 5;
    sr[ltid] = my_r;
    sg[ltid] = my_g;
    __syncthreads();
    // wave half wf holds F blocks 2 m + wf: blocks m = 0, 1 lie in the tile's first 128-feature
    // chunk, m = 2, 3 in its second; the wf = 1 halves hand their sums to the wf = 0 ones
    float ss0[4] = {0.f, 0.f, 0.f, 0.f}, ss1[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int fr = (2 * m + wf) * 32 + q * 8 + eh * 4;
        const f32x4 rv = *reinterpret_cast<const f32x4*>(sr + fr);
        const f32x4 gv = *reinterpret_cast<const f32x4*>(sg + fr);
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const float v0 = (acc[m][n][q * 4 + 0] + rv.x) * gv.x;
          const float v1 = (acc[m][n][q * 4 + 1] + rv.y) * gv.y;
          const float v2 = (acc[m][n][q * 4 + 2] + rv.z) * gv.z;
          const float v3 = (acc[m][n][q * 4 + 3] + rv.w) * gv.w;
          const float t = v0 * v0 + v1 * v1 + v2 * v2 + v3 * v3;
          if (m < 2) ss0[n] += t; else ss1[n] += t;
        }
      }
    }
    // the two half-waves' shares: v_permlane32_swap of a value with itself returns its
    // lower-half lanes' values in the first result and its upper half's in the second, in every
    // lane, so their sum is the half-waves' sum everywhere (no lane index, no LDS permute)
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const auto p0 = __builtin_amdgcn_permlane32_swap(__float_as_uint(ss0[n]), __float_as_uint(ss0[n]),
                                                       false, false);
      const auto p1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(ss1[n]), __float_as_uint(ss1[n]),
                                                       false, false);
      ss0[n] = __uint_as_float(p0[0]) + __uint_as_float(p0[1]);
      ss1[n] = __uint_as_float(p1[0]) + __uint_as_float(p1[1]);
    }
    if (wf == 1 && eh == 0) {
#pragma unroll
      for (int n = 0; n < 4; ++n) xch[wt][n][elane & 31] = make_float2(ss0[n], ss1[n]);
    }
    __syncthreads();
    if (wf == 0 && eh == 0) {
      const int chunk = f0 >> 7;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int tok = t0 + wt * 128 + n * 32 + (elane & 31);
        const float2 o = xch[wt][n][elane & 31];
        ssq[(size_t)chunk * a.mpad + tok] = ss0[n] + o.x;          // chunk-major: coalesced
        ssq[(size_t)(chunk + 1) * a.mpad + tok] = ss1[n] + o.y;
      }
    }
    if (!more) break;
    item = nitem;
    half = nhalf;
    cur = nxt;
  }
}

// RoPE on one pair of 32-feature MFMA blocks (mlo holds pair index j, mhi holds j + hd/2).
// cs, sn: this lane's entry for j = 4 h in the blocked tables (row-block of 32 rows, then
// groups of 4 consecutive j), so pair index j sits (j / 4) * 128 floats further on, and the
// 32 lanes of a half-wave read one contiguous 512-byte run.
template <int MLO, int MHI, int JOFF>
__device__ __forceinline__ void rope_pair(f32x16 (&acc)[4][4], int n, const float* cs,
                                          const float* sn) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int jb = (JOFF / 4 + q * 2) * 128;
    const f32x4 cv = *reinterpret_cast<const f32x4*>(cs + jb);
    const f32x4 sv = *reinterpret_cast<const f32x4*>(sn + jb);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = acc[MLO][n][q * 4 + e], hi = acc[MHI][n][q * 4 + e];
      acc[MLO][n][q * 4 + e] = lo * cv[e] - hi * sv[e];
      acc[MHI][n][q * 4 + e] = hi * cv[e] + lo * sv[e];
    }
  }
}

// Per-head sums of squares of token block n of the wave's 128 features: head 0 of the wave
// owns MFMA blocks m with m * 32 / hd == 0, head 1 (hd = 64 only) the others.  Each lane
// holds half of a head's entries for its token; the lane 32 apart holds the rest.
__device__ __forceinline__ void head_sumsq(const f32x16 (&acc)[4][4], int n, int hd, float& s0,
                                           float& s1) {
  s0 = 0.f;
  s1 = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    float t = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) t += acc[m][n][e] * acc[m][n][e];
    if (m * 32 < hd) s0 += t; else s1 += t;
  }
  s0 += __shfl_xor(s0, 32);
  s1 += __shfl_xor(s1, 32);
}

// MODE 0: fill (K and V tiles; RoPE, optional key norm and value rescale, paged stores).
// MODE 1: value norms (V tiles only): |v| of every (row, head) into a.vnorm.
template <int MODE>
__device__ __forceinline__ void fill_kv_tile(const FillKArgs& a, int tile) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kPipeLds];
  int g, tt, ft;
  decode_tile(tile, a.ntt, a.nft, g, tt, ft);
  ft += a.f_base;
  const FillLayerPtrs Lp = layer_ptrs(a, g);
  // Value norms take each layer's form from its pointers (a folded layer has c), so the
  // exact rows of the value rescale, plain layers, can share a launch with folded ones.
  const bool folded = MODE == 1 ? Lp.fc != nullptr : a.folded != 0;
  const int kdim = MODE == 1 ? (folded ? a.d_in : a.d) : a.kdim;
  const int t0 = tt * kTile, f0 = ft * kTile;
  const int tid = threadIdx.x;
  const uint16_t* hb = reinterpret_cast<const uint16_t*>(a.layer_ws + g * a.per_layer);
  const float* rs_tab = reinterpret_cast<const float*>(a.layer_ws + g * a.per_layer +
                                                       a.per_layer_h + a.per_layer_ssq);

  DmaOperand Fo, To;
  {
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int row[8];
    if (folded) gathered_rows(a, t0, wave, lane, row);
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int r0 = dma_block_row(p, wave), r = r0 + dma_lane_row(lane);
      const int ce = dma_chunk_elems(r, lane);
      const int f = f0 + r0;                 // 8-row blocks never straddle K and V (kv % 128 == 0)
      // value norms discard the K rows of a tile that straddles K and V: they read W_V's
      // first rows instead, so W_K is never needed there
      const uint16_t* wrow = f >= a.kv ? Lp.WV + (size_t)(f - a.kv) * kdim
                             : MODE == 1 ? Lp.WV : Lp.WK + (size_t)f * kdim;
      Fo.base[p] = reinterpret_cast<const unsigned char*>(wrow);
      Fo.off[p] = (uint32_t)((dma_lane_row(lane) * kdim + ce) * 2);
      if (folded) {                        // rows of x_S gathered through the index list
        To.base[p] = reinterpret_cast<const unsigned char*>(a.xS);
        To.off[p] = (uint32_t)(((size_t)row[p] * a.x_stride + ce) * 2);
      } else {
        To.base[p] = reinterpret_cast<const unsigned char*>(hb + (size_t)(t0 + r0) * a.d);
        To.off[p] = Fo.off[p];
      }
    }
  }

  // Per row of the tile: 1/sqrt(mean(x_hat^2) + eps), and the element offset of its slot in
  // the page pools (-1: skip the row); per feature of a key head the key-norm weight, per
  // value head its rescale factor.  Fetched under the main loop, parked in LDS after it.
  __shared__ float rstd[kTile];
  __shared__ long long rowoff[kTile];
  __shared__ __attribute__((aligned(16))) float skn[128];
  __shared__ float svs[kTile];
  __shared__ __attribute__((aligned(16))) float sfc[kTile];
  const float my_r = rs_tab[t0 + tid];
  long long my_off = -1;
  float my_kn = 1.f, my_vs = 1.f, my_c = 0.f;
  if (MODE == 0) {
    my_off = a.row_slot[t0 + tid];
    if (a.has_knorm && tid < a.hd) my_kn = bf16_to_f32(gload(Lp.kn + tid));
    if (Lp.vs && tid < a.n_kv) my_vs = gload(Lp.vs + tid);
  }
  if (folded) my_c = gload(Lp.fc + f0 + tid);

  f32x16 acc[4][4];
  gemm_pipeline(acc, Fo, To, kdim, smem);

  rstd[tid] = my_r;
  rowoff[tid] = my_off;
  if (tid < 128) skn[tid] = my_kn;
  svs[tid] = my_vs;
  sfc[tid] = my_c;
  // A tile with K features: the RoPE tables of its 256 rows (in the blocked layout, cos and
  // sin each one contiguous run of half KB) go by direct loads into the LDS the main loop has
  // left, cos at 0 and sin at 64 KB, and are waited for once here.  (Loaded from memory where
  // each 32-row block is rotated, they cost several round trips per block.)
  const int half = a.hd >> 1;
  const bool tabs = MODE == 0 && f0 < a.kv;
  if (tabs) {
    const int dwave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const size_t tbase = (size_t)(t0 >> 5) * (half >> 2) * 128;   // floats
    const uint32_t lbase = lds_addr(smem);
    const uint32_t voff = (uint32_t)(tid & 63) * 16;
    for (int c = dwave; c < 2 * half; c += 4) {    // 1 KB chunks: cos 0 .. half - 1, then sin
      const bool sinc = c >= half;
      const int cc = sinc ? c - half : c;
      dma16((sinc ? a.rsin : a.rcos) + tbase + (size_t)cc * 256, voff,
            lbase + (sinc ? 65536u : 0u) + (uint32_t)cc * 1024);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();

  const int lane = tid & 63, wave = tid >> 6, wf = wave >> 1, wt = wave & 1, h = lane >> 5;
  const int fw = f0 + wf * 128;                  // the wave's first feature
  const bool isK = fw < a.kv;                    // kv % 128 == 0: a wave is all K or all V
  if (MODE == 1) {
    if (isK) return;                             // a tile may straddle K and V (kv % 256 != 0)
    // heads (fw - kv) / hd and, for hd = 64, the next one
    const int h0 = (fw - a.kv) / a.hd;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int tl = wt * 128 + n * 32 + (lane & 31);
      const int tok = t0 + tl;
      const float r = rstd[tl];
      if (folded) {           // P x + c: the value before the 1/rms scale
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 cv = *reinterpret_cast<const f32x4*>(sfc + wf * 128 + m * 32 + q * 8 + h * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[m][n][q * 4 + e] += cv[e];
          }
      }
      float s0, s1;
      head_sumsq(acc, n, a.hd, s0, s1);
      if (h == 0 && tok < a.n_filled) {
        float* out = a.vnorm + ((size_t)g * a.mpad + tok) * a.n_kv;
        out[h0] = r * sqrtf(s0);
        if (a.hd == 64) out[h0 + 1] = r * sqrtf(s1);
      }
    }
    return;
  }
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int tl = wt * 128 + n * 32 + (lane & 31);
    const float r = rstd[tl];   // rows past n_filled: finite padding, never stored
    if (folded) {             // (P x + c) / rms
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 cv = *reinterpret_cast<const f32x4*>(sfc + wf * 128 + m * 32 + q * 8 + h * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[m][n][q * 4 + e] = (acc[m][n][q * 4 + e] + cv[e]) * r;
        }
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[m][n][e] *= r;
    }
    if (isK) {
      if (a.has_knorm) {
        float s0, s1;
        head_sumsq(acc, n, a.hd, s0, s1);
        const float k0 = 1.0f / sqrtf(s0 / (float)a.hd + a.eps);
        const float k1 = 1.0f / sqrtf(s1 / (float)a.hd + a.eps);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float km = (m * 32 < a.hd) ? k0 : k1;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 wk = *reinterpret_cast<const f32x4*>(skn + ((m * 32 + q * 8 + h * 4) & (a.hd - 1)));
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[m][n][q * 4 + e] *= km * wk[e];
          }
        }
      }
      const int e0 = ((tl >> 5) * (half >> 2) + h) * 128 + (tl & 31) * 4;   // tile-relative
      const float* cs = reinterpret_cast<const float*>(smem) + e0;
      const float* sn = reinterpret_cast<const float*>(smem + 65536) + e0;
      if (a.hd == 128) {
        rope_pair<0, 2, 0>(acc, n, cs, sn);
        rope_pair<1, 3, 32>(acc, n, cs, sn);
      } else {
        rope_pair<0, 1, 0>(acc, n, cs, sn);
        rope_pair<2, 3, 0>(acc, n, cs, sn);
      }
    } else if (Lp.vs) {
      // value rescale: one factor per head
      const int hv = (fw - a.kv) / a.hd;
      const float v0 = svs[hv];
      const float v1 = a.hd == 64 ? svs[hv + 1] : v0;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float vm = (m * 32 < a.hd) ? v0 : v1;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[m][n][e] *= vm;
      }
    }
    // straight to the token's page slot (off < 0: the row is not stored)
    const long long off = rowoff[tl];
    uint16_t* row = (isK ? Lp.kp : Lp.vp) + off + (isK ? fw : fw - a.kv);
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int e = 8 * p;                   // runs q = 2 p and 2 p + 1
        store_run_pair(row + m * 32 + 16 * p, h, pack_bf16x2(acc[m][n][e], acc[m][n][e + 1]),
                       pack_bf16x2(acc[m][n][e + 2], acc[m][n][e + 3]),
                       pack_bf16x2(acc[m][n][e + 4], acc[m][n][e + 5]),
                       pack_bf16x2(acc[m][n][e + 6], acc[m][n][e + 7]), off >= 0);
      }
  }
}

template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void fill_kv_kernel(FillKArgs a) {
  fill_kv_tile<MODE>(a, xcd_remap(blockIdx.x, gridDim.x));
}

// cos/sin of angle t * theta^(-2j/hd) for every row of the padded filled list (padding
// rows use t = 0), computed in fp64 and stored in the blocked layout the kv epilogue reads:
// element ((row / 32) * (hd / 8) + j / 4) * 128 + (row % 32) * 4 + j % 4.
__global__ void rope_table_kernel(const int32_t* idx, int n_filled, int mpad, int64_t P, int hd,
                                  double theta, float* rcos, float* rsin) {
  const int half = hd >> 1, jg = half >> 2;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)mpad * half) return;
  const int e = (int)(i & 3), rl = (int)((i >> 2) & 31);
  const int64_t blk = i >> 7;
  const int rb = (int)(blk / jg), j = (int)(blk - (int64_t)rb * jg) * 4 + e;
  const int row = rb * 32 + rl;
  int t = row < n_filled ? idx[row] : 0;
  if (t < 0 || t >= P) t = 0;
  const double inv = pow(theta, -2.0 * (double)j / (double)hd);
  double s, cth;
  sincos((double)t * inv, &s, &cth);
  rcos[i] = (float)cth;
  rsin[i] = (float)s;
}

// Over the padded filled list: flags indices that are out of the prefix, not strictly
// increasing, or whose page is missing from the block table, and stores each row's
// element offset in the page pools (-1 for flagged and padding rows, which the kv
// epilogue skips).
__global__ void row_slot_kernel(const int32_t* idx, int n_filled, int mpad, int64_t P,
                                const int32_t* bt, int64_t n_logical, int ps, int num_pages,
                                int kv, int64_t* slot, unsigned* status) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= mpad) return;
  int64_t off = -1;
  if (i < n_filled) {
    const int t = idx[i];
    bool bad = t < 0 || t >= P;
    if (!bad && i > 0 && idx[i - 1] >= t) bad = true;
    if (!bad) {
      const int64_t lp = t / ps;
      if (lp >= n_logical) {
        bad = true;
      } else {
        const int pg = bt[lp];
        bad = pg < 0 || pg >= num_pages;
        if (!bad) off = ((int64_t)pg * ps + (t - lp * ps)) * kv;
      }
    }
    if (bad) atomicOr(status, kStatusRowsBit);
  }
  slot[i] = off;
}

// 1/sqrt(mean(x_hat^2) + eps) per padded row and layer of a launch group, from the map
// kernel's per-128-feature partial sums (added in a fixed order).
__global__ void rstd_kernel(unsigned char* layer_ws, size_t per_layer, size_t per_layer_h,
                            size_t per_layer_ssq, int mpad, int nchunk, int d, float eps) {
  const int row = blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= mpad) return;
  unsigned char* lw = layer_ws + (size_t)blockIdx.y * per_layer;
  const float* p = reinterpret_cast<const float*>(lw + per_layer_h) + row;
  float s = 0.f;
  for (int c = 0; c < nchunk; ++c) s += p[(size_t)c * mpad];
  reinterpret_cast<float*>(lw + per_layer_h + per_layer_ssq)[row] = 1.0f / sqrtf(s / (float)d + eps);
}

// Folded layers: 1/sqrt((sum of the partials + kappa) / d + eps), d the map's output width.
__global__ void rstd_folded_kernel(FillKArgs a) {
  const int row = blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= a.mpad) return;
  const int g = blockIdx.y;
  unsigned char* lw = a.layer_ws + (size_t)g * a.per_layer;
  const float* p = reinterpret_cast<const float*>(lw + a.per_layer_h) + row;
  float s = 0.f;
  for (int c = 0; c < a.nchunk; ++c) s += p[(size_t)c * a.mpad];
  s = fmaxf(s + gload(layer_ptrs(a, g).kap), 0.f);
  reinterpret_cast<float*>(lw + a.per_layer_h + a.per_layer_ssq)[row] =
      1.0f / sqrtf(s / (float)a.d + a.eps);
}

// Exact tail inputs of the value rescale, one wave per (row, exact entry): bf16(x * w) and
// 1/sqrt(mean(x^2) + eps), written where the map kernel and rstd_kernel put the predicted
// ones, so the value-norm pass reads both the same way.  Padding rows get zeros.  Entry l of
// the exact side is table entry G + l: its w is the layer's norm weight and its A field holds
// the layer's exact rows x (bf16 [c][d]), which no other kernel reads from those entries.
// The waves of entry 0 also write the identity index list (row i -> i) that the predicted
// side gathers its rows through.
struct ExactArgs {
  const FillLayerPtrs* tab;     // the exact entries
  int32_t* idx;
  int c, d;
  float eps;
  unsigned char* layer_ws;      // the first exact entry's area
  size_t per_layer, per_layer_h, per_layer_ssq;
};

__global__ __launch_bounds__(256) void exact_rows_kernel(ExactArgs a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), l = blockIdx.y, lane = threadIdx.x & 63;
  const uint16_t* xr = a.tab[l].A;    // read once, before any store
  const uint16_t* w = a.tab[l].w;
  const uint16_t* x = xr + (size_t)row * a.d;
  unsigned char* lw = a.layer_ws + (size_t)l * a.per_layer;
  uint16_t* hb = reinterpret_cast<uint16_t*>(lw) + (size_t)row * a.d;
  const bool live = row < a.c;
  const int nch = a.d >> 3;                     // 16-byte chunks of a row
  float s = 0.f;
  for (int c0 = 0; c0 < nch; c0 += 4 * 64) {    // four chunks per lane in flight
    u32x4 xv[4], wv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c8 = c0 + j * 64 + lane;
      xv[j] = u32x4{0u, 0u, 0u, 0u};
      wv[j] = u32x4{0u, 0u, 0u, 0u};
      if (live && c8 < nch) {
        xv[j] = *reinterpret_cast<const u32x4*>(x + c8 * 8);
        wv[j] = *reinterpret_cast<const u32x4*>(w + c8 * 8);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c8 = c0 + j * 64 + lane;
      u32x4 o;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float x0 = bf16_to_f32(xv[j][k] & 0xffffu), x1 = bf16_to_f32(xv[j][k] >> 16);
        s += x0 * x0;
        s += x1 * x1;
        o[k] = pack_bf16x2(x0 * bf16_to_f32(wv[j][k] & 0xffffu), x1 * bf16_to_f32(wv[j][k] >> 16));
      }
      if (c8 < nch) *reinterpret_cast<u32x4*>(hb + c8 * 8) = o;
    }
  }
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) s += __shfl_xor(s, m);   // fixed butterfly: deterministic
  if (lane == 0) {
    float* rs = reinterpret_cast<float*>(lw + a.per_layer_h + a.per_layer_ssq);
    rs[row] = live ? 1.0f / sqrtf(s / (float)a.d + a.eps) : 0.f;
    if (l == 0) a.idx[row] = row;
  }
}

// Layer-pointer table entries [first, first + n) from the arguments into device memory, one
// thread per entry.
constexpr int kTableChunk = 32;
struct LayerTableChunk {
  FillLayerPtrs e[kTableChunk];
  FillLayerPtrs* dst;
  int n;
};
static_assert(sizeof(LayerTableChunk) <= 4096, "kernel arguments must fit in 4 KB");

__global__ void layer_table_kernel(LayerTableChunk c) {
  const int i = threadIdx.x;
  if (i < c.n) c.dst[i] = c.e[i];
}

// v_scale[l][h] = mean over the c rows of |v_exact| / |v_pred|: one block per (l, h); thread
// t adds rows t, t + 256, ... in fp64, then a fixed-order tree adds the 256 partials
// (deterministic).
__global__ __launch_bounds__(256) void vscale_kernel(const float* vn_pred, const float* vn_exact,
                                                     int c, int cpad, int n_kv, float* out) {
  __shared__ double part[256];
  const int i = blockIdx.x, l = i / n_kv, hh = i - l * n_kv, t = threadIdx.x;
  double s = 0.0;
  for (int r = t; r < c; r += 256) {
    const size_t k = ((size_t)l * cpad + r) * n_kv + hh;
    s += (double)vn_exact[k] / (double)vn_pred[k];
  }
  part[t] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w) part[t] += part[t + w];
    __syncthreads();
  }
  if (t == 0) out[i] = (float)(part[0] / c);
}

}  // namespace

__global__ void clear_status_kernel(unsigned* status) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *status = 0u;
}

hipError_t launch_clear_status(unsigned* status, hipStream_t stream) {
  hipLaunchKernelGGL(clear_status_kernel, dim3(1), dim3(64), 0, stream, status);
  return hipGetLastError();
}

FillWsLayout fill_ws_layout(int d, int d_in, int hd, int kv, int64_t n_filled, unsigned flags) {
  FillWsLayout L = {};
  const int64_t mpad = (n_filled + kTile - 1) / kTile * kTile;
  const size_t table = align256((size_t)mpad * (hd / 2) * sizeof(float));
  L.rope_cos = kStatusBytes;
  L.rope_sin = L.rope_cos + table;
  L.row_slot = L.rope_sin + table;
  L.fixed = L.row_slot + align256((size_t)mpad * sizeof(int64_t));
  const bool folded = (flags & kWsFolded) != 0;
  L.per_layer_h = folded ? 0 : align256((size_t)mpad * d * 2);
  L.per_layer_ssq = align256((size_t)mpad * ((folded ? d_in : d) / 128) * sizeof(float));
  L.per_layer_rstd = align256((size_t)mpad * sizeof(float));
  const size_t map_elems = (size_t)d * d_in;
  L.land = L.per_layer_h + L.per_layer_ssq + L.per_layer_rstd;
  // a landing slot holds one layer's streamed map, or its whole folded buffer
  if (flags & kWsStreamed)
    L.land_slot = folded ? fold_layout(d_in, kv).total
                         : align256(map_elems * ((flags & kWsInt8) ? 1 : 2));
  L.per_layer = L.land + 2 * L.land_slot;
  L.hbuf = L.fixed;
  return L;
}

namespace {

constexpr int kMaxDevices = 64;   // per-device host caches

// Workgroups of a persistent tile launch: one per CU, a multiple of 8 (the XCD count), or
// the item count when that is smaller.  The CU count is read once per device (threads that
// race on the first read store the same value).
int persist_grid(int n_items) {
  static std::atomic<int> cus[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  int c = cus[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 256;
    c = n >= 8 ? n & ~7 : 8;
    cus[dev].store(c, std::memory_order_relaxed);
  }
  return n_items < c ? n_items : c;
}

// A persistent tile launch of n_items items.
template <typename Kernel>
void launch_tiles(Kernel kernel, FillKArgs& a, int n_items, hipStream_t stream) {
  a.n_items = n_items;
  if (n_items > 0)
    hipLaunchKernelGGL(kernel, dim3(persist_grid(n_items)), dim3(kThreads), 0, stream, a);
}

FillKArgs fill_args(const FillPlan& p, unsigned char* layer_ws) {
  FillKArgs a = {};
  a.xS = p.xS;
  a.x_stride = p.x_stride;
  a.idx = p.idx;
  a.P = p.P;
  a.n_filled = p.n_filled;
  a.d = p.d;
  a.d_in = p.d_in;
  a.kv = p.kv;
  a.hd = p.hd;
  a.n_kv = p.n_kv;
  a.eps = p.eps;
  a.mpad = p.mpad;
  a.folded = (p.flags & kWsFolded) ? 1 : 0;
  a.nchunk = (a.folded ? p.d_in : p.d) / 128;
  a.kdim = a.folded ? p.d_in : p.d;
  a.layer_ws = layer_ws;
  a.per_layer = p.L.per_layer;
  a.per_layer_h = p.L.per_layer_h;
  a.per_layer_ssq = p.L.per_layer_ssq;
  a.rcos = p.rope_cos;
  a.rsin = p.rope_sin;
  a.row_slot = p.row_slot;
  a.ntt = p.mpad / kTile;
  a.has_scale = (p.flags & kWsInt8) ? 1 : 0;
  a.has_knorm = p.has_knorm;
  return a;
}

// Status clear, row validation and page slots, RoPE tables: once per call.
hipError_t launch_fill_prep(const FillPlan& p, hipStream_t stream) {
  hipError_t e = launch_clear_status(p.status, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(row_slot_kernel, dim3(p.mpad / 256), dim3(256), 0, stream, p.idx, p.n_filled,
                     p.mpad, (int64_t)p.P, p.block_table, p.n_logical, p.page_size, p.num_pages,
                     p.kv, p.row_slot, p.status);
  const int64_t nt = (int64_t)p.mpad * (p.hd / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((nt + 255) / 256)), dim3(256), 0, stream,
                     p.idx, p.n_filled, p.mpad, (int64_t)p.P, p.hd, p.theta, p.rope_cos,
                     p.rope_sin);
  return hipGetLastError();
}

// Map GEMM, 1/RMS, K/V GEMM for the G layers in a.L (their maps already on the device).
hipError_t launch_fill_group(const FillPlan& p, FillKArgs& a, int G, hipStream_t stream) {
  a.f_base = 0;
  if (a.folded) {
    a.nft = (p.d_in / kTile + 1) / 2;          // pairs of R tiles
    {
      ProfileScope ps(RF_KERNEL_FILL_NORM, stream);
      launch_tiles(fill_norm_kernel, a, G * a.ntt * a.nft, stream);
    }
    hipLaunchKernelGGL(rstd_folded_kernel, dim3(p.mpad / 256, G), dim3(256), 0, stream, a);
    a.nft = 2 * p.kv / kTile;
    {
      ProfileScope ps(RF_KERNEL_FILL_KV, stream);
      hipLaunchKernelGGL(fill_kv_kernel<0>, dim3(G * a.ntt * a.nft), dim3(kThreads), 0, stream, a);
    }
    return hipGetLastError();
  }
  a.nft = p.d / kTile;
  {
    ProfileScope ps(RF_KERNEL_FILL_MAP, stream);
    if (a.has_scale)
      hipLaunchKernelGGL(fill_map_kernel<1>, dim3(G * a.ntt * a.nft), dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL(fill_map_kernel<0>, dim3(G * a.ntt * a.nft), dim3(kThreads), 0, stream, a);
  }
  hipLaunchKernelGGL(rstd_kernel, dim3(p.mpad / 256, G), dim3(256), 0, stream, a.layer_ws,
                     a.per_layer, a.per_layer_h, a.per_layer_ssq, p.mpad, a.nchunk, p.d, p.eps);
  a.nft = 2 * p.kv / kTile;
  {
    ProfileScope ps(RF_KERNEL_FILL_KV, stream);
    hipLaunchKernelGGL(fill_kv_kernel<0>, dim3(G * a.ntt * a.nft), dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

// Balanced groups of at most `group` layers: as few, equal launches as the workspace allows.
int group_size(int n_layers, int group) {
  const int ngroups = (n_layers + group - 1) / group;
  return (n_layers + ngroups - 1) / ngroups;
}

// A folded buffer from host memory into a landing slot: P whole; of R only what the norm
// kernel reads (block row f0 .. f0 + 255 from column f0 on: the zeros left of the diagonal
// blocks, about half of R, stay behind and the slot's bytes there are never read); then c,
// r and kappa.  d_in is a multiple of kTile.
hipError_t copy_folded(unsigned char* land, const unsigned char* src, const FoldLayout& F,
                       int d_in, hipStream_t s) {
  hipError_t e = hipMemcpyAsync(land + F.P, src + F.P, F.R - F.P, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return e;
  const size_t pitch = (size_t)d_in * 2;
  for (int f0 = 0; f0 < d_in; f0 += kTile) {
    const size_t off = F.R + (size_t)f0 * pitch + (size_t)f0 * 2;
    e = hipMemcpy2DAsync(land + off, pitch, src + off, pitch, (size_t)(d_in - f0) * 2, kTile,
                         hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return e;
  }
  return hipMemcpyAsync(land + F.c, src + F.c, F.total - F.c, hipMemcpyHostToDevice, s);
}

struct StreamEvents {
  hipEvent_t ready[2] = {nullptr, nullptr};
  hipEvent_t done[2] = {nullptr, nullptr};
  hipEvent_t start = nullptr;
};

}  // namespace

// ------------------------------------------------------------- fixed scratch
// The workspace of ridgefill_fill_noalloc: a file-scope device array, one copy per device
// (each device that loads the library holds it until the process ends).  Host code never
// passes the array's name to a kernel or a copy (on the host it is only a stand-in for the
// symbol): the per-device device address comes from hipGetSymbolAddress, looked up once per
// device on the first call made with that device current, and kernels receive it as a
// plain pointer.
namespace {
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
std::atomic<void*> g_scratch_addr[kMaxDevices];
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_fill(const FillPlan& p, const FillLayerPtrs* layers, int n_layers,
                       hipStream_t stream) {
  hipError_t e = launch_fill_prep(p, stream);
  if (e != hipSuccess) return e;
  unsigned char* lws = reinterpret_cast<unsigned char*>(p.hbuf);
  const int gsize = group_size(n_layers, p.group);
  for (int l0 = 0; l0 < n_layers; l0 += gsize) {
    const int G = (n_layers - l0) < gsize ? (n_layers - l0) : gsize;
    FillKArgs a = fill_args(p, lws);
    for (int g = 0; g < G; ++g) a.L[g] = layers[l0 + g];
    if ((e = launch_fill_group(p, a, G, stream)) != hipSuccess) return e;
  }
  return hipSuccess;
}

// Maps in (pinned) host memory: group g's maps are copied on copy_stream into landing slot
// g % 2 of its layer blocks while group g - 1 computes on `stream`; the copy into a slot
// waits until the group that used it two steps before has finished.
hipError_t launch_fill_streamed(const FillPlan& p, const FillLayerPtrs* layers, int n_layers,
                                hipStream_t stream, hipStream_t copy_stream) {
  // events per host thread and device, created on first use
  static thread_local StreamEvents evs[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  StreamEvents& ev = evs[dev];
  for (int i = 0; i < 2; ++i) {
    if (!ev.ready[i] && (e = hipEventCreateWithFlags(&ev.ready[i], hipEventDisableTiming)) != hipSuccess) return e;
    if (!ev.done[i] && (e = hipEventCreateWithFlags(&ev.done[i], hipEventDisableTiming)) != hipSuccess) return e;
  }
  if (!ev.start && (e = hipEventCreateWithFlags(&ev.start, hipEventDisableTiming)) != hipSuccess) return e;
  // this call's copies start after the work already on `stream`: a previous call's last
  // groups may still be reading the landing slots
  if ((e = hipEventRecord(ev.start, stream)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(copy_stream, ev.start, 0)) != hipSuccess) return e;
  if ((e = launch_fill_prep(p, stream)) != hipSuccess) return e;
  unsigned char* lws = reinterpret_cast<unsigned char*>(p.hbuf);
  const bool int8 = (p.flags & kWsInt8) != 0;
  const bool folded = (p.flags & kWsFolded) != 0;
  const FoldLayout F = fold_layout(p.d_in, p.kv);
  const size_t map_bytes = folded ? F.total : (size_t)p.d * p.d_in * (int8 ? 1 : 2);
  // Group sizes ramp up 1, 2, 3, ... to the workspace's group size: only the first
  // layer's copy waits with no compute to hide under, and each later group's copy is
  // about as long as the previous group's compute or shorter (a group of 4 folded 27B-shape
  // layers copies in ~7 ms, which a first group of that size would leave exposed).
  const int gmax = p.group;
  int gi = 0;
  for (int l0 = 0, G = 0; l0 < n_layers; l0 += G, ++gi) {
    const int want = gi + 1 < gmax ? gi + 1 : gmax;
    G = (n_layers - l0) < want ? (n_layers - l0) : want;
    const int slot = gi & 1;
    if (gi >= 2 && (e = hipStreamWaitEvent(copy_stream, ev.done[slot], 0)) != hipSuccess) return e;
    FillKArgs a = fill_args(p, lws);
    for (int g = 0; g < G; ++g) {
      a.L[g] = layers[l0 + g];
      unsigned char* land = lws + g * p.L.per_layer + p.L.land + slot * p.L.land_slot;
      if (folded) {
        // a folded layer's A points at R inside its host buffer: the buffer starts F.R before
        const unsigned char* src = reinterpret_cast<const unsigned char*>(layers[l0 + g].A) - F.R;
        if ((e = copy_folded(land, src, F, p.d_in, copy_stream)) != hipSuccess) return e;
      } else {
        const void* src = int8 ? static_cast<const void*>(layers[l0 + g].Aq)
                               : static_cast<const void*>(layers[l0 + g].A);
        if ((e = hipMemcpyAsync(land, src, map_bytes, hipMemcpyHostToDevice, copy_stream)) != hipSuccess)
          return e;
      }
      if (int8) {
        a.L[g].Aq = reinterpret_cast<const int8_t*>(land);
      } else if (folded) {
        const uint16_t* P = reinterpret_cast<const uint16_t*>(land + F.P);
        a.L[g].A = reinterpret_cast<const uint16_t*>(land + F.R);
        a.L[g].b = reinterpret_cast<const float*>(land + F.r);
        a.L[g].WK = P;
        a.L[g].WV = P + (size_t)p.kv * p.d_in;
        a.L[g].fc = reinterpret_cast<const float*>(land + F.c);
        a.L[g].kap = reinterpret_cast<const float*>(land + F.kappa);
        a.L[g].fg = reinterpret_cast<const float*>(land + F.g);
      } else {
        a.L[g].A = reinterpret_cast<const uint16_t*>(land);
      }
    }
    if ((e = hipEventRecord(ev.ready[slot], copy_stream)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(stream, ev.ready[slot], 0)) != hipSuccess) return e;
    if ((e = launch_fill_group(p, a, G, stream)) != hipSuccess) return e;
    if ((e = hipEventRecord(ev.done[slot], stream)) != hipSuccess) return e;
  }
  return hipSuccess;
}

// Value-rescale factors: the c tail rows (indices 0 .. c-1 of x_S_tail) through the map,
// RMSNorm and W_V, and the exact tail inputs through RMSNorm and W_V; per (row, head) the
// two value norms; per head the mean of their ratio.  A group of G layers runs as: the map
// (or the folded norm) and 1/rms of the predicted rows for all G layers in one launch; the
// exact rows' bf16(x_l * w) and 1/rms; then the value norms of both sides in one launch over
// 2 G table entries (the G layers, then G plain entries with the layers' own W_V whose
// staged rows are the exact ones); then the factors.  Layer pointers come from a table in
// the workspace, so a group may hold more layers than the kernel arguments could.
hipError_t launch_value_scale(const FillPlan& p, const FillLayerPtrs* layers,
                              const uint16_t* const* x_exact, const uint16_t* const* exact_wv,
                              int n_layers, float* out, const VsLayout& V, hipStream_t stream) {
  hipError_t e = launch_clear_status(p.status, stream);
  if (e != hipSuccess) return e;
  unsigned char* pred = reinterpret_cast<unsigned char*>(p.hbuf);
  const int gsize = group_size(n_layers, p.group);
  for (int l0 = 0; l0 < n_layers; l0 += gsize) {
    const int G = (n_layers - l0) < gsize ? (n_layers - l0) : gsize;
    // the table: entries 0 .. G-1 the layers, G .. 2G-1 the exact side (W_V, norm weight)
    for (int c0 = 0; c0 < 2 * G; c0 += kTableChunk) {
      LayerTableChunk t = {};
      t.n = (2 * G - c0) < kTableChunk ? (2 * G - c0) : kTableChunk;
      t.dst = V.table + c0;
      for (int i = 0; i < t.n; ++i) {
        const int k = c0 + i;
        if (k < G) {
          t.e[i] = layers[l0 + k];
        } else {
          t.e[i].w = layers[l0 + k - G].w;
          t.e[i].WV = exact_wv[l0 + k - G];
          t.e[i].A = x_exact[l0 + k - G];
        }
      }
      hipLaunchKernelGGL(layer_table_kernel, dim3(1), dim3(kTableChunk), 0, stream, t);
    }
    // the exact rows into the G blocks after the predicted ones (and the index list 0 .. mpad-1)
    ExactArgs x = {};
    x.tab = V.table + G;
    x.idx = const_cast<int32_t*>(p.idx);
    x.c = p.n_filled;
    x.d = p.d;
    x.eps = p.eps;
    x.layer_ws = pred + (size_t)G * p.L.per_layer;
    x.per_layer = p.L.per_layer;
    x.per_layer_h = p.L.per_layer_h;
    x.per_layer_ssq = p.L.per_layer_ssq;
    hipLaunchKernelGGL(exact_rows_kernel, dim3(p.mpad / 4, G), dim3(256), 0, stream, x);
    FillKArgs a = fill_args(p, pred);
    a.Ltab = V.table;
    a.f_base = 0;
    if (a.folded) {              // |x_hat|^2 from the triangular factor, then 1/rms
      a.nft = (p.d_in / kTile + 1) / 2;
      launch_tiles(fill_norm_kernel, a, G * a.ntt * a.nft, stream);
      hipLaunchKernelGGL(rstd_folded_kernel, dim3(p.mpad / 256, G), dim3(256), 0, stream, a);
    } else {
      a.nft = p.d / kTile;
      if (a.has_scale)
        hipLaunchKernelGGL(fill_map_kernel<1>, dim3(G * a.ntt * a.nft), dim3(kThreads), 0, stream, a);
      else
        hipLaunchKernelGGL(fill_map_kernel<0>, dim3(G * a.ntt * a.nft), dim3(kThreads), 0, stream, a);
      hipLaunchKernelGGL(rstd_kernel, dim3(p.mpad / 256, G), dim3(256), 0, stream, a.layer_ws,
                         a.per_layer, a.per_layer_h, a.per_layer_ssq, p.mpad, a.nchunk, p.d, p.eps);
    }
    // value norms of both sides: the tiles that hold V features of 2 G entries
    a.f_base = p.kv / kTile;
    a.nft = 2 * p.kv / kTile - a.f_base;
    a.vnorm = V.vn;
    hipLaunchKernelGGL(fill_kv_kernel<1>, dim3(2 * G * a.ntt * a.nft), dim3(kThreads), 0, stream, a);
    hipLaunchKernelGGL(vscale_kernel, dim3(G * p.n_kv), dim3(256), 0, stream, V.vn,
                       V.vn + (size_t)G * p.mpad * p.n_kv, p.n_filled, p.mpad, p.n_kv,
                       out + (size_t)l0 * p.n_kv);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace rf
