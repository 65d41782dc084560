// Exact-row selection from supplied row scores on gfx950.
//
// Source: English RidgeFill review (jaehun.me), section "Which rows to compute exactly",
// attention selection: the rows that receive the most attention are computed exactly; the
// rest of the prefix is filled.  Given one score per prefix row, the k rows with the
// largest score (ties to the lower row index) are marked exact and the others are
// compacted, in ascending order, into the filled-row list the fill takes.
//
// Order: every row gets a unique 64-bit key, high word = the score's bits mapped to an
// unsigned order (negative scores flipped, non-negative ones offset; -0.0 folded onto
// +0.0 so the two tie), low word = ~row, so equal scores rank the lower row higher.  The
// k-th largest key is found by a most-significant-digit radix select, 8 bits per pass:
// a histogram of the next digit over the keys that share the digits found so far, then a
// scan of that histogram from the top.  Keys >= the k-th are exactly the k selected rows.
// Counts are integers, so the atomics in the histogram leave the result deterministic.
#include "rf_common.h"
#include "rf_internal.h"
#include "ridgefill.h"

namespace rf {

namespace {

struct SelState {
  unsigned long long prefix;    // digits found so far, in place
  unsigned long long mask;      // which bits of prefix are found
  unsigned long long k_rem;     // rank still to find among keys matching prefix
  unsigned long long pad;
};

__device__ __forceinline__ uint32_t score_order(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;                     // -0.0 ties with +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ unsigned long long row_key(const float* scores, int64_t i,
                                                      unsigned* status) {
  float s = scores[i];
  if (s != s) {                                    // NaN: flagged, ranked lowest
    atomicOr(status, kStatusScoreBit);
    s = -__builtin_huge_valf();
  }
  return ((unsigned long long)score_order(s) << 32) | (unsigned long long)(0xffffffffu - (uint32_t)i);
}

__global__ void sel_init_kernel(SelState* st, unsigned* hist, unsigned long long k) {
  const int t = threadIdx.x;
  if (t == 0) {
    st->prefix = 0ull;
    st->mask = 0ull;
    st->k_rem = k;
  }
  hist[t] = 0u;
}

// Histogram of the digit at `shift` over the keys that match the found prefix.
__global__ void sel_hist_kernel(const float* scores, int64_t P, const SelState* st, unsigned* hist,
                                int shift, unsigned* status) {
  __shared__ unsigned h[256];
  h[threadIdx.x] = 0u;
  __syncthreads();
  const unsigned long long prefix = st->prefix, mask = st->mask;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < P;
       i += (int64_t)gridDim.x * blockDim.x) {
    const unsigned long long key = row_key(scores, i, status);
    if ((key & mask) == prefix) atomicAdd(&h[(key >> shift) & 0xffu], 1u);
  }
  __syncthreads();
  if (h[threadIdx.x]) atomicAdd(&hist[threadIdx.x], h[threadIdx.x]);
}

// One block of 256: the digit whose bucket holds the k_rem-th largest matching key.
__global__ void sel_digit_kernel(SelState* st, unsigned* hist, int shift) {
  __shared__ unsigned long long above[256];         // matching keys with a larger digit
  __shared__ unsigned hv[256];
  const int t = threadIdx.x;
  hv[t] = hist[t];
  __syncthreads();
  if (t == 0) {
    unsigned long long run = 0ull;
    for (int d = 255; d >= 0; --d) {
      above[d] = run;                               // keys with a larger digit
      run += hv[d];
    }
  }
  __syncthreads();
  const unsigned long long k = st->k_rem;
  const bool mine = above[t] < k && k <= above[t] + hv[t];
  __syncthreads();
  if (mine) {
    st->prefix |= (unsigned long long)t << shift;
    st->mask |= 0xffull << shift;
    st->k_rem = k - above[t];
  }
  hist[t] = 0u;                                     // ready for the next pass
}

// exact[i] = key(i) >= threshold; per block of 1024 rows, the count of filled rows.
__global__ void sel_mark_kernel(const float* scores, int64_t P, const SelState* st, int64_t k,
                                uint8_t* exact, unsigned* block_count, unsigned* status) {
  __shared__ unsigned cnt;
  if (threadIdx.x == 0) cnt = 0u;
  __syncthreads();
  const unsigned long long thr = st->prefix;
  unsigned mine = 0u;
  for (int j = 0; j < 4; ++j) {
    const int64_t i = (int64_t)blockIdx.x * 1024 + j * 256 + threadIdx.x;
    if (i < P) {
      const bool ex = k > 0 && row_key(scores, i, status) >= thr;
      if (exact) exact[i] = ex ? 1 : 0;
      mine += ex ? 0u : 1u;
    }
  }
  atomicAdd(&cnt, mine);
  __syncthreads();
  if (threadIdx.x == 0) block_count[blockIdx.x] = cnt;
}

// Exclusive scan of the per-block counts (one block, in order).
__global__ void sel_scan_kernel(unsigned* block_count, int64_t nb) {
  __shared__ unsigned long long part[1024];
  __shared__ unsigned long long carry;
  if (threadIdx.x == 0) carry = 0ull;
  __syncthreads();
  for (int64_t base = 0; base < nb; base += 1024) {
    const int64_t i = base + threadIdx.x;
    const unsigned v = i < nb ? block_count[i] : 0u;
    part[threadIdx.x] = v;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {      // Hillis-Steele inclusive scan
      const unsigned long long add = threadIdx.x >= off ? part[threadIdx.x - off] : 0ull;
      __syncthreads();
      part[threadIdx.x] += add;
      __syncthreads();
    }
    if (i < nb) block_count[i] = (unsigned)(carry + part[threadIdx.x] - v);
    __syncthreads();
    if (threadIdx.x == 1023) carry += part[1023];
    __syncthreads();
  }
}

// Filled rows of each 1024-row block, in order, at the block's offset.
__global__ void sel_compact_kernel(const float* scores, int64_t P, const SelState* st, int64_t k,
                                   const unsigned* block_off, int32_t* filled, unsigned* status) {
  __shared__ unsigned part[1024];
  const unsigned long long thr = st->prefix;
  const int t = threadIdx.x;
  const int64_t i = (int64_t)blockIdx.x * 1024 + t;
  const bool keep = i < P && !(k > 0 && row_key(scores, i, status) >= thr);
  part[t] = keep ? 1u : 0u;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const unsigned add = t >= off ? part[t - off] : 0u;
    __syncthreads();
    part[t] += add;
    __syncthreads();
  }
  if (keep) filled[block_off[blockIdx.x] + part[t] - 1] = (int32_t)i;
}

}  // namespace

SelLayout select_layout(int64_t P) {
  SelLayout L;
  L.state = kStatusBytes;
  L.hist = L.state + 256;
  L.blocks = L.hist + 1024;
  const int64_t nb = (P + 1023) / 1024;
  L.total = L.blocks + align256((size_t)(nb > 0 ? nb : 1) * 4);
  return L;
}

hipError_t launch_select(const float* scores, int64_t P, int64_t k, uint8_t* exact,
                         int32_t* filled, void* ws, hipStream_t stream) {
  const SelLayout L = select_layout(P);
  unsigned char* w = static_cast<unsigned char*>(ws);
  unsigned* status = reinterpret_cast<unsigned*>(w);
  SelState* st = reinterpret_cast<SelState*>(w + L.state);
  unsigned* hist = reinterpret_cast<unsigned*>(w + L.hist);
  unsigned* blocks = reinterpret_cast<unsigned*>(w + L.blocks);
  hipError_t e = launch_clear_status(status, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sel_init_kernel, dim3(1), dim3(256), 0, stream, st, hist,
                     (unsigned long long)k);
  if (k > 0 && k < P) {
    const int grid = (int)((P + 255) / 256 < 1024 ? (P + 255) / 256 : 1024);
    for (int shift = 56; shift >= 0; shift -= 8) {
      hipLaunchKernelGGL(sel_hist_kernel, dim3(grid), dim3(256), 0, stream, scores, P, st, hist,
                         shift, status);
      hipLaunchKernelGGL(sel_digit_kernel, dim3(1), dim3(256), 0, stream, st, hist, shift);
    }
  }
  // k == P: every key passes the threshold 0; k == 0: nothing is exact (k > 0 test).
  const int64_t nb = (P + 1023) / 1024;
  hipLaunchKernelGGL(sel_mark_kernel, dim3((unsigned)nb), dim3(256), 0, stream, scores, P, st, k,
                     exact, blocks, status);
  hipLaunchKernelGGL(sel_scan_kernel, dim3(1), dim3(1024), 0, stream, blocks, nb);
  hipLaunchKernelGGL(sel_compact_kernel, dim3((unsigned)nb), dim3(1024), 0, stream, scores, P, st, k,
                     blocks, filled, status);
  return hipGetLastError();
}

}  // namespace rf

// ------------------------------------------------------------------------------
// int8 map quantization.  Section "Ridge map ...", map size paragraph (maps held in int8):
// symmetric, one scale per output row, scale = max |A[o, :]| / 127 and
// q = round-half-even(A / scale) clipped to [-127, 127] (a zero row: scale 0, q = 0).  All
// rounding decisions in fp32 with correctly rounded division.
namespace rf {
namespace {

__global__ void quantize_rows_kernel(const float* A, int64_t cols, int8_t* q, float* scale) {
  const int64_t row = blockIdx.x;
  const float* a = A + row * cols;
  __shared__ float red[256];
  float m = 0.f;
  for (int64_t c = threadIdx.x; c < cols; c += 256) m = fmaxf(m, fabsf(a[c]));
  red[threadIdx.x] = m;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  const float s = red[0] / 127.0f;
  if (threadIdx.x == 0) scale[row] = s;
  int8_t* out = q + row * cols;
  for (int64_t c = threadIdx.x; c < cols; c += 256) {
    float v = 0.f;
    if (s > 0.f) v = fminf(fmaxf(rintf(a[c] / s), -127.f), 127.f);
    out[c] = (int8_t)(int)v;
  }
}

}  // namespace

hipError_t launch_quantize(const float* A, int64_t rows, int64_t cols, int8_t* q, float* scale,
                           hipStream_t stream) {
  hipLaunchKernelGGL(quantize_rows_kernel, dim3((unsigned)rows), dim3(256), 0, stream, A, cols, q,
                     scale);
  return hipGetLastError();
}

}  // namespace rf
