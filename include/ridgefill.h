/*
 * ridgefill.h -- C ABI of the RidgeFill upper-layer KV fill, its one-pass calibration
 * and its closed-form ridge solve, for AMD Instinct MI355X (gfx950).
 *
 * Method source: the English RidgeFill review (jaehun.me, "paper-2611-09709v1", English
 * edition).  Each entry point names the section it implements.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers marked "device" point to GPU memory the caller allocated; pointers
 *    marked "host" point to CPU memory.  The library allocates no device memory,
 *    keeps no device state between calls and creates no streams (the streamed fill
 *    creates five HIP events per host thread and device on first use and reuses them;
 *    ridgefill_fill_noalloc works in a fixed array of RIDGEFILL_NOALLOC_SCRATCH_BYTES
 *    that is part of the library's device code, one per device, whose contents the
 *    next such call on that device overwrites).
 *    Every buffer it needs beyond inputs and outputs is a caller-owned workspace whose
 *    size a *_workspace_bytes / *_state_bytes query returns.
 *  - bf16 tensors are passed as uint16_t bit patterns (bfloat16, round-to-nearest-
 *    even where the library produces them).  All matrices are row-major.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Device work is enqueued
 *    on it and the call returns without waiting, except where stated.  ridgefill_fill
 *    with resident maps (plain or folded) enqueues kernels only (the status word is
 *    cleared by a kernel, not a memset), so it can be captured into a HIP graph and
 *    replayed; the workspace, index list and pools must then stay at their addresses.
 *  - Errors found on the host (null pointers, shapes, sizes, workspace too small,
 *    invalid parameters) return a non-zero rf_status before anything is enqueued;
 *    ridgefill_last_error() then gives a description.  A failed launch returns
 *    RF_E_HIP.  Errors that only the device can see (an index out of range, a
 *    non-increasing index list, a non-positive pivot) set bits in the status word
 *    at the start of the workspace; ridgefill_read_status() returns them.  Rows whose
 *    index is invalid are skipped: the library never writes outside the rows it was
 *    given and never aborts.
 *  - Calls that share a workspace or state buffer must not run concurrently.
 */
#ifndef RIDGEFILL_H
#define RIDGEFILL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rf_status {
  RF_OK = 0,
  RF_E_INVALID = 1,      /* null pointer or invalid scalar parameter            */
  RF_E_SHAPE = 2,        /* unsupported or inconsistent sizes                   */
  RF_E_WORKSPACE = 3,    /* workspace / state buffer too small or mismatched    */
  RF_E_HIP = 4,          /* a HIP runtime call or kernel launch failed          */
  RF_E_NOT_SPD = 5,      /* device: X^T X + alpha I was not positive definite   */
  RF_E_ROWS = 6,         /* device: an index was out of range or not increasing */
  RF_E_UNSUPPORTED = 7   /* the requested variant is not built                  */
} rf_status;

/* Model shape shared by all layers of one fill call. */
typedef struct rf_shape {
  int32_t d;            /* hidden size of the upper layers (the map's output width);
                           multiple of 256                                             */
  int32_t n_kv_heads;   /* KV heads; n_kv_heads * head_dim must be a multiple of 128 */
  int32_t head_dim;     /* 64 or 128                                                 */
  float rms_eps;        /* RMSNorm epsilon (inside the square root), >= 0; also the
                           epsilon of the per-head key norm when one is given        */
  double rope_theta;    /* RoPE base, > 1                                            */
  int32_t d_in;         /* width of x_S, the map's input (section "Ridge map ...", map
                           size paragraph: a map's input width may differ from its
                           output width).  0 means d.  Multiple of 64.                */
  int32_t reserved;     /* must be 0                                                  */
} rf_shape;

/* One upper layer l >= S.  Every pointer is a device pointer owned by the caller.   */
typedef struct rf_layer {
  const uint16_t* A;       /* bf16 [d][d_in]: x_hat = A x_S + b (A[out][in]); NULL when
                              the map is given in int8 (A_q)                            */
  const float* b;          /* fp32 [d]                                                 */
  const uint16_t* norm_w;  /* bf16 [d]: the layer's RMSNorm weight                     */
  const uint16_t* W_K;     /* bf16 [n_kv_heads*head_dim][d]: key projection, no bias   */
  const uint16_t* W_V;     /* bf16 [n_kv_heads*head_dim][d]: value projection, no bias */
  uint16_t* k_pages;       /* bf16 [num_pages][page_size][n_kv_heads][head_dim]        */
  uint16_t* v_pages;       /* bf16 [num_pages][page_size][n_kv_heads][head_dim]        */
  /* Optional parts (NULL = absent). */
  const uint16_t* k_norm_w; /* bf16 [head_dim]: per-head key RMSNorm (Qwen-style layers;
                               section "Hybrid layers and two corrections": the Qwen
                               models apply a norm to the keys), applied to each key head after W_K and
                               before RoPE                                               */
  const float* v_scale;     /* fp32 [n_kv_heads]: value-rescale factors (same section,
                               value rescale); head h of every filled value is
                               multiplied by v_scale[h].  ridgefill_value_scale computes
                               them.                                                    */
  const int8_t* A_q;        /* int8 [d][d_in] with A_scale: the map is A_q[o][i] *
                               A_scale[o] (section "Ridge map ...", map size paragraph:
                               int8 maps).  Exactly one of A and A_q is set.             */
  const float* A_scale;     /* fp32 [d]: per-output-row scale of A_q                    */
  const void* folded;       /* buffer of ridgefill_fold_bytes(shape) bytes made by
                               ridgefill_fold_maps, 256-byte aligned: the layer's folded
                               form (device memory; host memory, ideally page-locked, for
                               ridgefill_fill_streamed).  When set, the fill reads it
                               instead of A, A_q, A_scale, b, norm_w, W_K and W_V (which
                               may then be NULL).                                          */
} rf_layer;

/* Paged KV layout of one prompt, shared by every layer's k_pages / v_pages. */
typedef struct rf_paged_kv {
  const int32_t* block_table;   /* device int32 [n_logical]: logical page -> physical */
  int64_t n_logical;            /* entries in block_table (>= ceil(N / page_size))    */
  int32_t page_size;            /* rows per page, >= 1                                */
  int32_t num_pages;            /* physical pages in each k_pages / v_pages pool      */
} rf_paged_kv;

/* ------------------------------------------------------------------------------
 * Row partition.  Section "Method: ..." -> "Two numbers set the skip range": the last
 * T rows are the tail; the N - T rows before them are the prefix, whose rows are each
 * computed exactly or filled from the maps.  Host-only, integer, no GPU.
 *
 *   exact_mask  host uint8 [N - T]: nonzero marks an exact row (may be NULL = none)
 *   filled_idx  host int32 [N - T] out: the filled rows in ascending order
 *   n_filled    host out: their count (N - T - number of exact rows)
 * Returns RF_E_SHAPE unless 0 <= T <= N and N - T fits in int32.
 * ------------------------------------------------------------------------------ */
rf_status ridgefill_partition(int64_t N, int64_t T, const uint8_t* exact_mask,
                              int32_t* filled_idx, int64_t* n_filled);

/* ------------------------------------------------------------------------------
 * Exact-row selection from scores, on the device.  Section "Which rows to compute
 * exactly", attention selection: the prefix rows that receive the most attention are
 * computed exactly (10% of them in the reference study's "+rows" arm).  Given one score
 * per prefix row, the k rows with the largest score, ties broken toward the lower row
 * index, are the exact rows; the other P - k rows, in ascending order, are written to
 * filled_idx, ready for ridgefill_fill with n_filled = P - k.
 *
 *   scores      device fp32 [P]; -0.0 and +0.0 tie; a NaN score ranks lowest and sets
 *               RF_E_INVALID in the device status (ridgefill_read_status(ws))
 *   k           0 <= k <= P
 *   exact_mask  device uint8 [P] out (1 = exact), or NULL
 *   filled_idx  device int32 [P - k] out
 *   ws          device workspace >= ridgefill_select_workspace_bytes(P); its first 256
 *               bytes hold the status
 * Integer and order decisions only: the result is exact and deterministic.
 * ------------------------------------------------------------------------------ */
size_t ridgefill_select_workspace_bytes(int64_t P);
rf_status ridgefill_select_rows(const float* scores, int64_t P, int64_t k, uint8_t* exact_mask,
                                int32_t* filled_idx, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------
 * Fill.  Section "Ridge map: predict the input, and the original projection runs
 * unchanged" (prediction equation; the paragraph on feeding the predicted input to the
 * layer's norm and K/V projections; Fig. 2):
 * for every filled row t and every given upper layer l,
 *     x_hat = A_l x_S[t] + b_l          (A_l = A_q,l * A_scale,l for an int8 map)
 *     h     = x_hat / sqrt(mean(x_hat^2) + eps) * norm_w_l
 *     k     = W_K,l h,  then per head k / sqrt(mean(k^2) + eps) * k_norm_w_l if given
 *     k     = RoPE_t(k)   (pairs (j, j + head_dim/2), angle t * theta^(-2j/head_dim))
 *     v     = W_V,l h,  times v_scale_l[head] if given
 * and k, v are written to row t of layer l's paged cache (page block_table[t /
 * page_size], slot t % page_size).  Nothing else in the caches is touched; with
 * n_filled = 0 or n_layers = 0 only the status word is cleared (if ws is given).  Layers
 * are independent, so a caller may also split them over several calls.
 *
 *   x_S         device bf16 [N][x_stride]: split-layer states of all prompt rows
 *               (x_stride >= d_in); the prefix rows must span at most 4 GiB
 *               ((N - T) x x_stride x 2 bytes), and x_stride is a multiple of 8
 *   filled_idx  device int32 [n_filled]: filled rows, strictly increasing, each
 *               < N - T (the tail never receives a filled entry).  Violations set
 *               RF_E_ROWS in the device status; out-of-range rows are skipped.
 *   layers      host array [n_layers] of device-pointer descriptors
 *   ws          device workspace of ws_bytes >= ridgefill_fill_workspace_bytes(shape,
 *               n_filled, 1); a larger workspace (up to the value for n_layers) lets
 *               more layers share one launch.  Its first 256 bytes hold the status.
 * Computation: bf16 inputs, fp32 accumulation, x_hat and the RMS in fp32, one bf16
 * rounding of x_hat * norm_w, one bf16 rounding of the stored k and v.  An int8 map's
 * codes are read by the map GEMM as they are and turned into bf16 numbers between LDS and
 * the matrix cores (exactly: |q| <= 127), and its row scale is applied to the fp32
 * product, so it adds no rounding of its own.  All
 * layers of one call must agree on which optional parts they use (int8 or bf16 map,
 * key norm); v_scale may be set per layer.
 * ------------------------------------------------------------------------------ */
size_t ridgefill_fill_workspace_bytes(const rf_shape* shape, int64_t n_filled,
                                      int32_t n_layers);
rf_status ridgefill_fill(const rf_shape* shape, const uint16_t* x_S, int64_t N, int64_t T,
                         int64_t x_stride, const int32_t* filled_idx, int64_t n_filled,
                         const rf_layer* layers, int32_t n_layers, const rf_paged_kv* kv,
                         void* ws, size_t ws_bytes, void* stream);

/* Map variants for the workspace query: RF_MAPS_INT8 when the layers carry A_q/A_scale
 * (the same workspace as for bf16 maps), RF_MAPS_STREAMED for
 * ridgefill_fill_streamed (two landing slots per layer), RF_MAPS_FOLDED when the layers
 * carry folded forms (no predicted-input buffer: a few MB per layer).  Returns 0 on
 * invalid input.
 * ridgefill_fill_workspace_bytes(...) is ridgefill_fill_workspace_bytes_ex(..., 0). */
#define RF_MAPS_INT8 1
#define RF_MAPS_STREAMED 2
#define RF_MAPS_FOLDED 4
size_t ridgefill_fill_workspace_bytes_ex(const rf_shape* shape, int64_t n_filled,
                                         int32_t n_layers, int32_t map_flags);

/* ------------------------------------------------------------------------------
 * Fill with host-resident maps.  Section "Ridge map ...", map size paragraph: maps can
 * stay in GPU memory or be streamed from host memory layer by layer.  Same
 * computation and arguments as ridgefill_fill, except that every layer's A (or A_q), or
 * for folded layers its whole folded buffer, is a HOST pointer, ideally page-locked
 * (hipHostMalloc) so that the copies run asynchronously.  Layers are processed in groups
 * sized by the workspace (ridgefill_fill_workspace_bytes_ex with RF_MAPS_STREAMED, plus
 * RF_MAPS_INT8 for int8 maps or RF_MAPS_FOLDED for folded layers); group g's maps (or
 * folded buffers) are copied on `copy_stream` into landing slot g % 2 while group g - 1
 * computes on `stream`.  Of a folded buffer only what the fill reads is copied: P, c, r1,
 * g, kappa, and R1 from each 256-row block's diagonal block rightwards (the zeros below the
 * diagonal blocks, about half of R, are not).  copy_stream must be a different stream; both must stay
 * valid until the work completes.  The first copy of a call waits for the work already
 * enqueued on `stream`, so back-to-back calls on one workspace are ordered.  The results
 * are bit-identical to ridgefill_fill's.
 * ------------------------------------------------------------------------------ */
rf_status ridgefill_fill_streamed(const rf_shape* shape, const uint16_t* x_S, int64_t N, int64_t T,
                                  int64_t x_stride, const int32_t* filled_idx, int64_t n_filled,
                                  const rf_layer* layers, int32_t n_layers, const rf_paged_kv* kv,
                                  void* ws, size_t ws_bytes, void* stream, void* copy_stream);

/* ------------------------------------------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph capture, serving
 * loops that must not call hipMalloc): the same computation and arguments as
 * ridgefill_fill with resident maps (plain bf16, int8 or folded layers), without a
 * workspace argument.  The library's own scratch array serves as the workspace:
 * RIDGEFILL_NOALLOC_SCRATCH_BYTES of device memory per device, part of the library's code
 * object (allocated when it is loaded on that device, held until the process ends).  The
 * call allocates nothing; layers are processed in groups as large as the scratch holds.
 *   status   device pointer to one uint32 (4-byte aligned) that receives the device status
 *            word of the call (cleared first); read it with ridgefill_read_status(status).
 * Returns RF_E_WORKSPACE, before anything is enqueued, when one layer's share of the
 * workspace (ridgefill_fill_workspace_bytes_ex(shape, n_filled, 1, flags)) exceeds the
 * scratch.  All calls on one device share its scratch, which keeps the last call's
 * contents: calls that overlap on one device (two streams, two threads) race and must be
 * ordered by the caller.  Nothing in the scratch needs to start at zero.
 * ------------------------------------------------------------------------------ */
#define RIDGEFILL_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
rf_status ridgefill_fill_noalloc(const rf_shape* shape, const uint16_t* x_S, int64_t N, int64_t T,
                                 int64_t x_stride, const int32_t* filled_idx, int64_t n_filled,
                                 const rf_layer* layers, int32_t n_layers, const rf_paged_kv* kv,
                                 uint32_t* status, void* stream);

/* ------------------------------------------------------------------------------
 * Folded layers.  Section "Ridge map: predict the input, and the original projection runs
 * unchanged": after x_hat = A x_S + b the layer's RMSNorm weight w and its projections
 * W_K, W_V are linear, so they can be multiplied into the map once per layer; the only
 * non-linear quantity left is |x_hat|^2, which equals |R x_S + r|^2 + kappa with R the
 * upper-triangular factor of A^T A (R^T R = A^T A, positive diagonal),
 * r = R^-T A^T b and kappa = |b|^2 - |r|^2.  The fill of a folded layer then computes
 *     k, v = (P x_S + c) / sqrt((|R x_S + r|^2 + kappa) / d + eps)
 * with P = [W_K; W_V] diag(w) A and c = [W_K; W_V] (w * b), followed by the same key norm,
 * RoPE, value rescale and paged store as the plain fill.  Same result up to rounding;
 * R x_S needs half the multiply-adds of A x_S, and x_hat is never stored.
 *
 * A^T A is accumulated in fp32 from the exact bf16 products; its diagonal is lifted by a
 * relative 2^-16 before the fp64 Cholesky (so that the accumulation's rounding cannot make
 * the factorization meet a non-positive pivot for maps of large condition number), which
 * adds 2^-16 sum_i |A_i|^2 x_i^2 to |x_hat|^2 (about 1.5e-5 of it where the columns A_i x_i
 * do not cancel).  A zero column of A still gives a zero pivot.
 * R is stored with a unit diagonal: R = diag(g) R1 with g = diag(R) in fp32 and R1 in
 * bf16 whose diagonal entries are exactly 1, and r as r1 = r / g, so that
 * |R x_S + r|^2 = sum_f g_f^2 (R1_f x_S + r1_f)^2 and the diagonal term (through which
 * alone feature 0 reaches the sum) is not rounded to bf16.
 *
 * Folded buffer of one layer (offsets from its start, each 256-byte aligned):
 *     P bf16 [2 kv][d_in] (K rows, then V rows), R1 bf16 [d_in][d_in] (unit diagonal,
 *     zeros below it), c fp32 [2 kv], r1 fp32 [d_in], g fp32 [d_in], kappa fp32;
 *     kv = n_kv_heads * head_dim.
 * ridgefill_fold_bytes returns its size, 0 when the shape cannot be folded: A^T A must be
 * positive definite, so d_in <= d, and d_in must be a multiple of 256.
 *
 * ridgefill_fold_maps computes every given layer's folded buffer from its plain fields
 * (A bf16, or A_q int8 with A_scale; b, norm_w, W_K, W_V).  All layers of a call carry
 * bf16 maps or all carry int8 maps:
 *   folded     host array [n_layers] of device pointers, each >= ridgefill_fold_bytes
 *              bytes and 256-byte aligned
 *   ws         device workspace >= ridgefill_fold_workspace_bytes(shape) for bf16 maps,
 *              >= ridgefill_fold_workspace_bytes_maps(shape, 1, RF_MAPS_INT8) for int8
 *              maps (RF_E_WORKSPACE otherwise, before anything is enqueued); its first
 *              256 bytes hold the status: RF_E_NOT_SPD when some layer's A^T A had a
 *              non-positive pivot (A not of full column rank; that layer's buffer is
 *              then not usable).  A workspace of ridgefill_fold_workspace_bytes_ex(shape, G)
 *              bytes (ridgefill_fold_workspace_bytes_maps(shape, G, RF_MAPS_INT8) for int8
 *              maps) folds G layers side by side (their Cholesky factorizations share one
 *              sequence of launches); a smaller one folds as many as it holds, at least
 *              one (at most 64) at a time.  The results do not depend on G.
 * Arithmetic: P = bf16-split(W diag(w)) times A on the matrix cores (products exact,
 * fp32 accumulation, one bf16 rounding of P); A^T A with exact products and fp32
 * accumulation; Cholesky, r and kappa in fp64; R rounded to bf16 once; c in fp64
 * rounded to fp32.  An int8 map A = diag(A_scale) A_q folds through its codes, which
 * bf16 holds exactly: P = bf16-split(W diag(w A_scale)) times A_q, and
 * A^T A = A_q^T diag(A_scale^2) A_q with the scaled side split into two bf16 parts
 * (about 2^-17 of each entry), as above otherwise; the buffer is the same as from the
 * bf16 map A_q * A_scale up to those roundings.
 * Folded layers work with ridgefill_fill and, from host memory, ridgefill_fill_streamed;
 * all layers of a fill call must be folded or none.  ridgefill_value_scale takes folded
 * layers too (see there).
 * ------------------------------------------------------------------------------ */
size_t ridgefill_fold_bytes(const rf_shape* shape);
size_t ridgefill_fold_workspace_bytes(const rf_shape* shape);
/* Workspace that folds layers_at_once (>= 1) layers side by side; 0 for a shape that
 * cannot be folded or layers_at_once < 1. */
size_t ridgefill_fold_workspace_bytes_ex(const rf_shape* shape, int32_t layers_at_once);
/* The same for the map kind of the layers: map_flags 0 (bf16 maps, as the _ex query) or
 * RF_MAPS_INT8 (int8 maps, which take a second operand slot per layer); 0 for other flags. */
size_t ridgefill_fold_workspace_bytes_maps(const rf_shape* shape, int32_t layers_at_once,
                                           uint32_t map_flags);
rf_status ridgefill_fold_maps(const rf_shape* shape, const rf_layer* layers, int32_t n_layers,
                              void* const* folded, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------
 * int8 maps.  Section "Ridge map ...", map size paragraph: maps held in int8 (1.2 GiB
 * for 48 upper layers at hidden size 5120).  Symmetric, one scale per output row:
 *     A_scale[o] = max_i |A[o][i]| / 127,  A_q[o][i] = round-half-even(A[o][i] / A_scale[o])
 * clipped to [-127, 127]; a zero row gets scale 0 and zero codes.  All decisions in fp32
 * with correctly rounded division.  The fill then uses A_q * A_scale as the map.
 *   A        device fp32 [rows][cols] (e.g. one layer of ridgefill_solve's A_out)
 *   A_q      device int8 [rows][cols] out;  A_scale  device fp32 [rows] out
 * ------------------------------------------------------------------------------ */
rf_status ridgefill_quantize_map(const float* A, int64_t rows, int64_t cols, int8_t* A_q,
                                 float* A_scale, void* stream);

/* ------------------------------------------------------------------------------
 * Value-rescale factors.  Section "Hybrid layers and two corrections", value rescale:
 * for each upper layer, the values of the first c tail rows are computed from both the
 * true layer input and the mapped input; per KV head, the mean over those rows of
 * |exact value| / |predicted value| scales the filled values.  For layer l and head h:
 *     v_e(t) = W_V,l RMSNorm_l(x_l,exact[t]),  v_p(t) = W_V,l RMSNorm_l(A_l x_S[t] + b_l)
 *     v_scale_out[l][h] = (1/c) sum_t |v_e(t)_h| / |v_p(t)_h|
 * Pass v_scale_out + l * n_kv_heads as layer l's v_scale to ridgefill_fill.
 *
 *   x_S_tail     device bf16 [c][x_stride]: split-layer states of the first c tail rows
 *   x_l_tail     host array [n_layers] of device bf16 [c][d] (contiguous): each layer's
 *                exact input for the same rows
 *   layers       A or A_q/A_scale, b, norm_w, W_V of each layer (W_K is not read and
 *                may be null; K and the pages are not written); or, for
 *                folded layers (all or none), folded with norm_w and W_V: the predicted
 *                values then come from the folded form, v_p = (P_V x_S + c_V) / rms with
 *                |x_hat|^2 = |R x_S + r|^2 + kappa, and the exact ones from W_V and norm_w
 *   v_scale_out  device fp32 [n_layers][n_kv_heads]
 *   ws           >= ridgefill_value_scale_workspace_bytes(shape, c, 1, map_flags) with
 *                map_flags 0, RF_MAPS_INT8 or RF_MAPS_FOLDED (the last two exclusive); a
 *                larger one lets more layers share a launch (up to 64: the size query for
 *                n_layers covers min(n_layers, 64) layers)
 * Norms are taken in fp32 on the fp32 projections (before any bf16 rounding of v); the
 * inputs to W_V are rounded to bf16 once, as in the fill (for folded layers P_V is the
 * rounded operand).  The mean is added in row order in fp64.  A predicted norm of 0
 * gives an infinite factor.
 * ------------------------------------------------------------------------------ */
size_t ridgefill_value_scale_workspace_bytes(const rf_shape* shape, int64_t c, int32_t n_layers,
                                             int32_t map_flags);
rf_status ridgefill_value_scale(const rf_shape* shape, const uint16_t* x_S_tail, int64_t x_stride,
                                const uint16_t* const* x_l_tail, int64_t c, const rf_layer* layers,
                                int32_t n_layers, float* v_scale_out, void* ws, size_t ws_bytes,
                                void* stream);

/* ------------------------------------------------------------------------------
 * Calibration.  Same section, paragraph on alpha and the one-pass statistics: one pass
 * accumulates X^T X, Y_l^T X and the two means; a new lambda needs only a new solve.
 * The state belongs to one split (one x_S source) and is caller-owned device memory.
 * x_S is accumulated about a per-feature shift s (fp32 holding bf16 values), fixed by the
 * first call that adds rows: where that call has at least 64 rows, s_i is the bf16
 * rounding of the mean of feature i over them if that mean exceeds twice their standard
 * deviation, else 0; a first call of fewer rows fixes s = 0.  Each call accumulates
 * x'_S = bf16(x_S - s) (exact wherever x_S lies within [s/2, 2s]), so that a feature whose
 * mean dwarfs its spread keeps its centred moments in fp32 (raw moments would lose them
 * to cancellation).  Layout:
 *   [0, 256)   header: int64 row count n, int32 d, int32 n_layers, magic, int32 d,
 *              int32 shift fixed, int32 state marked bad, int32 (internal)
 *   then       fp64 sum_t x'_S         [d]
 *              fp64 sum_t x_l          [n_layers][d]
 *              fp32 sum_t x'_S x'_S^T  [d][d]   (lower triangle valid; i >= j)
 *              fp32 sum_t x_l x'_S^T   [n_layers][d][d]  (row = output feature of x_l)
 *              fp32 s                  [d]
 *              scratch: 16384 rows of bf16 [d] where each call stages x'_S (a call of
 *              more rows is processed in pieces of 16384)
 * Each region starts on a 256-byte boundary.  Saving the state is a device-to-host copy
 * of everything before the scratch area.
 *
 * ridgefill_calib_reset clears the state for (d, n_layers); later calls on the state
 * must pass the same d and n_layers.  A calibrate call whose sizes differ from the
 * header's changes nothing and marks the state bad; a later solve on it then reports
 * RF_E_WORKSPACE through ridgefill_read_status.
 * ridgefill_calibrate adds n_rows rows: x_S device bf16 [n_rows][d]; x_l host array
 * [n_layers] of device bf16 [n_rows][d] pointers.  Sums in fp32 per call and fp64
 * across calls for the means; moments accumulated in fp32.  d: multiple of 256;
 * n_layers: 1 .. 64.
 * ------------------------------------------------------------------------------ */
size_t ridgefill_calib_state_bytes(int32_t d, int32_t n_layers);
rf_status ridgefill_calib_reset(void* state, size_t state_bytes, int32_t d, int32_t n_layers,
                                void* stream);
rf_status ridgefill_calibrate(void* state, size_t state_bytes, int32_t d, int32_t n_layers,
                              const uint16_t* x_S, const uint16_t* const* x_l, int64_t n_rows,
                              void* stream);

/* The same for maps whose input width differs from their output width (section "Ridge
 * map ...", map-size paragraph): x_S rows are d_in wide, x_l rows d_out wide (both
 * multiples of 256).  The state then holds
 *   [0, 256)   header: int64 n, int32 d_out, int32 n_layers, magic, int32 d_in, ...
 *   then       fp64 sum_t x'_S [d_in], fp64 sum_t x_l [n_layers][d_out],
 *              fp32 sum_t x'_S x'_S^T [d_in][d_in] (lower triangle valid),
 *              fp32 sum_t x_l x'_S^T [n_layers][d_out][d_in], fp32 s [d_in],
 *              scratch bf16 [16384][d_in].
 * The plain calls are these with d_in = d_out = d. */
size_t ridgefill_calib_state_bytes_ex(int32_t d_in, int32_t d_out, int32_t n_layers);
rf_status ridgefill_calib_reset_ex(void* state, size_t state_bytes, int32_t d_in, int32_t d_out,
                                   int32_t n_layers, void* stream);
rf_status ridgefill_calibrate_ex(void* state, size_t state_bytes, int32_t d_in, int32_t d_out,
                                 int32_t n_layers, const uint16_t* x_S, const uint16_t* const* x_l,
                                 int64_t n_rows, void* stream);

/* ------------------------------------------------------------------------------
 * Solve.  Same section, closed-form equation and the scale-free penalty: with
 * mu = sums / n (mu_S of the shifted rows x'_S),  C = sum x'_S x'_S^T - n mu_S mu_S^T,
 * C_l = sum x_l x'_S^T - n mu_l mu_S^T,  alpha = lambda * tr(C) / d,
 *     A_l = C_l (C + alpha I)^-1,     b_l = mu_l - A_l (mu_S + s).
 * (C + alpha I) is factored by a device Cholesky in fp64 and inverted in fp64.  The
 * product C_l M (M = (C + alpha I)^-1) is a bf16 matrix-core GEMM on operands split into
 * bf16 parts, fp32 accumulation: two parts per operand (hi + mid, three products, about
 * 2^-17 relative per operand) while kappa_F = |C + alpha I|_F |M|_F <= 16 d, else three
 * parts (hi + mid + lo, six products, about 2^-25 per operand; the product then takes
 * twice as long).  The relative error of A grows about as 5e-6 kappa_F / d with two parts
 * and 1e-7 kappa_F / d with three.  b_l is accumulated in fp64.
 *
 *   A_out       device fp32 [n_layers][d][d] (may be NULL if A_bf16_out is given)
 *   b_out       device fp32 [n_layers][d]
 *   A_bf16_out  device bf16 [n_layers][d][d] or NULL: the map as the fill takes it
 *   ws          device workspace >= ridgefill_solve_workspace_bytes(d, n_layers);
 *               its first 256 bytes hold the status (RF_E_NOT_SPD on a bad pivot).
 * lambda must be >= 0 and finite.  Repeated solves reuse the state unchanged.
 * ------------------------------------------------------------------------------ */
size_t ridgefill_solve_workspace_bytes(int32_t d, int32_t n_layers);
rf_status ridgefill_solve(const void* state, size_t state_bytes, int32_t d, int32_t n_layers,
                          double lambda, float* A_out, float* b_out, uint16_t* A_bf16_out,
                          void* ws, size_t ws_bytes, void* stream);

/* The solve for a state made by the _ex calls: alpha = lambda tr(C) / d_in, the Cholesky
 * on the d_in x d_in side, A_out fp32 [n_layers][d_out][d_in], b_out fp32
 * [n_layers][d_out], A_bf16_out bf16 [n_layers][d_out][d_in]. */
size_t ridgefill_solve_workspace_bytes_ex(int32_t d_in, int32_t d_out, int32_t n_layers);
rf_status ridgefill_solve_ex(const void* state, size_t state_bytes, int32_t d_in, int32_t d_out,
                             int32_t n_layers, double lambda, float* A_out, float* b_out,
                             uint16_t* A_bf16_out, void* ws, size_t ws_bytes, void* stream);

/* Waits for `stream`, then returns the device status word of a fill, solve or selection
 * workspace: RF_OK, RF_E_ROWS, RF_E_NOT_SPD, RF_E_WORKSPACE for a solve on a calibration
 * state whose header disagrees with the solve's sizes or that a calibrate call marked bad,
 * or RF_E_INVALID for a NaN score.  Each call
 * clears that word on the stream before its own kernels run, so the word reflects the
 * last call only. */
rf_status ridgefill_read_status(void* ws, void* stream);

/* Waits for `stream`, then reports the conditioning of the last solve on this solve
 * workspace: *kappa_f = |C + alpha I|_F |(C + alpha I)^-1|_F (an upper bound on the
 * 2-norm condition number) and *parts = the bf16 parts per operand the map product used
 * (3: hi, mid, hi pairs, three products; 6: six products).  Both outputs are host pointers;
 * either may be NULL. */
rf_status ridgefill_solve_info(void* ws, double* kappa_f, int32_t* parts, void* stream);

/* ------------------------------------------------------------------------------
 * Kernel timing for measurement.  While enabled, every compute-kernel launch of the
 * library is bracketed by a pair of HIP events recorded on the caller's stream (no
 * synchronisation is added).  ridgefill_profile_read waits for the recorded events and
 * returns, for one kernel, the launches seen since the last reset and their summed
 * duration in milliseconds.  Host-side only; thread safe.
 * ------------------------------------------------------------------------------ */
typedef enum rf_kernel_id {
  RF_KERNEL_FILL_MAP = 0,      /* map GEMM: x_hat = A x_S + b, RMS partials, x_hat * w   */
  RF_KERNEL_FILL_KV = 1,       /* K/V GEMM: RMS scale, RoPE, paged store                 */
  RF_KERNEL_CALIB_MOMENTS = 2, /* calibration: sum x_S x_S^T (lower) and every x_l x_S^T */
  RF_KERNEL_CALIB_SUMS = 3,    /* calibration: column sums and row count                 */
  RF_KERNEL_SOLVE_MAP = 4,     /* solve: A_l = C_l (C + alpha I)^-1 product              */
  RF_KERNEL_FILL_NORM = 5,     /* folded fill: per-row |R x_S + r|^2 partials            */
  RF_KERNEL_COUNT = 6
} rf_kernel_id;
rf_status ridgefill_profile_enable(int32_t enable);
rf_status ridgefill_profile_read(int32_t kernel, int64_t* launches, double* total_ms);
rf_status ridgefill_profile_reset(void);

const char* ridgefill_status_string(rf_status s);
/* Description of the last non-OK status returned on this thread ("" if none). */
const char* ridgefill_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* RIDGEFILL_H */
