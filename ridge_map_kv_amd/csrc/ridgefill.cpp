// C ABI of the RidgeFill library: argument checks, workspace carve-up, the host row
// partition and status reporting.  Device work is in rf_fill.hip, rf_calib.hip and
// rf_solve.hip.
#include "ridgefill.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "rf_internal.h"

namespace {

thread_local std::string g_last_error;

rf_status fail(rf_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
rf_status fail(rf_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

rf_status ok() {
  g_last_error.clear();
  return RF_OK;
}

rf_status hip_fail(hipError_t e, const char* what) {
  return fail(RF_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

rf_status check_shape(const rf_shape* s) {
  if (!s) return fail(RF_E_INVALID, "shape is NULL");
  if (s->d < rf::kTile || s->d % rf::kTile)
    return fail(RF_E_SHAPE, "d = %d must be a positive multiple of %d", s->d, rf::kTile);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(RF_E_SHAPE, "head_dim = %d must be 64 or 128", s->head_dim);
  if (s->n_kv_heads < 1) return fail(RF_E_SHAPE, "n_kv_heads = %d must be >= 1", s->n_kv_heads);
  const int64_t kv = (int64_t)s->n_kv_heads * s->head_dim;
  if (kv % 128) return fail(RF_E_SHAPE, "n_kv_heads * head_dim = %lld must be a multiple of 128",
                            (long long)kv);
  if (kv > (1 << 20)) return fail(RF_E_SHAPE, "n_kv_heads * head_dim too large");
  if (s->n_kv_heads > 256) return fail(RF_E_SHAPE, "n_kv_heads = %d must be <= 256", s->n_kv_heads);
  if (s->reserved != 0) return fail(RF_E_INVALID, "shape.reserved must be 0");
  if (s->d_in != 0 && (s->d_in < 64 || s->d_in % 64))
    return fail(RF_E_SHAPE, "d_in = %d must be 0 (= d) or a positive multiple of 64", s->d_in);
  if (!(s->rms_eps >= 0.f) || !std::isfinite(s->rms_eps))
    return fail(RF_E_INVALID, "rms_eps must be finite and >= 0");
  if (!(s->rope_theta > 1.0) || !std::isfinite(s->rope_theta))
    return fail(RF_E_INVALID, "rope_theta must be finite and > 1");
  return RF_OK;
}

int d_in_of(const rf_shape* s) { return s->d_in ? s->d_in : s->d; }

unsigned map_flags_of(int32_t f) {
  return ((f & RF_MAPS_INT8) ? rf::kWsInt8 : 0u) | ((f & RF_MAPS_STREAMED) ? rf::kWsStreamed : 0u) |
         ((f & RF_MAPS_FOLDED) ? rf::kWsFolded : 0u);
}

// A folded form needs A^T A positive definite (d_in <= d) and whole 256-wide tiles of R.
rf_status check_foldable(const rf_shape* s) {
  const int d_in = d_in_of(s);
  if (d_in > s->d)
    return fail(RF_E_SHAPE, "d_in = %d > d = %d: A^T A is singular, the map cannot be folded",
                d_in, s->d);
  if (d_in % rf::kTile)
    return fail(RF_E_SHAPE, "folded maps need d_in (%d) to be a multiple of %d", d_in, rf::kTile);
  return RF_OK;
}

// Checks shared by the resident and the streamed fill; fills the plan and the layer
// pointers.  `streamed`: the maps (A or A_q), or the folded buffers, are host pointers.
rf_status prepare_fill(const rf_shape* shape, const uint16_t* x_S, int64_t N, int64_t T,
                       int64_t x_stride, const int32_t* filled_idx, int64_t n_filled,
                       const rf_layer* layers, int32_t n_layers, const rf_paged_kv* kv, void* ws,
                       size_t ws_bytes, bool streamed, rf::FillPlan& p,
                       std::vector<rf::FillLayerPtrs>& lp) {
  const int64_t P = N - T;
  if (!x_S || !filled_idx || !layers || !kv || !ws)
    return fail(RF_E_INVALID, "null pointer among x_S, filled_idx, layers, kv, ws");
  const int d_in = d_in_of(shape);
  if (x_stride < d_in) return fail(RF_E_SHAPE, "x_stride < d_in");
  if (x_stride % 8 || !aligned(x_S, 16))
    return fail(RF_E_SHAPE, "x_S must be 16-byte aligned with x_stride a multiple of 8");
  if ((uint64_t)(P - 1) * (uint64_t)x_stride * 2u + (uint64_t)d_in * 2u > 0xffffffffull)
    return fail(RF_E_SHAPE, "the prefix rows of x_S span more than 4 GiB (rows x x_stride x 2 bytes)");
  if (!kv->block_table || kv->page_size < 1 || kv->num_pages < 1 || kv->n_logical < 1)
    return fail(RF_E_INVALID, "paged layout: block_table, page_size, num_pages, n_logical");
  if (kv->n_logical < (P + kv->page_size - 1) / kv->page_size)
    return fail(RF_E_SHAPE, "block table has %lld pages, the prefix needs %lld",
                (long long)kv->n_logical, (long long)((P + kv->page_size - 1) / kv->page_size));
  if (!aligned(ws, 256)) return fail(RF_E_WORKSPACE, "workspace must be 256-byte aligned");
  const bool folded = layers[0].folded != nullptr;
  const bool int8 = !folded && layers[0].A_q != nullptr;
  const bool knorm = layers[0].k_norm_w != nullptr;
  if (folded) {
    rf_status fs = check_foldable(shape);
    if (fs != RF_OK) return fs;
  }
  for (int i = 0; i < n_layers; ++i) {
    const rf_layer& l = layers[i];
    if ((l.folded != nullptr) != folded)
      return fail(RF_E_INVALID, "layer %d: all layers of a call must be folded or none", i);
    if ((l.k_norm_w != nullptr) != knorm)
      return fail(RF_E_INVALID, "layer %d: all layers of a call must have a key norm or none", i);
    if (folded) {
      if (!l.k_pages || !l.v_pages) return fail(RF_E_INVALID, "layer %d has a null page pool", i);
      if (!aligned(l.folded, 256) || !aligned(l.k_pages, 8) || !aligned(l.v_pages, 8) ||
          (l.v_scale && !aligned(l.v_scale, 4)) || (l.k_norm_w && !aligned(l.k_norm_w, 2)))
        return fail(RF_E_SHAPE, "layer %d: the folded buffer needs 256-byte, the pages 8-byte "
                    "alignment", i);
      continue;
    }
    if (!l.b || !l.norm_w || !l.W_K || !l.W_V || !l.k_pages || !l.v_pages)
      return fail(RF_E_INVALID, "layer %d has a null pointer", i);
    if ((l.A != nullptr) == (l.A_q != nullptr))
      return fail(RF_E_INVALID, "layer %d: exactly one of A and A_q must be set", i);
    if ((l.A_q != nullptr) != int8)
      return fail(RF_E_INVALID, "layer %d: all layers of a call must use bf16 maps or all int8", i);
    if (int8 && !l.A_scale) return fail(RF_E_INVALID, "layer %d: A_q without A_scale", i);
    if ((l.A && !aligned(l.A, 16)) || (l.A_q && !aligned(l.A_q, 16)) || !aligned(l.b, 16) ||
        !aligned(l.norm_w, 8) || !aligned(l.W_K, 16) || !aligned(l.W_V, 16) ||
        !aligned(l.k_pages, 8) || !aligned(l.v_pages, 8) ||
        (l.A_scale && !aligned(l.A_scale, 4)) || (l.v_scale && !aligned(l.v_scale, 4)) ||
        (l.k_norm_w && !aligned(l.k_norm_w, 2)))
      return fail(RF_E_SHAPE, "layer %d: A, A_q, b, W_K, W_V need 16-byte, norm_w and the pages "
                  "8-byte alignment", i);
  }
  const unsigned flags = (int8 ? rf::kWsInt8 : 0u) | (streamed ? rf::kWsStreamed : 0u) |
                         (folded ? rf::kWsFolded : 0u);
  const rf::FillWsLayout L = rf::fill_ws_layout(shape->d, d_in, shape->head_dim,
                                                shape->n_kv_heads * shape->head_dim, n_filled, flags);
  if (ws_bytes < L.fixed + L.per_layer)
    return fail(RF_E_WORKSPACE, "workspace %zu bytes < %zu needed for one layer", ws_bytes,
                L.fixed + L.per_layer);
  size_t group = (ws_bytes - L.fixed) / L.per_layer;
  if (group > (size_t)rf::kMaxGroup) group = rf::kMaxGroup;

  unsigned char* w = static_cast<unsigned char*>(ws);
  p = rf::FillPlan{};
  p.d = shape->d;
  p.d_in = d_in;
  p.n_kv = shape->n_kv_heads;
  p.hd = shape->head_dim;
  p.kv = shape->n_kv_heads * shape->head_dim;
  p.flags = flags;
  p.has_knorm = knorm ? 1 : 0;
  p.eps = shape->rms_eps;
  p.theta = shape->rope_theta;
  p.xS = x_S;
  p.x_stride = x_stride;
  p.N = N;
  p.P = P;
  p.idx = filled_idx;
  p.n_filled = (int)n_filled;
  p.mpad = (int)((n_filled + rf::kTile - 1) / rf::kTile * rf::kTile);
  p.block_table = kv->block_table;
  p.n_logical = kv->n_logical;
  p.page_size = kv->page_size;
  p.num_pages = kv->num_pages;
  p.status = reinterpret_cast<unsigned*>(w);
  p.rope_cos = reinterpret_cast<float*>(w + L.rope_cos);
  p.rope_sin = reinterpret_cast<float*>(w + L.rope_sin);
  p.row_slot = reinterpret_cast<int64_t*>(w + L.row_slot);
  p.hbuf = reinterpret_cast<uint16_t*>(w + L.hbuf);
  p.group = (int)group;
  p.L = L;

  lp.resize((size_t)n_layers);
  const rf::FoldLayout F = rf::fold_layout(d_in, p.kv);
  for (int i = 0; i < n_layers; ++i) {
    const rf_layer& l = layers[i];
    if (folded) {
      const unsigned char* f = static_cast<const unsigned char*>(l.folded);
      const uint16_t* P = reinterpret_cast<const uint16_t*>(f + F.P);
      lp[i] = {reinterpret_cast<const uint16_t*>(f + F.R), reinterpret_cast<const float*>(f + F.r),
               nullptr, P, P + (size_t)p.kv * d_in, l.k_pages, l.v_pages, l.k_norm_w, l.v_scale,
               nullptr, nullptr, reinterpret_cast<const float*>(f + F.c),
               reinterpret_cast<const float*>(f + F.kappa), reinterpret_cast<const float*>(f + F.g)};
    } else {
      lp[i] = {l.A, l.b, l.norm_w, l.W_K, l.W_V, l.k_pages, l.v_pages,
               l.k_norm_w, l.v_scale, l.A_q, l.A_scale, nullptr, nullptr, nullptr};
    }
  }
  return RF_OK;
}

// Common front of ridgefill_fill and ridgefill_fill_streamed: scalar checks and the empty
// call.  Returns RF_OK with *done set when nothing more is to be done.
rf_status fill_front(const rf_shape* shape, int64_t N, int64_t T, int64_t n_filled,
                     int32_t n_layers, void* ws, size_t ws_bytes, void* stream, bool* done) {
  *done = false;
  rf_status s = check_shape(shape);
  if (s != RF_OK) return s;
  if (N < 0 || T < 0 || T > N) return fail(RF_E_SHAPE, "need 0 <= T <= N");
  const int64_t P = N - T;
  if (n_filled < 0 || n_filled > P)
    return fail(RF_E_SHAPE, "n_filled = %lld must be in [0, N - T = %lld]", (long long)n_filled,
                (long long)P);
  if (n_filled > INT32_MAX - rf::kTile) return fail(RF_E_SHAPE, "n_filled too large");
  if (n_layers < 0) return fail(RF_E_INVALID, "n_layers < 0");
  if (n_filled == 0 || n_layers == 0) {
    if (ws) {
      if (!aligned(ws, 256) || ws_bytes < rf::kStatusBytes)
        return fail(RF_E_WORKSPACE, "workspace must be 256-byte aligned and >= 256 bytes");
      hipError_t e = rf::launch_clear_status(static_cast<unsigned*>(ws),
                                             static_cast<hipStream_t>(stream));
      if (e != hipSuccess) return hip_fail(e, "status clear");
    }
    *done = true;
  }
  return RF_OK;
}

}  // namespace

extern "C" {

const char* ridgefill_status_string(rf_status s) {
  switch (s) {
    case RF_OK: return "ok";
    case RF_E_INVALID: return "invalid argument";
    case RF_E_SHAPE: return "unsupported or inconsistent shape";
    case RF_E_WORKSPACE: return "workspace or state buffer too small or mismatched";
    case RF_E_HIP: return "HIP runtime error";
    case RF_E_NOT_SPD: return "X^T X + alpha I is not positive definite";
    case RF_E_ROWS: return "filled-row index out of range or not strictly increasing";
    case RF_E_UNSUPPORTED: return "unsupported";
  }
  return "unknown status";
}

const char* ridgefill_last_error(void) { return g_last_error.c_str(); }

rf_status ridgefill_partition(int64_t N, int64_t T, const uint8_t* exact_mask,
                              int32_t* filled_idx, int64_t* n_filled) {
  if (N < 0 || T < 0 || T > N) return fail(RF_E_SHAPE, "need 0 <= T <= N (N=%lld, T=%lld)",
                                          (long long)N, (long long)T);
  const int64_t P = N - T;
  if (P > INT32_MAX) return fail(RF_E_SHAPE, "prefix of %lld rows exceeds int32", (long long)P);
  if (!n_filled) return fail(RF_E_INVALID, "n_filled is NULL");
  if (P > 0 && !filled_idx) return fail(RF_E_INVALID, "filled_idx is NULL");
  int64_t k = 0;
  for (int64_t t = 0; t < P; ++t)
    if (!exact_mask || exact_mask[t] == 0) filled_idx[k++] = (int32_t)t;
  *n_filled = k;
  return ok();
}

size_t ridgefill_fill_workspace_bytes_ex(const rf_shape* shape, int64_t n_filled,
                                         int32_t n_layers, int32_t map_flags) {
  if (check_shape(shape) != RF_OK || n_filled < 0 || n_layers < 1 ||
      (map_flags & ~(RF_MAPS_INT8 | RF_MAPS_STREAMED | RF_MAPS_FOLDED)))
    return 0;
  if ((map_flags & RF_MAPS_FOLDED) && ((map_flags & RF_MAPS_INT8) || check_foldable(shape) != RF_OK))
    return 0;
  const rf::FillWsLayout L = rf::fill_ws_layout(shape->d, d_in_of(shape), shape->head_dim,
                                                shape->n_kv_heads * shape->head_dim, n_filled,
                                                map_flags_of(map_flags));
  const int g = n_layers < rf::kMaxGroup ? n_layers : rf::kMaxGroup;
  return L.fixed + (size_t)g * L.per_layer;
}

size_t ridgefill_fill_workspace_bytes(const rf_shape* shape, int64_t n_filled, int32_t n_layers) {
  return ridgefill_fill_workspace_bytes_ex(shape, n_filled, n_layers, 0);
}

rf_status ridgefill_fill(const rf_shape* shape, const uint16_t* x_S, int64_t N, int64_t T,
                         int64_t x_stride, const int32_t* filled_idx, int64_t n_filled,
                         const rf_layer* layers, int32_t n_layers, const rf_paged_kv* kv,
                         void* ws, size_t ws_bytes, void* stream) {
  bool done;
  rf_status s = fill_front(shape, N, T, n_filled, n_layers, ws, ws_bytes, stream, &done);
  if (s != RF_OK || done) return s == RF_OK ? ok() : s;
  rf::FillPlan p;
  std::vector<rf::FillLayerPtrs> lp;
  s = prepare_fill(shape, x_S, N, T, x_stride, filled_idx, n_filled, layers, n_layers, kv, ws,
                   ws_bytes, false, p, lp);
  if (s != RF_OK) return s;
  hipError_t e = rf::launch_fill(p, lp.data(), n_layers, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "fill launch");
  return ok();
}

rf_status ridgefill_fill_noalloc(const rf_shape* shape, const uint16_t* x_S, int64_t N, int64_t T,
                                 int64_t x_stride, const int32_t* filled_idx, int64_t n_filled,
                                 const rf_layer* layers, int32_t n_layers, const rf_paged_kv* kv,
                                 uint32_t* status, void* stream) {
  if (!status || !aligned(status, 4)) return fail(RF_E_INVALID, "status must be a 4-byte aligned device pointer");
  bool done;
  rf_status s = fill_front(shape, N, T, n_filled, n_layers, nullptr, 0, stream, &done);
  if (s != RF_OK) return s;
  hipError_t e;
  if (done) {
    e = rf::launch_clear_status(status, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "status clear");
    return ok();
  }
  void* scratch = nullptr;
  e = rf::noalloc_scratch(&scratch);
  if (e != hipSuccess) return hip_fail(e, "scratch address lookup");
  rf::FillPlan p;
  std::vector<rf::FillLayerPtrs> lp;
  s = prepare_fill(shape, x_S, N, T, x_stride, filled_idx, n_filled, layers, n_layers, kv, scratch,
                   rf::kNoAllocScratchBytes, false, p, lp);
  if (s == RF_E_WORKSPACE)
    return fail(RF_E_WORKSPACE, "one layer of this call needs more than the %zu-byte scratch of "
                "ridgefill_fill_noalloc (%s); use ridgefill_fill with a workspace",
                rf::kNoAllocScratchBytes, g_last_error.c_str());
  if (s != RF_OK) return s;
  p.status = status;                     // the caller's status word, not the scratch's
  e = rf::launch_fill(p, lp.data(), n_layers, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "fill launch");
  return ok();
}

rf_status ridgefill_fill_streamed(const rf_shape* shape, const uint16_t* x_S, int64_t N, int64_t T,
                                  int64_t x_stride, const int32_t* filled_idx, int64_t n_filled,
                                  const rf_layer* layers, int32_t n_layers, const rf_paged_kv* kv,
                                  void* ws, size_t ws_bytes, void* stream, void* copy_stream) {
  bool done;
  rf_status s = fill_front(shape, N, T, n_filled, n_layers, ws, ws_bytes, stream, &done);
  if (s != RF_OK || done) return s == RF_OK ? ok() : s;
  if (copy_stream == stream)
    return fail(RF_E_INVALID, "copy_stream must differ from stream for the copies to overlap");
  rf::FillPlan p;
  std::vector<rf::FillLayerPtrs> lp;
  s = prepare_fill(shape, x_S, N, T, x_stride, filled_idx, n_filled, layers, n_layers, kv, ws,
                   ws_bytes, true, p, lp);
  if (s != RF_OK) return s;
  hipError_t e = rf::launch_fill_streamed(p, lp.data(), n_layers, static_cast<hipStream_t>(stream),
                                          static_cast<hipStream_t>(copy_stream));
  if (e != hipSuccess) return hip_fail(e, "streamed fill launch");
  return ok();
}

// Value-rescale workspace: status, row list, two norm arrays, then per layer of a group a
// predicted block and an exact block (each laid out like a fill layer block).
static rf::VsLayout vs_layout(int64_t c, int n_kv, int group) {
  rf::VsLayout V = {};
  const int64_t cpad = (c + rf::kTile - 1) / rf::kTile * rf::kTile;
  V.idx = rf::kStatusBytes;
  V.vn_off = V.idx + rf::align256((size_t)cpad * 4);
  V.table_off = V.vn_off + rf::align256((size_t)2 * group * cpad * n_kv * 4);
  V.blocks = V.table_off + rf::align256((size_t)2 * group * sizeof(rf::FillLayerPtrs));
  V.total_fixed = V.blocks;
  return V;
}

size_t ridgefill_value_scale_workspace_bytes(const rf_shape* shape, int64_t c, int32_t n_layers,
                                             int32_t map_flags) {
  if (check_shape(shape) != RF_OK || c < 1 || n_layers < 1 ||
      (map_flags & ~(RF_MAPS_INT8 | RF_MAPS_FOLDED)) ||
      ((map_flags & RF_MAPS_INT8) && (map_flags & RF_MAPS_FOLDED)))
    return 0;
  if ((map_flags & RF_MAPS_FOLDED) && check_foldable(shape) != RF_OK) return 0;
  // folded layers use the plain layout: their partials fit where the plain ones go, and the
  // exact rows need the staged-input blocks either way
  const rf::FillWsLayout L = rf::fill_ws_layout(shape->d, d_in_of(shape), shape->head_dim,
                                                shape->n_kv_heads * shape->head_dim, c,
                                                map_flags_of(map_flags & RF_MAPS_INT8));
  const int g = n_layers < rf::kVsMaxGroup ? n_layers : rf::kVsMaxGroup;
  const rf::VsLayout V = vs_layout(c, shape->n_kv_heads, g);
  return V.total_fixed + (size_t)2 * g * L.per_layer;
}

rf_status ridgefill_value_scale(const rf_shape* shape, const uint16_t* x_S_tail, int64_t x_stride,
                                const uint16_t* const* x_l_tail, int64_t c, const rf_layer* layers,
                                int32_t n_layers, float* v_scale_out, void* ws, size_t ws_bytes,
                                void* stream) {
  rf_status s = check_shape(shape);
  if (s != RF_OK) return s;
  if (c < 1 || c > (1 << 20)) return fail(RF_E_SHAPE, "c = %lld must be in [1, 2^20]", (long long)c);
  if (n_layers < 1) return fail(RF_E_INVALID, "n_layers must be >= 1");
  if (!x_S_tail || !x_l_tail || !layers || !v_scale_out || !ws)
    return fail(RF_E_INVALID, "null pointer among x_S_tail, x_l_tail, layers, v_scale_out, ws");
  const int d_in = d_in_of(shape);
  if (x_stride < d_in || x_stride % 8 || !aligned(x_S_tail, 16))
    return fail(RF_E_SHAPE, "x_S_tail must be 16-byte aligned, x_stride >= d_in and a multiple of 8");
  if ((uint64_t)(c - 1) * (uint64_t)x_stride * 2u + (uint64_t)d_in * 2u > 0xffffffffull)
    return fail(RF_E_SHAPE, "the tail rows of x_S span more than 4 GiB");
  if (!aligned(ws, 256) || !aligned(v_scale_out, 4))
    return fail(RF_E_WORKSPACE, "workspace must be 256-byte aligned, v_scale_out 4-byte aligned");
  const bool folded = layers[0].folded != nullptr;
  const bool int8 = !folded && layers[0].A_q != nullptr;
  if (folded) {
    s = check_foldable(shape);
    if (s != RF_OK) return s;
  }
  for (int i = 0; i < n_layers; ++i) {
    const rf_layer& l = layers[i];
    if ((l.folded != nullptr) != folded)
      return fail(RF_E_INVALID, "layer %d: all layers of a call must be folded or none", i);
    if (folded) {                 // the folded buffer, and for the exact rows W_V and norm_w
      if (!l.norm_w || !l.W_V || !x_l_tail[i])
        return fail(RF_E_INVALID, "layer %d: a folded layer needs norm_w, W_V and its exact "
                    "tail rows", i);
      if (!aligned(l.folded, 256) || !aligned(l.norm_w, 16) || !aligned(l.W_V, 16) ||
          !aligned(x_l_tail[i], 16))
        return fail(RF_E_SHAPE, "layer %d: the folded buffer needs 256-byte, norm_w, W_V and "
                    "the exact rows 16-byte alignment", i);
      continue;
    }
    if (!l.b || !l.norm_w || !l.W_V || !x_l_tail[i])
      return fail(RF_E_INVALID, "layer %d: b, norm_w, W_V and its exact tail rows are required",
                  i);
    if ((l.A != nullptr) == (l.A_q != nullptr) || (l.A_q != nullptr) != int8 ||
        (int8 && !l.A_scale))
      return fail(RF_E_INVALID, "layer %d: exactly one of A and A_q (with A_scale), the same kind "
                  "for all layers", i);
    if ((l.A && !aligned(l.A, 16)) || (l.A_q && !aligned(l.A_q, 16)) || !aligned(l.b, 16) ||
        !aligned(l.norm_w, 16) || !aligned(l.W_V, 16) || !aligned(x_l_tail[i], 16))
      return fail(RF_E_SHAPE, "layer %d: A, A_q, b, norm_w, W_V and the exact rows need 16-byte "
                  "alignment", i);
  }
  const unsigned flags = int8 ? rf::kWsInt8 : folded ? rf::kWsFolded : 0u;
  const rf::FillWsLayout L = rf::fill_ws_layout(shape->d, d_in, shape->head_dim,
                                                shape->n_kv_heads * shape->head_dim, c,
                                                int8 ? rf::kWsInt8 : 0u);
  const int gmax = n_layers < rf::kVsMaxGroup ? n_layers : rf::kVsMaxGroup;
  // the largest group the workspace holds: fixed part for that group + 2 blocks per layer
  int group = 0;
  for (int g = gmax; g >= 1; --g) {
    const rf::VsLayout V = vs_layout(c, shape->n_kv_heads, g);
    if (ws_bytes >= V.total_fixed + (size_t)2 * g * L.per_layer) { group = g; break; }
  }
  if (group == 0)
    return fail(RF_E_WORKSPACE, "workspace %zu bytes too small for one layer", ws_bytes);
  rf::VsLayout V = vs_layout(c, shape->n_kv_heads, group);
  unsigned char* w = static_cast<unsigned char*>(ws);
  V.vn = reinterpret_cast<float*>(w + V.vn_off);
  V.table = reinterpret_cast<rf::FillLayerPtrs*>(w + V.table_off);

  rf::FillPlan p = {};
  p.d = shape->d;
  p.d_in = d_in;
  p.n_kv = shape->n_kv_heads;
  p.hd = shape->head_dim;
  p.kv = shape->n_kv_heads * shape->head_dim;
  p.flags = flags;
  p.eps = shape->rms_eps;
  p.theta = shape->rope_theta;
  p.xS = x_S_tail;
  p.x_stride = x_stride;
  p.N = c;
  p.P = c;
  p.idx = reinterpret_cast<const int32_t*>(w + V.idx);
  p.n_filled = (int)c;
  p.mpad = (int)((c + rf::kTile - 1) / rf::kTile * rf::kTile);
  p.status = reinterpret_cast<unsigned*>(w);
  p.hbuf = reinterpret_cast<uint16_t*>(w + V.blocks);
  p.group = group;
  p.L = L;
  std::vector<rf::FillLayerPtrs> lp((size_t)n_layers);
  std::vector<const uint16_t*> wv((size_t)n_layers);
  const rf::FoldLayout F = rf::fold_layout(d_in, p.kv);
  for (int i = 0; i < n_layers; ++i) {
    const rf_layer& l = layers[i];
    wv[i] = l.W_V;
    if (folded) {
      const unsigned char* f = static_cast<const unsigned char*>(l.folded);
      const uint16_t* P = reinterpret_cast<const uint16_t*>(f + F.P);
      lp[i] = {reinterpret_cast<const uint16_t*>(f + F.R), reinterpret_cast<const float*>(f + F.r),
               l.norm_w, nullptr, P + (size_t)p.kv * d_in, nullptr, nullptr, nullptr, nullptr,
               nullptr, nullptr, reinterpret_cast<const float*>(f + F.c),
               reinterpret_cast<const float*>(f + F.kappa), reinterpret_cast<const float*>(f + F.g)};
    } else {              // the value norms read W_V only (W_K is not needed)
      lp[i] = {l.A, l.b, l.norm_w, nullptr, l.W_V, nullptr, nullptr, nullptr, nullptr, l.A_q,
               l.A_scale, nullptr, nullptr, nullptr};
    }
  }
  hipError_t e = rf::launch_value_scale(p, lp.data(), x_l_tail, wv.data(), n_layers,
                                        v_scale_out, V, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "value-scale launch");
  return ok();
}

static bool dims_ok(int d_in, int d_out) {
  return d_in >= rf::kTile && d_in % rf::kTile == 0 && d_out >= rf::kTile && d_out % rf::kTile == 0;
}

size_t ridgefill_calib_state_bytes_ex(int32_t d_in, int32_t d_out, int32_t n_layers) {
  if (!dims_ok(d_in, d_out) || n_layers < 1) return 0;
  return rf::calib_layout(d_in, d_out, n_layers).total;
}

size_t ridgefill_calib_state_bytes(int32_t d, int32_t n_layers) {
  return ridgefill_calib_state_bytes_ex(d, d, n_layers);
}

static rf_status check_state(const void* state, size_t bytes, int d_in, int d_out, int n_layers) {
  if (!state) return fail(RF_E_INVALID, "state is NULL");
  if (!aligned(state, 256)) return fail(RF_E_WORKSPACE, "state must be 256-byte aligned");
  if (!dims_ok(d_in, d_out))
    return fail(RF_E_SHAPE, "d_in = %d and d_out = %d must be positive multiples of %d", d_in,
                d_out, rf::kTile);
  if (n_layers < 1 || n_layers > 64) return fail(RF_E_SHAPE, "n_layers = %d must be in 1..64", n_layers);
  if (bytes < rf::calib_layout(d_in, d_out, n_layers).total)
    return fail(RF_E_WORKSPACE, "state %zu bytes < %zu needed", bytes,
                rf::calib_layout(d_in, d_out, n_layers).total);
  return RF_OK;
}

rf_status ridgefill_calib_reset_ex(void* state, size_t state_bytes, int32_t d_in, int32_t d_out,
                                   int32_t n_layers, void* stream) {
  rf_status s = check_state(state, state_bytes, d_in, d_out, n_layers);
  if (s != RF_OK) return s;
  hipError_t e = rf::launch_calib_reset(state, d_in, d_out, n_layers,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "calibration reset");
  return ok();
}

rf_status ridgefill_calib_reset(void* state, size_t state_bytes, int32_t d, int32_t n_layers,
                                void* stream) {
  return ridgefill_calib_reset_ex(state, state_bytes, d, d, n_layers, stream);
}

rf_status ridgefill_calibrate_ex(void* state, size_t state_bytes, int32_t d_in, int32_t d_out,
                                 int32_t n_layers, const uint16_t* x_S, const uint16_t* const* x_l,
                                 int64_t n_rows, void* stream) {
  rf_status s = check_state(state, state_bytes, d_in, d_out, n_layers);
  if (s != RF_OK) return s;
  if (n_rows < 0 || n_rows > INT32_MAX) return fail(RF_E_SHAPE, "n_rows out of range");
  if (n_rows == 0) return ok();
  if (!x_S || !x_l) return fail(RF_E_INVALID, "x_S or x_l is NULL");
  if (!aligned(x_S, 16)) return fail(RF_E_SHAPE, "x_S must be 16-byte aligned");
  for (int l = 0; l < n_layers; ++l)
    if (!x_l[l] || !aligned(x_l[l], 16))
      return fail(RF_E_INVALID, "x_l[%d] is NULL or not 16-byte aligned", l);
  hipError_t e = rf::launch_calibrate(state, d_in, d_out, n_layers, x_S, x_l, n_rows,
                                      static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return fail(RF_E_UNSUPPORTED, "calibration kernels not built");
  if (e != hipSuccess) return hip_fail(e, "calibration launch");
  return ok();
}

rf_status ridgefill_calibrate(void* state, size_t state_bytes, int32_t d, int32_t n_layers,
                              const uint16_t* x_S, const uint16_t* const* x_l, int64_t n_rows,
                              void* stream) {
  return ridgefill_calibrate_ex(state, state_bytes, d, d, n_layers, x_S, x_l, n_rows, stream);
}

size_t ridgefill_solve_workspace_bytes_ex(int32_t d_in, int32_t d_out, int32_t n_layers) {
  if (!dims_ok(d_in, d_out) || n_layers < 1) return 0;
  return rf::solve_layout(d_in, d_out, n_layers).total;
}

size_t ridgefill_solve_workspace_bytes(int32_t d, int32_t n_layers) {
  return ridgefill_solve_workspace_bytes_ex(d, d, n_layers);
}

rf_status ridgefill_solve_ex(const void* state, size_t state_bytes, int32_t d_in, int32_t d_out,
                             int32_t n_layers, double lambda, float* A_out, float* b_out,
                             uint16_t* A_bf16_out, void* ws, size_t ws_bytes, void* stream) {
  rf_status s = check_state(state, state_bytes, d_in, d_out, n_layers);
  if (s != RF_OK) return s;
  if (!(lambda >= 0.0) || !std::isfinite(lambda))
    return fail(RF_E_INVALID, "lambda must be finite and >= 0");
  if (!b_out || (!A_out && !A_bf16_out))
    return fail(RF_E_INVALID, "b_out and at least one of A_out, A_bf16_out are required");
  if ((A_out && !aligned(A_out, 16)) || !aligned(b_out, 16) || (A_bf16_out && !aligned(A_bf16_out, 16)))
    return fail(RF_E_SHAPE, "outputs must be 16-byte aligned");
  if (!ws || !aligned(ws, 256)) return fail(RF_E_WORKSPACE, "workspace NULL or not 256-byte aligned");
  if (ws_bytes < rf::solve_layout(d_in, d_out, n_layers).total)
    return fail(RF_E_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes,
                rf::solve_layout(d_in, d_out, n_layers).total);
  hipError_t e = rf::launch_solve(state, d_in, d_out, n_layers, lambda, A_out, b_out, A_bf16_out,
                                  ws, static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return fail(RF_E_UNSUPPORTED, "solve kernels not built");
  if (e != hipSuccess) return hip_fail(e, "solve launch");
  return ok();
}

rf_status ridgefill_solve(const void* state, size_t state_bytes, int32_t d, int32_t n_layers,
                          double lambda, float* A_out, float* b_out, uint16_t* A_bf16_out,
                          void* ws, size_t ws_bytes, void* stream) {
  return ridgefill_solve_ex(state, state_bytes, d, d, n_layers, lambda, A_out, b_out, A_bf16_out,
                            ws, ws_bytes, stream);
}

rf_status ridgefill_read_status(void* ws, void* stream) {
  if (!ws) return fail(RF_E_INVALID, "workspace is NULL");
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "stream synchronize");
  unsigned word = 0;
  e = hipMemcpy(&word, ws, sizeof word, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "status read");
  if (word & rf::kStatusStateBit)     // first: a mismatched state explains any pivot failure
    return fail(RF_E_WORKSPACE, "calibration state does not match the sizes it was reset with");
  if (word & rf::kStatusRowsBit) return fail(RF_E_ROWS, "device flagged filled-row indices");
  if (word & rf::kStatusNotSpdBit) return fail(RF_E_NOT_SPD, "device flagged a non-positive pivot");
  if (word & rf::kStatusScoreBit) return fail(RF_E_INVALID, "device flagged a NaN selection score");
  return ok();
}

rf_status ridgefill_solve_info(void* ws, double* kappa_f, int32_t* parts, void* stream) {
  if (!ws) return fail(RF_E_INVALID, "workspace is NULL");
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "stream synchronize");
  unsigned char buf[rf::kSolveInfoBytes];
  e = hipMemcpy(buf, static_cast<unsigned char*>(ws) + rf::kSolveInfoOff, sizeof buf,
                hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "solve info read");
  double k;
  int32_t p;
  std::memcpy(&k, buf, sizeof k);
  std::memcpy(&p, buf + 8, sizeof p);
  if (kappa_f) *kappa_f = k;
  if (parts) *parts = p;
  return ok();
}

size_t ridgefill_fold_bytes(const rf_shape* shape) {
  if (check_shape(shape) != RF_OK || check_foldable(shape) != RF_OK) return 0;
  return rf::fold_layout(d_in_of(shape), shape->n_kv_heads * shape->head_dim).total;
}

size_t ridgefill_fold_workspace_bytes_maps(const rf_shape* shape, int32_t layers_at_once,
                                           uint32_t map_flags) {
  if (check_shape(shape) != RF_OK || check_foldable(shape) != RF_OK || layers_at_once < 1 ||
      (map_flags & ~(uint32_t)RF_MAPS_INT8))
    return 0;
  return rf::fold_ws_layout(shape->d, d_in_of(shape), shape->n_kv_heads * shape->head_dim,
                            layers_at_once, (map_flags & RF_MAPS_INT8) != 0).total;
}

size_t ridgefill_fold_workspace_bytes_ex(const rf_shape* shape, int32_t layers_at_once) {
  return ridgefill_fold_workspace_bytes_maps(shape, layers_at_once, 0);
}

size_t ridgefill_fold_workspace_bytes(const rf_shape* shape) {
  return ridgefill_fold_workspace_bytes_ex(shape, 1);
}

rf_status ridgefill_fold_maps(const rf_shape* shape, const rf_layer* layers, int32_t n_layers,
                              void* const* folded, void* ws, size_t ws_bytes, void* stream) {
  rf_status s = check_shape(shape);
  if (s != RF_OK) return s;
  if ((s = check_foldable(shape)) != RF_OK) return s;
  if (n_layers < 0) return fail(RF_E_INVALID, "n_layers < 0");
  if (n_layers > 0 && (!layers || !folded)) return fail(RF_E_INVALID, "layers or folded is NULL");
  if (!ws) return fail(RF_E_INVALID, "ws is NULL");
  const int d = shape->d, d_in = d_in_of(shape), kv = shape->n_kv_heads * shape->head_dim;
  // int8 maps (A_q, A_scale) or bf16 maps (A): one kind per call
  const bool int8 = n_layers > 0 && layers[0].A_q != nullptr;
  for (int i = 0; i < n_layers; ++i) {
    const rf_layer& l = layers[i];
    if ((l.A_q != nullptr) != int8)
      return fail(RF_E_INVALID, "layer %d: all layers of a call need int8 maps or none", i);
    if (int8 ? (!l.A_q || !l.A_scale || l.A) : !l.A)
      return fail(RF_E_INVALID, "layer %d: exactly one map, A or A_q with A_scale, is needed", i);
    if (!l.b || !l.norm_w || !l.W_K || !l.W_V || !folded[i])
      return fail(RF_E_INVALID, "layer %d: b, norm_w, W_K, W_V and its folded buffer are needed", i);
    if ((l.A && !aligned(l.A, 16)) || (l.A_scale && !aligned(l.A_scale, 4)) ||
        !aligned(l.W_K, 16) || !aligned(l.W_V, 16) || !aligned(l.b, 4) ||
        !aligned(l.norm_w, 2) || !aligned(folded[i], 256))
      return fail(RF_E_SHAPE, "layer %d: A, W_K, W_V need 16-byte, A_scale and b 4-byte, the "
                  "folded buffer 256-byte alignment", i);
  }
  const rf::FoldWsLayout W1 = rf::fold_ws_layout(d, d_in, kv, 1, int8);
  if (!aligned(ws, 256) || ws_bytes < W1.total)
    return fail(RF_E_WORKSPACE, "fold workspace must be 256-byte aligned and >= %zu bytes%s",
                W1.total, int8 ? " (int8 maps)" : "");
  // as many layers side by side as the workspace holds
  int cap = n_layers > 0 ? n_layers : 1;
  if (cap > rf::kMaxFoldGroup) cap = rf::kMaxFoldGroup;
  int n_par = 1;
  while (n_par < cap && rf::fold_ws_layout(d, d_in, kv, n_par + 1, int8).total <= ws_bytes) ++n_par;
  const rf::FoldWsLayout W = rf::fold_ws_layout(d, d_in, kv, n_par, int8);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = rf::launch_clear_status(static_cast<unsigned*>(ws), st);
  if (e != hipSuccess) return hip_fail(e, "status clear");
  rf::FoldLayerIn in[rf::kMaxFoldGroup];
  for (int l0 = 0; l0 < n_layers; l0 += n_par) {
    const int G = n_layers - l0 < n_par ? n_layers - l0 : n_par;
    for (int g = 0; g < G; ++g) {
      const rf_layer& l = layers[l0 + g];
      in[g] = {l.A, l.b, l.norm_w, l.W_K, l.W_V, l.A_q, l.A_scale};
    }
    e = rf::launch_fold(d, d_in, kv, in, G, folded + l0, ws, W, st);
    if (e != hipSuccess) return hip_fail(e, "fold launch");
  }
  return ok();
}

rf_status ridgefill_quantize_map(const float* A, int64_t rows, int64_t cols, int8_t* A_q,
                                 float* A_scale, void* stream) {
  if (rows < 1 || rows > INT32_MAX || cols < 1)
    return fail(RF_E_SHAPE, "rows = %lld, cols = %lld", (long long)rows, (long long)cols);
  if (!A || !A_q || !A_scale) return fail(RF_E_INVALID, "null pointer among A, A_q, A_scale");
  if (!aligned(A, 4) || !aligned(A_scale, 4)) return fail(RF_E_SHAPE, "A and A_scale need 4-byte alignment");
  hipError_t e = rf::launch_quantize(A, rows, cols, A_q, A_scale, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "quantize launch");
  return ok();
}

size_t ridgefill_select_workspace_bytes(int64_t P) {
  if (P < 0 || P > INT32_MAX) return 0;
  return rf::select_layout(P).total;
}

rf_status ridgefill_select_rows(const float* scores, int64_t P, int64_t k, uint8_t* exact_mask,
                                int32_t* filled_idx, void* ws, size_t ws_bytes, void* stream) {
  if (P < 0 || P > INT32_MAX) return fail(RF_E_SHAPE, "P = %lld must be in [0, 2^31)", (long long)P);
  if (k < 0 || k > P) return fail(RF_E_SHAPE, "k = %lld must be in [0, P = %lld]", (long long)k,
                                  (long long)P);
  if (!ws) return fail(RF_E_INVALID, "workspace is NULL");
  if (!aligned(ws, 256)) return fail(RF_E_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < rf::select_layout(P).total)
    return fail(RF_E_WORKSPACE, "workspace %zu bytes < %zu", ws_bytes, rf::select_layout(P).total);
  if (P == 0) {
    hipError_t e = rf::launch_clear_status(static_cast<unsigned*>(ws), static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, "status clear");
  }
  if (!scores || (P > k && !filled_idx))
    return fail(RF_E_INVALID, "scores and (unless k = P) filled_idx are required");
  if (!aligned(scores, 4) || !aligned(filled_idx, 4))
    return fail(RF_E_SHAPE, "scores and filled_idx need 4-byte alignment");
  hipError_t e = rf::launch_select(scores, P, k, exact_mask, filled_idx, ws,
                                   static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "selection launch");
  return ok();
}

}  // extern "C"
