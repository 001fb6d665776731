// The C-ABI of libnarrowcast: argument checks, batching into launches of at
// most kMaxSeg tensors, workspace layout.  No allocation; the only state is
// the per-device address of the static scratch that nc_cast_tensor_static
// uses in place of a workspace (looked up once per device).
#include <mutex>
#include <string.h>

#include "nc_launch.h"

using namespace nc;

// The workspace of nc_cast_tensor_static: one array per GPU the library runs
// on, held until the process ends.  Host code never uses this name as an
// address (on the host it stands for a shadow variable): the device address
// comes from hipGetSymbolAddress, per device, in scratch_for().
static __device__ __align__(256) uint8_t scratch[NC_STATIC_SCRATCH_BYTES];

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int in_bytes(nc_dtype d) { return d == NC_F32 ? 4 : 2; }

// Checks shared by the calls that read tensors.  need_x / need_codes /
// mx: which fields must be valid.
nc_status check_tensors(const nc_tensor* t, int32_t count, bool need_x, bool need_codes, bool mx) {
  if (count < 0) return NC_E_ARG;
  if (count > 0 && t == nullptr) return NC_E_ARG;
  for (int32_t i = 0; i < count; ++i) {
    const nc_tensor& x = t[i];
    if (x.n < 0) return NC_E_ARG;
    if (mx && x.mx_axis != NC_MX_ROWS && x.mx_axis != NC_MX_COLS) return NC_E_UNSUPPORTED;
    if (mx && x.mx_axis != t[0].mx_axis) return NC_E_SHAPE;
    if (mx && (x.cols <= 0 || x.cols % 32 != 0 || x.n % x.cols != 0)) return NC_E_SHAPE;
    if (mx && x.mx_axis == NC_MX_COLS && (x.n / x.cols) % 32 != 0) return NC_E_SHAPE;
    if (x.n == 0) continue;
    if ((need_x && x.x == nullptr) || (need_codes && x.codes == nullptr)) return NC_E_ARG;
    if (mx && x.scales == nullptr) return NC_E_ARG;
    if ((need_x && !aligned16(x.x)) || (need_codes && !aligned16(x.codes))) return NC_E_ALIGN;
  }
  return NC_OK;
}

// Launches cover consecutive tensors (so b.first + s indexes the caller's
// arrays): at most kMaxSeg of them and at most kMaxLaunchElems elements, a
// rule that does not depend on the tile size, so every call on the same
// tensors forms the same launches.  A tensor larger than one launch is an
// error.
constexpr int64_t kMaxLaunchElems = (int64_t)1 << 34;

// The two descriptor types in a launch's Seg: a cast tensor (x, codes,
// scales, optional dequant output y), or a weight/update pair of the
// monitor (w in x, d in y, flags in codes).
void fill_seg(Seg& g, const nc_tensor& x, void* y) {
  g.x = x.x;
  g.codes = x.codes;
  g.scales = x.scales;
  g.y = y;
  g.cols = x.cols;
}
void fill_seg(Seg& g, const nc_update_tensor& x, void*) {
  g.x = x.w;
  g.y = const_cast<float*>(x.d);
  g.codes = x.flags;
  g.scales = nullptr;
  g.cols = 0;
}

// Launch boundaries: calls fn(first, end) for each launch [first, end).
template <typename T, typename Fn>
nc_status for_launches(const T* t, int32_t count, Fn fn) {
  int32_t i = 0;
  while (i < count) {
    const int32_t first = i;
    int64_t elems = 0;
    while (i < count && i - first < kMaxSeg && elems + t[i].n <= kMaxLaunchElems) elems += t[i++].n;
    if (i == first) return NC_E_ARG;     // one tensor above the per-launch limit
    const nc_status st = fn(first, i);
    if (st != NC_OK) return st;
  }
  return NC_OK;
}

// Fills b for tensors [first, end) with tiles of `tile` units of `unit`
// elements (unit 1: element tiles; column-block MX: col_slots, which divide
// every tensor the checks admit).  b.last counts units.
template <typename T>
void make_batch(SegBatch& b, const T* t, int32_t first, int32_t end, int64_t tile, void* const* y,
                int64_t unit = 1) {
  memset(&b, 0, sizeof(b));
  b.first = first;
  b.count = end - first;
  for (int32_t s = 0; s < b.count; ++s) {
    const T& x = t[first + s];
    Seg& g = b.s[s];
    fill_seg(g, x, y ? y[first + s] : nullptr);
    g.n = x.n;
    const int64_t units = x.n / unit;
    const int64_t tiles = (units + tile - 1) / tile;
    b.tile0[s + 1] = (int32_t)(b.tile0[s] + tiles);
    b.chunk0[s + 1] = (int32_t)(b.chunk0[s] + (tiles + kChunk - 1) / kChunk);
    b.last[s] = tiles ? (int32_t)(units - (tiles - 1) * tile) : 0;
  }
  for (int s = b.count + 1; s <= kMaxSeg; ++s) {
    b.tile0[s] = b.tile0[b.count];
    b.chunk0[s] = b.chunk0[b.count];
  }
}

// Walk the call in launches; `fn(batch)` enqueues one launch (skipped when
// the launch has no element at all).
template <typename T, typename Fn>
nc_status for_batches(const T* t, int32_t count, int64_t tile, void* const* y, Fn fn, int64_t unit = 1) {
  SegBatch b;
  return for_launches(t, count, [&](int32_t first, int32_t end) {
    make_batch(b, t, first, end, tile, y, unit);
    if (b.tile0[b.count] == 0) return NC_OK;
    return fn(b);
  });
}

nc_status hip_status(hipError_t e) { return e == hipSuccess ? NC_OK : NC_E_HIP; }

bool valid_dtype(nc_dtype d) { return d == NC_F32 || d == NC_BF16; }
bool valid_fmt(nc_fmt f) { return f == NC_E4M3 || f == NC_E5M2; }

nc_status check_ws(const nc_tensor* t, int32_t count, void* ws, size_t ws_bytes) {
  if (ws == nullptr || ((uintptr_t)ws & 15u) != 0) return NC_E_WORKSPACE;
  if (ws_bytes < nc_workspace_bytes(t, count)) return NC_E_WORKSPACE;
  return NC_OK;
}

Ws ws_of(const SegBatch& b, void* ws) { return ws_layout(ws, b.tile0[b.count], b.chunk0[b.count]); }

// Per-workgroup and per-chunk slots of the largest launch at tile `tile`.
template <typename T>
size_t ws_need(const T* t, int32_t count, int64_t tile) {
  if (t == nullptr || count <= 0) return 0;
  size_t need = 0;
  SegBatch b;
  for_launches(t, count, [&](int32_t first, int32_t end) {
    make_batch(b, t, first, end, tile, nullptr);
    const size_t v = ws_bytes_for(b.tile0[b.count], b.chunk0[b.count]);
    if (v > need) need = v;
    return NC_OK;
  });
  return need;
}


// Device address of `scratch` on the device that runs `stream` (the calling
// thread's current device for the null stream), looked up on first use with
// that device current and kept for the rest of the process.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

nc_status scratch_for(hipStream_t stream, void** out) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return NC_E_HIP;
  int dev = cur;
  if (stream != nullptr && hipStreamGetDevice(stream, &dev) != hipSuccess) return NC_E_HIP;
  if (dev < 0 || dev >= kMaxDevices) return NC_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return NC_E_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return NC_E_HIP;
    if (e != hipSuccess || p == nullptr) return NC_E_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return NC_OK;
}

}  // namespace

extern "C" {

size_t nc_workspace_bytes(const nc_tensor* t, int32_t count) {
  // at the smallest tile any call uses
  return ws_need(t, count, kMinWsTile);
}

size_t nc_swamp_workspace_bytes(const nc_update_tensor* t, int32_t count) {
  return ws_need(t, count, kSwampTile);
}

const char* nc_status_string(nc_status s) {
  switch (s) {
    case NC_OK: return "ok";
    case NC_E_ARG: return "invalid argument (null pointer, negative size, tensor above 2^34 elements or bad policy field)";
    case NC_E_ALIGN: return "element pointer not 16-byte aligned";
    case NC_E_SHAPE:
      return "MX shape: cols must be a positive multiple of 32 dividing n (column blocks: rows a multiple of "
             "32 too), one mx_axis per call";
    case NC_E_UNSUPPORTED: return "unsupported dtype, format, rule or estimator";
    case NC_E_HIP: return "HIP launch failed";
    case NC_E_WORKSPACE: return "workspace missing, misaligned or smaller than nc_workspace_bytes()";
    case NC_E_SCRATCH:
      return "the batch needs a larger workspace than the static scratch of nc_cast_tensor_static "
             "(NC_STATIC_SCRATCH_BYTES); use nc_cast_tensor with a workspace";
  }
  return "unknown status";
}

nc_status nc_amax(const nc_tensor* t, int32_t count, nc_dtype dtype, const nc_loss_scale* ls,
                  nc_counts* out, void* ws, size_t ws_bytes, void* stream) {
  if (!valid_dtype(dtype)) return NC_E_UNSUPPORTED;
  nc_status s = check_tensors(t, count, true, false, false);
  if (s != NC_OK) return s;
  if (count == 0) return NC_OK;
  if (out == nullptr) return NC_E_ARG;
  if ((s = check_ws(t, count, ws, ws_bytes)) != NC_OK) return s;
  const int64_t tile = tile_elems(in_bytes(dtype), kAmaxVecs);
  return for_batches(t, count, tile, nullptr, [&](const SegBatch& b) {
    const Tail tl = tail_of(ws_of(b, ws), b.tile0[b.count], out, nullptr, ls, false);
    nc_status r = hip_status(launch_amax(b, dtype, tl, Launch{b.tile0[b.count], (hipStream_t)stream}));
    if (r == NC_OK && !tl.direct) r = hip_status(launch_reduce(b, tl, (hipStream_t)stream));
    return r;
  });
}

nc_status nc_scale_update(const nc_policy* p, int32_t count, nc_scale_state* st, float* hist,
                          const nc_counts* in, nc_loss_scale* ls, void* stream) {
  if (p == nullptr || count < 0) return NC_E_ARG;
  if (!valid_fmt((nc_fmt)p->fmt)) return NC_E_UNSUPPORTED;
  if (p->est != NC_EST_CURRENT && p->est != NC_EST_MOST_RECENT && p->est != NC_EST_MAX_WINDOW &&
      p->est != NC_EST_EMA)
    return NC_E_UNSUPPORTED;
  if (p->est == NC_EST_EMA && !(p->ema_alpha > 0.0f && p->ema_alpha <= 1.0f)) return NC_E_ARG;
  if (p->window < 1 || p->window > 1024 || p->margin < 0 || p->margin > 32 || p->interval < 1)
    return NC_E_ARG;
  if (p->ls_enable && (p->ls_growth_interval < 1 || p->ls_log2_min < 0 ||
                       p->ls_log2_max < p->ls_log2_min || p->ls_log2_max > 64))
    return NC_E_ARG;
  if (count == 0) return NC_OK;
  if (st == nullptr || in == nullptr) return NC_E_ARG;
  if (p->est != NC_EST_CURRENT && hist == nullptr) return NC_E_ARG;
  return hip_status(launch_scale_update(*p, count, st, hist, in, ls, (hipStream_t)stream));
}

nc_status nc_cast_tensor(const nc_tensor* t, int32_t count, nc_dtype dtype, nc_fmt fmt,
                         const nc_scale_state* st, const nc_loss_scale* ls, nc_counts* out,
                         nc_stats* stats, void* ws, size_t ws_bytes, void* stream) {
  if (!valid_dtype(dtype) || !valid_fmt(fmt)) return NC_E_UNSUPPORTED;
  nc_status s = check_tensors(t, count, true, true, false);
  if (s != NC_OK) return s;
  if (count == 0) return NC_OK;
  if (out == nullptr || st == nullptr) return NC_E_ARG;
  if ((s = check_ws(t, count, ws, ws_bytes)) != NC_OK) return s;
  const int64_t tile = tile_elems(in_bytes(dtype), stats ? kCastStatsVecs : kCastVecs);
  return for_batches(t, count, tile, nullptr, [&](const SegBatch& b) {
    const Tail tl = tail_of(ws_of(b, ws), b.tile0[b.count], out, stats, ls, true);
    nc_status r = hip_status(launch_cast_pt(b, dtype, fmt, st, ls, stats != nullptr, tl,
                                            Launch{b.tile0[b.count], (hipStream_t)stream}));
    if (r == NC_OK && !tl.direct) r = hip_status(launch_reduce(b, tl, (hipStream_t)stream));
    return r;
  });
}

nc_status nc_cast_tensor_static(const nc_tensor* t, int32_t count, nc_dtype dtype, nc_fmt fmt,
                                const nc_scale_state* st, const nc_loss_scale* ls, nc_counts* out,
                                nc_stats* stats, void* stream) {
  // every check of nc_cast_tensor except the workspace's, before anything is enqueued
  if (!valid_dtype(dtype) || !valid_fmt(fmt)) return NC_E_UNSUPPORTED;
  nc_status s = check_tensors(t, count, true, true, false);
  if (s != NC_OK) return s;
  if (count == 0) return NC_OK;
  if (out == nullptr || st == nullptr) return NC_E_ARG;
  if (nc_workspace_bytes(t, count) > NC_STATIC_SCRATCH_BYTES) return NC_E_SCRATCH;
  void* ws = nullptr;
  if ((s = scratch_for((hipStream_t)stream, &ws)) != NC_OK) return s;
  return nc_cast_tensor(t, count, dtype, fmt, st, ls, out, stats, ws, NC_STATIC_SCRATCH_BYTES, stream);
}

nc_status nc_cast_tensor_sr(const nc_tensor* t, int32_t count, nc_dtype dtype, nc_fmt fmt,
                            const nc_scale_state* st, const nc_loss_scale* ls, uint64_t seed, uint64_t offset,
                            nc_counts* out, void* ws, size_t ws_bytes, void* stream) {
  if (!valid_dtype(dtype) || !valid_fmt(fmt)) return NC_E_UNSUPPORTED;
  nc_status s = check_tensors(t, count, true, true, false);
  if (s != NC_OK) return s;
  if (count == 0) return NC_OK;
  if (out == nullptr || st == nullptr) return NC_E_ARG;
  if ((s = check_ws(t, count, ws, ws_bytes)) != NC_OK) return s;
  const int64_t tile = tile_elems(in_bytes(dtype), kCastSrVecs);
  return for_batches(t, count, tile, nullptr, [&](const SegBatch& b) {
    const Tail tl = tail_of(ws_of(b, ws), b.tile0[b.count], out, nullptr, ls, true);
    nc_status r = hip_status(launch_cast_sr(b, dtype, fmt, st, ls, seed, offset, tl,
                                            Launch{b.tile0[b.count], (hipStream_t)stream}));
    if (r == NC_OK && !tl.direct) r = hip_status(launch_reduce(b, tl, (hipStream_t)stream));
    return r;
  });
}

nc_status nc_cast_mx(const nc_tensor* t, int32_t count, nc_dtype dtype, nc_fmt fmt, nc_mx_rule rule,
                     nc_counts* out, nc_stats* stats, void* ws, size_t ws_bytes, void* stream) {
  if (!valid_dtype(dtype) || !valid_fmt(fmt)) return NC_E_UNSUPPORTED;
  if (rule != NC_MX_OCP && rule != NC_MX_PLUS1 && rule != NC_MX_CEIL) return NC_E_UNSUPPORTED;
  nc_status s = check_tensors(t, count, true, true, true);
  if (s != NC_OK) return s;
  if (count == 0) return NC_OK;
  if (out == nullptr) return NC_E_ARG;
  if ((s = check_ws(t, count, ws, ws_bytes)) != NC_OK) return s;
  if (t[0].mx_axis == NC_MX_COLS)
    return for_batches(t, count, kThreads / col_cast_split(dtype), nullptr, [&](const SegBatch& b) {
      const Tail tl = tail_of(ws_of(b, ws), b.tile0[b.count], out, stats, nullptr, true);
      nc_status r = hip_status(launch_cast_mx_col(b, dtype, fmt, rule, stats != nullptr, tl,
                                                  Launch{b.tile0[b.count], (hipStream_t)stream}));
      if (r == NC_OK && !tl.direct) r = hip_status(launch_reduce(b, tl, (hipStream_t)stream));
      return r;
    }, col_unit(in_bytes(dtype)));
  const int64_t tile = tile_elems(in_bytes(dtype), stats ? kCastStatsVecs : kCastVecs);
  return for_batches(t, count, tile, nullptr, [&](const SegBatch& b) {
    const Tail tl = tail_of(ws_of(b, ws), b.tile0[b.count], out, stats, nullptr, true);
    nc_status r = hip_status(launch_cast_mx(b, dtype, fmt, rule, stats != nullptr, tl,
                                            Launch{b.tile0[b.count], (hipStream_t)stream}));
    if (r == NC_OK && !tl.direct) r = hip_status(launch_reduce(b, tl, (hipStream_t)stream));
    return r;
  });
}

nc_status nc_dequant(const nc_tensor* t, int32_t count, nc_fmt fmt, const nc_scale_state* st,
                     void* const* y, nc_dtype out_dtype, void* stream) {
  if (!valid_fmt(fmt) || out_dtype != NC_BF16) return NC_E_UNSUPPORTED;
  const bool mx = st == nullptr;
  nc_status s = check_tensors(t, count, false, true, mx);
  if (s != NC_OK) return s;
  if (count > 0 && y == nullptr) return NC_E_ARG;
  for (int32_t i = 0; i < count; ++i) {
    if (t[i].n == 0) continue;
    if (y[i] == nullptr) return NC_E_ARG;
    if (!aligned16(y[i])) return NC_E_ALIGN;
  }
  if (mx && count > 0 && t[0].mx_axis == NC_MX_COLS)
    return for_batches(t, count, kDequantColSlots, y, [&](const SegBatch& b) {
      return hip_status(launch_dequant_col(b, fmt, Launch{b.tile0[b.count], (hipStream_t)stream}));
    }, kDequantColUnit);
  return for_batches(t, count, kDequantTile, y, [&](const SegBatch& b) {
    return hip_status(launch_dequant(b, fmt, st, Launch{b.tile0[b.count], (hipStream_t)stream}));
  });
}

nc_status nc_cast_stats(const nc_tensor* t, int32_t count, nc_dtype dtype, nc_fmt fmt,
                        const nc_scale_state* st, const nc_loss_scale* ls, nc_stats* out,
                        void* ws, size_t ws_bytes, void* stream) {
  if (!valid_dtype(dtype) || !valid_fmt(fmt)) return NC_E_UNSUPPORTED;
  const bool mx = st == nullptr;
  nc_status s = check_tensors(t, count, true, true, mx);
  if (s != NC_OK) return s;
  if (count == 0) return NC_OK;
  if (out == nullptr) return NC_E_ARG;
  if ((s = check_ws(t, count, ws, ws_bytes)) != NC_OK) return s;
  if (mx && t[0].mx_axis == NC_MX_COLS)
    return for_batches(t, count, kThreads, nullptr, [&](const SegBatch& b) {
      const Tail tl = tail_of(ws_of(b, ws), b.tile0[b.count], nullptr, out, nullptr, false);
      nc_status r = hip_status(launch_stats_col(b, dtype, fmt, tl, Launch{b.tile0[b.count], (hipStream_t)stream}));
      if (r == NC_OK && !tl.direct) r = hip_status(launch_reduce(b, tl, (hipStream_t)stream));
      return r;
    }, stats_col_unit(in_bytes(dtype)));
  const int64_t tile = tile_elems(in_bytes(dtype), kStatsVecs);
  return for_batches(t, count, tile, nullptr, [&](const SegBatch& b) {
    const Tail tl = tail_of(ws_of(b, ws), b.tile0[b.count], nullptr, out, mx ? nullptr : ls, false);
    nc_status r = hip_status(launch_stats(b, dtype, fmt, st, ls, tl, Launch{b.tile0[b.count], (hipStream_t)stream}));
    if (r == NC_OK && !tl.direct) r = hip_status(launch_reduce(b, tl, (hipStream_t)stream));
    return r;
  });
}

nc_status nc_swamp_watch(const nc_update_tensor* t, int32_t count, nc_wfmt wfmt, nc_swamp_counts* out,
                         void* ws, size_t ws_bytes, void* stream) {
  if (wfmt != NC_W_BF16 && wfmt != NC_W_FP16) return NC_E_UNSUPPORTED;
  if (count < 0 || (count > 0 && t == nullptr)) return NC_E_ARG;
  for (int32_t i = 0; i < count; ++i) {
    const nc_update_tensor& x = t[i];
    if (x.n < 0) return NC_E_ARG;
    if (x.n == 0) continue;
    if (x.w == nullptr || x.d == nullptr) return NC_E_ARG;
    if (!aligned16(x.w) || !aligned16(x.d) || ((uintptr_t)x.flags & 3u) != 0) return NC_E_ALIGN;
  }
  if (count == 0) return NC_OK;
  if (out == nullptr) return NC_E_ARG;
  if (ws == nullptr || ((uintptr_t)ws & 15u) != 0 || ws_bytes < nc_swamp_workspace_bytes(t, count))
    return NC_E_WORKSPACE;
  return for_batches(t, count, kSwampTile, nullptr, [&](const SegBatch& b) {
    const Ws w = ws_of(b, ws);
    nc_status r = hip_status(launch_swamp(b, wfmt, w, Launch{b.tile0[b.count], (hipStream_t)stream}));
    if (r == NC_OK) r = hip_status(launch_swamp_reduce(b, w, out, (hipStream_t)stream));
    return r;
  });
}

nc_status nc_swamp_window(const nc_swamp_policy* p, int32_t count, nc_swamp_state* st,
                          const nc_swamp_counts* in, void* stream) {
  if (p == nullptr || count < 0) return NC_E_ARG;
  if (p->window < 1 || p->den < 1 || p->den > 65536 || p->num > p->den) return NC_E_ARG;
  if (count == 0) return NC_OK;
  if (st == nullptr || in == nullptr) return NC_E_ARG;
  return hip_status(launch_swamp_window(*p, count, st, in, (hipStream_t)stream));
}

}  // extern "C"
