// The C-ABI of libnarrowcast: argument checks, batching into launches of at
// most kMaxSeg tensors, grid sizing.  No allocation, no global state.
#include <string.h>

#include "nc_launch.h"

using namespace nc;

namespace {

// Workgroups per CU for the streaming kernels: 16 x 256 threads of grid
// (resident as registers allow), enough 16-byte loads in flight to cover
// HBM latency; measured best for read+write streams on MI355X.
constexpr int kWGPerCU = 16;

int grid_for(int64_t tiles) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      cus = v;
  }
  int64_t cap = (int64_t)cus * kWGPerCU;
  if (cap > kMaxGrid) cap = kMaxGrid;
  return (int)(tiles < cap ? tiles : cap);
}

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
    if (mx && (x.cols <= 0 || x.cols % 32 != 0 || x.n % x.cols != 0)) return NC_E_SHAPE;
    if (x.n == 0) continue;
    if ((need_x && x.x == nullptr) || (need_codes && x.codes == nullptr)) return NC_E_ARG;
    if (mx && x.scales == nullptr) return NC_E_ARG;
    if ((need_x && !aligned16(x.x)) || (need_codes && !aligned16(x.codes))) return NC_E_ALIGN;
  }
  return NC_OK;
}

// Walk the batch in launches of at most kMaxSeg tensors; `fn(batch)` enqueues
// one launch.  Empty tensors are skipped.
template <typename Fn>
nc_status for_batches(const nc_tensor* t, int32_t count, int64_t tile, void* const* y, Fn fn) {
  SegBatch b;
  memset(&b, 0, sizeof(b));
  int32_t i = 0;
  while (i < count) {
    b.count = 0;
    b.first = i;
    b.tile0[0] = 0;
    // a launch covers consecutive tensors so that b.first + s indexes the
    // caller's arrays; empty tensors inside keep a zero-tile slot
    while (i < count && b.count < kMaxSeg) {
      const nc_tensor& x = t[i];
      Seg& s = b.s[b.count];
      s.x = x.x;
      s.codes = x.codes;
      s.scales = x.scales;
      s.y = y ? y[i] : nullptr;
      s.n = x.n;
      const int64_t tiles = (x.n + tile - 1) / tile;
      b.tile0[b.count + 1] = b.tile0[b.count] + tiles;
      b.last[b.count] = tiles ? (int32_t)(x.n - (tiles - 1) * tile) : 0;
      ++b.count;
      ++i;
    }
    for (int s = b.count + 1; s <= kMaxSeg; ++s) b.tile0[s] = b.tile0[b.count];
    if (b.tile0[b.count] == 0) continue;
    const nc_status st = fn(b);
    if (st != NC_OK) return st;
  }
  return NC_OK;
}

nc_status hip_status(hipError_t e) { return e == hipSuccess ? NC_OK : NC_E_HIP; }

bool valid_dtype(nc_dtype d) { return d == NC_F32 || d == NC_BF16; }
bool valid_fmt(nc_fmt f) { return f == NC_E4M3 || f == NC_E5M2; }

nc_status check_ws(const nc_tensor* t, int32_t count, void* ws, size_t ws_bytes) {
  if (ws == nullptr || ((uintptr_t)ws & 7u) != 0) return NC_E_WORKSPACE;
  if (ws_bytes < nc_workspace_bytes(t, count)) return NC_E_WORKSPACE;
  return NC_OK;
}

}  // namespace

extern "C" {

size_t nc_workspace_bytes(const nc_tensor* t, int32_t count) {
  // one slot of 6 binary64 per (tensor of a launch, workgroup)
  if (t == nullptr || count <= 0) return 0;
  const int32_t per_launch = count < kMaxSeg ? count : kMaxSeg;
  return (size_t)per_launch * kMaxGrid * 6 * sizeof(double);
}

const char* nc_status_string(nc_status s) {
  switch (s) {
    case NC_OK: return "ok";
    case NC_E_ARG: return "invalid argument (null pointer, negative size or bad policy field)";
    case NC_E_ALIGN: return "element pointer not 16-byte aligned";
    case NC_E_SHAPE: return "MX shape: cols must be a positive multiple of 32 dividing n";
    case NC_E_UNSUPPORTED: return "unsupported dtype, format, rule or estimator";
    case NC_E_HIP: return "HIP launch failed";
    case NC_E_WORKSPACE: return "workspace missing, misaligned or smaller than nc_workspace_bytes()";
  }
  return "unknown status";
}

nc_status nc_amax(const nc_tensor* t, int32_t count, nc_dtype dtype, const nc_loss_scale* ls,
                  nc_counts* out, void* stream) {
  if (!valid_dtype(dtype)) return NC_E_UNSUPPORTED;
  nc_status s = check_tensors(t, count, true, false, false);
  if (s != NC_OK) return s;
  if (count > 0 && out == nullptr) return NC_E_ARG;
  const int64_t tile = tile_elems(in_bytes(dtype), kUnrollRead);
  return for_batches(t, count, tile, nullptr, [&](const SegBatch& b) {
    Launch l{grid_for(b.tile0[b.count]), (hipStream_t)stream};
    return hip_status(launch_amax(b, dtype, ls, out, l));
  });
}

nc_status nc_scale_update(const nc_policy* p, int32_t count, nc_scale_state* st, float* hist,
                          const nc_counts* in, nc_loss_scale* ls, void* stream) {
  if (p == nullptr || count < 0) return NC_E_ARG;
  if (!valid_fmt((nc_fmt)p->fmt)) return NC_E_UNSUPPORTED;
  if (p->est != NC_EST_CURRENT && p->est != NC_EST_MOST_RECENT && p->est != NC_EST_MAX_WINDOW)
    return NC_E_UNSUPPORTED;
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
  if (count > 0 && (out == nullptr || st == nullptr)) return NC_E_ARG;
  if (stats && (s = check_ws(t, count, ws, ws_bytes)) != NC_OK) return s;
  const int64_t tile = tile_elems(in_bytes(dtype), kUnrollCast);
  double* part = stats ? static_cast<double*>(ws) : nullptr;
  return for_batches(t, count, tile, nullptr, [&](const SegBatch& b) {
    Launch l{grid_for(b.tile0[b.count]), (hipStream_t)stream};
    nc_status r = hip_status(launch_cast_pt(b, dtype, fmt, st, ls, out, part, l));
    if (r == NC_OK && stats) r = hip_status(launch_stats_finalize(b, part, l.grid, stats, l.stream));
    return r;
  });
}

nc_status nc_cast_mx(const nc_tensor* t, int32_t count, nc_dtype dtype, nc_fmt fmt, nc_mx_rule rule,
                     nc_counts* out, nc_stats* stats, void* ws, size_t ws_bytes, void* stream) {
  if (!valid_dtype(dtype) || !valid_fmt(fmt)) return NC_E_UNSUPPORTED;
  if (rule != NC_MX_OCP && rule != NC_MX_PLUS1 && rule != NC_MX_CEIL) return NC_E_UNSUPPORTED;
  nc_status s = check_tensors(t, count, true, true, true);
  if (s != NC_OK) return s;
  if (count > 0 && out == nullptr) return NC_E_ARG;
  if (stats && (s = check_ws(t, count, ws, ws_bytes)) != NC_OK) return s;
  const int64_t tile = tile_elems(in_bytes(dtype), kUnrollCast);
  double* part = stats ? static_cast<double*>(ws) : nullptr;
  return for_batches(t, count, tile, nullptr, [&](const SegBatch& b) {
    Launch l{grid_for(b.tile0[b.count]), (hipStream_t)stream};
    nc_status r = hip_status(launch_cast_mx(b, dtype, fmt, rule, out, part, l));
    if (r == NC_OK && stats) r = hip_status(launch_stats_finalize(b, part, l.grid, stats, l.stream));
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
  return for_batches(t, count, kDequantTile, y, [&](const SegBatch& b) {
    Launch l{grid_for(b.tile0[b.count]), (hipStream_t)stream};
    return hip_status(launch_dequant(b, fmt, st, l));
  });
}

nc_status nc_cast_stats(const nc_tensor* t, int32_t count, nc_dtype dtype, nc_fmt fmt,
                        const nc_scale_state* st, const nc_loss_scale* ls, nc_stats* out,
                        void* ws, size_t ws_bytes, void* stream) {
  if (!valid_dtype(dtype) || !valid_fmt(fmt)) return NC_E_UNSUPPORTED;
  const bool mx = st == nullptr;
  nc_status s = check_tensors(t, count, true, true, mx);
  if (s != NC_OK) return s;
  if (count > 0 && out == nullptr) return NC_E_ARG;
  if (count > 0 && (s = check_ws(t, count, ws, ws_bytes)) != NC_OK) return s;
  const int64_t tile = tile_elems(in_bytes(dtype), kUnrollRead);
  double* part = static_cast<double*>(ws);
  return for_batches(t, count, tile, nullptr, [&](const SegBatch& b) {
    Launch l{grid_for(b.tile0[b.count]), (hipStream_t)stream};
    nc_status r = hip_status(launch_stats(b, dtype, fmt, st, ls, part, l));
    if (r == NC_OK) r = hip_status(launch_stats_finalize(b, part, l.grid, out, l.stream));
    return r;
  });
}

}  // extern "C"
