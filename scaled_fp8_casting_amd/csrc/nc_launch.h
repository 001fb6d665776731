// Internal launch interface between the C-ABI layer (nc_api.hip) and the
// kernel files.  Each launcher enqueues one batch of at most kMaxSeg tensors.
#pragma once

#include "nc_device.h"

namespace nc {

// Elements per workgroup tile: 256 lanes x a few 16-byte input vectors --
// two for the casts, eight when they also form statistics (and for the
// statistics pass), four for the amax pass (read only: tile size does not
// matter for bandwidth there, and larger tiles spread the per-workgroup
// reductions over more elements); dequant: 256 lanes x two vectors of 8
// codes (a 16-byte bf16 store each).  Measured best on MI355X.
constexpr int kCastVecs = 2;
constexpr int kCastStatsVecs = 8;   // casts with fused statistics (more work per element)
constexpr int kCastSrVecs = 8;      // the stochastic-rounding cast (ALU-bound: larger tiles)
constexpr int kStatsVecs = 8;       // the statistics pass (read only)
constexpr int kAmaxVecs = 4;
template <bool STATS> constexpr int cast_vecs() { return STATS ? kCastStatsVecs : kCastVecs; }
constexpr int kDequantVecs = 2;
constexpr int64_t kDequantTile = (int64_t)kThreads * 8 * kDequantVecs;
inline int64_t tile_elems(int in_bytes, int vecs) { return (int64_t)kThreads * (16 / in_bytes) * vecs; }
// smallest tile of any call that uses the workspace (fp32 cast / statistics)
constexpr int64_t kMinWsTile = (int64_t)kThreads * 4 * kCastVecs;

// Column-block MX (col_slot): a lane reads 8 input bytes per row (4 bf16 or
// 2 fp32 columns), or 8 codes per row in dequant, or 16 input bytes per row
// in the statistics pass.  Rows per slot, measured best on MI355X: the cast
// needs whole 32-row bands; the statistics pass is fastest with them too.  Dequant takes whole bands as well, but each lane
// only kDequantColRows of a band's rows: the four waves of a workgroup hold
// the four 8-row parts of the same 64 slots (a tile of 16 KiB of codes), so
// a band's scale bytes are fetched once and hit in cache for the other
// waves.  A cast or statistics tile is at least kMinWsTile elements, so the
// workspace bound above covers those calls too.
constexpr int kColBytes = 8;
constexpr int kDequantColCodes = 8;
constexpr int kDequantColRows = 8;                                   // rows per lane
constexpr int kDequantColSlots = kThreads / (32 / kDequantColRows);  // slots per tile
constexpr int kStatsColRows = 32;
// Lanes per slot in the column cast: two for bf16 (16 rows each, half the
// registers of a whole band), one for fp32 (measured faster whole).
constexpr int col_cast_split(int dtype) { return dtype == NC_BF16 ? 2 : 1; }
inline int64_t col_unit(int in_bytes, int rows = 32) { return rows * (kColBytes / in_bytes); }
// The column statistics pass reads 16 input bytes per row (8 bf16 or 4 fp32
// columns per slot).
inline int64_t stats_col_unit(int in_bytes) { return 32 * (16 / in_bytes); }
constexpr int64_t kDequantColUnit = 32 * kDequantColCodes;          // codes per slot
static_assert(kThreads * kStatsColRows * 2 >= kMinWsTile, "column tiles are no smaller than kMinWsTile");
static_assert(kThreads / col_cast_split(NC_BF16) * 32 * 2 >= kMinWsTile, "column tiles are no smaller than kMinWsTile");

// The update/step-ratio monitor: 256 lanes x eight 16-byte vectors of w (and
// of d) per tile -- read-only, like the amax pass.
constexpr int kSwampVecs = 8;
constexpr int64_t kSwampTile = (int64_t)kThreads * 4 * kSwampVecs;

// Workspace of one launch: per-tile slots, then per-chunk statistics slots
// (counts go from the chunk sums straight into the caller's counts).
struct Ws {
  CountSlot* cnt1;      // [tiles]
  double* st1;          // [tiles][6]    (statistics only)
  double* st2;          // [chunks][6]   (statistics only)
};

// Byte size of the workspace a launch with `tiles` tiles and `chunks`
// chunks needs (statistics included), and its layout inside `base`.
inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
inline size_t ws_bytes_for(int64_t tiles, int64_t chunks) {
  return align256((size_t)tiles * sizeof(CountSlot)) + align256((size_t)tiles * 48) +
         align256((size_t)chunks * 48);
}
inline Ws ws_layout(void* base, int64_t tiles, int64_t chunks) {
  uint8_t* p = static_cast<uint8_t*>(base);
  Ws w;
  w.cnt1 = reinterpret_cast<CountSlot*>(p);
  p += align256((size_t)tiles * sizeof(CountSlot));
  w.st1 = reinterpret_cast<double*>(p);
  p += align256((size_t)tiles * 48);
  w.st2 = reinterpret_cast<double*>(p);
  return w;
}

// What a reducing kernel does with its workgroups' partial results, and
// where the totals go (a kernel argument).  Normally each workgroup writes a
// slot and the separate reduction kernels follow the launch.  direct: a
// launch of at most kDirectMaxTiles workgroups that forms counts only has
// each workgroup add its counts straight into the caller's (integer sums and
// a max: the order does not matter), so no slot and no second launch.
// Statistics (binary64 sums in a fixed order) always go through the slots.
struct Tail {
  CountSlot* cnt1;          // per-workgroup counts
  double* st1;              // per-workgroup statistics
  double* st2;              // per-chunk statistics of tensors of several chunks
  nc_counts* out;           // the caller's counts (null: none)
  nc_stats* stats;          // the caller's statistics (null: none)
  const nc_loss_scale* ls;  // unscale of the amax and of the statistics (nullable)
  int32_t clips;            // the counts report clips (the amax pass reports none)
  int32_t direct;
};

// The largest launch whose workgroups add their counts directly.  Measured
// on MI355X: same-address atomics serialise, so the direct form pays only
// while few workgroups share the caller's counts (a 65,536-element fp32
// cast: 32 workgroups).
constexpr int64_t kDirectMaxTiles = 64;

inline Tail tail_of(const Ws& w, int64_t tiles, nc_counts* out, nc_stats* stats, const nc_loss_scale* ls,
                    bool clips) {
  return Tail{w.cnt1, w.st1, w.st2, out, stats, ls, clips ? 1 : 0,
              (stats == nullptr && out != nullptr && tiles <= kDirectMaxTiles) ? 1 : 0};
}

struct Launch {
  int64_t grid;        // workgroups (one per tile)
  hipStream_t stream;
};

hipError_t launch_amax(const SegBatch& b, int dtype, const Tail& t, const Launch& l);
hipError_t launch_cast_pt(const SegBatch& b, int dtype, int fmt, const nc_scale_state* st,
                          const nc_loss_scale* ls, bool stats, const Tail& t, const Launch& l);
hipError_t launch_cast_mx(const SegBatch& b, int dtype, int fmt, int rule, bool stats, const Tail& t,
                          const Launch& l);
hipError_t launch_cast_sr(const SegBatch& b, int dtype, int fmt, const nc_scale_state* st,
                          const nc_loss_scale* ls, uint64_t seed, uint64_t offset, const Tail& t, const Launch& l);
hipError_t launch_stats(const SegBatch& b, int dtype, int fmt, const nc_scale_state* st,
                        const nc_loss_scale* ls, const Tail& t, const Launch& l);
// Column-block MX forms of the MX cast, dequant and statistics pass; the
// batch's tiles are 256 col_slots.
hipError_t launch_cast_mx_col(const SegBatch& b, int dtype, int fmt, int rule, bool stats, const Tail& t,
                              const Launch& l);
hipError_t launch_dequant_col(const SegBatch& b, int fmt, const Launch& l);
hipError_t launch_stats_col(const SegBatch& b, int dtype, int fmt, const Tail& t, const Launch& l);
// The separate reductions of a launch's slots into t.out (nullable) and
// t.stats (nullable), for launches that do not reduce in-kernel.
hipError_t launch_reduce(const SegBatch& b, const Tail& t, hipStream_t stream);
hipError_t launch_dequant(const SegBatch& b, int fmt, const nc_scale_state* st, const Launch& l);
// The monitor's main kernel, its slot reduction into out, and the
// promotion window.
hipError_t launch_swamp(const SegBatch& b, int wfmt, const Ws& w, const Launch& l);
hipError_t launch_swamp_reduce(const SegBatch& b, const Ws& w, nc_swamp_counts* out, hipStream_t stream);
hipError_t launch_swamp_window(const nc_swamp_policy& p, int32_t count, nc_swamp_state* st,
                               const nc_swamp_counts* in, hipStream_t stream);
hipError_t launch_scale_update(const nc_policy& p, int32_t count, nc_scale_state* st, float* hist,
                               const nc_counts* in, nc_loss_scale* ls, hipStream_t stream);

}  // namespace nc
