// Internal launch interface between the C-ABI layer (nc_api.hip) and the
// kernel files.  Each launcher enqueues one batch of at most kMaxSeg tensors.
#pragma once

#include "nc_device.h"

namespace nc {

// Elements per tile of a kernel that reads `in_bytes`-wide elements with
// `unroll` 16-byte loads per thread (dequant reads codes: 256 * 16 * 2).
inline int64_t tile_elems(int in_bytes, int unroll) { return (int64_t)kThreads * (16 / in_bytes) * unroll; }
constexpr int64_t kDequantTile = (int64_t)kThreads * 16 * 2;

struct Launch {
  int grid;            // workgroups
  hipStream_t stream;
};

hipError_t launch_amax(const SegBatch& b, int dtype, const nc_loss_scale* ls, nc_counts* out,
                       const Launch& l);
hipError_t launch_cast_pt(const SegBatch& b, int dtype, int fmt, const nc_scale_state* st,
                          const nc_loss_scale* ls, nc_counts* out, double* part, const Launch& l);
hipError_t launch_cast_mx(const SegBatch& b, int dtype, int fmt, int rule, nc_counts* out,
                          double* part, const Launch& l);
hipError_t launch_stats(const SegBatch& b, int dtype, int fmt, const nc_scale_state* st,
                        const nc_loss_scale* ls, double* part, const Launch& l);
hipError_t launch_stats_finalize(const SegBatch& b, const double* part, int grid, nc_stats* out,
                                 hipStream_t stream);
hipError_t launch_dequant(const SegBatch& b, int fmt, const nc_scale_state* st, const Launch& l);
hipError_t launch_scale_update(const nc_policy& p, int32_t count, nc_scale_state* st, float* hist,
                               const nc_counts* in, nc_loss_scale* ls, hipStream_t stream);

}  // namespace nc
