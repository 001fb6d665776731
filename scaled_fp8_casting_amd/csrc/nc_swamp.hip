// The update/step-ratio ("swamping") monitor: a read-only pass over fp32
// master weights w and their updates d that classifies each update against
// the step of w's narrow copy ([E3, "Worked solution"]: watch the ratio of
// the update to the step at the weight; [SP, "Master weights and the
// optimizer step"]: a small enough update is exactly a no-op in 16 bits),
// and the per-tensor promotion window.
//
// One workgroup per tile of 8192 elements (32 per lane, eight 16-byte loads
// of w and eight of d; measured best on MI355X); the four per-lane counts go
// to a workspace slot and two small kernels reduce the slots per tensor in a
// fixed order.
#include "nc_launch.h"

namespace nc {
namespace {

// Narrow weight formats: significand bits, exponent bias, field masks.
template <int WF> struct WFmt;
template <> struct WFmt<NC_W_BF16> {
  static constexpr int MB = 7, BIAS = 127;
  static constexpr uint32_t MMASK = 0x7F, MAG = 0x7FFF, INF = 0x7F80;
  // RNE of an fp32 pattern to bf16 (IEEE overflow to Inf)
  __device__ static uint32_t round(uint32_t b) { return f32_to_bf16_rne(b) & 0xFFFFu; }
};
template <> struct WFmt<NC_W_FP16> {
  static constexpr int MB = 10, BIAS = 15;
  static constexpr uint32_t MMASK = 0x3FF, MAG = 0x7FFF, INF = 0x7C00;
  // the hardware conversion rounds to nearest even, keeps subnormals and
  // overflows to Inf
  __device__ static uint32_t round(uint32_t b) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)__uint_as_float(b));
  }
};

// 1 if a < b, for a, b < 2^31 (the sign of a - b).
__device__ __forceinline__ uint32_t lt31(uint32_t a, uint32_t b) { return (a - b) >> 31; }

// Flags of one element (bit 0 below, 1 no-op, 2 zero update, 3 excluded).
// The narrow copy w_F keeps w's sign.  The add w_F + d leaves w_F iff |d| is
// below half the gap to the neighbour on d's side, or exactly half with
// w_F's last significand bit even (ties to even).  That gap is the step,
// except toward zero from a power of two above the smallest normal, where
// the binade below has half the spacing.  Every decision compares |d| with
// a power of two, 2^j for j >= -135 (exact fp32 values, subnormal ones
// included, formed by v_ldexp_f32; the compare of two finite fp32 values is
// exact) -- never through a rounded sum.
template <int WF>
__device__ __forceinline__ uint32_t swamp_flags(uint32_t wb, uint32_t db) {
  using F = WFmt<WF>;
  const uint32_t ad = db & kAbsMask;
  const float fd = __uint_as_float(ad);
  const uint32_t h = F::round(wb);
  const uint32_t hm = h & F::MAG, mf = h & F::MMASK, ef = hm >> F::MB;
  const uint32_t excl = lt31(kMaxFinite, max(wb & kAbsMask, ad)) | lt31(F::INF - 1u, hm);
  const int se = max((int)ef, 1) - (F::BIAS + F::MB);          // log2 of the step
  const uint32_t halved = ((wb ^ db) >> 31) & lt31(0u, hm) & lt31(mf, 1u) & lt31(1u, ef);
  const float half = __builtin_amdgcn_ldexpf(1.0f, se - 1 - (int)halved);
  const uint32_t zero = lt31(ad, 1u);
  const uint32_t below = fd < __builtin_amdgcn_ldexpf(1.0f, se) ? 1u : 0u;
  const uint32_t noop = (fd < half || (fd == half && (mf & 1u) == 0u)) ? 1u : 0u;
  const uint32_t ok = excl ^ 1u, cons = ok & (zero ^ 1u);
  return (below & cons) | (noop & cons) << 1 | (zero & ok) << 2 | excl << 3;
}

struct SwampAcc {
  uint32_t zero, below, noop, excl;
  // four flag bytes of a packed word at once: popcount of each bit plane
  __device__ void add4(uint32_t f4) {
    below += __popc(f4 & 0x01010101u);
    noop += __popc(f4 & 0x02020202u);
    zero += __popc(f4 & 0x04040404u);
    excl += __popc(f4 & 0x08080808u);
  }
};

// The workgroup's four sums -> its slot (as write_count_slot, all sums).
__device__ inline void write_swamp_slot(const SwampAcc& a, uint4* slot, uint32_t* lds) {
  const uint32_t z = row_sum_u32(a.zero), b = row_sum_u32(a.below), n = row_sum_u32(a.noop),
                 x = row_sum_u32(a.excl);
  if ((threadIdx.x & 15) == 0) {
    const int r = threadIdx.x >> 4;
    lds[r * 4 + 0] = z;
    lds[r * 4 + 1] = b;
    lds[r * 4 + 2] = n;
    lds[r * 4 + 3] = x;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint4 c = {0u, 0u, 0u, 0u};
    for (int r = 0; r < kRows; ++r) {
      c.x += lds[r * 4 + 0];
      c.y += lds[r * 4 + 1];
      c.z += lds[r * 4 + 2];
      c.w += lds[r * 4 + 3];
    }
    *slot = c;
  }
}

template <int WF>
NC_STREAM_KERNEL
k_swamp(const SegBatch b, uint4* __restrict__ slots) {
  constexpr int U = kSwampVecs;
  constexpr int64_t TILE = kSwampTile;
  __shared__ uint32_t lds[kRows * 4];
  const int64_t tile = blockIdx.x;
  const int s = seg_of(b.tile0, b.count, tile);
  const Seg& g = b.s[s];
  const int64_t e0 = (tile - b.tile0[s]) * TILE;
  const int rem = tile_len<TILE>(b, s, tile);
  const u32x4* wv = reinterpret_cast<const u32x4*>(static_cast<const float*>(g.x) + e0);
  const u32x4* dv = reinterpret_cast<const u32x4*>(static_cast<const float*>(g.y) + e0);
  uint8_t* fl = g.codes ? g.codes + e0 : nullptr;
  SwampAcc acc{0u, 0u, 0u, 0u};
  if (rem == (int)TILE) {
    u32x4 w[U], d[U];
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = ld_stream(wv + u * kThreads + threadIdx.x);
#pragma unroll
    for (int u = 0; u < U; ++u) d[u] = ld_stream(dv + u * kThreads + threadIdx.x);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t f = swamp_flags<WF>(w[u].x, d[u].x) | swamp_flags<WF>(w[u].y, d[u].y) << 8 |
                         swamp_flags<WF>(w[u].z, d[u].z) << 16 | swamp_flags<WF>(w[u].w, d[u].w) << 24;
      acc.add4(f);
      if (fl) st_stream(reinterpret_cast<uint32_t*>(fl) + u * kThreads + threadIdx.x, f);
    }
  } else {
    const uint32_t* ws = static_cast<const uint32_t*>(g.x) + e0;
    const uint32_t* ds = static_cast<const uint32_t*>(g.y) + e0;
    for (int i = threadIdx.x; i < rem; i += kThreads) {
      const uint32_t f = swamp_flags<WF>(ws[i], ds[i]);
      acc.add4(f);
      if (fl) fl[i] = (uint8_t)f;
    }
  }
  write_swamp_slot(acc, slots + tile, lds);
}

// Slot reductions: chunks of kChunk tiles, then per tensor (fixed order).
__global__ void __launch_bounds__(kThreads)
k_swamp_reduce1(const SegBatch b, const uint4* __restrict__ s1, uint64_t* __restrict__ s2) {
  __shared__ uint64_t lds[kWaves * 4];
  const int64_t c = blockIdx.x;
  const int s = seg_of(b.chunk0, b.count, c);
  const int64_t t0 = b.tile0[s] + (c - b.chunk0[s]) * kChunk;
  const int64_t t1 = min(t0 + (int64_t)kChunk, b.tile0[s + 1]);
  uint64_t v[4] = {0, 0, 0, 0};
  for (int64_t t = t0 + threadIdx.x; t < t1; t += kThreads) {
    const uint4 x = s1[t];
    v[0] += x.x;
    v[1] += x.y;
    v[2] += x.z;
    v[3] += x.w;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint64_t r = wave_sum_u64(v[j]);
    if (lane == 0) lds[wave * 4 + j] = r;
  }
  __syncthreads();
  if (threadIdx.x < 4) {
    uint64_t r = 0;
    for (int w = 0; w < kWaves; ++w) r += lds[w * 4 + threadIdx.x];
    s2[c * 4 + threadIdx.x] = r;
  }
}

__global__ void __launch_bounds__(64)
k_swamp_reduce2(const SegBatch b, const uint64_t* __restrict__ s2, nc_swamp_counts* __restrict__ out) {
  const int s = blockIdx.x;
  uint64_t v[4] = {0, 0, 0, 0};
  for (int64_t c = b.chunk0[s] + threadIdx.x; c < b.chunk0[s + 1]; c += 64) {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] += s2[c * 4 + j];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = wave_sum_u64(v[j]);
  if (threadIdx.x == 0) {
    nc_swamp_counts* o = out + b.first + s;
    const uint64_t cons = (uint64_t)b.s[s].n - v[0] - v[3];
    if (cons) atomicAdd((unsigned long long*)&o->n_considered, (unsigned long long)cons);
    if (v[0]) atomicAdd((unsigned long long*)&o->n_zero, (unsigned long long)v[0]);
    if (v[1]) atomicAdd((unsigned long long*)&o->n_below, (unsigned long long)v[1]);
    if (v[2]) atomicAdd((unsigned long long*)&o->n_noop, (unsigned long long)v[2]);
    if (v[3]) atomicAdd((unsigned long long*)&o->n_excluded, (unsigned long long)v[3]);
  }
}

// The promotion window, one thread per tensor.
__global__ void __launch_bounds__(kThreads)
k_swamp_window(const nc_swamp_policy p, int32_t count, nc_swamp_state* __restrict__ st,
               const nc_swamp_counts* __restrict__ in) {
  const int32_t j = blockIdx.x * kThreads + threadIdx.x;
  if (j >= count) return;
  const nc_swamp_counts c = in[j];
  nc_swamp_state s = st[j];
  // n_below <= n_considered < 2^34 and num, den <= 2^16: both products < 2^50
  const bool below = c.n_considered > 0 && c.n_below * (uint64_t)p.den >= (uint64_t)p.num * c.n_considered;
  s.run = below ? s.run + 1 : 0;
  s.promoted = (s.promoted || s.run >= p.window) ? 1 : 0;
  s.steps += 1;
  st[j] = s;
}

}  // namespace

hipError_t launch_swamp(const SegBatch& b, int wfmt, const Ws& w, const Launch& l) {
  uint4* slots = reinterpret_cast<uint4*>(w.cnt1);
  if (wfmt == NC_W_BF16)
    hipLaunchKernelGGL((k_swamp<NC_W_BF16>), dim3((uint32_t)l.grid), dim3(kThreads), 0, l.stream, b, slots);
  else
    hipLaunchKernelGGL((k_swamp<NC_W_FP16>), dim3((uint32_t)l.grid), dim3(kThreads), 0, l.stream, b, slots);
  return hipGetLastError();
}

hipError_t launch_swamp_reduce(const SegBatch& b, const Ws& w, nc_swamp_counts* out, hipStream_t stream) {
  hipLaunchKernelGGL(k_swamp_reduce1, dim3((uint32_t)b.chunk0[b.count]), dim3(kThreads), 0, stream, b,
                     reinterpret_cast<const uint4*>(w.cnt1), w.cnt2);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_swamp_reduce2, dim3((uint32_t)b.count), dim3(64), 0, stream, b, w.cnt2, out);
  return hipGetLastError();
}

hipError_t launch_swamp_window(const nc_swamp_policy& p, int32_t count, nc_swamp_state* st,
                               const nc_swamp_counts* in, hipStream_t stream) {
  hipLaunchKernelGGL(k_swamp_window, dim3((uint32_t)((count + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                     stream, p, count, st, in);
  return hipGetLastError();
}

}  // namespace nc
