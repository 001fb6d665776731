// The update/step-ratio ("swamping") monitor: a read-only pass over fp32
// master weights w and their updates d that classifies each update against
// the step of w's narrow copy ([E3, "Worked solution"]: compare each update
// with the grid spacing where its weight sits; [SP, "Master weights and the
// optimizer step"]: a small enough update is exactly a no-op in 16 bits),
// and the per-tensor promotion window.
//
// One workgroup per tile of 8192 elements (32 per lane, eight 16-byte loads
// of w and eight of d; measured best on MI355X); the four counts (per lane
// where flag bytes are written, per wave otherwise) go to a workspace slot
// and one small kernel adds the slots of each chunk of tiles into the
// caller's counts.
#include "nc_launch.h"

namespace nc {
namespace {

// Narrow weight formats.  narrow(wb) rounds the fp32 pattern wb to the
// format (RNE, IEEE overflow to Inf) and gives the result's exponent field,
// whether its fraction field is zero and whether its last significand bit is
// even.  STEP0 = 2^-(BIAS + MB): the step of a binade with exponent field f
// is STEP0 2^max(f, 1).
template <int WF> struct WFmt;
template <> struct WFmt<NC_W_BF16> {
  static constexpr uint32_t EFULL = 0xFF;    // Inf/NaN exponent field
  static constexpr float STEP0 = 0x1p-134f;
  // the bf16 value sits in the high half of the rounded fp32 pattern
  __device__ static void narrow(uint32_t wb, uint32_t& ef, bool& frac0, uint32_t& even) {
    const uint32_t h = wb + 0x7FFFu + ((wb >> 16) & 1u);
    ef = (h >> 23) & 0xFFu;
    frac0 = (h & 0x007F0000u) == 0u;
    even = (~h >> 16) & 1u;
  }
};
template <> struct WFmt<NC_W_FP16> {
  static constexpr uint32_t EFULL = 0x1F;
  static constexpr float STEP0 = 0x1p-25f;
  // the hardware conversion rounds to nearest even, keeps subnormals and
  // overflows to Inf
  __device__ static void narrow(uint32_t wb, uint32_t& ef, bool& frac0, uint32_t& even) {
    const uint32_t h = __builtin_bit_cast(uint16_t, (_Float16)__uint_as_float(wb));
    ef = (h >> 10) & 0x1Fu;
    frac0 = (h & 0x3FFu) == 0u;
    even = (~h) & 1u;
  }
};

// Classes of one element.  The narrow copy w_F keeps w's sign.  The add
// w_F + d leaves w_F iff |d| is below half the gap to the neighbour on d's
// side, or exactly half with w_F's last significand bit even (ties to even).
// That gap is the step, except toward zero from a power of two above the
// smallest normal, where the binade below has half the spacing.  Every
// decision compares |d| with a power of two, 2^j for j >= -135 (exact fp32
// values, subnormal ones included, formed by v_ldexp_f32), never through a
// rounded sum; the tie test folds into the compare of non-negative patterns
// (|d| <= half iff bits(|d|) < bits(half) + 1).
struct SwampCls {
  bool below, noop, zero, excl;
};
template <int WF>
__device__ __forceinline__ SwampCls swamp_classify(uint32_t wb, uint32_t db) {
  using F = WFmt<WF>;
  const uint32_t ad = db & kAbsMask;
  uint32_t ef, even;
  bool frac0;
  F::narrow(wb, ef, frac0, even);
  const float step = __builtin_amdgcn_ldexpf(F::STEP0, (int)max(ef, 1u));
  const bool halved = (int32_t)(wb ^ db) < 0 && frac0 && ef > 1u;
  const float half = __builtin_amdgcn_ldexpf(step, halved ? -2 : -1);
  SwampCls c;
  c.excl = max(wb & kAbsMask, ad) > kMaxFinite || ef == F::EFULL;
  c.zero = ad == 0u;
  c.below = __uint_as_float(ad) < step;
  c.noop = ad < __float_as_uint(half) + even;
  return c;
}

// Flag byte of one element: bit 0 below, 1 no-op, 2 zero update, 3 excluded.
// below and no-op are counted over considered elements (finite, nonzero d),
// so the byte is 8 for an excluded element, else 4 for a zero update, else
// below | no-op << 1.  Returned in byte `pos` of a word (three selects on the
// compares' own results, no boolean arithmetic).
template <int WF>
__device__ __forceinline__ uint32_t swamp_flags(uint32_t wb, uint32_t db, int pos = 0) {
  const SwampCls c = swamp_classify<WF>(wb, db);
  const int sh = 8 * pos;
  uint32_t f = (c.below ? 1u << sh : 0u) + (c.noop ? 2u << sh : 0u);
  f = c.zero ? 4u << sh : f;
  return c.excl ? 8u << sh : f;
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
  // one element per active lane, counted for the whole wave: each test is
  // taken as the wave's lane mask (a compare's own result), the masks are
  // combined and popcounted on the scalar unit, and the sums are
  // wave-uniform; inactive lanes are in no mask
  template <int WF>
  __device__ void add_wave(uint32_t wb, uint32_t db) {
    const SwampCls c = swamp_classify<WF>(wb, db);
    const uint64_t mx = __ballot(c.excl), mz = __ballot(c.zero), mb = __ballot(c.below), mn = __ballot(c.noop);
    const uint64_t cons = ~(mx | mz);
    below += __popcll(mb & cons);
    noop += __popcll(mn & cons);
    zero += __popcll(mz & ~mx);
    excl += __popcll(mx);
  }
};

// The workgroup's four sums -> its slot (as write_count_slot, all sums).
// WAVE: the sums are per wave (equal in every lane), not per lane.
template <bool WAVE>
__device__ inline void write_swamp_slot(const SwampAcc& a, uint4* slot, uint32_t* lds) {
  constexpr int N = WAVE ? kWaves : kRows;
  uint32_t z = a.zero, b = a.below, n = a.noop, x = a.excl;
  if constexpr (!WAVE) {
    z = row_sum_u32(z);
    b = row_sum_u32(b);
    n = row_sum_u32(n);
    x = row_sum_u32(x);
  }
  if ((threadIdx.x & (WAVE ? 63 : 15)) == 0) {
    const int r = WAVE ? threadIdx.x >> 6 : threadIdx.x >> 4;
    lds[r * 4 + 0] = z;
    lds[r * 4 + 1] = b;
    lds[r * 4 + 2] = n;
    lds[r * 4 + 3] = x;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint4 c = {0u, 0u, 0u, 0u};
    for (int r = 0; r < N; ++r) {
      c.x += lds[r * 4 + 0];
      c.y += lds[r * 4 + 1];
      c.z += lds[r * 4 + 2];
      c.w += lds[r * 4 + 3];
    }
    *slot = c;
  }
}

// FLAGS: some tensor of the launch wants its flag bytes (those with a null
// flag pointer in such a launch are counted per lane too); otherwise only
// the counts are formed, per wave.
template <int WF, bool FLAGS>
NC_STREAM_KERNEL
k_swamp(const SegBatch b, uint4* __restrict__ slots) {
  constexpr int U = kSwampVecs;
  constexpr int64_t TILE = kSwampTile;
  __shared__ uint32_t lds[kRows * 4];
  // tile order (measured): 32 tiles per XCD in turn for the counts, 256 with
  // flag bytes
  const int64_t tile = FLAGS ? xcd_tile<256>() : xcd_tile<32>();
  const int s = seg_of(b.tile0, b.count, tile);
  const Seg& g = b.s[s];
  const int64_t e0 = (tile - b.tile0[s]) * TILE;
  const int rem = tile_len<TILE>(b, s, tile);
  const u32x4* wv = reinterpret_cast<const u32x4*>(static_cast<const float*>(g.x) + e0);
  const u32x4* dv = reinterpret_cast<const u32x4*>(static_cast<const float*>(g.y) + e0);
  uint8_t* fl = FLAGS && g.codes ? g.codes + e0 : nullptr;
  SwampAcc acc{0u, 0u, 0u, 0u};
  if (rem == (int)TILE) {
    u32x4 w[U], d[U];
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = ld_stream(wv + u * kThreads + threadIdx.x);
#pragma unroll
    for (int u = 0; u < U; ++u) d[u] = ld_stream(dv + u * kThreads + threadIdx.x);
    __builtin_amdgcn_sched_barrier(0);
    uint32_t fw[FLAGS ? U : 1];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (FLAGS) {
        fw[u] = swamp_flags<WF>(w[u].x, d[u].x, 0) | swamp_flags<WF>(w[u].y, d[u].y, 1) |
                swamp_flags<WF>(w[u].z, d[u].z, 2) | swamp_flags<WF>(w[u].w, d[u].w, 3);
        acc.add4(fw[u]);
      } else {
        acc.add_wave<WF>(w[u].x, d[u].x);
        acc.add_wave<WF>(w[u].y, d[u].y);
        acc.add_wave<WF>(w[u].z, d[u].z);
        acc.add_wave<WF>(w[u].w, d[u].w);
      }
    }
    // the tile's flag words go out together after its classification (5%
    // faster than a store after each vector, measured)
    if constexpr (FLAGS) {
      if (fl) {
#pragma unroll
        for (int u = 0; u < U; ++u) st_stream(reinterpret_cast<uint32_t*>(fl) + u * kThreads + threadIdx.x, fw[u]);
      }
    }
  } else {
    const uint32_t* ws = static_cast<const uint32_t*>(g.x) + e0;
    const uint32_t* ds = static_cast<const uint32_t*>(g.y) + e0;
    for (int i = threadIdx.x; i < rem; i += kThreads) {
      if constexpr (FLAGS) {
        const uint32_t f = swamp_flags<WF>(ws[i], ds[i]);
        acc.add4(f);
        if (fl) fl[i] = (uint8_t)f;
      } else {
        acc.add_wave<WF>(ws[i], ds[i]);    // inactive lanes are not in the masks
      }
    }
  }
  write_swamp_slot<!FLAGS>(acc, slots + tile, lds);
}

// Slot reduction: workgroup c sums chunk c (at most kChunk tiles of one
// tensor) and adds it into the caller's counts with atomics (integer sums:
// the order does not matter).  n_considered = n - zero - excluded: the
// tensor's first chunk adds n, every chunk takes off its own zero and
// excluded counts, modulo 2^64.
__global__ void __launch_bounds__(kThreads)
k_swamp_reduce(const SegBatch b, const uint4* __restrict__ s1, nc_swamp_counts* __restrict__ out) {
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
  if (threadIdx.x == 0) {
    uint64_t r[4] = {0, 0, 0, 0};
    for (int w = 0; w < kWaves; ++w)
      for (int j = 0; j < 4; ++j) r[j] += lds[w * 4 + j];
    nc_swamp_counts* o = out + b.first + s;
    const uint64_t cons = (c == b.chunk0[s] ? (uint64_t)b.s[s].n : 0u) - r[0] - r[3];   // modulo 2^64
    if (cons) atomicAdd((unsigned long long*)&o->n_considered, (unsigned long long)cons);
    if (r[0]) atomicAdd((unsigned long long*)&o->n_zero, (unsigned long long)r[0]);
    if (r[1]) atomicAdd((unsigned long long*)&o->n_below, (unsigned long long)r[1]);
    if (r[2]) atomicAdd((unsigned long long*)&o->n_noop, (unsigned long long)r[2]);
    if (r[3]) atomicAdd((unsigned long long*)&o->n_excluded, (unsigned long long)r[3]);
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
  bool flags = false;
  for (int j = 0; j < b.count; ++j) flags = flags || b.s[j].codes != nullptr;
  const dim3 grid((uint32_t)l.grid), block(kThreads);
  if (wfmt == NC_W_BF16) {
    if (flags) hipLaunchKernelGGL((k_swamp<NC_W_BF16, true>), grid, block, 0, l.stream, b, slots);
    else hipLaunchKernelGGL((k_swamp<NC_W_BF16, false>), grid, block, 0, l.stream, b, slots);
  } else {
    if (flags) hipLaunchKernelGGL((k_swamp<NC_W_FP16, true>), grid, block, 0, l.stream, b, slots);
    else hipLaunchKernelGGL((k_swamp<NC_W_FP16, false>), grid, block, 0, l.stream, b, slots);
  }
  return hipGetLastError();
}

hipError_t launch_swamp_reduce(const SegBatch& b, const Ws& w, nc_swamp_counts* out, hipStream_t stream) {
  hipLaunchKernelGGL(k_swamp_reduce, dim3((uint32_t)b.chunk0[b.count]), dim3(kThreads), 0, stream, b,
                     reinterpret_cast<const uint4*>(w.cnt1), out);
  return hipGetLastError();
}

hipError_t launch_swamp_window(const nc_swamp_policy& p, int32_t count, nc_swamp_state* st,
                               const nc_swamp_counts* in, hipStream_t stream) {
  hipLaunchKernelGGL(k_swamp_window, dim3((uint32_t)((count + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                     stream, p, count, st, in);
  return hipGetLastError();
}

}  // namespace nc
