// The scale-update state machine, dequant to bf16, and the statistics pass
// with its fixed-order finalisation.
#include "nc_launch.h"

namespace nc {
namespace {


// ---------------------------------------------------------------------------
// Scale rule ([E3, "Worked solution"]): the largest k with
// A * 2^k <= 1.75 * 2^EMAX * 2^-margin.  For A = m * 2^e, m in [1, 2):
// k = EMAX - margin - e - [m > 1.75].  Returned unclamped; A = 0 has no bound.
constexpr int kNoBound = 1 << 20;

__device__ inline int scale_k_unclamped(uint32_t a, int emax, int margin) {
  if (a == 0) return kNoBound;
  int e;
  uint32_t frac;
  if (a >= 0x800000u) {
    e = (int)(a >> 23) - 127;
    frac = a & 0x7FFFFFu;
  } else {
    const int lz = __clz(a);
    e = (31 - lz) - 149;
    frac = (a << (lz - 8)) & 0x7FFFFFu;
  }
  return emax - margin - e - (frac > 0x600000u ? 1 : 0);
}

// Hysteresis (the pages' factor-of-two rule read for power-of-two scales):
// reset k when the kept scale would overflow at the estimate, or when the
// estimate has fallen to half of a_ref or below; keep it otherwise.
__device__ inline void set_scale(const nc_policy& p, nc_scale_state& s, uint32_t a) {
  const int emax = p.fmt == NC_E4M3 ? Fp8<NC_E4M3>::EMAX : Fp8<NC_E5M2>::EMAX;
  const int ku = scale_k_unclamped(a, emax, p.margin);
  bool reset = !p.hysteresis || !s.has_ref;
  if (!reset) reset = s.k > ku;                                              // (i)
  if (!reset) reset = 2.0 * (double)__uint_as_float(a) <= (double)__uint_as_float(s.a_ref_bits);  // (ii)
  if (reset) {
    s.k = min(127, max(-127, ku));
    s.a_ref_bits = a;
    s.has_ref = 1;
  }
}

__global__ void __launch_bounds__(kThreads)
k_scale_update(const nc_policy p, int32_t count, nc_scale_state* __restrict__ st,
               float* __restrict__ hist, const nc_counts* __restrict__ in,
               nc_loss_scale* __restrict__ ls) {
  int local = 0;
  for (int i = threadIdx.x; i < count; i += kThreads) local |= in[i].n_nonfinite != 0;
  const int any_nf = __syncthreads_or(local);
  if (threadIdx.x == 0 && ls != nullptr && p.ls_enable) {
    nc_loss_scale l = *ls;
    if (any_nf) {
      l.s_log2 = max(p.ls_log2_min, l.s_log2 - 1);
      l.clean_steps = 0;
    } else if (++l.clean_steps >= p.ls_growth_interval) {
      l.s_log2 = min(p.ls_log2_max, l.s_log2 + 1);
      l.clean_steps = 0;
    }
    *ls = l;
  }
  if (p.est == NC_EST_CURRENT) {
    for (int i = threadIdx.x; i < count; i += kThreads) {
      nc_scale_state s = st[i];
      set_scale(p, s, in[i].amax_bits);
      st[i] = s;
    }
    return;
  }
  if (p.skip_on_nonfinite && any_nf) return;
  const int W = p.window;
  for (int i = threadIdx.x; i < count; i += kThreads) {
    nc_scale_state s = st[i];
    // a state from a call with a different window restarts its ring
    if (s.head < 0 || s.head >= W || s.n_hist < 0 || s.n_hist > W) s.head = s.n_hist = 0;
    uint32_t* h = reinterpret_cast<uint32_t*>(hist) + (int64_t)i * W;
    const uint32_t a = in[i].amax_bits;
    h[s.head] = a;
    s.head = (s.head + 1 == W) ? 0 : s.head + 1;
    s.n_hist = min(s.n_hist + 1, W);
    s.step += 1;
    if (s.step % p.interval == 0) {
      uint32_t A = a;                                   // most recent
      if (p.est == NC_EST_MAX_WINDOW)                   // valid slots are 0 .. n_hist-1
        for (int j = 0; j < s.n_hist; ++j) A = max(A, h[j]);
      set_scale(p, s, A);
    }
    st[i] = s;
  }
}

// ---------------------------------------------------------------------------
// Dequant: y = RNE_bf16(decode(q) * 2^-K).  The value decode(q) * 2^-K is
// exact in fp32 for |K| <= 127 (at most 4 significant bits, exponent within
// [-143, 143]) unless it overflows fp32, where bf16 rounds to Inf as well, so
// one ldexp followed by the fp32 -> bf16 rounding gives the exact result.
template <int FMT>
__device__ __forceinline__ uint32_t dq_bf16(uint32_t dec_bits, int K) {
  if ((dec_bits & kAbsMask) > kInfBits) return 0x7FC0u;
  const float v = __builtin_amdgcn_ldexpf(__uint_as_float(dec_bits), -K);
  return f32_to_bf16_rne(__float_as_uint(v));
}

template <int FMT, bool MX>
NC_STREAM_KERNEL
k_dequant(const SegBatch b, const nc_scale_state* __restrict__ st) {
  constexpr int64_t TILE = kDequantTile;      // 16 codes per lane per step, 2 steps
  __shared__ uint32_t tab[256];               // per-tensor: bf16 result; MX: decode bits
  if constexpr (MX) {
    tab[threadIdx.x] = decode_bits<FMT>(threadIdx.x);
    __syncthreads();
  }
  const int64_t total = b.tile0[b.count];
  int seg = -1, k = 0;
  for (int64_t tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const int s = seg_of(b, tile, seg);
    if (s != seg) {
      seg = s;
      if constexpr (!MX) {
        k = st[b.first + s].k;
        __syncthreads();
        tab[threadIdx.x] = dq_bf16<FMT>(decode_bits<FMT>(threadIdx.x), k);
        __syncthreads();
      }
    }
    const Seg& g = b.s[s];
    const int64_t e0 = (tile - b.tile0[s]) * TILE;
    const int rem = tile_len<TILE>(b, s, tile);
    const uint8_t* src = g.codes + e0;
    uint16_t* dst = static_cast<uint16_t*>(g.y) + e0;
    if (rem == (int)TILE) {
      u32x4 c[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) c[u] = ld_stream(reinterpret_cast<const u32x4*>(src) + u * kThreads + threadIdx.x);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int vi = u * kThreads + threadIdx.x;
        int K = 0;
        if constexpr (MX) K = 127 - (int)g.scales[(e0 + (int64_t)vi * 16) / 32];   // K = -X
        const uint32_t w[4] = {c[u].x, c[u].y, c[u].z, c[u].w};
        uint32_t o[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t h[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const uint32_t q = (w[j] >> (8 * t)) & 0xFFu;
            if constexpr (MX) h[t] = dq_bf16<FMT>(tab[q], K);
            else h[t] = tab[q];
          }
          o[2 * j] = h[0] | (h[1] << 16);
          o[2 * j + 1] = h[2] | (h[3] << 16);
        }
        u32x4* d = reinterpret_cast<u32x4*>(dst) + (int64_t)vi * 2;
        d[0] = u32x4{o[0], o[1], o[2], o[3]};
        d[1] = u32x4{o[4], o[5], o[6], o[7]};
      }
    } else {
      for (int i = threadIdx.x; i < rem; i += kThreads) {
        const uint32_t q = src[i];
        if constexpr (MX) {
          const int K = 127 - (int)g.scales[(e0 + i) / 32];
          dst[i] = (uint16_t)dq_bf16<FMT>(tab[q], K);
        } else {
          dst[i] = (uint16_t)tab[q];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Statistics as a separate pass over x and the codes (and the MX scales).
template <int FMT, int DT, bool MX>
NC_STREAM_KERNEL
k_stats(const SegBatch b, const nc_scale_state* __restrict__ st,
        const nc_loss_scale* __restrict__ ls, double* __restrict__ part) {
  constexpr int VEC = In<DT>::VEC;
  constexpr int64_t TILE = (int64_t)kThreads * VEC * kUnrollRead;
  __shared__ double tab[256];
  __shared__ double lds_st[kWaves * 6];
  if constexpr (MX) {
    fill_stat_table<FMT>(tab, 0);
    __syncthreads();
  }
  const int s_log2 = (!MX && ls) ? ls->s_log2 : 0;
  const int64_t total = b.tile0[b.count];
  StatAcc sa;
  sa.reset();
  int seg = -1;
  // buf always holds the current tile when it is full (prefetch invariant)
  u32x4 buf[kUnrollRead];
  prefetch_tile<In<DT>::BYTES, kUnrollRead, TILE>(b, blockIdx.x, -1, buf);
  for (int64_t tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const int s = seg_of(b, tile, seg);
    if (s != seg) {
      if (seg >= 0) stats_seg_flush(sa, stat_slot(part, seg, blockIdx.x), lds_st, s_log2);
      seg = s;
      if constexpr (!MX) {
        __syncthreads();
        fill_stat_table<FMT>(tab, st[b.first + s].k - s_log2);
        __syncthreads();
      }
    }
    const Seg& g = b.s[s];
    const int64_t e0 = (tile - b.tile0[s]) * TILE;
    const int rem = tile_len<TILE>(b, s, tile);
    const uint8_t* cs = g.codes + e0;
    if (rem == (int)TILE) {
      u32x4 v[kUnrollRead];
#pragma unroll
      for (int u = 0; u < kUnrollRead; ++u) v[u] = buf[u];
      prefetch_tile<In<DT>::BYTES, kUnrollRead, TILE>(b, tile + gridDim.x, s, buf);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kUnrollRead; ++u) {
        const int vi = u * kThreads + threadIdx.x;
        uint32_t xb[VEC], q[VEC];
        unpack<DT>(v[u], xb);
        if constexpr (DT == NC_F32) {
          const uint32_t w = reinterpret_cast<const uint32_t*>(cs)[vi];
#pragma unroll
          for (int i = 0; i < 4; ++i) q[i] = (w >> (8 * i)) & 0xFFu;
        } else {
          const uint64_t w = reinterpret_cast<const uint64_t*>(cs)[vi];
#pragma unroll
          for (int i = 0; i < 8; ++i) q[i] = (uint32_t)(w >> (8 * i)) & 0xFFu;
        }
        double blk = 1.0;
        if constexpr (MX) blk = pow2_f64((int)g.scales[(e0 + (int64_t)vi * VEC) / 32] - 127);
        stats_vec<VEC, MX>(xb, q, tab, blk, sa);
      }
    } else {
      prefetch_tile<In<DT>::BYTES, kUnrollRead, TILE>(b, tile + gridDim.x, s, buf);
      for (int i = threadIdx.x; i < rem; i += kThreads) {
        const uint32_t xb = load_one<DT>(g.x, e0 + i);
        const uint32_t q = cs[i];
        double blk = 1.0;
        if constexpr (MX) blk = pow2_f64((int)g.scales[(e0 + i) / 32] - 127);
        stats_vec<1, MX>(&xb, &q, tab, blk, sa);
      }
    }
  }
  if (seg >= 0) stats_seg_flush(sa, stat_slot(part, seg, blockIdx.x), lds_st, s_log2);
}

// One workgroup per tensor: sum the partials of the workgroups that worked
// on it, in the order of the tensor's first tiles (the producer grid of G
// workgroups strides over tiles, so tile t went to workgroup t mod G), and
// add the result into out (only this workgroup writes that tensor's stats).
__global__ void __launch_bounds__(kThreads)
k_stats_finalize(const SegBatch b, const double* __restrict__ part, int grid,
                 nc_stats* __restrict__ out) {
  __shared__ double lds[kWaves * 6];
  const int s = blockIdx.x;
  const int64_t t0 = b.tile0[s], t1 = min(b.tile0[s + 1], b.tile0[s] + grid);
  double acc[6] = {0, 0, 0, 0, 0, 0};
  for (int64_t t = t0 + threadIdx.x; t < t1; t += kThreads) {
    const double* p = part + ((int64_t)s * kMaxGrid + t % grid) * 6;
    for (int j = 0; j < 6; ++j) acc[j] += p[j];
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int j = 0; j < 6; ++j) {
    const double v = wave_sum_f64(acc[j]);
    if (lane == 0) lds[wave * 6 + j] = v;
  }
  __syncthreads();
  if (threadIdx.x < 6) {
    double t = 0.0;
    for (int w = 0; w < kWaves; ++w) t += lds[w * 6 + threadIdx.x];
    double* o = reinterpret_cast<double*>(out + b.first + s);
    o[threadIdx.x] += t;
  }
}

template <int FMT, int DT>
hipError_t stats_t(const SegBatch& b, const nc_scale_state* st, const nc_loss_scale* ls,
                   double* part, const Launch& l) {
  if (st)
    hipLaunchKernelGGL((k_stats<FMT, DT, false>), dim3(l.grid), dim3(kThreads), 0, l.stream, b, st, ls, part);
  else
    hipLaunchKernelGGL((k_stats<FMT, DT, true>), dim3(l.grid), dim3(kThreads), 0, l.stream, b, st, ls, part);
  return hipGetLastError();
}

template <int FMT>
hipError_t dequant_t(const SegBatch& b, const nc_scale_state* st, const Launch& l) {
  if (st)
    hipLaunchKernelGGL((k_dequant<FMT, false>), dim3(l.grid), dim3(kThreads), 0, l.stream, b, st);
  else
    hipLaunchKernelGGL((k_dequant<FMT, true>), dim3(l.grid), dim3(kThreads), 0, l.stream, b, st);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scale_update(const nc_policy& p, int32_t count, nc_scale_state* st, float* hist,
                               const nc_counts* in, nc_loss_scale* ls, hipStream_t stream) {
  hipLaunchKernelGGL(k_scale_update, dim3(1), dim3(kThreads), 0, stream, p, count, st, hist, in, ls);
  return hipGetLastError();
}

hipError_t launch_dequant(const SegBatch& b, int fmt, const nc_scale_state* st, const Launch& l) {
  return fmt == NC_E4M3 ? dequant_t<NC_E4M3>(b, st, l) : dequant_t<NC_E5M2>(b, st, l);
}

hipError_t launch_stats(const SegBatch& b, int dtype, int fmt, const nc_scale_state* st,
                        const nc_loss_scale* ls, double* part, const Launch& l) {
  if (fmt == NC_E4M3)
    return dtype == NC_F32 ? stats_t<NC_E4M3, NC_F32>(b, st, ls, part, l)
                           : stats_t<NC_E4M3, NC_BF16>(b, st, ls, part, l);
  return dtype == NC_F32 ? stats_t<NC_E5M2, NC_F32>(b, st, ls, part, l)
                         : stats_t<NC_E5M2, NC_BF16>(b, st, ls, part, l);
}

hipError_t launch_stats_finalize(const SegBatch& b, const double* part, int grid, nc_stats* out,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(k_stats_finalize, dim3(b.count), dim3(kThreads), 0, stream, b, part, grid, out);
  return hipGetLastError();
}

}  // namespace nc
