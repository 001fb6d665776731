// Reductions of the per-workgroup slots of a launch into the caller's counts
// and statistics.
//
// Each workgroup of a reducing kernel writes its partial counts (and
// statistics) to a slot of its own.  A chunk is at most kChunk consecutive
// tiles of one tensor.  k_reduce1 sums each chunk (reduce_chunk): the counts
// (integer sums and a max, order-free) go into the caller's counts by
// atomics; the statistics of a tensor of one chunk are added to the caller's
// statistics, those of a tensor of several chunks go to a chunk slot, and
// k_reduce2 adds a tensor's chunk slots in index order
// (reduce_tensor_stats).  Every floating-point sum runs in a fixed order
// (threads over slots in index order, lanes by butterfly, waves in index
// order), so the results do not depend on scheduling.
//
// A small launch that forms counts only skips the slots (Tail::direct): each
// workgroup adds its counts into the caller's with add_counts.  A
// last-workgroup-done reduction inside every launch was built and measured
// instead and cost far more than the second launch it saves on large
// launches: agent-scope release fences write back the whole L2 of an XCD
// (the 2^30-element MX cast went from 0.50 to 19 ms), and even without them
// the per-workgroup arrival atomics and their round trip tripled it.
#pragma once

#include "nc_launch.h"

namespace nc {

// The unscale by 2^-s scales sums 0, 1, 3 (e, |e|, sign(x) e) by 2^-s and
// the others (e^2, x e, x^2) by 2^-2s.
__device__ __forceinline__ int stat_shift(int j, int s_log2) {
  return (j == 0 || j == 1 || j == 3) ? -s_log2 : -2 * s_log2;
}

// Adds one part of tensor s -- a chunk of slots, or (Tail::direct) one
// workgroup's tile -- into the caller's counts: the finite amax (after the
// unscale, which is monotone, so the max of the unscaled values is the
// unscaled max), and the counts.  n_finite: the tensor's first part adds the
// tensor's size, every part takes off its non-finite elements (modulo 2^64).
// n_big counts clips and non-finite elements together.  One thread.
__device__ inline void add_counts(const SegBatch& b, int s, bool first, uint32_t amax, uint64_t n_nf,
                                  uint64_t n_big, uint64_t n_uf, const Tail& t) {
  nc_counts* o = t.out + b.first + s;
  const uint64_t fin = (first ? (uint64_t)b.s[s].n : 0u) - n_nf;
  atomicMax(&o->amax_bits, unscale_bits(amax, t.ls ? t.ls->s_log2 : 0));
  if (fin) atomicAdd((unsigned long long*)&o->n_finite, (unsigned long long)fin);
  if (n_nf) atomicAdd((unsigned long long*)&o->n_nonfinite, (unsigned long long)n_nf);
  if (t.clips && n_big - n_nf) atomicAdd((unsigned long long*)&o->n_clip, (unsigned long long)(n_big - n_nf));
  if (n_uf) atomicAdd((unsigned long long*)&o->n_underflow, (unsigned long long)n_uf);
}

// Sums chunk c of tensor s.  Called by all threads of a 256-thread
// workgroup.  Tensors of several chunks leave their statistics in t.st2.
template <bool COUNTS, bool STATS>
__device__ void reduce_chunk(const SegBatch& b, int s, int64_t c, const Tail& t) {
  __shared__ uint64_t lds_c[kWaves * 4];
  __shared__ double lds_s[kWaves * 6];
  const int64_t t0 = b.tile0[s] + (c - b.chunk0[s]) * kChunk;
  const int64_t t1 = min(t0 + (int64_t)kChunk, (int64_t)b.tile0[s + 1]);
  uint32_t mx = 0;
  uint64_t nf = 0, big = 0, uf = 0;
  double a[6] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
  for (int64_t i = t0 + threadIdx.x; i < t1; i += kThreads) {
    if constexpr (COUNTS) {
      const CountSlot v = t.cnt1[i];
      mx = max(mx, v.amax);
      nf += v.n_nf;
      big += v.n_big;
      uf += v.n_uf;
    }
    if constexpr (STATS) {
#pragma unroll
      for (int j = 0; j < 6; ++j) a[j] += t.st1[i * 6 + j];
    }
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if constexpr (COUNTS) {
    mx = wave_max_u32(mx);
    nf = wave_sum_u64(nf);
    big = wave_sum_u64(big);
    uf = wave_sum_u64(uf);
    if (lane == 0) {
      lds_c[wave * 4 + 0] = mx;
      lds_c[wave * 4 + 1] = nf;
      lds_c[wave * 4 + 2] = big;
      lds_c[wave * 4 + 3] = uf;
    }
  }
  if constexpr (STATS) {
#pragma unroll
    for (int j = 0; j < 6; ++j) {
      const double v = wave_sum_f64(a[j]);
      if (lane == 0) lds_s[wave * 6 + j] = v;
    }
  }
  __syncthreads();
  const int s_log2 = t.ls ? t.ls->s_log2 : 0;
  if (COUNTS && threadIdx.x == 0) {
    uint64_t m = 0, n_nf = 0, n_big = 0, n_uf = 0;
    for (int w = 0; w < kWaves; ++w) {
      m = max(m, lds_c[w * 4]);
      n_nf += lds_c[w * 4 + 1];
      n_big += lds_c[w * 4 + 2];
      n_uf += lds_c[w * 4 + 3];
    }
    add_counts(b, s, c == b.chunk0[s], (uint32_t)m, n_nf, n_big, n_uf, t);
  }
  if (STATS && threadIdx.x >= 64 && threadIdx.x < 70) {
    const int j = threadIdx.x - 64;
    double r = 0.0;
    for (int w = 0; w < kWaves; ++w) r += lds_s[w * 6 + j];
    if (b.chunk0[s + 1] - b.chunk0[s] == 1)
      atomicAdd(reinterpret_cast<double*>(t.stats + b.first + s) + j, ldexp(r, stat_shift(j, s_log2)));
    else
      t.st2[c * 6 + j] = r;
  }
}

// Adds tensor s's chunk statistics in index order into the caller's.  Run by
// one whole wave (64 lanes).
__device__ inline void reduce_tensor_stats(const SegBatch& b, int s, const Tail& t) {
  const int lane = threadIdx.x & 63;
  const int64_t c0 = b.chunk0[s], c1 = b.chunk0[s + 1];
  const int s_log2 = t.ls ? t.ls->s_log2 : 0;
  double a[6] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
  for (int64_t c = c0 + lane; c < c1; c += 64) {
#pragma unroll
    for (int j = 0; j < 6; ++j) a[j] += t.st2[c * 6 + j];
  }
  double r[6];
#pragma unroll
  for (int j = 0; j < 6; ++j) r[j] = wave_sum_f64(a[j]);
  if (lane < 6) {
    double v = r[0];
#pragma unroll
    for (int i = 1; i < 6; ++i) v = lane == i ? r[i] : v;
    atomicAdd(reinterpret_cast<double*>(t.stats + b.first + s) + lane, ldexp(v, stat_shift(lane, s_log2)));
  }
}

// A count-only workgroup's totals: into its slot, or (Tail::direct) straight
// into the caller's counts.  Called by all threads.
__device__ inline void flush_counts(const Acc& acc, const SegBatch& b, int s, int64_t tile, const Tail& t,
                                    uint32_t* lds) {
  const CountSlot c = workgroup_counts(acc, lds);
  if (threadIdx.x != 0) return;
  if (t.direct) add_counts(b, s, tile == b.tile0[s], c.amax, c.n_nf, c.n_big, c.n_uf, t);
  else t.cnt1[tile] = c;
}

}  // namespace nc
