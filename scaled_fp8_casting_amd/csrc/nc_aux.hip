// The scale-update state machine, dequant to bf16, the statistics pass, and
// the fixed-order reductions of the per-workgroup slots.
#include "nc_reduce.h"

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

// Exponential smoothing ([MaxWin, "Experimental Variables"]): E + alpha *
// (a - E), three fp32 operations each rounded to nearest even -- contraction
// into a fused multiply-add is off, so the result is defined bit for bit.
__device__ __noinline__ uint32_t ema_step(float alpha, uint32_t E_bits, uint32_t a_bits) {
#pragma clang fp contract(off)
  const float E = __uint_as_float(E_bits);
  const float d = __uint_as_float(a_bits) - E;
  const float m = alpha * d;
  return __float_as_uint(E + m);
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
    if (p.est == NC_EST_EMA) {
      const uint32_t E = s.n_hist > 0 ? ema_step(p.ema_alpha, h[0], a) : a;
      h[0] = E;
      s.head = 0;
      s.n_hist = 1;
      s.step += 1;
      if (s.step % p.interval == 0) set_scale(p, s, E);
      st[i] = s;
      continue;
    }
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

// The bf16 output is written with non-temporal stores (measured faster on
// MI355X, as for the casts' code stores).
//
// Full tiles decode in hardware: v_cvt_pk_f32_fp8 / _bf8 turns two codes
// into their exact fp32 values, v_ldexp_f32 applies the scale (exact, as
// above), v_cvt_pk_bf16_f32 rounds two values to bf16 (nearest even, IEEE
// overflow).  NaN codes -- the only codes where the hardware result is not
// the defined one (0x7FC0) -- are rare: a wave whose vector holds any takes
// a uniform branch that rewrites them.  Every code at every k is checked
// against the exact definition by the tests.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int FMT, bool HI>
__device__ __forceinline__ f32x2 decode_pair(uint32_t w) {
  if constexpr (FMT == NC_E4M3) return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
  else return __builtin_amdgcn_cvt_pk_f32_bf8((int)w, HI);
}

__device__ __forceinline__ uint32_t bf16_pair(f32x2 v, int sh) {
  v.x = __builtin_amdgcn_ldexpf(v.x, sh);
  v.y = __builtin_amdgcn_ldexpf(v.y, sh);
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Bytes of w that are NaN codes: bit 7 of each byte set for E4M3 x.1111.111
// and E5M2 x.11111.01..11.
template <int FMT>
__device__ __forceinline__ uint32_t nan_bytes(uint32_t w) {
  constexpr uint32_t kBump = FMT == NC_E4M3 ? 0x01010101u : 0x03030303u;
  return ((w & 0x7F7F7F7Fu) + kBump) & 0x80808080u;
}

template <int FMT, bool MX>
NC_STREAM_KERNEL
k_dequant(const SegBatch b, const nc_scale_state* __restrict__ st) {
  constexpr int64_t TILE = kDequantTile;      // 8 codes per lane per vector
  const int64_t tile = xcd_tile<32>();
  const int s = seg_of(b.tile0, b.count, tile);
  const Seg& g = b.s[s];
  const int64_t e0 = (tile - b.tile0[s]) * TILE;
  const int rem = tile_len<TILE>(b, s, tile);
  const uint8_t* src = g.codes + e0;
  uint16_t* dst = static_cast<uint16_t*>(g.y) + e0;
  if (rem == (int)TILE) {
    constexpr int U = kDequantVecs;
    u32x2 c[U];
    // Plain loads: for this read-1/write-2 stream they measured about one
    // point of HBM peak faster than non-temporal ones (the stores stay
    // non-temporal); the casts, which read more than they write, are the
    // other way round.
#pragma unroll
    for (int u = 0; u < U; ++u) c[u] = reinterpret_cast<const u32x2*>(src)[u * kThreads + threadIdx.x];
    int sh[U];                                // the value is decode(q) * 2^sh
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (MX) sh[u] = (int)g.scales[(e0 + (int64_t)(u * kThreads + threadIdx.x) * 8) / 32] - 127;   // X
      else sh[u] = -st[b.first + s].k;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      u32x4 o;
      o.x = bf16_pair(decode_pair<FMT, false>(c[u].x), sh[u]);
      o.y = bf16_pair(decode_pair<FMT, true>(c[u].x), sh[u]);
      o.z = bf16_pair(decode_pair<FMT, false>(c[u].y), sh[u]);
      o.w = bf16_pair(decode_pair<FMT, true>(c[u].y), sh[u]);
      const uint32_t nb0 = nan_bytes<FMT>(c[u].x), nb1 = nan_bytes<FMT>(c[u].y);
      if (__ballot((nb0 | nb1) != 0) != 0) {    // wave-uniform, rare
        uint32_t h[8] = {o.x & 0xFFFFu, o.x >> 16, o.y & 0xFFFFu, o.y >> 16,
                         o.z & 0xFFFFu, o.z >> 16, o.w & 0xFFFFu, o.w >> 16};
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (((i < 4 ? nb0 : nb1) >> (8 * (i % 4) + 7)) & 1u) h[i] = 0x7FC0u;
        o = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
      }
      __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(dst) + u * kThreads + threadIdx.x);
    }
  } else {
    const int k = MX ? 0 : st[b.first + s].k;
    for (int i = threadIdx.x; i < rem; i += kThreads) {
      const uint32_t q = src[i];
      const int K = MX ? 127 - (int)g.scales[(e0 + i) / 32] : k;
      dst[i] = (uint16_t)dq_bf16<FMT>(decode_bits<FMT>(q), K);
    }
  }
}

// Dequant of column-block MX codes.  A slot is 8 columns of a 32-row band
// (col_slot); lane l of wave w takes rows 8w .. 8w + 7 of the tile's slot l,
// reads the slot's 8 scale bytes (the same bytes as the other three waves)
// and then, per row, 8 codes (8 bytes) and writes 8 bf16 values (16 bytes);
// each column has its own shift.
__device__ __forceinline__ uint32_t bf16_pair2(f32x2 v, int sh0, int sh1) {
  v.x = __builtin_amdgcn_ldexpf(v.x, sh0);
  v.y = __builtin_amdgcn_ldexpf(v.y, sh1);
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

template <int FMT>
NC_STREAM_KERNEL
k_dequant_col(const SegBatch b) {
  constexpr int VC = kDequantColCodes, R = kDequantColRows, SLOTS = kDequantColSlots;
  static_assert(SLOTS == 64, "one slot per lane of a wave, one 8-row part per wave");
  const int64_t tile = xcd_tile<32>();
  const int s = seg_of_scan(b.tile0, b.count, tile);
  const Seg& g = b.s[s];
  const int rem = tile_len<SLOTS>(b, s, tile);                 // slots in this tile
  const uint32_t slot = threadIdx.x % SLOTS, part = threadIdx.x / SLOTS;
  const ColSlot cs = col_slot_at<VC>(g, (uint32_t)(tile - b.tile0[s]) * SLOTS + slot, (int)slot < rem);
  if (!cs.act) return;                      // no barriers below
  const int64_t cols = g.cols;
  const uint8_t* src = g.codes + cs.e0 + (int64_t)part * R * cols;
  uint16_t* dst = static_cast<uint16_t*>(g.y) + cs.e0 + (int64_t)part * R * cols;
  u32x2 c[R];
#pragma unroll
  for (int r = 0; r < R; ++r) c[r] = ld_stream(reinterpret_cast<const u32x2*>(src + r * cols));
  int sh[VC];                               // X of each column
  if (((uintptr_t)g.scales & 7u) == 0) {    // wave-uniform: one 8-byte load
    const u32x2 sw = *reinterpret_cast<const u32x2*>(g.scales + cs.sc);
#pragma unroll
    for (int i = 0; i < VC; ++i) sh[i] = (int)(((i < 4 ? sw.x : sw.y) >> (8 * (i % 4))) & 0xFFu) - 127;
  } else {
#pragma unroll
    for (int i = 0; i < VC; ++i) sh[i] = (int)g.scales[cs.sc + i] - 127;
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    u32x4 o;
    o.x = bf16_pair2(decode_pair<FMT, false>(c[r].x), sh[0], sh[1]);
    o.y = bf16_pair2(decode_pair<FMT, true>(c[r].x), sh[2], sh[3]);
    o.z = bf16_pair2(decode_pair<FMT, false>(c[r].y), sh[4], sh[5]);
    o.w = bf16_pair2(decode_pair<FMT, true>(c[r].y), sh[6], sh[7]);
    const uint32_t nb0 = nan_bytes<FMT>(c[r].x), nb1 = nan_bytes<FMT>(c[r].y);
    if (__ballot((nb0 | nb1) != 0) != 0) {    // wave-uniform, rare
      uint32_t h[8] = {o.x & 0xFFFFu, o.x >> 16, o.y & 0xFFFFu, o.y >> 16,
                       o.z & 0xFFFFu, o.z >> 16, o.w & 0xFFFFu, o.w >> 16};
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (((i < 4 ? nb0 : nb1) >> (8 * (i % 4) + 7)) & 1u) h[i] = 0x7FC0u;
      o = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
    }
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(dst + r * cols));
  }
}

// ---------------------------------------------------------------------------
// Statistics as a separate pass over x and the codes (and the MX scales).

// Vector vi of a full tile: its elements, their codes and (MX) the block's 2^X.
// Codes of vector vi of a tile (VEC per 16-byte input vector).
template <int DT>
struct CodeVec;
template <> struct CodeVec<NC_F32> {
  typedef uint32_t T;
  __device__ static T load(const uint8_t* cs, int vi) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(cs) + vi);
  }
  __device__ static void split(T w, uint32_t* q) {
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = (w >> (8 * i)) & 0xFFu;
  }
};
template <> struct CodeVec<NC_BF16> {
  typedef u32x2 T;
  __device__ static T load(const uint8_t* cs, int vi) { return ld_stream(reinterpret_cast<const u32x2*>(cs) + vi); }
  __device__ static void split(T w, uint32_t* q) {
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = (w.x >> (8 * i)) & 0xFFu;
#pragma unroll
    for (int i = 0; i < 4; ++i) q[4 + i] = (w.y >> (8 * i)) & 0xFFu;
  }
};

template <int FMT, int DT, bool MX>
NC_STREAM_KERNEL
k_stats(const SegBatch b, const nc_scale_state* __restrict__ st,
        const nc_loss_scale* __restrict__ ls, const Tail t) {
  constexpr int VEC = In<DT>::VEC;
  constexpr int U = kStatsVecs;
  constexpr int64_t TILE = (int64_t)kThreads * VEC * U;
  typedef typename CodeVec<DT>::T CT;
  constexpr int NSC = MX ? (int)(TILE / 32) : 16;        // scale bytes of a full tile
  __shared__ double tab[256];
  __shared__ double lds_st[kStatLds];
  __shared__ __align__(16) uint8_t lds_sc[NSC];
  const int64_t tile = xcd_tile<32>();
  const int s = seg_of(b.tile0, b.count, tile);
  const Seg& g = b.s[s];
  const int64_t e0 = (tile - b.tile0[s]) * TILE;
  const int rem = tile_len<TILE>(b, s, tile);
  const uint8_t* cs = g.codes + e0;
  const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(g.x) + e0 * In<DT>::BYTES);
  const bool full = rem == (int)TILE;
  // a full tile's loads go out first (an MX tile's scale bytes first of all,
  // staged through LDS: one 16-byte load by each of the first NSC / 16
  // lanes, or NSC / 256 bytes per lane where the scale array is not 16-byte
  // aligned); the table fill overlaps them
  u32x4 v[U];
  CT c[U];
  if (full) {
    if constexpr (MX) {
      const uint8_t* sb = g.scales + e0 / 32;
      if (((uintptr_t)g.scales & 15u) == 0) {
        if ((int)threadIdx.x < NSC / 16)
          reinterpret_cast<u32x4*>(lds_sc)[threadIdx.x] = reinterpret_cast<const u32x4*>(sb)[threadIdx.x];
      } else {
#pragma unroll
        for (int j = 0; j < NSC / kThreads; ++j) lds_sc[j * kThreads + threadIdx.x] = sb[j * kThreads + threadIdx.x];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = ld_stream(src + u * kThreads + threadIdx.x);
#pragma unroll
    for (int u = 0; u < U; ++u) c[u] = CodeVec<DT>::load(cs, u * kThreads + threadIdx.x);
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (MX) fill_stat_table<FMT>(tab, 0);
  else fill_stat_table<FMT>(tab, st[b.first + s].k - (ls ? ls->s_log2 : 0));
  __syncthreads();
  StatAcc sa;
  sa.reset();
  if (full) {
    // every element unmasked; a lane that met an Inf/NaN starts over with
    // the masked form (rare)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      uint32_t xb[VEC], q[VEC];
      unpack<DT>(v[u], xb);
      CodeVec<DT>::split(c[u], q);
      double blk = 1.0;
      if constexpr (MX) blk = pow2_f64((int)lds_sc[(u * kThreads + threadIdx.x) * VEC / 32] - 127);
      stats_vec<VEC, MX, true>(xb, q, tab, blk, sa);
      __builtin_amdgcn_sched_barrier(0);   // one vector's table reads at a time (register pressure)
    }
    if (!stats_all_finite(sa)) {
      sa.reset();
      for (int u = 0; u < U; ++u) {       // reloads: the vectors above are not kept
        const int vi = u * kThreads + threadIdx.x;
        uint32_t xb[VEC], q[VEC];
        unpack<DT>(src[vi], xb);
        CodeVec<DT>::split(CodeVec<DT>::load(cs, vi), q);
        double blk = 1.0;
        if constexpr (MX) blk = pow2_f64((int)g.scales[(e0 + (int64_t)vi * VEC) / 32] - 127);
        stats_vec<VEC, MX, false>(xb, q, tab, blk, sa);
      }
    }
  } else {
    for (int i = threadIdx.x; i < rem; i += kThreads) {
      const uint32_t xb = load_one<DT>(g.x, e0 + i);
      const uint32_t q = cs[i];
      double blk = 1.0;
      if constexpr (MX) blk = pow2_f64((int)g.scales[(e0 + i) / 32] - 127);
      stats_vec<1, MX, false>(&xb, &q, tab, blk, sa);
    }
  }
  write_stat_slot(sa, t.st1 + tile * 6, lds_st);
}

// Statistics of column-block MX codes: a lane owns one col_slot (VC =
// 16 / BYTES columns -- 8 bf16 or 4 fp32 -- of a 32-row band), reads its VC
// scale bytes once, then per row 16 input bytes and VC codes (8 or 4
// bytes), eight rows at a time.  Accumulation is unmasked as in k_stats,
// with the masked redo when an Inf/NaN was met.
template <int DT>
struct ColCodes;
template <> struct ColCodes<NC_F32> {      // 4 codes per row
  __device__ static u32x2 load(const uint8_t* p) {
    return u32x2{__builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p)), 0u};
  }
};
template <> struct ColCodes<NC_BF16> {     // 8 codes per row
  __device__ static u32x2 load(const uint8_t* p) { return ld_stream(reinterpret_cast<const u32x2*>(p)); }
};

template <int DT, bool FINITE>
__device__ __forceinline__ void stats_col_row(u32x4 v, u32x2 w, const double* tab, const double* blk,
                                              StatAcc& sa) {
  constexpr int VC = In<DT>::VEC;
  uint32_t xb[VC];
  unpack<DT>(v, xb);
#pragma unroll
  for (int i = 0; i < VC; ++i) {
    if (!FINITE && (xb[i] & kAbsMask) > kMaxFinite) continue;
    const uint32_t q = ((i < 4 ? w.x : w.y) >> (8 * (i % 4))) & 0xFFu;
    stat_term_blk((double)__uint_as_float(xb[i]), tab[q], blk[i], sa);
  }
}

template <int FMT, int DT>
NC_STREAM_KERNEL
k_stats_col(const SegBatch b, const Tail t) {
  constexpr int VC = In<DT>::VEC, R = kStatsColRows;
  constexpr int Q = 8;                      // rows per batch of loads
  __shared__ double tab[256];
  __shared__ double lds_st[kStatLds];
  const int64_t tile = xcd_tile<32>();
  const int s = seg_of(b.tile0, b.count, tile);
  const Seg& g = b.s[s];
  const ColSlot cs = col_slot<VC, R>(g, tile - b.tile0[s], tile_len<kThreads>(b, s, tile));
  const int64_t cols = g.cols;
  const uint8_t* xs = static_cast<const uint8_t*>(g.x) + cs.e0 * In<DT>::BYTES;
  const uint8_t* qs = g.codes + cs.e0;
  double blk[VC];
#pragma unroll
  for (int i = 0; i < VC; ++i) blk[i] = pow2_f64((int)g.scales[cs.sc + i] - 127);
  StatAcc sa;
  sa.reset();
#pragma unroll
  for (int h = 0; h < R / Q; ++h) {
    u32x4 v[Q];
    u32x2 w[Q];
#pragma unroll
    for (int r = 0; r < Q; ++r) {
      const int64_t row = h * Q + r;
      v[r] = ld_stream(reinterpret_cast<const u32x4*>(xs + row * cols * In<DT>::BYTES));
      w[r] = ColCodes<DT>::load(qs + row * cols);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (!cs.act) {                          // idle lane (last tile): zeros add nothing
#pragma unroll
      for (int r = 0; r < Q; ++r) {
        v[r] = u32x4{0u, 0u, 0u, 0u};
        w[r] = u32x2{0u, 0u};
      }
    }
    if (h == 0) {                           // the table fill overlaps the first loads
      fill_stat_table<FMT>(tab, 0);
      __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < Q; ++r) {
      stats_col_row<DT, true>(v[r], w[r], tab, blk, sa);
      __builtin_amdgcn_sched_barrier(0);    // one row's table reads at a time (register pressure)
    }
  }
  if (!stats_all_finite(sa)) {              // an Inf/NaN met: redo masked (rare; reloads)
    __asm__ volatile("" ::: "memory");      // keeps the compiler from holding the first loads for this
    sa.reset();
    for (int row = 0; row < R && cs.act; ++row) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(xs + row * cols * In<DT>::BYTES);
      stats_col_row<DT, false>(v, ColCodes<DT>::load(qs + row * cols), tab, blk, sa);
    }
  }
  write_stat_slot(sa, t.st1 + tile * 6, lds_st);
}

// ---------------------------------------------------------------------------
// The separate reductions of a launch's slots (when it does not reduce
// in-kernel): one workgroup per chunk, then one wave per tensor of several
// chunks (statistics only).  The sums are those of nc_reduce.h.
template <bool COUNTS, bool STATS>
__global__ void __launch_bounds__(kThreads)
k_reduce1(const SegBatch b, const Tail t) {
  const int64_t c = blockIdx.x;
  reduce_chunk<COUNTS, STATS>(b, seg_of(b.chunk0, b.count, c), c, t);
}

__global__ void __launch_bounds__(64)
k_reduce2(const SegBatch b, const Tail t) {
  const int s = blockIdx.x;
  if (b.chunk0[s + 1] - b.chunk0[s] <= 1) return;    // done by the first reduction (or empty)
  reduce_tensor_stats(b, s, t);
}

template <int FMT, int DT>
hipError_t stats_t(const SegBatch& b, const nc_scale_state* st, const nc_loss_scale* ls,
                   const Tail& t, const Launch& l) {
  if (st)
    hipLaunchKernelGGL((k_stats<FMT, DT, false>), dim3((uint32_t)l.grid), dim3(kThreads), 0, l.stream, b, st, ls, t);
  else
    hipLaunchKernelGGL((k_stats<FMT, DT, true>), dim3((uint32_t)l.grid), dim3(kThreads), 0, l.stream, b, st, ls, t);
  return hipGetLastError();
}

template <int FMT>
hipError_t dequant_t(const SegBatch& b, const nc_scale_state* st, const Launch& l) {
  if (st)
    hipLaunchKernelGGL((k_dequant<FMT, false>), dim3((uint32_t)l.grid), dim3(kThreads), 0, l.stream, b, st);
  else
    hipLaunchKernelGGL((k_dequant<FMT, true>), dim3((uint32_t)l.grid), dim3(kThreads), 0, l.stream, b, st);
  return hipGetLastError();
}

template <bool COUNTS, bool STATS>
hipError_t reduce_t(const SegBatch& b, const Tail& t, hipStream_t stream) {
  const int64_t chunks = b.chunk0[b.count];
  hipLaunchKernelGGL((k_reduce1<COUNTS, STATS>), dim3((uint32_t)chunks), dim3(kThreads), 0, stream, b, t);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !STATS) return e;
  bool several = false;
  for (int s = 0; s < b.count; ++s) several = several || b.chunk0[s + 1] - b.chunk0[s] > 1;
  if (!several) return hipSuccess;
  hipLaunchKernelGGL(k_reduce2, dim3((uint32_t)b.count), dim3(64), 0, stream, b, t);
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
                        const nc_loss_scale* ls, const Tail& t, const Launch& l) {
  if (fmt == NC_E4M3)
    return dtype == NC_F32 ? stats_t<NC_E4M3, NC_F32>(b, st, ls, t, l)
                           : stats_t<NC_E4M3, NC_BF16>(b, st, ls, t, l);
  return dtype == NC_F32 ? stats_t<NC_E5M2, NC_F32>(b, st, ls, t, l)
                         : stats_t<NC_E5M2, NC_BF16>(b, st, ls, t, l);
}

hipError_t launch_reduce(const SegBatch& b, const Tail& t, hipStream_t stream) {
  if (t.out && t.stats) return reduce_t<true, true>(b, t, stream);
  if (t.out) return reduce_t<true, false>(b, t, stream);
  return reduce_t<false, true>(b, t, stream);
}

hipError_t launch_dequant_col(const SegBatch& b, int fmt, const Launch& l) {
  if (fmt == NC_E4M3)
    hipLaunchKernelGGL((k_dequant_col<NC_E4M3>), dim3((uint32_t)l.grid), dim3(kThreads), 0, l.stream, b);
  else
    hipLaunchKernelGGL((k_dequant_col<NC_E5M2>), dim3((uint32_t)l.grid), dim3(kThreads), 0, l.stream, b);
  return hipGetLastError();
}

template <int FMT, int DT>
hipError_t stats_col_t(const SegBatch& b, const Tail& t, const Launch& l) {
  hipLaunchKernelGGL((k_stats_col<FMT, DT>), dim3((uint32_t)l.grid), dim3(kThreads), 0, l.stream, b, t);
  return hipGetLastError();
}

hipError_t launch_stats_col(const SegBatch& b, int dtype, int fmt, const Tail& t, const Launch& l) {
  if (fmt == NC_E4M3)
    return dtype == NC_F32 ? stats_col_t<NC_E4M3, NC_F32>(b, t, l) : stats_col_t<NC_E4M3, NC_BF16>(b, t, l);
  return dtype == NC_F32 ? stats_col_t<NC_E5M2, NC_F32>(b, t, l) : stats_col_t<NC_E5M2, NC_BF16>(b, t, l);
}

}  // namespace nc
