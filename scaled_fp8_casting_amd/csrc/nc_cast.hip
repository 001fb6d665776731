// Streaming kernels that read the input tensor: the per-tensor amax pass,
// the per-tensor cast (unscale + cast + counts + next-step amax, optional
// statistics) and the MX block-scaled cast (blocks along rows or down
// columns).
//
// One workgroup per tile (256 threads x a few 16-byte vectors each; see
// nc_device.h for why).  Each 16-byte load instruction of a wave covers
// 1 KiB of contiguous input and each code store 256-512 B of contiguous
// output.  A ragged last tile runs per element with lanes past the end fed
// zeros (a zero is finite and never counted).  The workgroup's counts and
// statistics go to its workspace slot.
#include "nc_reduce.h"

namespace nc {
namespace {

// ---------------------------------------------------------------------------
// Per-tensor amax pass.
template <int DT>
NC_STREAM_KERNEL
k_amax(const SegBatch b, const Tail t) {
  constexpr int VEC = In<DT>::VEC;
  constexpr int64_t TILE = (int64_t)kThreads * VEC * kAmaxVecs;
  __shared__ uint32_t lds[kRows * 4];
  const int64_t tile = xcd_tile<32>();
  const int s = seg_of(b.tile0, b.count, tile);
  const Seg& g = b.s[s];
  const int64_t e0 = (tile - b.tile0[s]) * TILE;
  const int rem = tile_len<TILE>(b, s, tile);
  Acc acc;
  acc.reset();
  if (rem == (int)TILE) {
    const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(g.x) + e0 * In<DT>::BYTES);
    u32x4 v[kAmaxVecs];
#pragma unroll
    for (int u = 0; u < kAmaxVecs; ++u) v[u] = ld_stream(src + u * kThreads + threadIdx.x);
    __builtin_amdgcn_sched_barrier(0);   // all loads in flight before any use
#pragma unroll
    for (int u = 0; u < kAmaxVecs; ++u) {
      uint32_t xb[VEC];
      unpack<DT>(v[u], xb);
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < VEC; ++i) m = max(m, xb[i] & kAbsMask);
      if (__ballot(m > kMaxFinite) == 0) {     // wave-uniform: no Inf/NaN in this vector
        acc.amax = max(acc.amax, m);
      } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc.amax = max(acc.amax, finite_mag(xb[i] & kAbsMask, acc));
      }
    }
  } else {
    for (int i = threadIdx.x; i < rem; i += kThreads)
      acc.amax = max(acc.amax, finite_mag(load_one<DT>(g.x, e0 + i) & kAbsMask, acc));
  }
  flush_counts(acc, b, s, tile, t, lds);   // n_big stays 0: the amax pass reports no clips
}

// ---------------------------------------------------------------------------
// Per-tensor cast: code = RNE-sat(x * 2^(k - s)).

// A full tile: U vectors per lane, loaded already.
template <int FMT, int DT, bool STATS, bool SCALED, int U>
__device__ __forceinline__ void cast_pt_full(const u32x4* v, const CastParams& p, float scale, Acc& acc,
                                             StatAcc& sa, const double* tab, uint8_t* dst) {
  constexpr int VEC = In<DT>::VEC;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    uint32_t xb[VEC], w[VEC / 4];
    unpack<DT>(v[u], xb);
    const bool clean = cast_vec<FMT, DT, SCALED>(v[u], xb, p, scale, acc, w);
    if constexpr (STATS) {
      uint32_t q[VEC];
#pragma unroll
      for (int i = 0; i < VEC; ++i) q[i] = (w[i / 4] >> (8 * (i % 4))) & 0xFFu;
      if (clean) stats_vec<VEC, false, true>(xb, q, tab, 1.0, sa);
      else stats_vec<VEC, false, false>(xb, q, tab, 1.0, sa);
    }
    const int vi = u * kThreads + threadIdx.x;
    if constexpr (DT == NC_F32) st_stream(reinterpret_cast<uint32_t*>(dst) + vi, w[0]);
    else st_stream(reinterpret_cast<u32x2*>(dst) + vi, u32x2{w[0], w[1]});
    if constexpr (STATS) __builtin_amdgcn_sched_barrier(0);   // one vector at a time (register pressure)
  }
}
template <int FMT, int DT, bool STATS>
NC_STREAM_KERNEL
k_cast_pt(const SegBatch b, const nc_scale_state* __restrict__ st,
          const nc_loss_scale* __restrict__ ls, const Tail t) {
  constexpr int VEC = In<DT>::VEC;
  constexpr int U = cast_vecs<STATS>();
  constexpr int64_t TILE = (int64_t)kThreads * VEC * U;
  __shared__ uint32_t lds[kRows * 4];
  __shared__ double lds_st[STATS ? kStatLds : 1];
  __shared__ double tab[STATS ? 256 : 1];
  const int64_t tile = xcd_tile<256>();
  const int s = seg_of_scan(b.tile0, b.count, tile);
  const Seg& g = b.s[s];
  const int64_t e0 = (tile - b.tile0[s]) * TILE;
  const int rem = tile_len<TILE>(b, s, tile);
  const bool full = rem == (int)TILE;
  const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(g.x) + e0 * In<DT>::BYTES);
  // a full tile's loads go out first; the scale and table set-up overlap them
  u32x4 v[U];
  if (full) {
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = ld_stream(src + u * kThreads + threadIdx.x);
  }
  __builtin_amdgcn_sched_barrier(0);
  const int K = st[b.first + s].k - (ls ? ls->s_log2 : 0);
  const CastParams p = cast_params<FMT>(K);
  if constexpr (STATS) {
    fill_stat_table<FMT>(tab, K);
    __syncthreads();
  }
  Acc acc;
  acc.reset();
  StatAcc sa;
  if constexpr (STATS) sa.reset();
  uint8_t* dst = g.codes + e0;
  if (full) {
    // scaled converts while 2^-K is an fp32 value; a loss-scale unscale can
    // push K below -127, where ldexp + convert takes over (uniform branch)
    if (K >= -127 && K <= 127)
      cast_pt_full<FMT, DT, STATS, true, U>(v, p, __builtin_amdgcn_ldexpf(1.0f, -K), acc, sa, tab, dst);
    else
      cast_pt_full<FMT, DT, STATS, false, U>(v, p, 0.0f, acc, sa, tab, dst);
  } else {
    for (int base = 0; base < rem; base += kThreads) {
      const int i = base + (int)threadIdx.x;
      const bool act = i < rem;
      const uint32_t xb = act ? load_one<DT>(g.x, e0 + i) : 0u;
      const uint32_t q = cast_one<FMT>(xb, p, acc);
      if constexpr (STATS) stats_vec<1, false, false>(&xb, &q, tab, 1.0, sa);
      if (act) dst[i] = (uint8_t)q;
    }
  }
  if constexpr (STATS) write_count_stat_slots(acc, sa, t.cnt1 + tile, t.st1 + tile * 6, lds, lds_st);
  else flush_counts(acc, b, s, tile, t, lds);
}

// ---------------------------------------------------------------------------
// Stochastic-rounding cast ([Drift, "The part I would rather not write"]:
// its expected code at one step is the input itself, with no bias).
//
// Uniforms: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random
// Numbers: As Easy as 1, 2, 3", SC11): ten rounds, each two 32 x 32 -> 64-bit
// products of counter words 0 and 2 with the generator's multipliers, whose
// high halves are xored with the other counter words and the key; the key
// is bumped by two Weyl constants between rounds.  Element i of tensor j
// reads word i % 4 of the block at counter (i / 4, j, offset lo, offset hi)
// under key (seed lo, seed hi).  The key schedule is the same for every
// lane (scalar registers); a block costs 20 multiplies for 4 elements.
__device__ __forceinline__ void philox10(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)c[0] * 0xD2511F53u;
    const uint64_t p1 = (uint64_t)c[2] * 0xCD9E8D57u;
    // three-input xors in one instruction each (truth table 0x96)
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c[1], k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c[3], k1, 0x96);
    c[0] = n0;
    c[1] = (uint32_t)p1;
    c[2] = n2;
    c[3] = (uint32_t)p0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

struct SrKey {
  uint32_t k0, k1;    // seed
  uint32_t j;         // tensor index in the call
  uint32_t o0, o1;    // offset
};

// The four uniforms of block `blk` (elements 4 blk .. 4 blk + 3).
__device__ __forceinline__ void sr_block(uint32_t blk, const SrKey& key, uint32_t (&r)[4]) {
  r[0] = blk;
  r[1] = key.j;
  r[2] = key.o0;
  r[3] = key.o1;
  philox10(r, key.k0, key.k1);
}

// Only word 0 of a block's counter (blk, j, o0, o1) differs between the
// blocks of a tensor, so part of the first three rounds is the same for all
// of them: round 1's product of word 2 and the words it yields, and round
// 2's product of word 0.  SrPre holds those parts, each already xored with
// its round key, formed once per workgroup from wave-uniform values (scalar
// unit).  Round r (0-based) uses key (k0 + r W0, k1 + r W1).
struct SrPre {
  uint32_t x0;    // round 1: o1 ^ k1
  uint32_t x1;    // round 2: lo(o0 M1) ^ (k0 + W0)
  uint32_t x2;    // round 2: hi(A M0) ^ (k1 + W1), A = hi(o0 M1) ^ j ^ k0
  uint32_t x3;    // round 3: lo(A M0) ^ (k1 + 2 W1)
  uint32_t k0, k1;
};

__device__ __forceinline__ SrPre sr_pre(const SrKey& key) {
  const uint32_t k0 = __builtin_amdgcn_readfirstlane(key.k0), k1 = __builtin_amdgcn_readfirstlane(key.k1);
  const uint32_t j = __builtin_amdgcn_readfirstlane(key.j), o0 = __builtin_amdgcn_readfirstlane(key.o0);
  const uint32_t o1 = __builtin_amdgcn_readfirstlane(key.o1);
  const uint64_t q1 = (uint64_t)o0 * 0xCD9E8D57u;
  const uint32_t a = (uint32_t)(q1 >> 32) ^ j ^ k0;
  const uint64_t q0 = (uint64_t)a * 0xD2511F53u;
  return SrPre{o1 ^ k1, (uint32_t)q1 ^ (k0 + 0x9E3779B9u), (uint32_t)(q0 >> 32) ^ (k1 + 0xBB67AE85u),
               (uint32_t)q0 ^ (k1 + 2u * 0xBB67AE85u), k0, k1};
}

// The four uniforms of block `blk`, complemented (~r[i], the operand the
// hardware stochastic-rounding converts take): the same ten rounds as
// sr_block with the shared parts taken from `pre`, and the last round's
// xors complemented in the same instruction (truth table 0x69).
__device__ __forceinline__ void sr_block_inv(uint32_t blk, const SrPre& pre, uint32_t (&r)[4]) {
  uint32_t c0, c1, c2, c3;
  {                                                 // round 1: word 2's product is shared
    const uint64_t p0 = (uint64_t)blk * 0xD2511F53u;
    c2 = (uint32_t)(p0 >> 32) ^ pre.x0;
    c3 = (uint32_t)p0;
  }
  {                                                 // round 2: word 0's product is shared
    const uint64_t p1 = (uint64_t)c2 * 0xCD9E8D57u;
    c0 = (uint32_t)(p1 >> 32) ^ pre.x1;
    c1 = (uint32_t)p1;
    c2 = c3 ^ pre.x2;
  }
  {                                                 // round 3: word 3 is shared
    const uint64_t p0 = (uint64_t)c0 * 0xD2511F53u;
    const uint64_t p1 = (uint64_t)c2 * 0xCD9E8D57u;
    c0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, pre.k0 + 2u * 0x9E3779B9u, 0x96);
    c1 = (uint32_t)p1;
    c2 = (uint32_t)(p0 >> 32) ^ pre.x3;
    c3 = (uint32_t)p0;
  }
  uint32_t k0 = pre.k0 + 3u * 0x9E3779B9u, k1 = pre.k1 + 3u * 0xBB67AE85u;
#pragma unroll
  for (int i = 3; i < 9; ++i) {
    const uint64_t p0 = (uint64_t)c0 * 0xD2511F53u;
    const uint64_t p1 = (uint64_t)c2 * 0xCD9E8D57u;
    c0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
    c1 = (uint32_t)p1;
    c2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
    c3 = (uint32_t)p0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  const uint64_t p0 = (uint64_t)c0 * 0xD2511F53u;
  const uint64_t p1 = (uint64_t)c2 * 0xCD9E8D57u;
  r[0] = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x69);
  r[1] = ~(uint32_t)p1;
  r[2] = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x69);
  r[3] = ~(uint32_t)p0;
}

// Stochastic rounding of one |x| (bits ax, finite, |x| 2^K <= max) at
// exponent K with uniform u: returns m 2^(K - s), m the drawn multiple of
// the grid spacing q at y = |x| 2^K (q = 2^(max(floor(log2 y), EMIN) - MB)).
// With |x| = f 2^ex, f in [0.5, 1), yq = y / q = |x| 2^s for
// s = min(MB + 1 - ex, K - EMIN + MB) (c2 = K - EMIN + MB).  Where yq >=
// 2^-32 it is a normal binary32 number, so yq, fl = floor(yq), yq - fl and
// (yq - fl) 2^32 are exact, and T = ceil((yq - fl) 2^32) = ceil(t 2^32):
// u < t 2^32 iff u < T for an integer u.  Below 2^-32, yq may lose bits or
// underflow, but there 0 < t 2^32 < 1 for any nonzero x and T must be 1:
// yq is raised to min(|x|, 2^-33), positive exactly when x is, and
// ceil(2^-33 2^32) = 1.  The raise is an integer max and min on the bit
// patterns (non-negative floats order as their bits).  No branch and no
// 64-bit shift.
template <int FMT>
__device__ __forceinline__ float sr_value(uint32_t ax, int K, int c2, uint32_t u, float& m) {
  using F = Fp8<FMT>;
  const float xf = __uint_as_float(ax);
  const int s = min(F::MB + 1 - __builtin_amdgcn_frexp_expf(xf), c2);
  const float yq = __uint_as_float(max(__float_as_uint(__builtin_amdgcn_ldexpf(xf, s)), min(ax, 0x2F000000u)));
  const float fl = __builtin_floorf(yq);
  // v_cvt_u32_f32 saturates (NaN -> 0): defined for a discarded lane's Inf
  // or NaN, where a C conversion would not be
  uint32_t T;
  __asm__("v_cvt_u32_f32 %0, %1" : "=v"(T) : "v"(__builtin_ceilf(__builtin_amdgcn_ldexpf(yq - fl, 32))));
  m = fl + (u < T ? 1.0f : 0.0f);
  return __builtin_amdgcn_ldexpf(m, K - s);
}

// Four elements -> four codes (byte i = element i), counts and amax to acc.
// Clips saturate; non-finite elements are rewritten by the caller's uniform
// branch (as in the round-to-nearest cast).
template <int FMT>
__device__ __forceinline__ uint32_t sr4(const uint32_t* xb, const CastParams& p, int c2, const uint32_t (&r)[4],
                                        Acc& acc) {
  constexpr float kMaxF = 1.75f * (float)(1u << Fp8<FMT>::EMAX);
  float v[4];
  uint32_t sgn = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t ax = xb[i] & kAbsMask;
    float m;
    const float val = sr_value<FMT>(ax, p.K, c2, r[i], m);
    const bool big = ax > p.t_clip;            // clips and non-finite
    acc.n_big += big ? 1u : 0u;
    acc.n_uf += (!big && ax != 0u && m == 0.0f) ? 1u : 0u;
    v[i] = big ? kMaxF : val;
    sgn |= (xb[i] >> 31) << (8 * i + 7);
  }
  int w = cvt_pair<FMT, false>(v[0], v[1], 0);
  w = cvt_pair<FMT, true>(v[2], v[3], w);
  return (uint32_t)w | sgn;
}

// gfx950's stochastic-rounding scaled converts (v_cvt_scalef32_sr_fp8_f32 /
// _bf8_f32): x / scale rounded to the format with a 32-bit random operand
// per element.  Given ~u they follow the rule above -- up exactly when
// u < ceil(t 2^32) -- whenever the fraction t has at most 23 - MB
// fractional bits; with more, they resolve t to 23 - MB bits and round up
// only when the top 23 - MB bits of u lie below t's, so for u just under
// ceil(t 2^32) they round down where the rule rounds up (never the other
// way).  A probe with u set at the threshold and one below it, over every
// fraction length from 1 to 44 bits, both formats and scales 2^-127 ..
// 2^127, showed exactly this boundary.  t has at most 23 - MB fractional
// bits whenever the result is in the normal range (y >= 2^EMIN: 24
// significant bits of x above the grid's last MB), and for bf16 inputs (8
// significant bits) whenever y >= 2^(EMIN - 16); below those bounds
// sr_fix_region marks the elements for the software rule.  (The bf16-input
// forms differ further, so bf16 inputs are widened to fp32 first.)  Past the
// largest finite value they give the overflow code, which sat4 saturates.
// Four elements (fp32 patterns) and their complemented uniforms -> four
// codes, byte i = element i.
template <int FMT>
__device__ __forceinline__ uint32_t sr_cvt4(const uint32_t* xb, const uint32_t (&nr)[4], float scale) {
  // every byte is written, so the word starts from any live value
  int w = (int)nr[0];
  if constexpr (FMT == NC_E4M3) {
    w = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(w, __uint_as_float(xb[0]), nr[0], scale, 0);
    w = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(w, __uint_as_float(xb[1]), nr[1], scale, 1);
    w = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(w, __uint_as_float(xb[2]), nr[2], scale, 2);
    w = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(w, __uint_as_float(xb[3]), nr[3], scale, 3);
  } else {
    w = __builtin_amdgcn_cvt_scalef32_sr_bf8_f32(w, __uint_as_float(xb[0]), nr[0], scale, 0);
    w = __builtin_amdgcn_cvt_scalef32_sr_bf8_f32(w, __uint_as_float(xb[1]), nr[1], scale, 1);
    w = __builtin_amdgcn_cvt_scalef32_sr_bf8_f32(w, __uint_as_float(xb[2]), nr[2], scale, 2);
    w = __builtin_amdgcn_cvt_scalef32_sr_bf8_f32(w, __uint_as_float(xb[3]), nr[3], scale, 3);
  }
  return (uint32_t)w;
}

// Bytes of w whose code has magnitude zero (a signed zero): bit 7 of each
// such byte set.
__device__ __forceinline__ uint32_t zero_code_bytes(uint32_t w) {
  return ~((w & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) & 0x80808080u;
}

// Where the hardware converts may differ from the rule (see sr_cvt4): |x|
// bits below `thr`, i.e. y = |x| 2^K below 2^EMIN (fp32 inputs) or below
// 2^(EMIN - 16) (bf16 inputs).  For bf16 inputs such a y lies below the
// grid by more than 2^(16 - MB) (t < 2^(MB - 16), so the rule can only round
// up when u < 2^(MB + 16)): `nr_min` is the smallest complemented word of
// such a u, and an element needs the software rule only if it is in the
// region and its word is at least nr_min.
struct SrFix {
  uint32_t thr;        // region: 0 < |x| bits < thr (a zero input is exact: t = 0); thr >= 1
  uint32_t nr_min;     // bf16: ~u >= nr_min  <=>  u < 2^(MB + 16)
  __device__ bool in(uint32_t ax) const { return ax - 1u < thr - 1u; }
};

template <int FMT, int DT>
__device__ __forceinline__ SrFix sr_fix_region(int K) {
  using F = Fp8<FMT>;
  const int j = (DT == NC_BF16 ? F::EMIN - 16 : F::EMIN) - K;     // region: |x| < 2^j
  uint32_t thr;
  if (j > 127) thr = kInfBits;                     // every finite |x|
  else if (j >= -126) thr = (uint32_t)(j + 127) << 23;
  else if (j >= -149) thr = 1u << (j + 149);       // a subnormal power of two
  else thr = 1u;                                   // no nonzero |x|
  return SrFix{thr, 0u - (1u << (F::MB + 16))};
}

// The rule in software for four elements of the region from their
// complemented uniforms: four codes, byte i = element i (elements outside
// the region give bytes the caller discards).  In the region y < 2^EMIN, so
// the result is a subnormal code or the smallest normal one, on the grid of
// q = 2^(EMIN - MB): with z = y / q = |x| 2^c2 (< 2^MB) the code's magnitude
// is floor(z) + [u < ceil(frac(z) 2^32)].  z is exact where it is at least
// 2^-126; below 2^-32 the threshold is 1 for any nonzero x, which raising z
// to 2^-40 gives also where it rounded or underflowed (a nonzero element is
// in the region).  floor, the difference, the scaling by 2^32 and ceil are
// exact binary32 steps (sr_value, in the general form).
template <int FMT>
__device__ __forceinline__ uint32_t sr4_region(const uint32_t* xb, int c2, const uint32_t* nr) {
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float z = __builtin_fmaxf(__builtin_amdgcn_ldexpf(__uint_as_float(xb[i] & kAbsMask), c2), 0x1p-40f);
    const float fl = __builtin_floorf(z);
    // v_cvt_u32_f32 saturates (NaN -> 0): defined for a discarded element's
    // Inf or NaN, where a C conversion would not be
    uint32_t T, f;
    __asm__("v_cvt_u32_f32 %0, %1" : "=v"(T) : "v"(__builtin_ceilf(__builtin_amdgcn_ldexpf(z - fl, 32))));
    __asm__("v_cvt_u32_f32 %0, %1" : "=v"(f) : "v"(fl));
    const uint32_t code = f + (~nr[i] < T ? 1u : 0u);
    w |= ((code & 0x7Fu) | ((xb[i] >> 24) & 0x80u)) << (8 * i);
  }
  return w;
}

// A full tile of the stochastic-rounding cast with the hardware converts
// (scale 2^-K, |K| <= 127).  Counts: a drawn zero of a nonzero finite input
// is an underflow, and a zero input always gives a zero code, so underflows
// are the zero codes less the zero inputs (non-finite inputs never give a
// zero code).  The zero inputs are counted only in a wave whose vector holds
// one (uniform branch, rare).  Saturation and the clip counts run only in a
// wave whose vector holds an element above the clip bound (uniform branch).
template <int FMT, int DT, int U>
__device__ __forceinline__ void sr_full_hw(const u32x4* v, int64_t e0, const CastParams& p, int c2, float scale,
                                           const SrPre& pre, const SrFix& fx, Acc& acc, uint8_t* dst) {
  constexpr int VEC = In<DT>::VEC;
  uint32_t zc = 0, n0 = 0;     // zero codes, zero inputs (per lane)
  // Philox block of a lane's first element: element index / 4 (< 2^32, as
  // the element index is < 2^34; e0 is a multiple of the tile)
  const uint32_t blk0 = (uint32_t)(e0 >> 2) + threadIdx.x * (uint32_t)(VEC / 4);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int vi = u * kThreads + threadIdx.x;
    const uint32_t blk = blk0 + (uint32_t)(u * kThreads * (VEC / 4));
    uint32_t xb[VEC], w[VEC / 4], nr[VEC];
    unpack<DT>(v[u], xb);
#pragma unroll
    for (int j = 0; j < VEC / 4; ++j) {
      uint32_t q[4];
      sr_block_inv(blk + j, pre, q);
      w[j] = sr_cvt4<FMT>(xb + 4 * j, q, scale);
#pragma unroll
      for (int i = 0; i < 4; ++i) nr[4 * j + i] = q[i];
    }
    // the software rule for the elements of the region, where some element
    // of the wave's vector needs it (wave-uniform)
    auto fix_region = [&](bool fix) {
      if (__ballot(fix) == 0) return;
#pragma unroll
      for (int j = 0; j < VEC / 4; ++j) {
        const uint32_t sw = sr4_region<FMT>(xb + 4 * j, c2, nr + 4 * j);
        uint32_t sel = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) sel |= (fx.in(xb[4 * j + i] & kAbsMask) ? 0xFFu : 0u) << (8 * i);
        w[j] = (w[j] & ~sel) | (sw & sel);
      }
    };
    uint32_t m = 0;
    if constexpr (DT == NC_BF16) {               // packed 16-bit magnitudes
      const u16x2 h[4] = {mag16(v[u].x), mag16(v[u].y), mag16(v[u].z), mag16(v[u].w)};
      const u16x2 hm = __builtin_elementwise_max(__builtin_elementwise_max(h[0], h[1]),
                                                 __builtin_elementwise_max(h[2], h[3]));
      const u16x2 hn = __builtin_elementwise_min(__builtin_elementwise_min(h[0], h[1]),
                                                 __builtin_elementwise_min(h[2], h[3]));
      m = (uint32_t)max(hm.x, hm.y) << 16;
      if (__ballot(min(hn.x, hn.y) == 0) != 0) {    // wave-uniform: exact zeros
        const u16x2 one = {1, 1};
        u16x2 z = {0, 0};
#pragma unroll
        for (int j = 0; j < 4; ++j) z += one - __builtin_elementwise_min(h[j], one);
        n0 += (uint32_t)z.x + z.y;
      }
      // far below the grid only an element whose u < 2^(MB + 16) can
      // differ: screen on the vector's largest complemented word, about one
      // element in 2^(16 - MB) passes
      uint32_t nmax = nr[0];
#pragma unroll
      for (int i = 1; i < VEC; ++i) nmax = max(nmax, nr[i]);
      if (__ballot(nmax >= fx.nr_min) != 0) {    // wave-uniform
        bool fix = false;
#pragma unroll
        for (int i = 0; i < VEC; ++i) fix |= fx.in(xb[i] & kAbsMask) && nr[i] >= fx.nr_min;
        fix_region(fix);
      }
    } else {
      uint32_t mn = ~0u;                         // least magnitude
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        m = max(m, xb[i] & kAbsMask);
        mn = min(mn, xb[i] & kAbsMask);
      }
      if (__ballot(mn == 0u) != 0) {             // wave-uniform: exact zeros
        bool fix = false;
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          n0 += (xb[i] & kAbsMask) == 0u ? 1u : 0u;
          fix |= fx.in(xb[i] & kAbsMask);
        }
        fix_region(fix);
      } else {
        fix_region(mn < fx.thr);                 // every magnitude nonzero here
      }
    }
#pragma unroll
    for (int j = 0; j < VEC / 4; ++j) zc += __popc(zero_code_bytes(w[j]));
    if (__ballot(m > p.t_clip) != 0) {           // wave-uniform: some element clips (or is Inf/NaN)
#pragma unroll
      for (int j = 0; j < VEC / 4; ++j) w[j] = sat4<FMT>(w[j]);
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc.n_big += (xb[i] & kAbsMask) > p.t_clip ? 1u : 0u;
      if (__ballot(m > kMaxFinite) != 0) {       // wave-uniform: Inf/NaN present
        uint32_t mf = 0;
#pragma unroll
        for (int i = 0; i < VEC; ++i) mf = max(mf, finite_mag(xb[i] & kAbsMask, acc));
        m = mf;
#pragma unroll
        for (int j = 0; j < VEC / 4; ++j) w[j] = fix_nonfinite4<FMT>(w[j], xb + 4 * j);
      }
    }
    acc.amax = max(acc.amax, m);
    if constexpr (DT == NC_F32) st_stream(reinterpret_cast<uint32_t*>(dst) + vi, w[0]);
    else st_stream(reinterpret_cast<u32x2*>(dst) + vi, u32x2{w[0], w[1]});
  }
  acc.n_uf += zc - n0;
}

template <int FMT, int DT>
NC_STREAM_KERNEL
k_cast_sr(const SegBatch b, const nc_scale_state* __restrict__ st, const nc_loss_scale* __restrict__ ls,
          uint64_t seed, uint64_t offset, const Tail t) {
  constexpr int VEC = In<DT>::VEC;
  constexpr int U = kCastSrVecs;
  constexpr int64_t TILE = (int64_t)kThreads * VEC * U;
  __shared__ uint32_t lds[kRows * 4];
  const int64_t tile = xcd_tile<1>();
  const int s = seg_of(b.tile0, b.count, tile);
  const Seg& g = b.s[s];
  const int64_t e0 = (tile - b.tile0[s]) * TILE;
  const int rem = tile_len<TILE>(b, s, tile);
  const bool full = rem == (int)TILE;
  const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(g.x) + e0 * In<DT>::BYTES);
  u32x4 v[U];
  if (full) {
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = ld_stream(src + u * kThreads + threadIdx.x);
  }
  __builtin_amdgcn_sched_barrier(0);
  const int K = st[b.first + s].k - (ls ? ls->s_log2 : 0);
  const CastParams p = cast_params<FMT>(K);
  const int c2 = K - Fp8<FMT>::EMIN + Fp8<FMT>::MB;
  const SrKey key{(uint32_t)seed, (uint32_t)(seed >> 32), (uint32_t)(b.first + s), (uint32_t)offset,
                  (uint32_t)(offset >> 32)};
  Acc acc;
  acc.reset();
  uint8_t* dst = g.codes + e0;
  if (full && K >= -127 && K <= 127) {
    // hardware converts while 2^-K is an fp32 value (uniform branch); a full
    // tile at a scale beyond that (a loss-scale unscale far outside the
    // usual range) runs per element, like a ragged one
    sr_full_hw<FMT, DT, U>(v, e0, p, c2, __builtin_amdgcn_ldexpf(1.0f, -K), sr_pre(key), sr_fix_region<FMT, DT>(K),
                           acc, dst);
  } else {
    for (int base = 0; base < rem; base += kThreads) {
      const int i = base + (int)threadIdx.x;
      const bool act = i < rem;
      const int64_t e = e0 + i;
      uint32_t xb[4] = {act ? load_one<DT>(g.x, e) : 0u, 0u, 0u, 0u};
      uint32_t r[4];
      sr_block((uint32_t)(e >> 2), key, r);
      r[0] = r[e & 3];                         // this element's word
      uint32_t q = sr4<FMT>(xb, p, c2, r, acc) & 0xFFu;
      const uint32_t ax = xb[0] & kAbsMask;
      acc.amax = max(acc.amax, finite_mag(ax, acc));
      if (ax > kMaxFinite) q = nonfinite_code<FMT>(xb[0]);
      if (act) dst[i] = (uint8_t)q;
    }
  }
  flush_counts(acc, b, s, tile, t, lds);
}

// ---------------------------------------------------------------------------
// MX: shared block exponent X ([Drift, "What the measurements said"]) from
// the finite amax a of each 32-element block (a = 0 -> -127).
// Only the floor-based rule can put a block's largest magnitude above the
// format's largest finite value: with one bit of headroom |x| 2^-X < 2^EMAX,
// and the rounded-up scale keeps every |x| 2^-X <= max (a value the rounding
// cannot exceed).  The other rules need neither saturation nor clip counts.
constexpr bool mx_rule_clips(int rule) { return rule == NC_MX_OCP; }

template <int FMT, int RULE>
__device__ __forceinline__ int mx_exponent(uint32_t a) {
  using F = Fp8<FMT>;
  // binade and fraction of a, normalising a subnormal fp32 amax (selects only)
  const int lz = __clz(a | 1u);
  const bool normal = a >= 0x800000u;
  const int e = normal ? (int)(a >> 23) - 127 : (31 - lz) - 149;
  const uint32_t frac = normal ? (a & 0x7FFFFFu) : ((a << ((lz - 8) & 31)) & 0x7FFFFFu);
  int X = e - F::EMAX;                                    // OCP: floor based
  if constexpr (RULE == NC_MX_PLUS1) X += 1;              // one bit of headroom
  if constexpr (RULE == NC_MX_CEIL) X += (frac > 0x600000u) ? 1 : 0;   // smallest X that fits
  X = min(127, max(-127, X));
  return a == 0 ? -127 : X;
}

// What a block's cast needs from its exponent X: the scale byte X + 127, the
// scaled converts' divisor 2^X, and the clip / underflow thresholds of
// cast_params(-X).
struct MxBlock {
  int sb;           // X + 127
  float scale;      // 2^X (any positive normal value for an all-zero block)
  uint32_t t_clip;  // as CastParams
  uint32_t t_uf;
};

// The general form: any block amax bits a (finite).
template <int FMT, int RULE>
__device__ __forceinline__ MxBlock mx_block(uint32_t a) {
  const int X = mx_exponent<FMT, RULE>(a);
  const CastParams p = cast_params<FMT>(-X);
  return MxBlock{X + 127, __builtin_amdgcn_ldexpf(1.0f, X), p.t_clip, p.t_uf};
}

// Block amax bits for which mx_block_fast applies: 0, or a normal fp32 with
// exponent field 33 .. 253 (2^-94 <= a < 2^127).
__device__ __forceinline__ bool mx_fast_ok(uint32_t a) {
  return a == 0u || a - (33u << 23) < ((254u - 33u) << 23);
}

// The same values by exponent-field arithmetic, for a block amax bits a with
// mx_fast_ok(a).  With E the exponent field of a (e(a) = E - 127) the rule
// gives X + 127 = E - EMAX (+1; ceil: +[m(a) > 1.75]), between 18 and 247 here,
// so no clamp applies; 2^X has exponent field X + 127; the clip bound
// 1.75 * 2^(EMAX + X) has exponent field X + 127 + EMAX <= 254 and mantissa
// 0x600000; the underflow bound 2^(X + EMIN - MB - 1) has exponent field
// X + 127 + EMIN - MB - 1 >= 1.  All are normal fp32 patterns, equal bit for
// bit to mx_block's.  An all-zero block (a = 0) has X = -127: its clip bound
// is still normal, and since its elements are zeros or non-finite, an
// underflow bound of 0 and a scale of 2^-126 give the same codes and counts.
template <int FMT, int RULE>
__device__ __forceinline__ MxBlock mx_block_fast(uint32_t a) {
  using F = Fp8<FMT>;
  int sb = (int)(a >> 23) - F::EMAX;                       // OCP: floor based
  if constexpr (RULE == NC_MX_PLUS1) sb += 1;              // one bit of headroom
  if constexpr (RULE == NC_MX_CEIL) sb += (a & 0x7FFFFFu) > 0x600000u ? 1 : 0;   // smallest X that fits
  sb = a == 0u ? 0 : sb;
  MxBlock b;
  b.sb = sb;
  b.scale = __uint_as_float((uint32_t)max(sb, 1) << 23);
  b.t_clip = ((uint32_t)(sb + F::EMAX) << 23) | 0x600000u;
  b.t_uf = (uint32_t)max(sb + F::EMIN - F::MB - 1, 0) << 23;
  return b;
}

// Max over the lanes of one block: 4 lanes (bf16, 8 elements each) or 8
// lanes (fp32, 4 each), by DPP moves inside rows of the wave.
template <int GROUP>
__device__ __forceinline__ uint32_t group_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
  if constexpr (GROUP == 8)
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  return v;
}

// One tile of the MX cast, from this lane's vectors v.  FULL: every lane's
// vector is inside the tensor (no predicates at all); otherwise lanes past
// `rem` hold zeros and skip their stores (rem is a multiple of 32, so a
// block is all in or all out).
template <int FMT, int DT, int RULE, bool STATS, bool FULL, int U>
__device__ __forceinline__ void mx_tile(const Seg& g, int64_t e0, int rem, const u32x4* v,
                                        Acc& acc, StatAcc& sa, const double* tab) {
  constexpr int VEC = In<DT>::VEC;
  constexpr int GROUP = 32 / VEC;
  constexpr bool CLIPS = mx_rule_clips(RULE);
  uint8_t* dst = g.codes + e0;
  uint8_t* sdst = g.scales + e0 / 32;
  // the scales may be stored a row's worth at a time (4 bytes for bf16, 2
  // for fp32) when their array is aligned for it (wave-uniform)
  const bool sc_word = ((uintptr_t)g.scales & (GROUP == 4 ? 3u : 1u)) == 0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int vi = u * kThreads + threadIdx.x;
    uint32_t xb[VEC], w[VEC / 4];
    unpack<DT>(v[u], xb);
    uint32_t m = 0;
    u16x2 h[4];
    if constexpr (DT == NC_BF16) {               // packed 16-bit magnitudes (see count16)
      h[0] = mag16(v[u].x); h[1] = mag16(v[u].y); h[2] = mag16(v[u].z); h[3] = mag16(v[u].w);
      const u16x2 hm = __builtin_elementwise_max(__builtin_elementwise_max(h[0], h[1]),
                                                 __builtin_elementwise_max(h[2], h[3]));
      m = (uint32_t)max(hm.x, hm.y) << 16;
    } else {
#pragma unroll
      for (int i = 0; i < VEC; ++i) m = max(m, xb[i] & kAbsMask);
    }
    const bool clean = __ballot(m > kMaxFinite) == 0;   // wave-uniform
    if (!clean) {                                       // finite amax, count non-finite
      m = 0;
#pragma unroll
      for (int i = 0; i < VEC; ++i) m = max(m, finite_mag(xb[i] & kAbsMask, acc));
    }
    acc.amax = max(acc.amax, m);
    const uint32_t gm = group_max<GROUP>(m);
    // exponent-field arithmetic unless some block of the wave has an amax
    // below 2^-94 or above 2^127 (wave-uniform)
    const MxBlock blk = __ballot(!mx_fast_ok(gm)) == 0 ? mx_block_fast<FMT, RULE>(gm) : mx_block<FMT, RULE>(gm);
    const int X = blk.sb - 127;
    CastParams p;
    p.K = -X;
    p.t_clip = blk.t_clip;
    p.t_uf = blk.t_uf;
    // scaled converts divide by the block's scale 2^X
#pragma unroll
    for (int j = 0; j < VEC / 4; ++j) w[j] = scvt4<FMT, DT, CLIPS>(v[u], j, blk.scale);
    if constexpr (DT == NC_BF16) {
      const u16x2 tc = splat16(p.t_clip), tu = splat16(p.t_uf);
#pragma unroll
      for (int j = 0; j < 4; ++j) count16<CLIPS>(h[j], tc, tu, acc);
    } else {
#pragma unroll
      for (int i = 0; i < VEC; ++i) count_elem<CLIPS>(xb[i] & kAbsMask, p, acc);
    }
    if (!clean) {
#pragma unroll
      for (int j = 0; j < VEC / 4; ++j) w[j] = fix_nonfinite4<FMT>(w[j], xb + 4 * j);
    }
    if constexpr (STATS) {
      uint32_t q[VEC];
#pragma unroll
      for (int i = 0; i < VEC; ++i) q[i] = (w[i / 4] >> (8 * (i % 4))) & 0xFFu;
      if (clean) stats_vec<VEC, true, true>(xb, q, tab, pow2_f64(X), sa);
      else stats_vec<VEC, true, false>(xb, q, tab, pow2_f64(X), sa);
    }
    if (FULL || vi * VEC < rem) {
      if constexpr (DT == NC_F32) st_stream(reinterpret_cast<uint32_t*>(dst) + vi, w[0]);
      else st_stream(reinterpret_cast<u32x2*>(dst) + vi, u32x2{w[0], w[1]});
      const uint32_t sb = (uint32_t)blk.sb;
      if (FULL && sc_word) {
        // a 16-lane row holds 16 / GROUP whole blocks: each lane shifts its
        // block's scale byte to that block's place in the row's word, and
        // DPP row shifts OR them into the row's first lane, which stores the
        // word (vi is a multiple of 16 there)
        const uint32_t placed = sb << (8 * ((threadIdx.x / GROUP) & (16 / GROUP - 1)));
        if constexpr (GROUP == 4) {
          const uint32_t b8 = placed | dpp_u32<0x108>(placed);   // row_shl:8
          const uint32_t b4 = b8 | dpp_u32<0x104>(b8);            // row_shl:4
          if ((threadIdx.x & 15) == 0) reinterpret_cast<uint32_t*>(sdst)[vi / 16] = b4;
        } else {
          const uint32_t b2 = placed | dpp_u32<0x108>(placed);
          if ((threadIdx.x & 15) == 0) reinterpret_cast<uint16_t*>(sdst)[vi / 16] = (uint16_t)b2;
        }
      } else {
        // every lane of the block holds the same X: all store it (same byte,
        // same value), which keeps the tile free of divergent branches
        sdst[vi / GROUP] = (uint8_t)sb;
      }
    }
    __builtin_amdgcn_sched_barrier(0);   // keep each vector's ballots short-lived
  }
}

template <int FMT, int DT, int RULE, bool STATS>
NC_STREAM_KERNEL
k_cast_mx(const SegBatch b, const Tail t) {
  constexpr int VEC = In<DT>::VEC;
  constexpr int U = cast_vecs<STATS>();
  constexpr int64_t TILE = (int64_t)kThreads * VEC * U;
  __shared__ uint32_t lds[kRows * 4];
  __shared__ double lds_st[STATS ? kStatLds : 1];
  __shared__ double tab[STATS ? 256 : 1];
  const int64_t tile = xcd_tile<256>();
  const int s = seg_of_scan(b.tile0, b.count, tile);
  const Seg& g = b.s[s];
  const int64_t e0 = (tile - b.tile0[s]) * TILE;
  const int rem = tile_len<TILE>(b, s, tile);      // a multiple of 32
  const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(g.x) + e0 * In<DT>::BYTES);
  // loads first (a ragged tile: lanes past the end hold zeros); the table
  // fill overlaps them
  u32x4 v[U];
  const bool full = rem == (int)TILE;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int vi = u * kThreads + threadIdx.x;
    v[u] = (full || vi * VEC < rem) ? ld_stream(src + vi) : u32x4{0u, 0u, 0u, 0u};
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (STATS) {
    fill_stat_table<FMT>(tab, 0);
    __syncthreads();
  }
  Acc acc;
  acc.reset();
  StatAcc sa;
  if constexpr (STATS) sa.reset();
  if (full) mx_tile<FMT, DT, RULE, STATS, true, U>(g, e0, rem, v, acc, sa, tab);
  else mx_tile<FMT, DT, RULE, STATS, false, U>(g, e0, rem, v, acc, sa, tab);
  if constexpr (!mx_rule_clips(RULE)) acc.no_clips();
  if constexpr (STATS) write_count_stat_slots(acc, sa, t.cnt1 + tile, t.st1 + tile * 6, lds, lds_st);
  else flush_counts(acc, b, s, tile, t, lds);
}

// ---------------------------------------------------------------------------
// MX with blocks down the columns (32 consecutive rows of one column share
// X): the layout of an operand consumed transposed.  A slot (col_slot) is
// VC = 8 / BYTES adjacent columns of a 32-row band, 8 input bytes per row;
// SPLIT adjacent lanes share it (two for bf16), each loading 32 / SPLIT of
// its rows.  Each lane takes its columns' finite max over its rows in
// registers, the lanes of a slot exchange theirs by one DPP swap, and each
// casts and stores its own rows.
template <int FMT, int DT, int RULE, bool STATS>
NC_STREAM_KERNEL
k_cast_mx_col(const SegBatch b, const Tail t) {
  constexpr int VC = kColBytes / In<DT>::BYTES;    // 4 bf16 or 2 fp32 columns
  constexpr int SPLIT = col_cast_split(DT), RL = 32 / SPLIT, SLOTS = kThreads / SPLIT;
  static_assert(SPLIT == 1 || SPLIT == 2, "lanes per slot");
  __shared__ uint32_t lds[kRows * 4];
  __shared__ double lds_st[STATS ? kStatLds : 1];
  __shared__ double tab[STATS ? 256 : 1];
  const int64_t tile = xcd_tile<1>();
  const int s = seg_of(b.tile0, b.count, tile);
  const Seg& g = b.s[s];
  const int rem = tile_len<SLOTS>(b, s, tile);                 // slots in this tile
  const uint32_t slot = threadIdx.x / SPLIT, part = threadIdx.x % SPLIT;
  const ColSlot cs = col_slot_at<VC>(g, (uint32_t)(tile - b.tile0[s]) * SLOTS + slot, (int)slot < rem);
  const int64_t cols = g.cols;
  const int64_t stride = cols * In<DT>::BYTES;
  const int64_t r0 = (int64_t)part * RL;                       // this lane's first row of the band
  const uint8_t* src = static_cast<const uint8_t*>(g.x) + (cs.e0 + r0 * cols) * In<DT>::BYTES;
  u32x2 v[RL];
#pragma unroll
  for (int r = 0; r < RL; ++r) v[r] = ld_stream(reinterpret_cast<const u32x2*>(src + r * stride));
  __builtin_amdgcn_sched_barrier(0);
  if (rem < SLOTS && !cs.act) {             // the tensor's last tile: idle lanes hold zeros
#pragma unroll
    for (int r = 0; r < RL; ++r) v[r] = u32x2{0u, 0u};
  }
  if constexpr (STATS) {
    fill_stat_table<FMT>(tab, 0);
    __syncthreads();
  }
  Acc acc;
  acc.reset();
  // per-column max of |x| bits (an idle lane holds zeros: X = -127, no
  // counts).  Formed on the packed words with operations of its own -- bf16
  // magnitudes by packed 16-bit max, fp32 magnitudes as x << 1 -- so the
  // compiler keeps no unpacked copy of the rows alive into the cast loop.
  uint32_t m[VC], mall = 0;
  if constexpr (DT == NC_BF16) {
    u16x2 mx = {0, 0}, my = {0, 0};
#pragma unroll
    for (int r = 0; r < RL; ++r) {
      mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, v[r].x & 0x7FFF7FFFu));
      my = __builtin_elementwise_max(my, __builtin_bit_cast(u16x2, v[r].y & 0x7FFF7FFFu));
    }
    m[0] = (uint32_t)mx.x << 16; m[1] = (uint32_t)mx.y << 16;
    m[2] = (uint32_t)my.x << 16; m[3] = (uint32_t)my.y << 16;
  } else {
    uint32_t m2[2] = {0u, 0u};
#pragma unroll
    for (int r = 0; r < RL; ++r) {
      m2[0] = max(m2[0], v[r].x << 1);
      m2[1] = max(m2[1], v[r].y << 1);
    }
    m[0] = m2[0] >> 1; m[1] = m2[1] >> 1;
  }
#pragma unroll
  for (int i = 0; i < VC; ++i) mall = max(mall, m[i]);
  const bool clean = __ballot(mall > kMaxFinite) == 0;   // wave-uniform
  if (!clean) {                                          // finite max, count non-finite
#pragma unroll
    for (int i = 0; i < VC; ++i) m[i] = 0;
#pragma unroll
    for (int r = 0; r < RL; ++r) {
      uint32_t xb[VC];
      unpack8<DT>(v[r], xb);
#pragma unroll
      for (int i = 0; i < VC; ++i) m[i] = max(m[i], finite_mag(xb[i] & kAbsMask, acc));
    }
  }
  if constexpr (SPLIT == 2) {                            // the partner lane's rows: quad_perm [1,0,3,2]
#pragma unroll
    for (int i = 0; i < VC; ++i) m[i] = max(m[i], dpp_u32<0xB1>(m[i]));
  }
  int X[VC];
  CastParams p[VC];
#pragma unroll
  for (int i = 0; i < VC; ++i) {
    acc.amax = max(acc.amax, m[i]);
    X[i] = mx_exponent<FMT, RULE>(m[i]);
    p[i] = cast_params<FMT>(-X[i]);
  }
  StatAcc sa;
  if constexpr (STATS) sa.reset();
  uint8_t* dst = g.codes + cs.e0 + r0 * cols;
#pragma unroll
  for (int r = 0; r < RL; ++r) {
    // the row's words pass through an empty asm: values derived from them
    // above (the non-finite path) cannot be hoisted and held for this loop
    u32x2 vr = v[r];
    __asm__ volatile("" : "+v"(vr));
    uint32_t xb[VC];
    unpack8<DT>(vr, xb);
    float y[VC];
#pragma unroll
    for (int i = 0; i < VC; ++i) y[i] = __builtin_amdgcn_ldexpf(__uint_as_float(xb[i]), p[i].K);
    int wi = cvt_pair<FMT, false>(y[0], y[1], 0);
    if constexpr (VC == 4) wi = cvt_pair<FMT, true>(y[2], y[3], wi);
    uint32_t w = mx_rule_clips(RULE) ? sat4<FMT>((uint32_t)wi) : (uint32_t)wi;
#pragma unroll
    for (int i = 0; i < VC; ++i) count_elem<mx_rule_clips(RULE)>(xb[i] & kAbsMask, p[i], acc);
    if (!clean) {
#pragma unroll
      for (int i = 0; i < VC; ++i)
        if ((xb[i] & kAbsMask) > kMaxFinite)
          w = (w & ~(0xFFu << (8 * i))) | (nonfinite_code<FMT>(xb[i]) << (8 * i));
    }
    if constexpr (STATS) {
#pragma unroll
      for (int i = 0; i < VC; ++i) {
        if (!clean && (xb[i] & kAbsMask) > kMaxFinite) continue;
        stat_term_blk((double)__uint_as_float(xb[i]), tab[(w >> (8 * i)) & 0xFFu], pow2_f64(X[i]), sa);
      }
    }
    // the row's counts are taken here: left alone, the compiler sinks every
    // compare to the end of the loop and keeps all the rows' magnitudes live
    __asm__ volatile("" : "+v"(acc.n_big), "+v"(acc.n_uf));
    __builtin_amdgcn_sched_barrier(0);   // one row at a time (register pressure)
    if (cs.act) {
      uint8_t* d = dst + r * stride / In<DT>::BYTES;
      if constexpr (VC == 4) st_stream(reinterpret_cast<uint32_t*>(d), w);
      else __builtin_nontemporal_store((uint16_t)w, reinterpret_cast<uint16_t*>(d));
    }
  }
  if (cs.act && part == 0) {
    uint8_t* sd = g.scales + cs.sc;
    uint32_t sb = 0;
#pragma unroll
    for (int i = 0; i < VC; ++i) sb |= (uint32_t)(X[i] + 127) << (8 * i);
    // one word per slot when the scale array allows it (wave-uniform)
    if (((uintptr_t)g.scales & (VC - 1)) == 0) {
      if constexpr (VC == 4) *reinterpret_cast<uint32_t*>(sd) = sb;
      else *reinterpret_cast<uint16_t*>(sd) = (uint16_t)sb;
    } else {
#pragma unroll
      for (int i = 0; i < VC; ++i) sd[i] = (uint8_t)(sb >> (8 * i));
    }
  }
  if constexpr (!mx_rule_clips(RULE)) acc.no_clips();
  if constexpr (STATS) write_count_stat_slots(acc, sa, t.cnt1 + tile, t.st1 + tile * 6, lds, lds_st);
  else flush_counts(acc, b, s, tile, t, lds);
}

template <int FMT, int DT>
hipError_t cast_pt_t(const SegBatch& b, const nc_scale_state* st, const nc_loss_scale* ls, bool stats,
                     const Tail& t, const Launch& l) {
  if (stats)
    hipLaunchKernelGGL((k_cast_pt<FMT, DT, true>), dim3((uint32_t)l.grid), dim3(kThreads), 0, l.stream, b, st, ls, t);
  else
    hipLaunchKernelGGL((k_cast_pt<FMT, DT, false>), dim3((uint32_t)l.grid), dim3(kThreads), 0, l.stream, b, st, ls, t);
  return hipGetLastError();
}

template <int FMT, int DT, int RULE>
hipError_t cast_mx_r(const SegBatch& b, bool stats, const Tail& t, const Launch& l) {
  if (stats)
    hipLaunchKernelGGL((k_cast_mx<FMT, DT, RULE, true>), dim3((uint32_t)l.grid), dim3(kThreads), 0, l.stream, b, t);
  else
    hipLaunchKernelGGL((k_cast_mx<FMT, DT, RULE, false>), dim3((uint32_t)l.grid), dim3(kThreads), 0, l.stream, b, t);
  return hipGetLastError();
}

template <int FMT, int DT>
hipError_t cast_mx_t(const SegBatch& b, int rule, bool stats, const Tail& t, const Launch& l) {
  if (rule == NC_MX_OCP) return cast_mx_r<FMT, DT, NC_MX_OCP>(b, stats, t, l);
  if (rule == NC_MX_PLUS1) return cast_mx_r<FMT, DT, NC_MX_PLUS1>(b, stats, t, l);
  return cast_mx_r<FMT, DT, NC_MX_CEIL>(b, stats, t, l);
}

template <int FMT, int DT>
hipError_t cast_sr_t(const SegBatch& b, const nc_scale_state* st, const nc_loss_scale* ls, uint64_t seed,
                     uint64_t offset, const Tail& t, const Launch& l) {
  hipLaunchKernelGGL((k_cast_sr<FMT, DT>), dim3((uint32_t)l.grid), dim3(kThreads), 0, l.stream, b, st, ls, seed,
                     offset, t);
  return hipGetLastError();
}

template <int FMT, int DT, int RULE>
hipError_t cast_mx_col_r(const SegBatch& b, bool stats, const Tail& t, const Launch& l) {
  if (stats)
    hipLaunchKernelGGL((k_cast_mx_col<FMT, DT, RULE, true>), dim3((uint32_t)l.grid), dim3(kThreads), 0, l.stream,
                       b, t);
  else
    hipLaunchKernelGGL((k_cast_mx_col<FMT, DT, RULE, false>), dim3((uint32_t)l.grid), dim3(kThreads), 0, l.stream,
                       b, t);
  return hipGetLastError();
}

template <int FMT, int DT>
hipError_t cast_mx_col_t(const SegBatch& b, int rule, bool stats, const Tail& t, const Launch& l) {
  if (rule == NC_MX_OCP) return cast_mx_col_r<FMT, DT, NC_MX_OCP>(b, stats, t, l);
  if (rule == NC_MX_PLUS1) return cast_mx_col_r<FMT, DT, NC_MX_PLUS1>(b, stats, t, l);
  return cast_mx_col_r<FMT, DT, NC_MX_CEIL>(b, stats, t, l);
}

}  // namespace

hipError_t launch_amax(const SegBatch& b, int dtype, const Tail& t, const Launch& l) {
  if (dtype == NC_F32)
    hipLaunchKernelGGL((k_amax<NC_F32>), dim3((uint32_t)l.grid), dim3(kThreads), 0, l.stream, b, t);
  else
    hipLaunchKernelGGL((k_amax<NC_BF16>), dim3((uint32_t)l.grid), dim3(kThreads), 0, l.stream, b, t);
  return hipGetLastError();
}

hipError_t launch_cast_pt(const SegBatch& b, int dtype, int fmt, const nc_scale_state* st,
                          const nc_loss_scale* ls, bool stats, const Tail& t, const Launch& l) {
  if (fmt == NC_E4M3)
    return dtype == NC_F32 ? cast_pt_t<NC_E4M3, NC_F32>(b, st, ls, stats, t, l)
                           : cast_pt_t<NC_E4M3, NC_BF16>(b, st, ls, stats, t, l);
  return dtype == NC_F32 ? cast_pt_t<NC_E5M2, NC_F32>(b, st, ls, stats, t, l)
                         : cast_pt_t<NC_E5M2, NC_BF16>(b, st, ls, stats, t, l);
}

hipError_t launch_cast_mx(const SegBatch& b, int dtype, int fmt, int rule, bool stats, const Tail& t,
                          const Launch& l) {
  if (fmt == NC_E4M3)
    return dtype == NC_F32 ? cast_mx_t<NC_E4M3, NC_F32>(b, rule, stats, t, l)
                           : cast_mx_t<NC_E4M3, NC_BF16>(b, rule, stats, t, l);
  return dtype == NC_F32 ? cast_mx_t<NC_E5M2, NC_F32>(b, rule, stats, t, l)
                         : cast_mx_t<NC_E5M2, NC_BF16>(b, rule, stats, t, l);
}

hipError_t launch_cast_mx_col(const SegBatch& b, int dtype, int fmt, int rule, bool stats, const Tail& t,
                              const Launch& l) {
  if (fmt == NC_E4M3)
    return dtype == NC_F32 ? cast_mx_col_t<NC_E4M3, NC_F32>(b, rule, stats, t, l)
                           : cast_mx_col_t<NC_E4M3, NC_BF16>(b, rule, stats, t, l);
  return dtype == NC_F32 ? cast_mx_col_t<NC_E5M2, NC_F32>(b, rule, stats, t, l)
                         : cast_mx_col_t<NC_E5M2, NC_BF16>(b, rule, stats, t, l);
}

hipError_t launch_cast_sr(const SegBatch& b, int dtype, int fmt, const nc_scale_state* st,
                          const nc_loss_scale* ls, uint64_t seed, uint64_t offset, const Tail& t, const Launch& l) {
  if (fmt == NC_E4M3)
    return dtype == NC_F32 ? cast_sr_t<NC_E4M3, NC_F32>(b, st, ls, seed, offset, t, l)
                           : cast_sr_t<NC_E4M3, NC_BF16>(b, st, ls, seed, offset, t, l);
  return dtype == NC_F32 ? cast_sr_t<NC_E5M2, NC_F32>(b, st, ls, seed, offset, t, l)
                         : cast_sr_t<NC_E5M2, NC_BF16>(b, st, ls, seed, offset, t, l);
}

}  // namespace nc
