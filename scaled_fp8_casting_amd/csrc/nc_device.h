// Device-side building blocks of libnarrowcast for CDNA4 (gfx950).
//
// The cast of an input x at exponent K (the value quantised is y = x * 2^K,
// formed exactly) is round-to-nearest-even onto the FP8 grid, saturating at
// the largest finite value ([MP-card, item (3)]: E4M3 max 448, E5M2 max
// 57344).  On gfx950 it runs as:
//
//  1. y = ldexp(x, K) in fp32.  Exact whenever y is at least fp32's smallest
//     normal and not above fp32's range.  Outside that: a y above range is a
//     clip (saturated in step 3); a y below 2^-126 is far below half the
//     smallest FP8 subnormal, so its code is zero however it rounds.
//  2. The hardware pair convert (v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32) rounds
//     y to nearest even.  Measured against the exact definition over all 2^32
//     fp32 patterns it agrees on every finite y with |y| <= max -- normals,
//     subnormals, ties and signed zeros -- and differs only where y is out of
//     range (E4M3 gives the NaN code S.1111.111, E5M2 gives Inf) or not a
//     number.
//  3. Saturation, on four packed codes at once: a byte whose low seven bits
//     are the overflow code (E4M3 0x7F, E5M2 0x7C) is decremented to the
//     largest finite code of the same sign; no in-range result has those
//     bits, so nothing else changes.
//  4. Inputs that are Inf/NaN are rare: a wave whose current vector holds any
//     takes a uniform branch that rewrites their codes (NaN -> 0x7F, +-Inf ->
//     +-max) and masks them out of the amax.
//  5. Clip, underflow and non-finite are decided on |x|'s bit pattern against
//     per-scale thresholds (exact comparisons on the input, never on the
//     fp32 product) and counted per lane.
//
// Sources cited by title and section: [MP-card] "Mixed Precision
// FP16/BF16/FP8", [Drift] "what actually breaks low precision training",
// [E3] practice exercise c06/E3 "Worked solution", [MaxWin] "Max-Window
// Scale Estimation for Near-Lossless HiF8 W8A8 Quantization-Aware Training".
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "narrowcast.h"

namespace nc {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// Input element types: elements per 16-byte vector, bytes per element.
template <int DT> struct In;
template <> struct In<NC_F32> { static constexpr int VEC = 4, BYTES = 4; };
template <> struct In<NC_BF16> { static constexpr int VEC = 8, BYTES = 2; };

constexpr int kThreads = 256;       // 4 wave64s per workgroup
constexpr int kMaxSeg = 64;         // tensors per launch (descriptors travel as kernel arguments)
constexpr int kWaves = kThreads / 64;
constexpr int kChunk = 1024;        // per-workgroup slots summed by one workgroup of the first reduction

// Work distribution.  Every streaming kernel gives each workgroup ONE small
// tile (a few KiB of input) and launches as many workgroups as there are
// tiles: the hardware then keeps a compact window of addresses in flight,
// which on MI355X sustains far more HBM bandwidth for mixed read/write
// streams than a persistent grid striding over the tensor (measured: a
// cast-shaped stream 82% of peak vs 72%, a dequant-shaped one 81% vs 69%).
// Each workgroup writes its partial results (counts, amax, statistics) to
// its own workspace slot (one same-address atomic per workgroup would
// serialise); a small kernel then sums each chunk of slots, adding the
// counts into the caller's and the statistics in a fixed order (through a
// second small kernel for a tensor of several chunks).
#define NC_STREAM_KERNEL __global__ void __launch_bounds__(nc::kThreads)

// ---------------------------------------------------------------------------
// Formats.  E4M3: bias 7, no Inf, S.1111.111 is NaN, max 1.75*2^8 = 448.
// E5M2: bias 15, IEEE specials, max 1.75*2^15 = 57344.  Both maxima are
// 1.75 * 2^EMAX.
template <int FMT> struct Fp8;
template <> struct Fp8<NC_E4M3> {
  static constexpr int MB = 3, BIAS = 7, EMIN = -6, EMAX = 8;
  static constexpr uint32_t MAXCODE = 0x7E;
};
template <> struct Fp8<NC_E5M2> {
  static constexpr int MB = 2, BIAS = 15, EMIN = -14, EMAX = 15;
  static constexpr uint32_t MAXCODE = 0x7B;
};

constexpr uint32_t kAbsMask = 0x7FFFFFFFu;
constexpr uint32_t kMaxFinite = 0x7F7FFFFFu;   // |x| bits above this: Inf/NaN
constexpr uint32_t kInfBits = 0x7F800000u;     // |x| bits above this: NaN
constexpr uint32_t kNaNCode = 0x7Fu;

// Largest fp32 pattern whose value is <= 1.75 * 2^j (the clip bound at
// exponent K is 1.75 * 2^(EMAX - K)).
// Written without branches (selects only): it runs per lane per MX block.
__host__ __device__ inline uint32_t clip_threshold(int j) {
  const uint32_t normal = ((uint32_t)(j + 127) << 23) | 0x600000u;   // j in [-126, 127]
  // subnormal range: 1.75 * 2^j = 7 * 2^(j + 147) units of 2^-149
  const int up = j + 147;
  const uint32_t left = 7u << (up < 0 ? 0 : (up > 20 ? 20 : up));
  const uint32_t right = 7u >> (up >= 0 ? 0 : (-up > 3 ? 3 : -up));
  const uint32_t sub = up >= 0 ? left : right;
  return j > 127 ? kMaxFinite : (j >= -126 ? normal : sub);
}

// Largest fp32 pattern whose value is <= 2^j (the underflow bound at
// exponent K is half the smallest subnormal: 2^(EMIN - MB - 1 - K)).
__host__ __device__ inline uint32_t pow2_threshold(int j) {
  const uint32_t normal = (uint32_t)(j + 127) << 23;
  const int sh = j + 149;
  const uint32_t sub = sh < 0 ? 0u : (1u << (sh > 31 ? 31 : sh));
  return j > 127 ? kMaxFinite : (j >= -126 ? normal : sub);
}

// Thresholds of a cast at exponent K.
struct CastParams {
  int K;
  uint32_t t_clip;  // finite |x| bits > t_clip  <=>  |x| * 2^K > max
  uint32_t t_uf;    // 0 < |x| bits <= t_uf      <=>  rounds to a zero code
};

template <int FMT>
__host__ __device__ inline CastParams cast_params(int K) {
  using F = Fp8<FMT>;
  CastParams p;
  p.K = K;
  p.t_clip = clip_threshold(F::EMAX - K);
  p.t_uf = pow2_threshold(F::EMIN - F::MB - 1 - K);
  return p;
}

// Per-lane running totals: each lane counts its own elements (a compare
// and an add per count, no scalar traffic); the workgroup reduces them into
// its slot.  A workgroup handles at most a few thousand elements.
struct Acc {
  uint32_t n_nf;     // non-finite elements
  uint32_t n_big;    // |x| bits above t_clip: every clip plus every non-finite
  uint32_t n_uf;
  uint32_t amax;     // largest finite |x| bits
  u16x2 big16, uf16; // the bf16 paths' packed per-half counters (wave_counts adds them in)
  __device__ void reset() {
    n_nf = n_big = n_uf = 0;
    amax = 0;
    big16 = u16x2{0, 0};
    uf16 = u16x2{0, 0};
  }
  // Without clip counting (CLIPS = false) n_big must still hold the
  // non-finite elements, which the slot reduction subtracts from it.
  __device__ void no_clips() { n_big = n_nf; }
};

// bf16 inputs, two per 32-bit word: the magnitude, clip and underflow tests
// on packed 16-bit halves.  A bf16 x has fp32 bits X << 16, so |x| bits >
// t_clip <=> X > t_clip >> 16, and 0 < |x| bits <= t_uf <=> 1 <= X <=
// t_uf >> 16 (integer thresholds, exact).  Counts: saturating subtract,
// clamp to 1, packed add; each half counts at most a few dozen elements per
// tile, far below 2^16.
__device__ __forceinline__ u16x2 mag16(uint32_t w) { return __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu); }
// [a > b] per 16-bit half: min(max(a - b, 0), 1) -- v_pk_sub_u16 with clamp,
// then v_pk_min_u16 against 1 in both halves (a register operand: an inline
// constant reaches the low half only).  Written as asm: the compiler
// otherwise turns it into a compare, a select and a repack per half.
__device__ __forceinline__ u16x2 gt16(u16x2 a, u16x2 b) {
  uint32_t r;
  __asm__("v_pk_sub_u16 %0, %1, %2 clamp\n\tv_pk_min_u16 %0, %0, %3"
          : "=&v"(r) : "v"(__builtin_bit_cast(uint32_t, a)), "v"(__builtin_bit_cast(uint32_t, b)),
            "v"(0x00010001u));
  return __builtin_bit_cast(u16x2, r);
}
// CLIPS = false: the caller knows no finite element exceeds the clip bound
// (the MX rules with headroom), so only underflows are counted.
template <bool CLIPS = true>
__device__ __forceinline__ void count16(u16x2 h, u16x2 tc, u16x2 tu, Acc& acc) {
  const u16x2 one = {1, 1};
  if constexpr (CLIPS) acc.big16 += gt16(h, tc);   // |x| > t_clip
  acc.uf16 += gt16(tu, h - one);                   // 1 <= |x| <= t_uf (h = 0 wraps to 0xFFFF)
}
__device__ __forceinline__ u16x2 splat16(uint32_t t) {
  const uint16_t v = (uint16_t)(t >> 16);
  return u16x2{v, v};
}

// |x| bits with Inf/NaN mapped to 0 (for the amax), counting non-finite
// elements.
__device__ __forceinline__ uint32_t finite_mag(uint32_t ax, Acc& acc) {
  const bool nf = ax > kMaxFinite;
  acc.n_nf += nf ? 1u : 0u;
  return nf ? 0u : ax;
}

// Saturation of four packed codes (step 3).
template <int FMT>
__device__ __forceinline__ uint32_t sat4(uint32_t w) {
  // (low 7 bits) + (0x80 - overflow code) reaches bit 7 exactly for the
  // overflow code and the codes above it (NaN codes, absent here)
  constexpr uint32_t kBump = FMT == NC_E4M3 ? 0x01010101u : 0x04040404u;
  const uint32_t t = ((w & 0x7F7F7F7Fu) + kBump) & 0x80808080u;
  return w - (t >> 7);
}

// Two fp32 values -> two codes in the low (HI = false) or high (HI = true)
// half of `old`.
template <int FMT, bool HI>
__device__ __forceinline__ int cvt_pair(float a, float b, int old) {
  if constexpr (FMT == NC_E4M3) return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
  else return __builtin_amdgcn_cvt_pk_bf8_f32(a, b, old, HI);
}

// Four elements (fp32 patterns) at exponent K -> four codes, byte i =
// element i, saturated (steps 1-3).  Exact for every finite input.
template <int FMT>
__device__ __forceinline__ uint32_t cvt4(const uint32_t* xb, int K) {
  const float y0 = __builtin_amdgcn_ldexpf(__uint_as_float(xb[0]), K);
  const float y1 = __builtin_amdgcn_ldexpf(__uint_as_float(xb[1]), K);
  const float y2 = __builtin_amdgcn_ldexpf(__uint_as_float(xb[2]), K);
  const float y3 = __builtin_amdgcn_ldexpf(__uint_as_float(xb[3]), K);
  int w = cvt_pair<FMT, false>(y0, y1, 0);
  w = cvt_pair<FMT, true>(y2, y3, w);
  return sat4<FMT>((uint32_t)w);
}

// One element -> its code (for ragged tails), saturated.
template <int FMT>
__device__ __forceinline__ uint32_t cvt1(uint32_t xb, int K) {
  const float y = __builtin_amdgcn_ldexpf(__uint_as_float(xb), K);
  return sat4<FMT>((uint32_t)cvt_pair<FMT, false>(y, 0.0f, 0) & 0xFFu);
}

// gfx950's scaled converts (v_cvt_scalef32_pk_{fp8,bf8}_{bf16,f32}): two
// elements -> the codes of RNE(x / scale) in half HI of `old`.  Measured
// against the exact definition for every bf16 pattern, and for random and
// grid-midpoint fp32 values, at every scale 2^j, j in [-127, 127]: identical
// to steps 1-2 above on every finite in-range input; out of range and
// non-finite inputs give the same overflow/NaN codes, which steps 3-4 fix.
// bf16 pairs convert straight from the packed input word (no unpacking).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x2_t __attribute__((ext_vector_type(2)));

template <int FMT, bool HI>
__device__ __forceinline__ uint32_t scvt_bf16(uint32_t pair, float scale, uint32_t old) {
  const bf16x2_t x = __builtin_bit_cast(bf16x2_t, pair);
  const s16x2_t o = __builtin_bit_cast(s16x2_t, old);
  if constexpr (FMT == NC_E4M3) return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o, x, scale, HI));
  else return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(o, x, scale, HI));
}
template <int FMT, bool HI>
__device__ __forceinline__ uint32_t scvt_f32(uint32_t a, uint32_t b, float scale, uint32_t old) {
  const s16x2_t o = __builtin_bit_cast(s16x2_t, old);
  if constexpr (FMT == NC_E4M3)
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, __uint_as_float(a), __uint_as_float(b), scale, HI));
  else
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(o, __uint_as_float(a), __uint_as_float(b), scale, HI));
}

// Four elements of an input vector -> four codes (byte i = element i),
// saturated: the scaled-convert form of cvt4 (x * 2^K with scale = 2^-K).
// j: which group of four (bf16: words 2j, 2j+1 of the vector; fp32: the
// whole vector).
// SAT = false: no element can round above the largest finite value (the MX
// rules with headroom), so the codes need no saturation.
template <int FMT, int DT, bool SAT = true>
__device__ __forceinline__ uint32_t scvt4(const u32x4& v, int j, float scale) {
  uint32_t w;
  if constexpr (DT == NC_BF16) {
    const uint32_t lo = j == 0 ? v.x : v.z, hi = j == 0 ? v.y : v.w;
    w = scvt_bf16<FMT, false>(lo, scale, 0u);
    w = scvt_bf16<FMT, true>(hi, scale, w);
  } else {
    w = scvt_f32<FMT, false>(v.x, v.y, scale, 0u);
    w = scvt_f32<FMT, true>(v.z, v.w, scale, w);
  }
  return SAT ? sat4<FMT>(w) : w;
}

// Code of a non-finite element (step 4): NaN -> 0x7F, +-Inf -> +-max.
template <int FMT>
__device__ __forceinline__ uint32_t nonfinite_code(uint32_t xb) {
  return (xb & kAbsMask) > kInfBits ? kNaNCode : (((xb >> 24) & 0x80u) | Fp8<FMT>::MAXCODE);
}

// Step 4 on a packed word of four codes of elements xb[0..3].
template <int FMT>
__device__ inline uint32_t fix_nonfinite4(uint32_t w, const uint32_t* xb) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if ((xb[i] & kAbsMask) > kMaxFinite)
      w = (w & ~(0xFFu << (8 * i))) | (nonfinite_code<FMT>(xb[i]) << (8 * i));
  return w;
}

// Clip and underflow counts of one element (step 5).  Clip counts include
// every non-finite element (Acc::n_big); the flush subtracts them.
template <bool CLIPS = true>
__device__ __forceinline__ void count_elem(uint32_t ax, const CastParams& p, Acc& acc) {
  if constexpr (CLIPS) acc.n_big += (ax > p.t_clip) ? 1u : 0u;
  acc.n_uf += ((ax - 1u) < p.t_uf) ? 1u : 0u;
}

// Cast one input vector (VEC elements, unpacked in xb) at one exponent into
// VEC/4 packed words; counts and the finite amax go to acc.  SCALED: the
// scaled converts with scale = 2^-K (|K| <= 127), else ldexp + convert.
// Returns the wave-uniform "no Inf/NaN in this vector anywhere in the wave".
template <int FMT, int DT, bool SCALED>
__device__ __forceinline__ bool cast_vec(const u32x4& v, const uint32_t* xb, const CastParams& p, float scale,
                                         Acc& acc, uint32_t* w) {
  constexpr int VEC = In<DT>::VEC;
  if constexpr (DT == NC_BF16 && SCALED) {
    // packed 16-bit magnitudes: max and counts without unpacking
    const u16x2 h0 = mag16(v.x), h1 = mag16(v.y), h2 = mag16(v.z), h3 = mag16(v.w);
    const u16x2 hm = __builtin_elementwise_max(__builtin_elementwise_max(h0, h1), __builtin_elementwise_max(h2, h3));
    const uint32_t m = (uint32_t)max(hm.x, hm.y) << 16;
    w[0] = scvt4<FMT, DT>(v, 0, scale);
    w[1] = scvt4<FMT, DT>(v, 1, scale);
    const u16x2 tc = splat16(p.t_clip), tu = splat16(p.t_uf);
    count16(h0, tc, tu, acc);
    count16(h1, tc, tu, acc);
    count16(h2, tc, tu, acc);
    count16(h3, tc, tu, acc);
    if (__ballot(m > kMaxFinite) == 0) {      // wave-uniform: no Inf/NaN here
      acc.amax = max(acc.amax, m);
      return true;
    }
    uint32_t mf = 0;
#pragma unroll
    for (int i = 0; i < VEC; ++i) mf = max(mf, finite_mag(xb[i] & kAbsMask, acc));
    acc.amax = max(acc.amax, mf);
#pragma unroll
    for (int j = 0; j < VEC / 4; ++j) w[j] = fix_nonfinite4<FMT>(w[j], xb + 4 * j);
    return false;
  }
  uint32_t ax[VEC];
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < VEC; ++i) {
    ax[i] = xb[i] & kAbsMask;
    m = max(m, ax[i]);
  }
#pragma unroll
  for (int j = 0; j < VEC / 4; ++j) w[j] = SCALED ? scvt4<FMT, DT>(v, j, scale) : cvt4<FMT>(xb + 4 * j, p.K);
#pragma unroll
  for (int i = 0; i < VEC; ++i) count_elem(ax[i], p, acc);
  if (__ballot(m > kMaxFinite) == 0) {        // wave-uniform: no Inf/NaN here
    acc.amax = max(acc.amax, m);
    return true;
  }
  uint32_t mf = 0;
#pragma unroll
  for (int i = 0; i < VEC; ++i) mf = max(mf, finite_mag(ax[i], acc));
  acc.amax = max(acc.amax, mf);
#pragma unroll
  for (int j = 0; j < VEC / 4; ++j) w[j] = fix_nonfinite4<FMT>(w[j], xb + 4 * j);
  return false;
}

// One element (ragged tails): its code; counts and amax to acc.
template <int FMT>
__device__ __forceinline__ uint32_t cast_one(uint32_t xb, const CastParams& p, Acc& acc) {
  const uint32_t ax = xb & kAbsMask;
  count_elem(ax, p, acc);
  acc.amax = max(acc.amax, finite_mag(ax, acc));
  const uint32_t q = cvt1<FMT>(xb, p.K);
  return ax > kMaxFinite ? nonfinite_code<FMT>(xb) : q;
}

// fp32 bits of RNE(value(a) * 2^-s) for finite non-negative a, s >= 0 (the
// unscaled amax; exact unless the result is below fp32's normal range).
__host__ __device__ inline uint32_t unscale_bits(uint32_t a, int s) {
  if (s <= 0 || a == 0) return a;
  const uint32_t E = a >> 23;
  if (E > (uint32_t)s) return a - ((uint32_t)s << 23);
  const uint32_t sig = E ? ((a & 0x7FFFFFu) | 0x800000u) : (a & 0x7FFFFFu);
  const int sh = s + 1 - (E ? (int)E : 1);   // result in units of 2^-149
  if (sh > 26) return 0u;
  const uint32_t half_m1 = (1u << (sh - 1)) - 1u;
  return (sig + half_m1 + ((sig >> sh) & 1u)) >> sh;
}

// Wave64 reductions (used at flushes only, never per element).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Row (16-lane) reductions by DPP moves: quad_perm [1,0,3,2], quad_perm
// [2,3,0,1], row_half_mirror, row_mirror.  Afterwards every lane of a row
// holds the row's result; for floating point the result is the same in all
// 16 lanes (each step adds two equal partial sums in either order) and does
// not depend on scheduling.  Full EXEC only.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = dpp_u32<CTRL>((uint32_t)b), hi = dpp_u32<CTRL>((uint32_t)(b >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ uint32_t row_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));
  v = max(v, dpp_u32<0x4E>(v));
  v = max(v, dpp_u32<0x141>(v));
  return max(v, dpp_u32<0x140>(v));
}
__device__ __forceinline__ uint32_t row_sum_u32(uint32_t v) {
  v += dpp_u32<0xB1>(v);
  v += dpp_u32<0x4E>(v);
  v += dpp_u32<0x141>(v);
  return v + dpp_u32<0x140>(v);
}
constexpr int kRows = kThreads / 16;    // 16-lane rows per workgroup

// ---------------------------------------------------------------------------
// Batches.  Up to kMaxSeg tensors per launch; tensor s owns tiles
// [tile0[s], tile0[s+1]) of the launch (one workgroup per tile) and
// first-reduction chunks [chunk0[s], chunk0[s+1]); the entries past `count`
// repeat the launch's totals.
struct Seg {
  const void* x;
  uint8_t* codes;
  uint8_t* scales;
  void* y;
  int64_t n;
  int64_t cols;    // MX: row length
};

struct SegBatch {
  Seg s[kMaxSeg];
  int32_t tile0[kMaxSeg + 1];    // < 2^31: a launch has at most 2^34 elements, 2048 or more per tile
  int32_t chunk0[kMaxSeg + 1];
  int32_t last[kMaxSeg];   // elements in tensor s's last tile (1..tile size; 0 if empty)
  int32_t count;   // tensors in this launch
  int32_t first;   // index of s[0] in the caller's arrays (counts, states, stats)
};
static_assert(sizeof(SegBatch) <= 4096, "a SegBatch travels as a kernel argument");
static_assert(kMaxSeg % 8 == 0, "seg_of_scan takes the prefix entries in groups of eight");

// Tensor owning entry `i` of a prefix array (tile0 or chunk0): the last s
// with start[s] <= i, i.e. the number of s' in [1, count) with start[s'] <=
// i (start is non-decreasing).  Lane l tests start[l + 1] and the wave
// counts the hits: one load per lane instead of a chain of up to 31
// dependent scalar loads.  A one-tensor launch loads nothing.  Called by
// whole waves; the result is wave-uniform.
__device__ __forceinline__ int seg_of(const int32_t* start, int count, int64_t i) {
  if (count == 1) return 0;
  const int l = threadIdx.x & 63;
  const bool hit = l + 1 < count && i >= start[l + 1];
  return __builtin_amdgcn_readfirstlane(__popcll(__ballot(hit)));
}

// The same lookup on the scalar unit: the entries start[8], start[16], ...,
// start[56] pick a group of eight, whose entries then give the tensor, so
// two rounds of independent scalar loads of the kernel arguments and about
// 40 scalar instructions per wave, no vector memory access.  Relies on the
// entries past `count` holding the launch's total (never <= i).  Which of the
// two is faster depends on the kernel: with 2^30 elements split over eight
// tensors, the scalar form made the per-tensor and row-block casts and the
// column-block dequant 2-5% of HBM peak faster, the lane form kept amax and
// the per-tensor dequant 1-2% faster, the rest measured level.
__device__ __forceinline__ int seg_of_scan(const int32_t* start, int count, int64_t i) {
  if (count == 1) return 0;
  const int32_t k = (int32_t)i;
  int c = 0;   // groups of eight whose first entry is <= k, past group 0
#pragma unroll
  for (int j = 1; j < kMaxSeg / 8; ++j) c += (int)((uint32_t)(start[8 * j] - k - 1) >> 31);
  const int32_t* g = start + 8 * c;
  int s = 8 * c;
#pragma unroll
  for (int j = 1; j < 8; ++j) s += (int)((uint32_t)(g[j] - k - 1) >> 31);
  return s;
}

// The tile of this workgroup.  Workgroups are handed to the eight XCDs in
// turn (g mod 8), so with tile = g every XCD streams every eighth tile of
// the launch.  Here each group of 8C consecutive workgroups takes 8C
// consecutive tiles, XCD x the C of them starting at x C: XCD x's j-th
// workgroup of the group gets tile 8C group + x C + j.  A trailing partial
// group keeps tile = g.  C = 1 is the plain order.  Nothing is reused
// across tiles, so this is about how the eight XCDs' request streams meet
// in HBM, not about L2 hits.  Measured on 2^30 elements against the plain
// order, in points of HBM peak: C = 256 lifts the per-tensor cast by 2-3
// and the row-block MX cast by 1-2; C = 32 lifts amax by 4-6, the
// statistics passes and the monitor by 1-8, the column-block dequant by 1;
// the column-block cast and stochastic rounding measured best or level in
// the plain order.  One contiguous region per XCD (C = G / 8) helped the
// read-only kernels as much but cost the dequants 3-4 points.
template <uint32_t C>
__device__ __forceinline__ int64_t xcd_tile() {
  const uint32_t g = blockIdx.x, G = gridDim.x;
  if constexpr (C == 1) return (int64_t)g;
  constexpr uint32_t span = 8u * C;
  if (g >= G / span * span) return (int64_t)g;
  return (int64_t)(g / span * span + (g % 8u) * C + (g / 8u) % C);
}

// Elements in tile t of tensor s: TILE, except in the tensor's last tile.
// Written as a 64-bit equality plus a 32-bit select on purpose.  The gfx950
// backend of this ROCm toolchain has been seen to lower min(n - e0, TILE)
// (a 64-bit ordered compare whose result feeds both a select and a branch)
// with the vector compare's copy into the scalar condition code dropped, so
// the select read a stale carry flag and a ragged tile ran as a full one.
// The library build scans the device assembly for that signature.
template <int64_t TILE>
__device__ __forceinline__ int tile_len(const SegBatch& b, int s, int64_t t) {
  return t == b.tile0[s + 1] - 1 ? b.last[s] : (int)TILE;
}

// Column-block MX (blocks of 32 consecutive rows of one column).  A "slot"
// is VC adjacent columns of R consecutive rows inside one 32-row band (R
// divides 32): R * VC elements, all under the same VC scale bytes.  Slots
// are numbered row group by row group, left to right; tile t of a tensor is
// slots [S t, S t + S), S = 256 / (lanes per slot), in lane order, so the
// lanes of a wave hold consecutive pieces of the same rows and every row
// access of a wave is one contiguous run per group of lanes that share a row.  The cast needs whole bands (R = 32: a block's max before
// any code); dequant and statistics take shorter slots, which keep their
// tiles small.  A tensor has n / (R VC) < 2^30 slots (rows are a multiple
// of 32, so cols <= n / 32), which keeps the division 32-bit.
struct ColSlot {
  int64_t e0;   // element index of the slot's top-left element
  int64_t sc;   // index of the slot's first scale byte ((rows / 32) x cols, row-major)
  bool act;     // the lane has a slot (the tensor's last tile may be short)
};
// An idle lane gets the tensor's slot 0 -- in bounds, so its loads need no
// predicate (they would otherwise become a branch per row) -- and must
// discard what it reads and store nothing.
template <int VC, int R = 32>
__device__ __forceinline__ ColSlot col_slot_at(const Seg& g, uint32_t j, bool act) {
  static_assert(32 % R == 0, "a slot stays inside one band");
  const uint32_t per_group = (uint32_t)(g.cols / VC);
  const uint32_t grp = j / per_group;
  const uint32_t cg = j - grp * per_group;
  ColSlot c;
  c.act = act;
  c.e0 = act ? (int64_t)grp * R * g.cols + (int64_t)cg * VC : 0;
  c.sc = act ? (int64_t)(grp / (32 / R)) * g.cols + (int64_t)cg * VC : 0;
  return c;
}
// Slot of this lane in tile t (one slot per lane; rem slots in the tile).
template <int VC, int R = 32>
__device__ __forceinline__ ColSlot col_slot(const Seg& g, int64_t t, int rem) {
  return col_slot_at<VC, R>(g, (uint32_t)t * (uint32_t)kThreads + threadIdx.x, (int)threadIdx.x < rem);
}

// Workspace slots.  A workgroup's counts: finite-|x| max (bits), non-finite,
// |x| above the clip bound (clips + non-finite), underflows.
struct CountSlot {
  uint32_t amax, n_nf, n_big, n_uf;
};

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  for (int o = 32; o > 0; o >>= 1) v += (uint32_t)__shfl_xor((int)v, o, 64);
  return v;
}
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
  for (int o = 32; o > 0; o >>= 1) v += (uint64_t)__shfl_xor((long long)v, o, 64);
  return v;
}

// One wave's count totals, the same in every lane (wave-uniform): DPP row
// reductions, then the four row totals read across rows.  n_big and n_uf
// travel packed in one word (low and high half): a lane counts at most a
// few dozen elements -- 64 in the largest tiles -- so a wave's totals stay
// far below 2^16.  n_nf is reduced only in a wave that met an Inf or NaN
// (uniform branch).  Called with full EXEC.
struct WaveCounts {
  uint32_t amax, big_uf, n_nf;
};

__device__ __forceinline__ uint32_t rows_sum(uint32_t v) {     // v: row totals in lanes 0, 16, 32, 48
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 0) + (uint32_t)__builtin_amdgcn_readlane((int)v, 16) +
         (uint32_t)__builtin_amdgcn_readlane((int)v, 32) + (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
}
__device__ __forceinline__ uint32_t rows_max(uint32_t v) {
  return max(max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
             max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}

__device__ __forceinline__ WaveCounts wave_counts(Acc acc) {
  const uint32_t big = acc.n_big + acc.big16.x + acc.big16.y;
  const uint32_t uf = acc.n_uf + acc.uf16.x + acc.uf16.y;
  WaveCounts w;
  w.amax = rows_max(row_max_u32(acc.amax));
  w.big_uf = rows_sum(row_sum_u32(big | (uf << 16)));
  w.n_nf = __ballot(acc.n_nf != 0u) != 0 ? rows_sum(row_sum_u32(acc.n_nf)) : 0u;
  return w;
}

// The workgroup's totals, valid in thread 0: one LDS entry per wave, thread
// 0 over the waves.  Called by all threads (full EXEC); lds holds at least
// kWaves * 3 words.
__device__ inline CountSlot workgroup_counts(Acc acc, uint32_t* lds) {
  const WaveCounts w = wave_counts(acc);
  if ((threadIdx.x & 63) == 0) {
    const int i = threadIdx.x >> 6;
    lds[i * 3 + 0] = w.amax;
    lds[i * 3 + 1] = w.big_uf;
    lds[i * 3 + 2] = w.n_nf;
  }
  __syncthreads();
  CountSlot c{0u, 0u, 0u, 0u};
  if (threadIdx.x == 0) {
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      c.amax = max(c.amax, lds[i * 3 + 0]);
      c.n_big += lds[i * 3 + 1] & 0xFFFFu;
      c.n_uf += lds[i * 3 + 1] >> 16;
      c.n_nf += lds[i * 3 + 2];
    }
  }
  return c;
}

// ---------------------------------------------------------------------------
// Decoding.  fp32 bits of the value a code stands for (at exponent 0);
// NaN codes give 0x7FC00000, E5M2 Inf codes give +-Inf.
template <int FMT>
__host__ __device__ inline uint32_t decode_bits(uint32_t q) {
  using F = Fp8<FMT>;
  const uint32_t sign = (q & 0x80u) << 24;
  const uint32_t e = (q >> F::MB) & ((1u << (7 - F::MB)) - 1u);
  const uint32_t m = q & ((1u << F::MB) - 1u);
  constexpr uint32_t etop = (1u << (7 - F::MB)) - 1u;
  if (FMT == NC_E4M3 && e == etop && m == 7u) return 0x7FC00000u;
  if (FMT == NC_E5M2 && e == etop) return m ? 0x7FC00000u : (sign | kInfBits);
  if (e == 0) {
    // m * 2^(EMIN - MB): m < 2^MB, normalise into fp32
    if (m == 0) return sign;
    int lz = 0;
    while (!(m & (1u << (F::MB - 1 - lz)))) ++lz;
    const int top = F::MB - 1 - lz;                      // value = 1.f * 2^(top + EMIN - MB)
    const uint32_t frac = (m ^ (1u << top)) << (23 - top);
    return sign | ((uint32_t)(top + F::EMIN - F::MB + 127) << 23) | frac;
  }
  return sign | ((uint32_t)((int)e - F::BIAS + 127) << 23) | (m << (23 - F::MB));
}

// bf16 pattern of RNE(fp32 value) -- IEEE overflow to Inf; quiet NaN kept.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(uint32_t b) {
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------------------
// Input vectors and error statistics (shared by the casts and the
// separate statistics pass).

// Streaming loads: every input byte is read once per pass, so the loads are
// non-temporal (the cache lines are not kept for reuse).
__device__ __forceinline__ u32x4 ld_stream(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ u32x2 ld_stream(const u32x2* p) { return __builtin_nontemporal_load(p); }

// Code stores of the casts are streamed too (measured faster on MI355X for
// these read-2/write-1 streams).
__device__ __forceinline__ void st_stream(uint32_t* p, uint32_t v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void st_stream(u32x2* p, u32x2 v) { __builtin_nontemporal_store(v, p); }


// 16 input bytes -> VEC fp32 bit patterns (bf16 widens exactly by a shift).
template <int DT>
__device__ __forceinline__ void unpack(const u32x4 v, uint32_t* xb) {
  if constexpr (DT == NC_F32) {
    xb[0] = v.x; xb[1] = v.y; xb[2] = v.z; xb[3] = v.w;
  } else {
    xb[0] = v.x << 16; xb[1] = v.x & 0xFFFF0000u;
    xb[2] = v.y << 16; xb[3] = v.y & 0xFFFF0000u;
    xb[4] = v.z << 16; xb[5] = v.z & 0xFFFF0000u;
    xb[6] = v.w << 16; xb[7] = v.w & 0xFFFF0000u;
  }
}

// 8 input bytes -> 8 / BYTES fp32 bit patterns (the column-block kernels).
template <int DT>
__device__ __forceinline__ void unpack8(const u32x2 v, uint32_t* xb) {
  if constexpr (DT == NC_F32) {
    xb[0] = v.x; xb[1] = v.y;
  } else {
    xb[0] = v.x << 16; xb[1] = v.x & 0xFFFF0000u;
    xb[2] = v.y << 16; xb[3] = v.y & 0xFFFF0000u;
  }
}

template <int DT>
__device__ __forceinline__ uint32_t load_one(const void* x, int64_t i) {
  if constexpr (DT == NC_F32) return static_cast<const uint32_t*>(x)[i];
  else return (uint32_t)static_cast<const uint16_t*>(x)[i] << 16;
}

// ---------------------------------------------------------------------------
// Error statistics ([Drift, "What the measurements said"]): over finite
// x, sums of e, |e|, e^2, sign(x) e, x e, x^2 with e = xhat - x, in binary64.
// They are accumulated in the kernel's input domain (x as stored, xhat =
// decode(q) * 2^-K with K = k - s); the loss-scale unscale multiplies x and
// e by 2^-s, so the final reduction scales the first, second and fourth
// sums by 2^-s and the others by 2^-2s -- exact power-of-two factors.
struct StatAcc {
  double s[6];
  __device__ void reset() {
#pragma unroll
    for (int j = 0; j < 6; ++j) s[j] = 0.0;
  }
};

// LDS table of decode(q) * 2^-K in binary64 (exact: at most 4 significant
// bits).  NaN codes never meet a finite x; they hold 0.  Threads 0..255
// each fill one entry.
template <int FMT>
__device__ inline void fill_stat_table(double* tab, int K) {
  const uint32_t b = decode_bits<FMT>(threadIdx.x);
  tab[threadIdx.x] = ((b & kAbsMask) > kInfBits) ? 0.0 : ldexp((double)__uint_as_float(b), -K);
}

__device__ __forceinline__ double pow2_f64(int X) {   // 2^X for |X| <= 1022
  return __longlong_as_double((long long)(X + 1023) << 52);
}

__device__ __forceinline__ void stat_term(double x, double xh, StatAcc& a) {
  const double e = xh - x;
  a.s[0] += e;
  a.s[1] += fabs(e);
  a.s[2] = fma(e, e, a.s[2]);
  a.s[3] += fabs(xh) - fabs(x);    // = sign(x) e: a code keeps its input's sign
  a.s[4] = fma(x, e, a.s[4]);
  a.s[5] = fma(x, x, a.s[5]);
}

// The same for an MX element, xhat = t * blk with blk = 2^X: the product is
// exact in binary64 (|t| in [2^-16, 2^16], |X| <= 128), so an fma that takes
// it rounds once, as the difference of the product does -- the same sums
// with one operation fewer.
__device__ __forceinline__ void stat_term_blk(double x, double t, double blk, StatAcc& a) {
  const double e = fma(t, blk, -x);
  a.s[0] += e;
  a.s[1] += fabs(e);
  a.s[2] = fma(e, e, a.s[2]);
  a.s[3] += fma(fabs(t), blk, -fabs(x));
  a.s[4] = fma(x, e, a.s[4]);
  a.s[5] = fma(x, x, a.s[5]);
}

// Terms of VEC elements (fp32 patterns xb, codes q); xhat = tab[q] (* blk
// for MX, the block's 2^X).  FINITE: the caller knows every x is finite (no
// test); otherwise Inf/NaN elements are skipped.
template <int VEC, bool MX, bool FINITE>
__device__ __forceinline__ void stats_vec(const uint32_t* xb, const uint32_t* q, const double* tab,
                                          double blk, StatAcc& a) {
#pragma unroll
  for (int i = 0; i < VEC; ++i) {
    if (!FINITE && (xb[i] & kAbsMask) > kMaxFinite) continue;
    if constexpr (MX) stat_term_blk((double)__uint_as_float(xb[i]), tab[q[i]], blk, a);
    else stat_term((double)__uint_as_float(xb[i]), tab[q[i]], a);
  }
}

// After unmasked accumulation: was every x finite?  A finite fp32 x has
// x^2 <= 2^256, so the binary64 sum of x^2 over a tile stays finite; an
// Inf/NaN x makes it Inf/NaN.
__device__ __forceinline__ bool stats_all_finite(const StatAcc& a) {
  return __builtin_isfinite(a.s[5]);
}

// The workgroup's six partial sums, in a fixed order (so the sums are
// reproducible): every thread stores its six sums in LDS, sum-major; after a
// barrier lane 8j + r of wave 0 (j < 6, r < 8) adds sum j of threads r,
// r + 8, ..., r + 248 in four interleaved chains, then the eight lanes of
// each group combine their partials by three DPP steps inside the group
// (quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror); each step adds
// two equal partial sums in either order, so every lane of the group ends
// with the same value.  Lanes 48..63 repeat group 5 to keep EXEC full for the
// DPP moves.  A workgroup spends about 60 VALU instructions here, against
// about 120 per wave for six 16-lane DPP sums.
constexpr int kStatStride = kThreads + 8;   // doubles per sum: the groups' reads start 64 bytes apart in the banks
constexpr int kStatLds = 6 * kStatStride;   // doubles of LDS the stat sums take

__device__ __forceinline__ void stat_store(const StatAcc& a, double* lds) {
#pragma unroll
  for (int j = 0; j < 6; ++j) lds[j * kStatStride + threadIdx.x] = a.s[j];
}

// Wave 0, full EXEC, after the barrier that follows stat_store: sum j of the
// workgroup in lanes 8j..8j+7.
__device__ __forceinline__ double stat_sum_wave0(const double* lds) {
  const int lane = threadIdx.x & 63;
  const double* p = lds + min(lane >> 3, 5) * kStatStride + (lane & 7);
  double c[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) c[k] = p[8 * k];
#pragma unroll
  for (int i = 4; i < kThreads / 8; i += 4) {
#pragma unroll
    for (int k = 0; k < 4; ++k) c[k] += p[8 * (i + k)];
  }
  double t = (c[0] + c[1]) + (c[2] + c[3]);
  t += dpp_f64<0xB1>(t);
  t += dpp_f64<0x4E>(t);
  return t + dpp_f64<0x141>(t);
}

// The workgroup's six partial sums -> its slot.  Called by all threads (full
// EXEC); lds holds kStatLds doubles.
__device__ inline void write_stat_slot(const StatAcc& a, double* slot, double* lds) {
  stat_store(a, lds);
  __syncthreads();
  if (threadIdx.x < 64) {
    const double v = stat_sum_wave0(lds);
    if ((threadIdx.x & 7) == 0 && threadIdx.x < 48) slot[threadIdx.x >> 3] = v;
  }
}

// The casts with fused statistics: both slots in one epilogue, one barrier.
// lds holds kWaves * 3 words, lds_st kStatLds doubles.  Wave 0 adds the
// statistics, thread 64 the counts beside it.
__device__ inline void write_count_stat_slots(Acc acc, const StatAcc& a, CountSlot* slot, double* stat_slot,
                                              uint32_t* lds, double* lds_st) {
  const WaveCounts w = wave_counts(acc);
  if ((threadIdx.x & 63) == 0) {
    const int i = threadIdx.x >> 6;
    lds[i * 3 + 0] = w.amax;
    lds[i * 3 + 1] = w.big_uf;
    lds[i * 3 + 2] = w.n_nf;
  }
  stat_store(a, lds_st);
  __syncthreads();
  if (threadIdx.x < 64) {
    const double v = stat_sum_wave0(lds_st);
    if ((threadIdx.x & 7) == 0 && threadIdx.x < 48) stat_slot[threadIdx.x >> 3] = v;
  } else if (threadIdx.x == 64) {
    CountSlot c{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      c.amax = max(c.amax, lds[i * 3 + 0]);
      c.n_big += lds[i * 3 + 1] & 0xFFFFu;
      c.n_uf += lds[i * 3 + 1] >> 16;
      c.n_nf += lds[i * 3 + 2];
    }
    *slot = c;
  }
}

}  // namespace nc
