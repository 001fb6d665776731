/*
 * libnarrowcast -- the scaled narrow-format (FP8) cast on AMD Instinct
 * MI355X (gfx950).
 *
 * Sources (web pages, cited by title and section):
 *   [E3]      practice exercise c06/E3, "Worked solution"
 *             (deeper.gabrielebattimelli.com): which quantity is measured and
 *             when, the rule that turns it into a scale, what the run claims.
 *   [MP-card] "Mixed Precision FP16/BF16/FP8" (talentme.airsota.com mind-map
 *             card), items (1)-(3): formats, loss scaling.
 *   [Drift]   "what actually breaks low precision training"
 *             (aarohigandhi.vercel.app/writing/drift), "What the measurements
 *             said": MX blocks of 32, the OCP rule and +1 headroom, clip and
 *             bias measurements.
 *   [MaxWin]  "Max-Window Scale Estimation for Near-Lossless HiF8 W8A8
 *             Quantization-Aware Training" (gist.science explainer),
 *             "Experimental Variables": amax estimators.
 *   [SP]      "Which parts of a mixed-precision training step must stay in
 *             single precision, and why?" (katajob.com), "Master weights and
 *             the optimizer step": a 16-bit weight update that is a no-op.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers marked (device) are HIP device memory owned by the caller; the
 *   library allocates nothing and keeps no state between calls (apart from
 *   nc_cast_tensor_static's static per-GPU scratch and its looked-up
 *   address).  Pointers marked (host) are read during the call only.
 * - Every call is asynchronous on `stream` (a hipStream_t; NULL is the null
 *   stream): argument checks happen on the host before anything is enqueued
 *   and return an error code; results land in device memory and the caller
 *   synchronises.  Calls on different streams are independent.
 * - Counts and statistics ACCUMULATE into caller-zeroed buffers (integer
 *   max/add; binary64 sums formed in a fixed order, then added), so a
 *   tensor may be processed in several calls.  All outputs of a call are
 *   deterministic.
 * - Element data (x, codes, y) must be 16-byte aligned.  n == 0 is a valid
 *   no-op; any 0 <= n <= 2^34 is accepted (ragged tails are handled in the
 *   kernels).
 * - Scale exponents: a per-tensor scale is 2^k -- the cast quantises
 *   x * 2^k and code q stands for decode(q) * 2^-k.  An MX block exponent is
 *   X -- elements are quantised as x * 2^-X and stand for decode(q) * 2^X; its
 *   scale byte is X + 127.  k and X lie in [-127, 127].
 * - The cast rounds to nearest, ties to even, saturating at the format's
 *   largest finite value (E4M3: 448, E5M2: 57344 [MP-card, item (3)]).
 *   NaN inputs become code 0x7F; +-Inf become +-max; a zero keeps its sign.
 *   clip: finite x with |x * 2^K| > max (the exact product, never the fp32
 *   one).  underflow: finite nonzero x that rounds to a zero code.
 */
#ifndef NARROWCAST_H
#define NARROWCAST_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NC_OK = 0,
  NC_E_ARG = 1,          /* null pointer, negative size, bad policy field */
  NC_E_ALIGN = 2,        /* element pointer not 16-byte aligned */
  NC_E_SHAPE = 3,        /* MX: cols not a positive multiple of 32, n % cols != 0, rows not a
                            multiple of 32 for NC_MX_COLS, or mixed mx_axis in one call */
  NC_E_UNSUPPORTED = 4,  /* unknown enum value */
  NC_E_HIP = 5,          /* a HIP launch failed */
  NC_E_WORKSPACE = 6,    /* workspace missing or smaller than nc_workspace_bytes() */
  NC_E_SCRATCH = 7       /* nc_cast_tensor_static: the batch needs more than NC_STATIC_SCRATCH_BYTES */
} nc_status;

typedef enum { NC_F32 = 0, NC_BF16 = 1 } nc_dtype;
typedef enum { NC_E4M3 = 0, NC_E5M2 = 1 } nc_fmt;

/* MX shared-exponent rules for a block with finite amax a = m * 2^e, m in [1,2)
 * ([Drift, "What the measurements said" and "The part I would rather not
 * write"]):  OCP (floor based): X = e - emax_F;  PLUS1: the exponent one
 * higher, X = e - emax_F + 1;  CEIL: the scale rounded up, the
 * smallest X with a * 2^-X <= max_F.  a == 0 gives X = -127. */
typedef enum { NC_MX_OCP = 0, NC_MX_PLUS1 = 1, NC_MX_CEIL = 2 } nc_mx_rule;

/* amax estimators ([MaxWin, "Experimental Variables"]): CURRENT uses the
 * amax passed in for this step (the two-pass "current scaling");
 * MOST_RECENT the last amax pushed into the history; MAX_WINDOW the largest
 * of the last `window` pushes; EMA exponential smoothing, E <- E + alpha *
 * (a - E) with each of the three operations rounded to fp32 (nearest even,
 * no fused multiply-add), E = a at the first push.  EMA keeps E in slot 0
 * of the tensor's history (window >= 1). */
typedef enum { NC_EST_CURRENT = 0, NC_EST_MOST_RECENT = 1, NC_EST_MAX_WINDOW = 2, NC_EST_EMA = 3 } nc_est;

/* Which elements share an MX block exponent.  ROWS: 32 consecutive elements
 * of a row; scales are row-major rows x (cols / 32).  COLS: 32 consecutive
 * rows of one column (the layout a transposed operand needs); scales are
 * row-major (rows / 32) x cols. */
typedef enum { NC_MX_ROWS = 0, NC_MX_COLS = 1 } nc_mx_axis;

/* One tensor of a batch (host array of these). */
typedef struct {
  const void *x;     /* (device) n input elements, fp32 or bf16; for nc_dequant unused */
  uint8_t *codes;    /* (device) n FP8 codes: written by the casts, read by dequant/stats */
  int64_t n;         /* element count, >= 0 */
  int64_t cols;      /* MX calls only: row length of the row-major rows x cols matrix,
                        a multiple of 32 dividing n (NC_MX_COLS: n / cols also a
                        multiple of 32) */
  uint8_t *scales;   /* MX calls only (device): n / 32 block-scale bytes X + 127 (layout
                        by mx_axis) */
  int32_t mx_axis;   /* MX calls only: nc_mx_axis; one value for all tensors of a call */
  int32_t reserved;  /* 0 */
} nc_tensor;

/* ---- The update/step-ratio ("swamping") monitor types ---------------------- */

/* The narrow format a weight copy is kept in. */
typedef enum { NC_W_BF16 = 0, NC_W_FP16 = 1 } nc_wfmt;

/* One weight tensor and its update (host array of these). */
typedef struct {
  const float *w;    /* (device) n fp32 master weights, 16-byte aligned */
  const float *d;    /* (device) n fp32 updates (what the optimizer adds), 16-byte aligned */
  uint8_t *flags;    /* (device, nullable, 4-byte aligned) n flag bytes: bit 0 below the step,
                        bit 1 no-op, bit 2 zero update, bit 3 excluded */
  int64_t n;         /* element count, >= 0 */
} nc_update_tensor;

/* Per-tensor monitor counts (device array, one per tensor; zero before the
 * call: the call adds into it). */
typedef struct {
  uint64_t n_considered;   /* finite weight in the format's range, finite nonzero update */
  uint64_t n_zero;         /* finite weight in range, zero update */
  uint64_t n_below;        /* considered, |d| < the step of w's narrow copy (ratio below one) */
  uint64_t n_noop;         /* considered, the narrow add leaves the weight unchanged */
  uint64_t n_excluded;     /* w or d not finite, or w overflows the narrow format */
} nc_swamp_counts;

/* Promotion rule: a step is "below" when n_below * den >= num * n_considered
 * (n_considered > 0); `window` below steps in a row promote the tensor. */
typedef struct {
  int32_t window;    /* >= 1 */
  uint32_t num;      /* threshold num / den, 0 <= num <= den */
  uint32_t den;      /* 1 .. 65536 */
  int32_t reserved;  /* 0 */
} nc_swamp_policy;

/* Per-tensor promotion state (device array; zero-initialise). */
typedef struct {
  int32_t run;       /* consecutive below steps */
  int32_t promoted;  /* 1 once run has reached the window; stays 1 */
  int32_t steps;     /* steps seen */
  int32_t reserved;
} nc_swamp_state;

/* Per-tensor counts (device array, one per tensor; zero before first use). */
typedef struct {
  uint64_t n_finite;
  uint64_t n_clip;
  uint64_t n_underflow;
  uint64_t n_nonfinite;  /* > 0 is the tensor's non-finite flag */
  uint32_t amax_bits;    /* fp32 bits of the largest finite |x| (after unscale),
                            rounded to nearest even if it falls below fp32's normal range */
  uint32_t reserved;
} nc_counts;

/* Per-tensor error statistics over finite elements (device array, zeroed),
 * e = xhat - x with xhat the exact value the code stands for and x the
 * (unscaled) input: the size of the change the cast makes, and apart from
 * it the direction of that change ([Drift, "What the measurements said"]). */
typedef struct {
  double sum_e, sum_abs_e, sum_e2;
  double sum_dir_e;  /* sum of sign(x) * e: negative when magnitudes shrink */
  double sum_xe;     /* with sum_x2: the kept fraction 1 + sum_xe / sum_x2 */
  double sum_x2;
} nc_stats;

/* Per-tensor scale state (device array; all-zero is a fresh state). */
typedef struct {
  int32_t k;            /* scale exponent used by the next cast */
  uint32_t a_ref_bits;  /* fp32 estimate at the last change of k (hysteresis) */
  int32_t has_ref;      /* 0 until the first recompute */
  int32_t n_hist;       /* valid history entries, <= window */
  int32_t head;         /* next history slot */
  int32_t step;         /* history pushes so far */
} nc_scale_state;

/* Loss scale S = 2^s_log2 (device, one per batch). */
typedef struct {
  int32_t s_log2;
  int32_t clean_steps;
} nc_loss_scale;

/* Scale policy (host).  [E3, "Worked solution"]: watch amax over a window
 * of steps; largest power of two keeping it at or below the format's max
 * with a margin; recompute every `interval` steps; hysteresis of a factor of
 * two.  [MP-card, item (1)]: dynamic loss scaling. */
typedef struct {
  int32_t fmt;                /* nc_fmt: the format the scale is for */
  int32_t est;                /* nc_est */
  int32_t window;             /* history length W, 1..1024 */
  int32_t margin;             /* binades of margin, 0..32 */
  int32_t hysteresis;         /* 0/1 */
  int32_t interval;           /* recompute every I pushes, >= 1 */
  int32_t skip_on_nonfinite;  /* 0/1: a batch with any Inf/NaN changes no scale state */
  int32_t ls_enable;          /* 0/1: run the loss-scale machine */
  int32_t ls_growth_interval; /* clean steps before S doubles, >= 1 */
  int32_t ls_log2_min;        /* bounds on s_log2, 0 <= min <= max <= 64 */
  int32_t ls_log2_max;
  float ema_alpha;            /* EMA smoothing coefficient, 0 < alpha <= 1 (other estimators ignore it) */
} nc_policy;

/* Per-tensor amax pass (a full read of the tensor, [E3, "Worked solution"];
 * the second look at the data that current scaling needs, [MaxWin,
 * "Experimental Variables"]).  Reads x only.  For each tensor: max-accumulates
 * amax_bits of |x| * 2^-s over finite elements and adds n_finite and
 * n_nonfinite into out[i].  ls (device, nullable): unscale by 2^-ls->s_log2.
 * ws: workspace of nc_workspace_bytes(t, count) bytes.  Input bytes per
 * element: 4 (fp32) or 2 (bf16). */
nc_status nc_amax(const nc_tensor *t, int32_t count, nc_dtype dtype,
                  const nc_loss_scale *ls, nc_counts *out, void *ws, size_t ws_bytes,
                  void *stream);

/* Scale update for a batch of `count` tensors ([E3, "Worked solution"];
 * [MaxWin, "Experimental Variables"]).  in[i] holds tensor i's counts from
 * the pass just run.  est == CURRENT: k is set from in[i].amax now (no
 * history).  Otherwise in[i].amax is pushed into tensor i's ring
 * hist[i*window .. i*window+window-1] (device fp32) and, every `interval`
 * pushes, k is recomputed from the estimator.  The rule: the largest k in
 * [-127, 127] with A * 2^k <= max_F * 2^-margin (A == 0 gives 127).
 * Hysteresis: k is reset when A * 2^k would exceed that bound or when
 * A <= a_ref / 2, and kept otherwise.  With skip_on_nonfinite, a batch in
 * which any tensor has n_nonfinite > 0 changes no scale state.  ls
 * (device, nullable): when policy->ls_enable, halves S on a non-finite batch
 * and doubles it after ls_growth_interval clean batches, within bounds. */
nc_status nc_scale_update(const nc_policy *policy, int32_t count, nc_scale_state *st,
                          float *hist, const nc_counts *in, nc_loss_scale *ls, void *stream);

/* Per-tensor scaled cast ([MP-card, item (3)]; [E3, "Worked solution"]).
 * Element i of tensor j becomes RNE-sat(x * 2^(st[j].k - s)), s =
 * ls->s_log2 or 0 -- the loss-scale unscale fused in front ([MP-card, item
 * (1)]).  Fused: counts (n_finite, n_clip, n_underflow, n_nonfinite) and the
 * next step's amax (of x * 2^-s) accumulate into out[j].  stats (device,
 * nullable): also accumulate the error statistics.  ws: workspace of
 * nc_workspace_bytes(t, count) bytes.  Bytes per element: in 4|2, out 1. */
nc_status nc_cast_tensor(const nc_tensor *t, int32_t count, nc_dtype dtype, nc_fmt fmt,
                         const nc_scale_state *st, const nc_loss_scale *ls, nc_counts *out,
                         nc_stats *stats, void *ws, size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: the
 * per-tensor cast of nc_cast_tensor, identical in arguments (less the
 * workspace), checks, results and kernels, with the workspace taken from a
 * static array of NC_STATIC_SCRATCH_BYTES bytes that the library holds on
 * each GPU it runs on until the process ends.  It allocates nothing and calls
 * no allocating routine.  A batch whose nc_workspace_bytes() exceeds
 * NC_STATIC_SCRATCH_BYTES (8 MiB: one launch of up to about 2^28 elements)
 * returns NC_E_SCRATCH before anything is enqueued.  The array's device
 * address is looked up on the first call for the device that runs `stream`
 * (the current device for the null stream) and kept.  Every call on a GPU
 * shares that GPU's array, which keeps the last call's contents (nothing in
 * it needs to start at zero): calls that overlap in time on one GPU --
 * different streams, or threads -- race and must be serialised by the
 * caller (one stream, or events). */
#define NC_STATIC_SCRATCH_BYTES ((size_t)8 << 20)
nc_status nc_cast_tensor_static(const nc_tensor *t, int32_t count, nc_dtype dtype, nc_fmt fmt,
                                const nc_scale_state *st, const nc_loss_scale *ls, nc_counts *out,
                                nc_stats *stats, void *stream);

/* Per-tensor cast with stochastic rounding ([Drift, "The part I would rather
 * not write": no bias within one step]).  As nc_cast_tensor, except the
 * rounding: with y = x * 2^(st[j].k - s) between grid neighbours lo <= |y| <
 * lo + q and t = (|y| - lo) / q, the magnitude rounds up iff u < t * 2^32,
 * u the element's uniform 32-bit integer -- word i % 4 of Philox4x32-10
 * (Salmon et al., SC11) with key `seed` (low word first) and counter
 * (i / 4, j, offset low word, offset high word), j the tensor's index in
 * this call.  Pass a new `offset` (e.g. the step number) per call for fresh
 * draws; the same (seed, offset) reproduces the codes bit for bit.  |y| >
 * max saturates (a clip); n_underflow counts finite nonzero elements whose
 * drawn code is a zero.  Counts and next-step amax as nc_cast_tensor; no
 * statistics (nc_cast_stats measures any codes).  Bytes per element: in
 * 4|2, out 1. */
nc_status nc_cast_tensor_sr(const nc_tensor *t, int32_t count, nc_dtype dtype, nc_fmt fmt,
                            const nc_scale_state *st, const nc_loss_scale *ls, uint64_t seed,
                            uint64_t offset, nc_counts *out, void *ws, size_t ws_bytes,
                            void *stream);

/* MX block-scaled cast ([Drift, "What the measurements said"]): blocks of
 * 32 elements (consecutive in a row, or in a column: mx_axis) share X from
 * the block's finite amax by `rule`; codes = RNE-sat(x * 2^-X), scales =
 * X + 127.  Counts, tensor amax
 * and optional statistics accumulate as in nc_cast_tensor.  Bytes per
 * element: in 4|2, out 1 + 1/32. */
nc_status nc_cast_mx(const nc_tensor *t, int32_t count, nc_dtype dtype, nc_fmt fmt,
                     nc_mx_rule rule, nc_counts *out, nc_stats *stats, void *ws,
                     size_t ws_bytes, void *stream);

/* Dequantise codes to bf16 ([Drift, "What the measurements said"]: the cast
 * is judged by what it does to the tensor, which needs the value each code
 * stands for; the formats of [MP-card, items (2) and (3)]):
 * y = RNE_bf16(decode(q) * 2^-k) (per-tensor, st non-NULL) or
 * RNE_bf16(decode(q) * 2^X) (MX, st == NULL, scales read), with IEEE
 * overflow to +-Inf; NaN codes give 0x7FC0; a signed zero keeps its sign.
 * t[i].codes and t[i].n (and, for MX, scales, cols and mx_axis) describe the
 * codes; t[i].x is unused.  y (host array of `count` device pointers, each
 * 16-byte aligned) receives n bf16 values per tensor; the caller owns them.
 * out_dtype must be NC_BF16, else NC_E_UNSUPPORTED.  Needs no workspace.
 * Bytes per element: in 1 (+1/32), out 2. */
nc_status nc_dequant(const nc_tensor *t, int32_t count, nc_fmt fmt, const nc_scale_state *st,
                     void *const *y, nc_dtype out_dtype, void *stream);

/* Error statistics as a separate pass over x and the codes already written
 * ([Drift, "What the measurements said"]: the size of the change the cast
 * makes, measured apart from its direction).  Over the
 * finite elements of each tensor, with x the input after the unscale by
 * 2^-ls->s_log2 (per-tensor only; ls nullable) and xhat = decode(q) * 2^-k
 * (per-tensor, st non-NULL) or decode(q) * 2^X (MX, st == NULL, scales
 * read), e = xhat - x: the sums of e, |e|, e^2, sign(x) e, x e and x^2, each
 * formed in binary64 in a fixed order and ADDED into out[i] (nc_stats, a
 * caller-zeroed device array).  The codes are read as they are: any codes
 * can be measured, not only the cast's own.  Over the codes a cast wrote,
 * the sums equal bit for bit those the cast forms when given `stats` (the
 * same terms in the same order).  ws: workspace of
 * nc_workspace_bytes(t, count) bytes.  Bytes per element: 4|2 + 1 (+1/32). */
nc_status nc_cast_stats(const nc_tensor *t, int32_t count, nc_dtype dtype, nc_fmt fmt,
                        const nc_scale_state *st, const nc_loss_scale *ls, nc_stats *out,
                        void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes that nc_amax, nc_cast_tensor, nc_cast_tensor_sr,
 * nc_cast_mx and nc_cast_stats need for this batch of tensors (any dtype,
 * statistics or not).  Every workgroup of a launch writes its partial counts
 * and sums to a slot of its own (64 bytes per 2048 input elements at most);
 * a small kernel sums each chunk of 1024 slots and adds the counts into the
 * caller's, and the statistics of a tensor with several chunks take a second
 * small kernel (48 bytes per chunk), every floating-point sum in a fixed
 * order -- about 3% of the input bytes of fp32, 1.6% of bf16.  A launch of at
 * most 64 workgroups that forms counts only (no statistics) skips the slots:
 * its workgroups add their counts into the caller's directly.  The workspace
 * is caller device memory (16-byte aligned), needs no initialisation, and may
 * be reused by the next call on the same stream; calls that run
 * concurrently need workspaces of their own.  0 for an empty batch. */
size_t nc_workspace_bytes(const nc_tensor *t, int32_t count);

/* Static description of a status code. */
const char *nc_status_string(nc_status s);

/* ---- The update/step-ratio ("swamping") monitor -----------------------------
 * [E3, "Worked solution"]: a format's step is what breaks at the weight, so
 * each update is compared with the grid spacing at its weight; a wide
 * master copy is kept while updates fall below that spacing, and a tensor
 * moves to a wider format once its updates have stayed below it for a full
 * window of steps.  [SP, "Master weights and the optimizer step"]: in 16
 * bits such an add changes nothing at all.
 *
 * Per element, with w_F = RNE_F(w) the narrow copy (F = bf16 or fp16, IEEE
 * overflow) and step = F's grid spacing in |w_F|'s binade (the subnormal
 * spacing below the normal range): excluded if w or d is not finite or w_F
 * overflows; zero if d == 0; otherwise considered, below if |d| < step, and
 * a no-op if RNE_F(w_F + d) == w_F for the exact sum.  Counts add into
 * out[j]; flags (if given) are written per element.  A read-only pass:
 * 8 bytes per element in (+1 with flags).  ws: nc_swamp_workspace_bytes(t,
 * count) bytes (at most 64 B per 8192 elements), 16-byte aligned. */
size_t nc_swamp_workspace_bytes(const nc_update_tensor *t, int32_t count);
nc_status nc_swamp_watch(const nc_update_tensor *t, int32_t count, nc_wfmt wfmt, nc_swamp_counts *out,
                         void *ws, size_t ws_bytes, void *stream);

/* One step of the promotion rule for `count` tensors: st[j] from in[j] (the
 * counts of this step) under the policy: run = run + 1 if the step is below,
 * else 0; promoted = promoted or run >= window; steps += 1. */
nc_status nc_swamp_window(const nc_swamp_policy *policy, int32_t count, nc_swamp_state *st,
                          const nc_swamp_counts *in, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* NARROWCAST_H */
