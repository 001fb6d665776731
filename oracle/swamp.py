"""The update/step-ratio ("swamping") monitor.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the pages fix:

* [E3, "Worked solution"]: range fails at a format's extremes, while the
  grid spacing is what fails where the weight sits.  So the
  procedure tracks, beside the amax, how large each update is compared with
  the grid spacing at its weight; a wide master copy is kept while updates
  are smaller than that spacing, and a tensor moves to a wider format once
  its updates have stayed under the spacing for a full window of steps.  The
  page's example is a weight of 1.0 that an update of 0.001 leaves unchanged.
* [SP, "Master weights and the optimizer step"]: late in training a weight
  of order 1 meets updates of order 1e-7; in 16 bits the add is exactly a
  no-op, in 32 bits the update lands.

Readings where the pages are silent:

* The watched copy of a weight is w_F = RNE_F(w), the fp32 master w rounded
  to the narrow weight format F (bf16 or fp16).  "The step at the weight" is
  F's grid spacing in |w_F|'s binade: 2^(e - mbits), or the subnormal
  spacing below the normal range (zero included).
* Per element, with d the fp32 update:
    excluded   w or d is not finite, or w_F overflows F;
    zero       d == 0 (either sign);
    below      0 < |d| < step_F(w_F)                  (the ratio is below one);
    no-op      d != 0 and RNE_F(w_F + d) == w_F        (the exact sum, rounded
               once, compared as values: the narrow add leaves the weight).
  "Considered" elements are those neither excluded nor zero.
* Window: a tensor's step counts as "below" when it has considered elements
  and n_below * den >= num * n_considered (a threshold num/den, 1/2 meaning
  at least half of its updates).  `run` counts consecutive below steps; at
  run >= window the tensor is promoted, and stays promoted (a widened format
  is not narrowed again by this rule).
"""

from dataclasses import dataclass
from fractions import Fraction

import numpy as np

from .formats import BF16, FP16, Fmt, Val, floor_log2, pow2

WFORMATS = {"bf16": BF16, "fp16": FP16}


def step_at(fmt: Fmt, mag: Fraction) -> Fraction:
    """F's grid spacing in the binade of a magnitude on F's grid."""
    e = floor_log2(mag) if mag != 0 else fmt.emin
    return pow2(max(e, fmt.emin) - fmt.mbits)


def element(fmt: Fmt, w: Val, d: Val):
    """Tier 0: (below, noop, zero, excluded) for one weight/update pair."""
    if not (w.finite and d.finite):
        return False, False, False, True
    r = fmt.round_mag(w.mag)
    if r > fmt.maxval:
        return False, False, False, True
    wf = -r if w.neg else r
    if d.mag == 0:
        return False, False, True, False
    dv = d.signed
    below = d.mag < step_at(fmt, r)
    s = wf + dv
    rs = fmt.round_mag(abs(s))
    moved = (rs > fmt.maxval) or ((-rs if s < 0 else rs) != wf)
    return below, not moved, False, False


def watch(fmt: Fmt, ws, ds):
    """Tier 0 over a tensor: (flags, counts).  flags[i] = below | noop << 1 |
    zero << 2 | excluded << 3."""
    flags = []
    c = dict(n_considered=0, n_zero=0, n_below=0, n_noop=0, n_excluded=0)
    for w, d in zip(ws, ds):
        b, n, z, x = element(fmt, w, d)
        flags.append(int(b) | int(n) << 1 | int(z) << 2 | int(x) << 3)
        c["n_below"] += b
        c["n_noop"] += n
        c["n_zero"] += z
        c["n_excluded"] += x
    c["n_considered"] = len(flags) - c["n_zero"] - c["n_excluded"]
    return flags, c


def _round_to(fmt: Fmt, v: np.ndarray) -> np.ndarray:
    """RNE of binary64 values onto F with IEEE overflow, as binary64."""
    if fmt is FP16:
        with np.errstate(over="ignore"):
            return v.astype(np.float16).astype(np.float64)
    from .bulk import bf16_bits_to_f64, round_bf16_bits
    return bf16_bits_to_f64(round_bf16_bits(v))


def watch_f64(fmt: Fmt, w: np.ndarray, d: np.ndarray):
    """Tier 1 (numpy): the same flags and counts.  w and d hold fp32 values
    in binary64.  The sum w_F + d is formed in binary64 before the one
    rounding to F: it is exact whenever the two are within 29 binades, and
    otherwise the smaller addend is far below half a step of the larger, so
    the no-op decision cannot change."""
    w = np.asarray(w, dtype=np.float64)
    d = np.asarray(d, dtype=np.float64)
    fin = np.isfinite(w) & np.isfinite(d)
    wf = _round_to(fmt, np.where(fin, w, 0.0))
    excl = ~fin | ~np.isfinite(wf)
    wf = np.where(excl, 0.0, wf)
    zero = ~excl & (d == 0)
    cons = ~excl & ~zero
    a = np.abs(wf)
    _, ex = np.frexp(a)
    e = np.where(a == 0, fmt.emin, ex.astype(np.int64) - 1)
    step = np.ldexp(1.0, np.maximum(e, fmt.emin) - fmt.mbits)
    dd = np.where(cons, d, 0.0)
    below = cons & (np.abs(dd) < step)
    with np.errstate(over="ignore", invalid="ignore"):
        moved = _round_to(fmt, wf + dd) != wf
    noop = cons & ~moved
    flags = (below.astype(np.uint8) | noop.astype(np.uint8) << 1 | zero.astype(np.uint8) << 2
             | excl.astype(np.uint8) << 3)
    c = dict(n_considered=int(cons.sum()), n_zero=int(zero.sum()), n_below=int(below.sum()),
             n_noop=int(noop.sum()), n_excluded=int(excl.sum()))
    return flags, c


@dataclass
class WindowPolicy:
    window: int = 8
    num: int = 1
    den: int = 2


@dataclass
class WindowState:
    run: int = 0
    promoted: int = 0
    steps: int = 0


def window_step(p: WindowPolicy, s: WindowState, counts: dict) -> WindowState:
    """One step of the promotion rule for one tensor."""
    n = counts["n_considered"]
    below = n > 0 and counts["n_below"] * p.den >= p.num * n
    run = s.run + 1 if below else 0
    return WindowState(run=run, promoted=1 if (s.promoted or run >= p.window) else 0, steps=s.steps + 1)
