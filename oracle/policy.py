"""Tier 0: the scale-update state machine and the loss-scale machine.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the pages fix:

* [E3, "Worked solution"]: track each tensor's largest magnitude across a
  span of recent steps; choose the biggest power-of-two scale under which
  that maximum, with a margin, still fits the format; recompute at a fixed
  step interval; leave the scale unchanged when the recomputed one is
  within a factor of two of it.
* [MaxWin, "Experimental Variables"]: the estimators -- most recent (the
  previous step's amax), a maximum over a window of recent steps (64 there),
  exponential smoothing, and current scaling (this step's own amax, which
  has to read the data one extra time).  The smoothing coefficient and the
  arithmetic are not given; read here as E <- E + alpha (a - E) in fp32 with
  each operation rounded to nearest even (no fused multiply-add), E = a at
  the first push.  [MaxWin, "Key Contributions"]: the
  window maximum guarantees no scale-induced saturation for a step whose amax
  is within the window.  A warmup fills the history before quantisation.
* [MP-card, item (1)]: dynamic loss scaling halves S and skips the step on an
  Inf/NaN, and doubles S once enough steps have passed with no overflow.

Readings adopted where the pages are silent or loose:

* Timing (delayed scaling): the history receives amax_t after step t's cast;
  the scale for step t+1 is computed from the last W pushes.  A step whose
  history is empty is cast with current scaling (the caller runs the amax
  pass first and calls ``update`` with est='current'), standing in for the
  warmup that fills the history.
* Current scaling sets k from the amax passed in, recomputing every call; it
  neither reads nor writes the history or the step counter.
* Interval I: with delayed estimators, after the push of step t the scale is
  recomputed when (t + 1) is a multiple of I (the step counter counts pushes).
* Hysteresis.  Read literally (no change within a factor of two) the rule
  is vacuous for power-of-two scales, which always differ by at least two.  Adopted per tensor: keep a_ref, the estimate at the last change of k.
  At a recompute with estimate A:
    (i)  if A * 2^k exceeds M_F * 2^-margin, k is reset from A (a forced
         decrease, so the scale never overflows at the estimate);
    (ii) else if A <= a_ref / 2 (the ideal scale has at least doubled since
         the last change), k is reset from A;
    (iii) else k is kept.
  A reset also sets a_ref = A.  The first recompute on a fresh state resets
  unconditionally.  Pinned by brute-force properties and by traces worked
  by hand from this reading (tests/golden/scale_update_hand.json).
* Skip: when skipping on non-finite is enabled and any tensor of the batch
  saw a non-finite element, the whole step is skipped -- no tensor's history,
  step counter or scale changes.  (The loss-scale machine still runs.)
* The loss-scale machine runs only when enabled; S = 2^s with s clamped to
  [s_min, s_max]; the overflow-free stretch before a doubling is the growth
  interval in clean steps.
"""

from dataclasses import dataclass, field
from fractions import Fraction
from typing import List

from .cast import scale_exponent
from .formats import FP32, Fmt, pow2

EST_CURRENT, EST_MOST_RECENT, EST_MAX_WINDOW, EST_EMA = "current", "most_recent", "max_window", "ema"


@dataclass
class Policy:
    fmt: Fmt
    est: str = EST_MAX_WINDOW
    window: int = 16
    margin: int = 0
    hysteresis: bool = True
    interval: int = 1
    skip_on_nonfinite: bool = False
    ls_enable: bool = False
    ls_growth_interval: int = 2000
    ls_log2_min: int = 0
    ls_log2_max: int = 24
    ema_alpha: Fraction = Fraction(1, 16)     # an fp32 value in (0, 1]


@dataclass
class ScaleState:
    """Per-tensor state.  A zeroed state is a fresh one."""
    k: int = 0
    a_ref: Fraction = Fraction(0)
    has_ref: bool = False
    hist: List[Fraction] = field(default_factory=list)   # oldest first, at most W
    step: int = 0


@dataclass
class LossScale:
    s_log2: int = 16
    clean_steps: int = 0


def set_scale(policy: Policy, st: ScaleState, a: Fraction) -> None:
    """Apply the scale rule with hysteresis to estimate a (readings above)."""
    fmt, margin = policy.fmt, policy.margin
    k_new = scale_exponent(fmt, a, margin)
    if not policy.hysteresis or not st.has_ref:
        reset = True
    elif a * pow2(st.k) > fmt.maxval * pow2(-margin):     # (i) overflow at the estimate
        reset = True
    elif 2 * a <= st.a_ref:                                # (ii) ideal scale doubled
        reset = True
    else:                                                  # (iii) keep
        reset = False
    if reset:
        st.k, st.a_ref, st.has_ref = k_new, a, True


def _rn32(v: Fraction) -> Fraction:
    """v rounded to the nearest fp32 value (ties to even; symmetric in sign)."""
    m = FP32.round_mag(abs(v))
    return -m if v < 0 else m


def ema_step(alpha: Fraction, e: Fraction, a: Fraction) -> Fraction:
    """Exponential smoothing ([MaxWin, "Experimental Variables"]) read with a
    defined fp32 operation order: d = rn(a - e), m = rn(alpha * d), result
    rn(e + m) -- three roundings, none fused."""
    d = _rn32(a - e)
    m = _rn32(alpha * d)
    return _rn32(e + m)


def estimate(policy: Policy, st: ScaleState) -> Fraction:
    if policy.est == EST_MOST_RECENT:
        return st.hist[-1]
    if policy.est == EST_MAX_WINDOW:
        return max(st.hist)
    raise ValueError(policy.est)


def update(policy: Policy, states: List[ScaleState], amaxes: List[Fraction],
           nonfinite: List[int], ls: LossScale = None) -> None:
    """One scale update for a batch of tensors, in place.

    amaxes[i] is tensor i's finite amax from the pass just run (the amax pass
    for current scaling, the cast for delayed scaling); nonfinite[i] is its
    count of non-finite elements.
    """
    any_nf = any(n > 0 for n in nonfinite)
    if ls is not None and policy.ls_enable:
        if any_nf:
            ls.s_log2 = max(policy.ls_log2_min, ls.s_log2 - 1)
            ls.clean_steps = 0
        else:
            ls.clean_steps += 1
            if ls.clean_steps >= policy.ls_growth_interval:
                ls.s_log2 = min(policy.ls_log2_max, ls.s_log2 + 1)
                ls.clean_steps = 0
    if policy.est == EST_CURRENT:
        for st, a in zip(states, amaxes):
            set_scale(policy, st, Fraction(a))
        return
    if policy.skip_on_nonfinite and any_nf:
        return
    W = policy.window
    if policy.est == EST_EMA:
        # the smoothed estimate E is the whole history: E = a at the first
        # push, then E <- ema_step(alpha, E, a)
        for st, a in zip(states, amaxes):
            a = Fraction(a)
            st.hist = [ema_step(policy.ema_alpha, st.hist[0], a) if st.hist else a]
            st.step += 1
            if st.step % policy.interval == 0:
                set_scale(policy, st, st.hist[0])
        return
    for st, a in zip(states, amaxes):
        st.hist.append(Fraction(a))
        if len(st.hist) > W:
            st.hist.pop(0)
        st.step += 1
        if st.step % policy.interval == 0:
            set_scale(policy, st, estimate(policy, st))
