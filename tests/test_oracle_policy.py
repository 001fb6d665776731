"""Properties of the scale-update state machine and the loss-scale machine,
and hand-worked traces of it.

The pages' hysteresis rule is ambiguous for power-of-two scales; the
reading taken (R7: a forced decrease whenever the kept scale would overflow
at the estimate, a reset when the estimate is at most half the estimate at
the last change, otherwise keep) is pinned by brute-force properties and by
traces worked by hand from that reading (tests/golden/scale_update_hand.json),
which planted mistakes in the oracle fail."""

import itertools
from fractions import Fraction

import pytest

from oracle import E4M3, E5M2
from oracle import cast as t0
from oracle import policy as pol_mod
from oracle.formats import pow2
from oracle.policy import (EST_CURRENT, EST_MAX_WINDOW, EST_MOST_RECENT, LossScale, Policy,
                           ScaleState, update)
from tests.conftest import load_golden

HAND = load_golden("scale_update_hand.json")
FMTS = {"e4m3": E4M3, "e5m2": E5M2}

VALUES = [pow2(j) * m for j in (-1, 0, 1) for m in (Fraction(1), Fraction(3, 2), Fraction(7, 4), Fraction(15, 8))]


def _run(policy, seq):
    """Step 0 by current scaling, then delayed updates; returns the k used at
    each step and the state snapshots before each recompute."""
    st = ScaleState()
    cur = Policy(**{**policy.__dict__, "est": EST_CURRENT})
    update(cur, [st], [seq[0]], [0])
    ks = [st.k]
    trace = []
    for a in seq:
        before = (st.k, st.a_ref)
        update(policy, [st], [a], [0])
        trace.append((before, (st.k, st.a_ref), list(st.hist)))
        ks.append(st.k)
    return ks, trace


@pytest.mark.parametrize("fmt", [E4M3, E5M2], ids=["e4m3", "e5m2"])
def test_brute_force_properties(fmt):
    """Every amax sequence of length 4 over 8 values (the mantissas 1, 1.75,
    1.875 that straddle the rule's threshold, and 1.5, over three binades,
    thinned), W in {1, 2, 3},
    hysteresis on/off, both delayed estimators:
    (i) the scale never overflows at the estimate it was computed from;
    (ii) k rises only when the estimate is at most half of a_ref;
    (iii) without hysteresis, k is the plain rule on the estimate."""
    for W, hyst, est in itertools.product((1, 2, 3), (False, True), (EST_MOST_RECENT, EST_MAX_WINDOW)):
        pol = Policy(fmt=fmt, est=est, window=W, hysteresis=hyst)
        for seq in itertools.product(VALUES[1:9], repeat=4):
            _, trace = _run(pol, seq)
            for (k0, aref0), (k1, aref1), hist in trace:
                A = hist[-1] if est == EST_MOST_RECENT else max(hist)
                assert len(hist) <= W
                assert A * pow2(k1) <= fmt.maxval                       # (i)
                if hyst and k1 > k0:
                    assert 2 * A <= aref0                               # (ii)
                if not hyst:
                    assert k1 == t0.scale_exponent(fmt, A)              # (iii)
                if k1 != k0:
                    assert aref1 == A


def test_window_guarantee():
    """[MaxWin, "Key Contributions"]: with the window maximum, a step whose
    amax does not exceed the maximum of the window it was scaled from does
    not clip (amax_t * 2^k_t <= M_F), with or without hysteresis."""
    for hyst in (False, True):
        pol = Policy(fmt=E4M3, est=EST_MAX_WINDOW, window=3, hysteresis=hyst)
        for seq in itertools.product(VALUES[::2], repeat=5):
            ks, trace = _run(pol, seq)
            for t in range(1, len(seq)):
                window = trace[t - 1][2]
                if seq[t] <= max(window):
                    assert seq[t] * pow2(ks[t]) <= E4M3.maxval


def test_most_recent_saturates_on_a_spike():
    """[MaxWin, "Key Contributions"]: the most-recent estimator saturates one
    step after a quiet step that follows a spike -- and the window maximum
    does not."""
    seq = [Fraction(1)] * 4 + [Fraction(100)] + [Fraction(1)] + [Fraction(100)]
    mr = Policy(fmt=E4M3, est=EST_MOST_RECENT, window=16, hysteresis=False)
    mw = Policy(fmt=E4M3, est=EST_MAX_WINDOW, window=16, hysteresis=False)
    ks_mr, _ = _run(mr, seq)
    ks_mw, _ = _run(mw, seq)
    over_mr = [a * pow2(k) > E4M3.maxval for a, k in zip(seq, ks_mr)]
    over_mw = [a * pow2(k) > E4M3.maxval for a, k in zip(seq, ks_mw)]
    assert over_mr == [False, False, False, False, True, False, True]
    assert over_mw == [False, False, False, False, True, False, False]


def test_hysteresis_keeps_scale_within_a_factor_of_two():
    pol = Policy(fmt=E4M3, est=EST_MOST_RECENT, window=1, hysteresis=True)
    ks, _ = _run(pol, [Fraction(1), Fraction(3, 4), Fraction(5, 8), Fraction(1, 2), Fraction(1, 4)])
    # 1 -> k=8; 0.75 and 0.625 keep k (ideal scale less than doubled);
    # 0.5 = a_ref / 2 resets to k=9; 0.25 = 0.5 / 2 resets to k=10
    assert ks == [8, 8, 8, 8, 9, 10]


def test_interval_recomputes_every_I_steps():
    pol = Policy(fmt=E4M3, est=EST_MOST_RECENT, window=1, hysteresis=False, interval=3)
    seq = [Fraction(1), Fraction(4), Fraction(16), Fraction(64), Fraction(1), Fraction(1), Fraction(1)]
    ks, _ = _run(pol, seq)
    # pushes 1..7; recompute after pushes 3 and 6 (a = 16, then 1)
    assert ks == [8, 8, 8, 4, 4, 4, 8, 8]


def test_skip_and_loss_scale_machine():
    pol = Policy(fmt=E4M3, est=EST_MAX_WINDOW, window=4, hysteresis=False, skip_on_nonfinite=True,
                 ls_enable=True, ls_growth_interval=3, ls_log2_min=2, ls_log2_max=18)
    sts = [ScaleState(), ScaleState()]
    ls = LossScale(s_log2=17)
    update(Policy(**{**pol.__dict__, "est": EST_CURRENT}), sts, [Fraction(1), Fraction(2)], [0, 0])
    update(pol, sts, [Fraction(1), Fraction(2)], [0, 0], ls)          # clean 1
    assert ls.s_log2 == 17 and ls.clean_steps == 1 and sts[0].step == 1
    update(pol, sts, [Fraction(1000), Fraction(2)], [0, 5], ls)       # overflow: halve, skip
    assert ls.s_log2 == 16 and ls.clean_steps == 0
    assert sts[0].step == 1 and sts[0].hist == [Fraction(1)] and sts[0].k == 8
    for _ in range(3):
        update(pol, sts, [Fraction(1), Fraction(2)], [0, 0], ls)
    assert ls.s_log2 == 17 and ls.clean_steps == 0 and sts[0].step == 4
    for _ in range(6):
        update(pol, sts, [Fraction(1), Fraction(2)], [0, 0], ls)
    assert ls.s_log2 == 18                                              # clamped at max
    for _ in range(20):
        update(pol, sts, [Fraction(1), Fraction(2)], [1, 0], ls)
    assert ls.s_log2 == 2                                               # clamped at min
    # without skipping, the finite amax is still pushed on a flagged step
    pol2 = Policy(fmt=E4M3, est=EST_MAX_WINDOW, window=4, hysteresis=False)
    st = ScaleState()
    update(pol2, [st], [Fraction(3)], [7])
    assert st.hist == [Fraction(3)] and st.step == 1


def test_zero_amax_and_fresh_state():
    pol = Policy(fmt=E4M3, est=EST_MOST_RECENT, window=2, hysteresis=True)
    ks, _ = _run(pol, [Fraction(0), Fraction(0), Fraction(3)])
    assert ks[:3] == [127, 127, 127] and ks[3] == t0.scale_exponent(E4M3, Fraction(3))


# -- exponential smoothing ----------------------------------------------------

def test_ema_step_against_numpy_float32():
    """ema_step (exact rationals, rounded to fp32 after each operation)
    against numpy's own float32 arithmetic (IEEE single, nearest even, no
    fused multiply-add) on random sequences and coefficients."""
    import numpy as np
    from oracle.policy import ema_step
    rng = np.random.default_rng(5)
    for alpha in (np.float32(1 / 16), np.float32(0.1), np.float32(0.9), np.float32(1.0), np.float32(1e-3)):
        a_seq = (10.0 ** rng.uniform(-40, 38, 400)).astype(np.float32)
        a_seq[::37] = 0.0
        e_np = a_seq[0]
        e_or = Fraction(float(a_seq[0]))
        for a in a_seq[1:]:
            e_np = np.float32(e_np + np.float32(alpha * np.float32(a - e_np)))
            e_or = ema_step(Fraction(float(alpha)), e_or, Fraction(float(a)))
            assert Fraction(float(e_np)) == e_or, (alpha, a)


def test_ema_worked_values_and_properties():
    from oracle.policy import EST_EMA, ema_step
    assert ema_step(Fraction(1, 2), Fraction(4), Fraction(2)) == 3
    assert ema_step(Fraction(1, 4), Fraction(8), Fraction(0)) == 6
    assert ema_step(Fraction(1, 16), Fraction(5), Fraction(5)) == 5             # constant input stays
    # the estimate stays between the smallest and largest amax seen; with
    # hysteresis off k is the rule applied to it at every recompute
    pol = Policy(fmt=E4M3, est=EST_EMA, window=1, hysteresis=False, ema_alpha=Fraction(1, 8))
    st = [ScaleState()]
    seq = [Fraction(2) ** j * m for j, m in zip((3, -2, 5, 0, 1, 7, -4), (1, Fraction(3, 2), 1, Fraction(7, 4), 1, 1, Fraction(5, 4)))]
    for i, a in enumerate(seq):
        update(pol, st, [a], [0])
        assert min(seq[:i + 1]) <= st[0].hist[0] <= max(seq[:i + 1])
        assert st[0].k == t0.scale_exponent(E4M3, st[0].hist[0])
        assert len(st[0].hist) == 1 and st[0].step == i + 1


# -- hand-worked traces -------------------------------------------------------------

def _policy(d):
    kw = {k: v for k, v in d.items() if k not in ("fmt",)}
    return Policy(fmt=FMTS[d["fmt"]], **kw)


def run_hand_trace(tr):
    """The oracle through one golden trace: step 0 by current scaling (no
    loss-scale step), then the delayed updates.  Returns per step (k, a_ref,
    s_log2, clean_steps)."""
    pol = _policy(tr["policy"])
    cur = Policy(**{**pol.__dict__, "est": EST_CURRENT})
    st = ScaleState()
    update(cur, [st], [Fraction(tr["start"]["amax"])], [0])
    out = [(st.k, st.a_ref, None, None)]
    ls = LossScale(**tr["loss_scale"]) if "loss_scale" in tr else None
    for s in tr["steps"]:
        update(pol, [st], [Fraction(s["amax"])], [s.get("nonfinite", 0)], ls)
        out.append((st.k, st.a_ref, ls.s_log2 if ls else None, ls.clean_steps if ls else None))
    return out


def hand_trace_mismatches(tr):
    got = run_hand_trace(tr)
    want = [tr["start"]] + tr["steps"]
    bad = []
    for i, (g, w) in enumerate(zip(got, want)):
        if g[0] != w["k"] or ("a_ref" in w and g[1] != Fraction(w["a_ref"])):
            bad.append((i, g[:2], w))
        if "s_log2" in w and i > 0 and (g[2] != w["s_log2"] or g[3] != w["clean_steps"]):
            bad.append((i, g[2:], w))
    return bad


@pytest.mark.parametrize("tr", HAND["traces"], ids=[t["name"] for t in HAND["traces"]])
def test_hand_worked_traces(tr):
    """The scale exponent, the reference estimate and the loss scale after
    every step equal the values worked by hand from the readings."""
    assert hand_trace_mismatches(tr) == []


def _set_scale_variant(kind):
    """set_scale with one plausible mistake planted."""
    def f(policy, st, a):
        fmt, margin = policy.fmt, policy.margin
        k_new = t0.scale_exponent(fmt, a, margin)
        over = a * pow2(st.k) > fmt.maxval * pow2(-margin)
        half = (2 * a < st.a_ref) if kind == "strict_half" else (2 * a <= st.a_ref)
        if kind == "no_forced_decrease":
            over = False
        reset = (not policy.hysteresis) or (not st.has_ref) or over or half
        if reset:
            st.k, st.a_ref, st.has_ref = k_new, a, True
        elif kind == "ref_every_recompute":
            st.a_ref = a
    return f


@pytest.mark.parametrize("kind", ["strict_half", "no_forced_decrease", "ref_every_recompute",
                                  "window_off_by_one", "interval_ignored"])
def test_hand_traces_catch_planted_mistakes(kind, monkeypatch):
    """Each planted mistake in the state machine changes at least one value
    of the hand-worked traces."""
    if kind == "window_off_by_one":
        real = pol_mod.estimate
        monkeypatch.setattr(pol_mod, "estimate",
                            lambda p, st: max(st.hist[1:] or st.hist) if p.est == EST_MAX_WINDOW else real(p, st))
    elif kind == "interval_ignored":
        def every_step(policy, states, amaxes, nonfinite, ls=None):
            return pol_mod.update(Policy(**{**policy.__dict__, "interval": 1}), states, amaxes, nonfinite, ls)
        monkeypatch.setitem(globals(), "update", every_step)
    else:
        monkeypatch.setattr(pol_mod, "set_scale", _set_scale_variant(kind))
    assert any(hand_trace_mismatches(tr) for tr in HAND["traces"]), kind
