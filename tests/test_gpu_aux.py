"""GPU parity of the scale-update state machine, dequant and the error
statistics (fused into the casts and as a separate pass)."""

import itertools
from fractions import Fraction

import numpy as np
import pytest
import torch

import scaled_fp8_casting_amd as nc
from oracle import E4M3, E5M2
from oracle import bulk
from oracle import cast as t0
from oracle.policy import EST_CURRENT, LossScale, Policy, ScaleState, update
import workloads
from tests._gpu import (assert_counts, codes_like, dev_bf16, dev_f32, host_u16, host_u8, state_with_k,
                        stats_close)

pytestmark = pytest.mark.gpu
FMTS = [("e4m3", E4M3), ("e5m2", E5M2)]


def _f32_bits(v: float) -> int:
    return int(np.array([v], dtype=np.float32).view(np.uint32)[0])


def _counts_from_amax(amaxes, nonfinite=None):
    c = nc.new_counts(len(amaxes))
    c[:, 4] = torch.tensor([_f32_bits(float(a)) for a in amaxes], dtype=torch.int64)
    if nonfinite is not None:
        c[:, 3] = torch.tensor(nonfinite, dtype=torch.int64)
    return c


# -- scale update ------------------------------------------------------------------

VALUES = [Fraction(2) ** j * m for j in (-1, 0, 1) for m in (Fraction(1), Fraction(3, 2), Fraction(7, 4), Fraction(15, 8))]


def _hand_traces():
    from tests.conftest import load_golden
    return load_golden("scale_update_hand.json")["traces"]


@pytest.mark.parametrize("tr", _hand_traces(), ids=lambda t: t["name"])
def test_scale_update_hand_worked_traces(tr):
    """The device state machine through the traces worked by hand from the
    readings (tests/golden/scale_update_hand.json), compared with the hand
    values directly: k and the reference estimate (as fp32) after every
    step, and the loss scale where the trace runs it.  Each amax is passed
    as the nearest fp32 value; the hand derivations hold for those too
    (doubling an fp32 value is exact, so the halving comparisons are
    unchanged)."""
    p = dict(tr["policy"])
    st = nc.new_state(1)
    hist = nc.new_history(1, p["window"])
    ls = nc.new_loss_scale(tr["loss_scale"]["s_log2"]) if "loss_scale" in tr else None
    pol_cur = nc.policy(**{**p, "est": "current"})
    nc.nc_scale_update(pol_cur, st, _counts_from_amax([Fraction(tr["start"]["amax"])]))
    pol = nc.policy(**p)
    rows = [tr["start"]] + tr["steps"]
    for i, w in enumerate(rows):
        if i > 0:
            nc.nc_scale_update(pol, st, _counts_from_amax([Fraction(w["amax"])], [w.get("nonfinite", 0)]), hist, ls)
        got = st.cpu().numpy()[0]
        assert int(got[0]) == w["k"], (tr["name"], i, w)
        if "a_ref" in w:
            assert int(np.array([got[1]]).view(np.uint32)[0]) == _f32_bits(float(Fraction(w["a_ref"]))), (tr["name"], i)
        if i > 0 and "s_log2" in w:
            assert ls.cpu().tolist() == [w["s_log2"], w["clean_steps"]], (tr["name"], i)


@pytest.mark.parametrize("name,fmt", FMTS)
def test_scale_update_brute_force(name, fmt):
    """Every amax sequence of length 3 over 12 values (one tensor each, all
    in one batch), W in {1, 2, 3}, hysteresis on/off, both delayed
    estimators: GPU state after every step equals the oracle's."""
    seqs = list(itertools.product(VALUES, repeat=3))
    T = len(seqs)
    for W, hyst, est in itertools.product((1, 2, 3), (False, True), ("most_recent", "max_window")):
        pol_o = Policy(fmt=fmt, est=est, window=W, hysteresis=hyst)
        pol_c = Policy(fmt=fmt, est=EST_CURRENT, window=W, hysteresis=hyst)
        sts = [ScaleState() for _ in seqs]
        update(pol_c, sts, [s[0] for s in seqs], [0] * T)
        st = nc.new_state(T)
        hist = nc.new_history(T, W)
        nc.nc_scale_update(nc.policy(name, "current", W, hysteresis=hyst), st, _counts_from_amax([s[0] for s in seqs]))
        for step in range(3):
            amaxes = [s[step] for s in seqs]
            update(pol_o, sts, amaxes, [0] * T)
            nc.nc_scale_update(nc.policy(name, est, W, hysteresis=hyst), st, _counts_from_amax(amaxes), hist)
            got = st.cpu().numpy()
            want_k = np.array([s.k for s in sts])
            want_ref = np.array([_f32_bits(float(s.a_ref)) for s in sts], dtype=np.uint32)
            assert np.array_equal(got[:, 0], want_k), (W, hyst, est, step)
            assert np.array_equal(got[:, 1].view(np.uint32), want_ref)
            assert np.all(got[:, 5] == step + 1) and np.all(got[:, 3] == min(step + 1, W))


def test_scale_update_edges_interval_skip_loss_scale():
    pol_o = Policy(fmt=E4M3, est="max_window", window=4, hysteresis=True, interval=2,
                   skip_on_nonfinite=True, ls_enable=True, ls_growth_interval=3, ls_log2_min=2, ls_log2_max=18)
    pol_d = nc.policy("e4m3", "max_window", 4, hysteresis=True, interval=2, skip_on_nonfinite=True,
                      ls_enable=True, ls_growth_interval=3, ls_log2_min=2, ls_log2_max=18)
    rng = np.random.default_rng(2)
    T = 300                                     # more tensors than threads in the update kernel
    sts = [ScaleState() for _ in range(T)]
    ls_o = LossScale(s_log2=17)
    st = nc.new_state(T)
    hist = nc.new_history(T, 4)
    ls = nc.new_loss_scale(17)
    for step in range(40):
        am = [Fraction(float(np.float32(v))) for v in 10.0 ** rng.uniform(-45, 38, T)]
        am[step % T] = Fraction(0)
        nf = [0] * T
        if step % 7 == 3:
            nf[rng.integers(0, T)] = 5
        update(pol_o, sts, am, nf, ls_o)
        nc.nc_scale_update(pol_d, st, _counts_from_amax(am, nf), hist, ls)
        got = st.cpu().numpy()
        assert np.array_equal(got[:, 0], [s.k for s in sts]), step
        assert ls.cpu().tolist() == [ls_o.s_log2, ls_o.clean_steps]


@pytest.mark.parametrize("margin", [0, 2])
def test_scale_rule_extremes(margin):
    am = [Fraction(0), Fraction(1, 2 ** 149), Fraction(7, 2 ** 149), Fraction(float(np.float32(3e38))),
          Fraction(448), Fraction(449), Fraction(57344), Fraction(7, 2), Fraction(7, 2) + Fraction(1, 2 ** 21)]
    for name, fmt in FMTS:
        st = nc.new_state(len(am))
        nc.nc_scale_update(nc.policy(name, "current", hysteresis=False, margin=margin), st, _counts_from_amax(am))
        got = st[:, 0].cpu().tolist()
        assert got == [t0.scale_exponent(fmt, a, margin) for a in am]


# -- dequant --------------------------------------------------------------------------

@pytest.mark.parametrize("name,fmt", FMTS)
def test_dequant_per_tensor_every_code_every_k(name, fmt):
    ks = list(range(-127, 128))
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).repeat(33).cuda()   # ragged: 8448
    ys = [torch.empty(codes.numel(), dtype=torch.bfloat16, device="cuda") for _ in ks]
    nc.nc_dequant([codes] * len(ks), ys, name, st=state_with_k(ks))
    torch.cuda.synchronize()
    cnp = host_u8(codes)
    for k, y in zip(ks, ys):
        assert np.array_equal(host_u16(y), bulk.dequant_bf16_f64(fmt, cnp, k)), k


@pytest.mark.parametrize("name,fmt", FMTS)
def test_dequant_mx(name, fmt):
    rng = np.random.default_rng(1)
    n, cols = 32 * 1000 + 8192, 64
    n -= n % cols
    codes = rng.integers(0, 256, n).astype(np.uint8)
    scales = rng.integers(0, 255, n // 32).astype(np.uint8)
    scales[:8] = [0, 1, 254, 253, 127, 126, 128, 2]
    y = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    nc.nc_dequant([torch.from_numpy(codes).cuda()], [y], name,
                  scales=[torch.from_numpy(scales).cuda()], cols=[cols])
    torch.cuda.synchronize()
    K = np.repeat(127 - scales.astype(np.int64), 32)
    assert np.array_equal(host_u16(y), bulk.dequant_bf16_f64(fmt, codes, K))


# -- statistics ------------------------------------------------------------------------

def _stats_input(dtype, n, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_t(3, n) * 10.0 ** rng.uniform(-3, 3, n)).astype(np.float32)
    x[7], x[9] = np.inf, np.nan
    x[11] = np.float32(3e30)                    # clips far out of range
    if dtype == "bf16":
        bits = workloads.to_bf16_bits(x.astype(np.float64))
        return dev_bf16(bits), bulk.bf16_bits_to_f64(bits)
    return dev_f32(x), x.astype(np.float64)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name,fmt", FMTS)
def test_stats_per_tensor_fused_and_separate(dtype, name, fmt):
    n = 3 * 8192 + 77
    xd, x64 = _stats_input(dtype, n, 3)
    k, s = 4, 3
    ls = nc.new_loss_scale(s)
    codes = codes_like(n)
    out = nc.new_counts(1)
    fused = nc.new_stats(1)
    desc, cnt = nc.tensors([xd], [codes])
    ws = nc.new_workspace(desc, cnt)
    st = state_with_k([k])
    nc.nc_cast_tensor([xd], [codes], name, st, out, ls=ls, stats=fused, ws=ws)
    sep = nc.new_stats(1)
    nc.nc_cast_stats([xd], [codes], name, sep, ws, st=st, ls=ls)
    torch.cuda.synchronize()
    xu = np.ldexp(x64, -s)
    want_codes = bulk.cast_f64(fmt, x64, k - s)[0]
    assert np.array_equal(host_u8(codes), want_codes)
    want = bulk.stats_f64(fmt, xu, want_codes, k)
    stats_close(fused[0].cpu().tolist(), want)
    stats_close(sep[0].cpu().tolist(), want)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rule,off", [("ocp", 0), ("plus1", 0), ("ocp", 5)])
def test_stats_mx_fused_and_separate(dtype, rule, off):
    """Several full tiles and a ragged one; the scale array at a 16-byte
    aligned and at an odd address (the two ways a full tile's scale bytes
    are staged)."""
    rows, cols = 70, 1024
    xd, x64 = _stats_input(dtype, rows * cols, 5)
    n = rows * cols
    codes = codes_like(n)
    scales = torch.empty(n // 32 + 16, dtype=torch.uint8, device="cuda")[off:off + n // 32]
    out = nc.new_counts(1)
    fused = nc.new_stats(1)
    desc, cnt = nc.tensors([xd], [codes])
    ws = nc.new_workspace(desc, cnt)
    nc.nc_cast_mx([xd], [codes], [scales], [cols], "e4m3", rule, out, stats=fused, ws=ws)
    sep = nc.new_stats(1)
    nc.nc_cast_stats([xd], [codes], "e4m3", sep, ws, scales=[scales], cols=[cols])
    torch.cuda.synchronize()
    wc, wsc, _ = bulk.cast_mx_f64(E4M3, x64, cols, rule)
    assert np.array_equal(host_u8(codes), wc) and np.array_equal(host_u8(scales), wsc)
    want = bulk.stats_f64(E4M3, x64, wc, np.repeat(127 - wsc.astype(np.int64), 32))
    stats_close(fused[0].cpu().tolist(), want)
    stats_close(sep[0].cpu().tolist(), want)


def test_stats_batch_of_many_tensors():
    """70 tensors (two launches), ragged sizes, statistics per tensor."""
    rng = np.random.default_rng(6)
    sizes = [int(v) for v in rng.integers(1, 20000, 70)]
    sizes[3] = 0
    xs = [(rng.standard_normal(m) * 10.0 ** rng.uniform(-4, 4)).astype(np.float32) for m in sizes]
    xd = [dev_f32(x) for x in xs]
    codes = [codes_like(m) for m in sizes]
    ks = [int(v) for v in rng.integers(-5, 20, 70)]
    out = nc.new_counts(70)
    stats = nc.new_stats(70)
    desc, cnt = nc.tensors(xd, codes)
    ws = nc.new_workspace(desc, cnt)
    nc.nc_cast_tensor(xd, codes, "e5m2", state_with_k(ks), out, stats=stats, ws=ws)
    torch.cuda.synchronize()
    got = stats.cpu().tolist()
    for i, x in enumerate(xs):
        wc = bulk.cast_f64(E5M2, x.astype(np.float64), ks[i])[0]
        assert np.array_equal(host_u8(codes[i]), wc)
        stats_close(got[i], bulk.stats_f64(E5M2, x.astype(np.float64), wc, ks[i]))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_stats_and_counts_over_many_chunks(dtype):
    """A tensor of more than 1024 workgroup tiles (several chunks in the
    first reduction) plus a tiny one in the same launch: codes, counts and
    both statistics paths against the oracle."""
    rng = np.random.default_rng(8)
    n_big = 3 * 1024 * 2048 + 1234
    xs, x64s = [], []
    for n in (n_big, 100):
        x = (rng.standard_t(4, n) * 10.0 ** rng.uniform(-2, 2, n)).astype(np.float32)
        x[::100003] = np.inf
        if dtype == "bf16":
            bits = workloads.to_bf16_bits(x.astype(np.float64))
            xs.append(dev_bf16(bits))
            x64s.append(bulk.bf16_bits_to_f64(bits))
        else:
            xs.append(dev_f32(x))
            x64s.append(x.astype(np.float64))
    ks = [5, -3]
    codes = [codes_like(x.numel()) for x in xs]
    out, fused, sep = nc.new_counts(2), nc.new_stats(2), nc.new_stats(2)
    st = state_with_k(ks)
    nc.nc_cast_tensor(xs, codes, "e4m3", st, out, stats=fused)
    nc.nc_cast_stats(xs, codes, "e4m3", sep, st=st)
    am = nc.new_counts(2)
    nc.nc_amax(xs, am)
    torch.cuda.synchronize()
    got = nc.counts_list(out)
    got_am = nc.counts_list(am)
    for i, x64 in enumerate(x64s):
        wc, want = bulk.cast_tensor_f64(E4M3, x64, ks[i])
        assert np.array_equal(host_u8(codes[i]), wc), i
        for f in ("n_finite", "n_clip", "n_underflow", "n_nonfinite", "amax"):
            assert got[i][f] == want[f], (i, f, got[i][f], want[f])
        assert got_am[i]["amax"] == want["amax"] and got_am[i]["n_nonfinite"] == want["n_nonfinite"]
        assert got_am[i]["n_clip"] == 0
        ws_ = bulk.stats_f64(E4M3, x64, wc, ks[i])
        stats_close(fused[i].cpu().tolist(), ws_)
        stats_close(sep[i].cpu().tolist(), ws_)


@pytest.mark.parametrize("hyst,interval", [(False, 1), (True, 1), (True, 3)])
def test_scale_update_ema(hyst, interval):
    """Exponential smoothing: per step, the smoothed estimate (history slot 0),
    k, a_ref and the push count against the oracle, for exact and inexact
    fp32 coefficients and amaxes over the whole fp32 range (zeros too)."""
    from oracle.policy import EST_EMA
    rng = np.random.default_rng(31)
    alphas = [np.float32(1 / 16), np.float32(0.1), np.float32(0.9), np.float32(1.0)]
    T = 160                                          # 40 tensors per coefficient
    for j, alpha in enumerate(alphas):
        pol_o = Policy(fmt=E4M3, est=EST_EMA, window=4, hysteresis=hyst, interval=interval,
                       ema_alpha=Fraction(float(alpha)))
        pol_d = nc.policy("e4m3", "ema", 4, hysteresis=hyst, interval=interval, ema_alpha=float(alpha))
        sts = [ScaleState() for _ in range(T)]
        st = nc.new_state(T)
        hist = nc.new_history(T, 4)
        for step in range(50):
            am = (10.0 ** rng.uniform(-44, 38, T)).astype(np.float32)
            am[rng.integers(0, T, 5)] = 0.0
            amx = [Fraction(float(v)) for v in am]
            update(pol_o, sts, amx, [0] * T)
            nc.nc_scale_update(pol_d, st, _counts_from_amax(am), hist)
            g = st.cpu().numpy()
            e = hist[:, 0].cpu().numpy().view(np.uint32)
            assert np.array_equal(g[:, 0], [s.k for s in sts]), (alpha, step)
            assert np.array_equal(e, [_f32_bits(float(s.hist[0])) for s in sts]), (alpha, step)
            assert np.array_equal(g[:, 1].view(np.uint32), [_f32_bits(float(s.a_ref)) for s in sts])
            assert np.all(g[:, 5] == step + 1) and np.all(g[:, 3] == 1)


# -- MX, blocks down the columns ---------------------------------------------------

@pytest.mark.parametrize("name,fmt", FMTS)
@pytest.mark.parametrize("rows,cols", [(32, 32), (64, 96), (160, 2080)])
def test_dequant_mx_column_blocks(name, fmt, rows, cols):
    """Every code under random scale bytes (and the extremes), column
    layout; ragged last tiles; output guarded against writes past the end;
    scale arrays at an aligned and an odd offset."""
    rng = np.random.default_rng(rows + cols)
    n = rows * cols
    codes = rng.integers(0, 256, n).astype(np.uint8)
    codes[:256] = np.arange(256)
    scales = rng.integers(0, 256, n // 32).astype(np.uint8)
    scales[:8] = [0, 1, 254, 253, 127, 126, 128, 255]
    K = -bulk.mx_element_exponents(scales.astype(np.int64) - 127, n, cols, "cols")
    want = bulk.dequant_bf16_f64(fmt, codes, K)
    for off in (0, 3):
        sbig = torch.zeros(n // 32 + 8, dtype=torch.uint8, device="cuda")
        sbig[off:off + n // 32] = torch.from_numpy(scales).cuda()
        ybig = torch.full((n + 64,), -7.0, dtype=torch.bfloat16, device="cuda")
        nc.nc_dequant([torch.from_numpy(codes).cuda()], [ybig[:n]], name,
                      scales=[sbig[off:off + n // 32]], cols=[cols], axis="cols")
        torch.cuda.synchronize()
        y = host_u16(ybig)
        assert np.array_equal(y[:n], want), off
        assert np.all(ybig[n:].float().cpu().numpy() == -7.0), off


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rule", ["ocp", "ceil"])
def test_stats_mx_column_blocks_fused_and_separate(dtype, rule):
    rows, cols = 96, 1056
    n = rows * cols
    xd, x64 = _stats_input(dtype, n, 8)
    codes = codes_like(n)
    scales = torch.empty(n // 32, dtype=torch.uint8, device="cuda")
    out = nc.new_counts(1)
    fused = nc.new_stats(1)
    desc, cnt = nc.tensors([xd], [codes])
    ws = nc.new_workspace(desc, cnt)
    nc.nc_cast_mx([xd], [codes], [scales], [cols], "e5m2", rule, out, stats=fused, ws=ws, axis="cols")
    sep = nc.new_stats(1)
    nc.nc_cast_stats([xd], [codes], "e5m2", sep, ws, scales=[scales], cols=[cols], axis="cols")
    torch.cuda.synchronize()
    wc, wsc, wn = bulk.cast_mx_f64(E5M2, x64, cols, rule, axis="cols")
    assert np.array_equal(host_u8(codes), wc) and np.array_equal(host_u8(scales), wsc)
    assert_counts(nc.counts_list(out)[0], wn)
    K = -bulk.mx_element_exponents(wsc.astype(np.int64) - 127, n, cols, "cols")
    want = bulk.stats_f64(E5M2, x64, wc, K)
    stats_close(fused[0].cpu().tolist(), want)
    stats_close(sep[0].cpu().tolist(), want)
