"""GPU parity on the full workloads, in the launch configurations the
benchmark and a training step use:

* the 2^30 heavy-tailed bf16 tensor through the benchmark's step (amax,
  current scaling, per-tensor E4M3, MXFP8 E4M3 OCP, both dequants, both
  statistics passes): every code, scale byte, dequantised value, count and
  statistic checked against the oracle -- per-tensor codes through a lookup
  table over the 65,536 bf16 patterns built by the oracle's element cast,
  MX codes through one such table per block exponent present, statistics
  exactly from histograms of (pattern, exponent);
* 64 gradient tensors (2^12 .. 2^22 elements) over 32 steps with delayed
  scaling, E5M2, most-recent and 16-step-window estimators with
  hysteresis: every code, scale, amax and count of every tensor at every
  step, and the whole scale state (k, reference estimate, history ring)
  after the last;
* loss-scaled Llama-7B-shaped fp32 gradients at full size (225 tensors,
  6.6 G elements, one call per step) over 1024 steps: fused 2^-16 unscale,
  Inf/NaN injection, 16-step window -- the scale state machine replayed on
  every step; at steps 0, 1, 2, 512 and 1023 every count and the amax of all
  225 tensors, and every code of one tensor of each shape (4096 x 4096,
  4096 x 11008 and the 32000 x 4096 embedding).

The oracle's work runs on a thread pool (numpy releases the interpreter lock
in its array operations); progress lines go to stderr.
"""

import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor
from fractions import Fraction

import numpy as np
import pytest
import torch

import scaled_fp8_casting_amd as nc
import workloads
from oracle import E4M3, E5M2, bulk
from oracle.cast import scale_exponent
from oracle.policy import EST_CURRENT, EST_MAX_WINDOW, EST_MOST_RECENT, Policy, ScaleState, update
from tests._gpu import host_u8, host_u16, stats_close

pytestmark = pytest.mark.gpu

COLS = 4096


def _procs():
    return max(1, min(16, os.cpu_count() or 1))


def _f32(bits: int) -> float:
    return float(np.array([bits], dtype=np.uint32).view(np.float32)[0])


# -- the 2^30 heavy-tailed tensor ------------------------------------------------

def test_heavy_tailed_full_size():
    rows = 262144
    n = rows * COLS
    bits = workloads.heavy_tailed_parallel(rows, COLS, procs=_procs(), context="spawn").reshape(-1)
    x = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    codes_pt = torch.empty(n, dtype=torch.uint8, device="cuda")
    codes_mx = torch.empty(n, dtype=torch.uint8, device="cuda")
    scales = torch.empty(n // 32, dtype=torch.uint8, device="cuda")
    y_pt = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    y_mx = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    desc, cnt = nc.tensors([x], [codes_pt])
    ws = nc.new_workspace(desc, cnt)
    am, cpt, cmx = nc.new_counts(1), nc.new_counts(1), nc.new_counts(1)
    spt, smx, fpt, fmx = (nc.new_stats(1) for _ in range(4))
    st = nc.new_state(1)
    nc.nc_amax([x], am, ws=ws)
    nc.nc_scale_update(nc.policy("e4m3", "current", hysteresis=False), st, am)
    nc.nc_cast_tensor([x], [codes_pt], "e4m3", st, cpt, ws=ws)
    nc.nc_cast_mx([x], [codes_mx], [scales], [COLS], "e4m3", "ocp", cmx, ws=ws)
    nc.nc_dequant([codes_pt], [y_pt], "e4m3", st=st)
    nc.nc_dequant([codes_mx], [y_mx], "e4m3", scales=[scales], cols=[COLS])
    nc.nc_cast_stats([x], [codes_pt], "e4m3", spt, ws, st=st)
    nc.nc_cast_stats([x], [codes_mx], "e4m3", smx, ws, scales=[scales], cols=[COLS])
    # the casts with statistics fused: same codes and counts as without
    fused_c, fused_cm = nc.new_counts(1), nc.new_counts(1)
    fused_codes = torch.empty_like(codes_pt)
    nc.nc_cast_tensor([x], [fused_codes], "e4m3", st, fused_c, stats=fpt, ws=ws)
    assert torch.equal(fused_codes, codes_pt) and torch.equal(fused_c, cpt)
    fused_scales = torch.empty_like(scales)
    nc.nc_cast_mx([x], [fused_codes], [fused_scales], [COLS], "e4m3", "ocp", fused_cm, stats=fmx, ws=ws)
    assert torch.equal(fused_codes, codes_mx) and torch.equal(fused_scales, scales) and torch.equal(fused_cm, cmx)
    del fused_codes
    torch.cuda.synchronize()

    # amax, scale, per-tensor counts
    vals = bulk.bf16_bits_to_f64(np.arange(65536, dtype=np.uint16))          # every bf16 pattern
    hist = np.bincount(bits, minlength=65536)
    present = hist > 0
    fin = np.isfinite(vals)
    amax = float(np.max(np.abs(vals[present & fin])))
    got_am = nc.counts_list(am)[0]
    assert got_am["amax"] == amax and got_am["n_nonfinite"] == int(hist[~fin].sum())
    k = scale_exponent(E4M3, Fraction(amax))
    assert int(st[0, 0]) == k
    lut, clip, uf, nf = bulk.cast_f64(E4M3, vals, k)                        # code of every pattern
    want = dict(n_finite=int(hist[fin].sum()), n_clip=int(hist[clip].sum()),
                n_underflow=int(hist[uf].sum()), n_nonfinite=int(hist[nf].sum()))
    got = nc.counts_list(cpt)[0]
    for f, v in want.items():
        assert got[f] == v, (f, got[f], v)
    assert got["amax"] == amax

    # every per-tensor code and dequantised value
    gc = host_u8(codes_pt)
    assert np.array_equal(gc, lut[bits])
    dq = bulk.dequant_bf16_f64(E4M3, np.arange(256, dtype=np.uint8), k)
    assert np.array_equal(host_u16(y_pt), dq[gc])
    del gc

    # MX: block exponents, then a code table per exponent present
    X = np.empty(n // 32, dtype=np.int64)
    step = 1 << 24
    for i in range(0, n, step):
        X[i // 32:(i + step) // 32] = bulk.mx_exponents(E4M3, vals[bits[i:i + step]], "ocp")
    gs = host_u8(scales)
    assert np.array_equal(gs, (X + 127).astype(np.uint8))
    xs = np.unique(X)
    tab = np.stack([bulk.cast_f64(E4M3, vals, int(-v))[0] for v in xs])    # [exponent, pattern] -> code
    clip_tab = np.stack([bulk.cast_f64(E4M3, vals, int(-v))[1] for v in xs])
    xi = np.searchsorted(xs, X)
    dq_mx = np.stack([bulk.dequant_bf16_f64(E4M3, np.arange(256, dtype=np.uint8), int(-v)) for v in xs])
    gm = host_u8(codes_mx)
    gy = host_u16(y_mx)
    n_clip_mx = 0
    key = np.zeros(xs.size * 65536, dtype=np.int64)
    for i in range(0, n, step):                 # one pass per chunk: codes, clips, dequant, histogram
        bi = np.repeat(xi[i // 32:(i + step) // 32], 32)
        bc = bits[i:i + step]
        assert np.array_equal(gm[i:i + step], tab[bi, bc]), i
        n_clip_mx += int(clip_tab[bi, bc].sum())
        assert np.array_equal(gy[i:i + step], dq_mx[bi, gm[i:i + step]]), i
        key += np.bincount(bi * 65536 + bc, minlength=key.size)
    del gy, gm
    gotm = nc.counts_list(cmx)[0]
    assert gotm["n_clip"] == n_clip_mx and gotm["n_finite"] == want["n_finite"] and gotm["amax"] == amax

    # statistics, exactly, from histograms
    want_pt = bulk.stats_from_histogram(E4M3, vals, lut, k, hist)
    stats_close(spt[0].cpu().tolist(), want_pt)
    stats_close(fpt[0].cpu().tolist(), want_pt)
    want_mx = bulk.stats_from_histogram(E4M3, np.tile(vals, xs.size), tab.reshape(-1),
                                        np.repeat(-xs, 65536), key)
    stats_close(smx[0].cpu().tolist(), want_mx)
    stats_close(fmx[0].cpu().tolist(), want_mx)


# -- oracle work on a thread pool ------------------------------------------------

CHUNK = 1 << 21


def _progress(capsys, msg):
    """A progress line on the real stderr (pytest's capture set aside), so
    that a long test is seen to be alive."""
    with capsys.disabled():
        sys.stderr.write(f"[progress] {msg}\n")
        sys.stderr.flush()


def _oracle_codes(pool, fmt, x32: np.ndarray, K: int) -> np.ndarray:
    """Every code of x32 (fp32) cast at exponent K, by the oracle's element
    cast, in chunks over the pool."""
    parts = pool.map(lambda i: bulk.cast_f64(fmt, x32[i:i + CHUNK].astype(np.float64), K)[0],
                     range(0, x32.size, CHUNK))
    return np.concatenate(list(parts)) if x32.size else np.zeros(0, np.uint8)


def _oracle_counts(pool, fmt, x32: np.ndarray, K: int) -> dict:
    """The oracle's counts and finite amax of x32 at exponent K, in chunks."""
    parts = list(pool.map(lambda i: bulk.counts_threshold(fmt, x32[i:i + 4 * CHUNK], K),
                          range(0, x32.size, 4 * CHUNK)))
    out = {f: sum(p[f] for p in parts) for f in ("n_finite", "n_clip", "n_underflow", "n_nonfinite")}
    out["amax"] = max((p["amax"] for p in parts), default=0.0)
    return out


def _f32_bits(v) -> int:
    return int(np.array([float(v)], dtype=np.float32).view(np.uint32)[0])


def _assert_states(st: torch.Tensor, hist: torch.Tensor, sts, W: int):
    """The device scale states and history rings equal the oracle's states:
    k, the reference estimate's fp32 bits, has_ref, the number of pushes
    kept, the push count, and the ring read oldest first."""
    gs, gh = st.cpu().numpy(), hist.cpu().numpy()
    for i, o in enumerate(sts):
        k, a_ref, has_ref, n_hist, head, step = (int(v) for v in gs[i])
        assert (k, a_ref & 0xFFFFFFFF, has_ref, n_hist, step) == (
            o.k, _f32_bits(o.a_ref), int(o.has_ref), len(o.hist), o.step), i
        ring = gh[i, :n_hist] if n_hist < W else np.roll(gh[i], -head)
        assert [Fraction(float(v)) for v in ring] == o.hist, i


# -- gradient steps: delayed scaling ------------------------------------------------

def test_gradient_steps_delayed_scaling_every_code(capsys):
    """32 steps of 64 fp32 gradient tensors (44M elements a step), E5M2 with
    delayed scaling under the most-recent and the 16-step-window estimators
    (hysteresis on), step 0 by current scaling from the oracle's own amax.
    Every step: each tensor's scale against the oracle's replayed state,
    every code against the oracle's element cast, every count and the amax
    against the oracle's counts; the window guarantee (an amax within the
    window never clips).  After the last step, the whole state and history."""
    W = 16
    gen = workloads.GradientSteps()
    T = len(gen.sizes)
    ests = (EST_MOST_RECENT, EST_MAX_WINDOW)
    pol_cur = Policy(fmt=E5M2, est=EST_CURRENT, window=W, hysteresis=True)
    run = {}
    for est in ests:
        run[est] = dict(pol_o=Policy(fmt=E5M2, est=est, window=W, hysteresis=True),
                        pol_d=nc.policy("e5m2", est, W, hysteresis=True),
                        sts=[ScaleState() for _ in range(T)], st=nc.new_state(T), hist=nc.new_history(T, W),
                        codes=[torch.empty(m, dtype=torch.uint8, device="cuda") for m in gen.sizes],
                        past=[[] for _ in range(T)])
    xd = [torch.empty(m, dtype=torch.float32, device="cuda") for m in gen.sizes]
    desc, cnt = nc.tensors(xd, run[ests[0]]["codes"])
    ws = nc.new_workspace(desc, cnt)
    t_start = time.time()
    with ThreadPoolExecutor(_procs()) as pool:
        for t in range(gen.steps):
            xs = gen.step(t)
            for d, x in zip(xd, xs):
                d.copy_(torch.from_numpy(x))
            if t == 0:
                a0 = [Fraction(_oracle_counts(pool, E5M2, x, 0)["amax"]) for x in xs]
            for est in ests:
                r = run[est]
                if t == 0:                          # empty history: current scaling
                    am = nc.new_counts(T)
                    nc.nc_amax(xd, am, ws=ws)
                    nc.nc_scale_update(nc.policy("e5m2", "current", W, hysteresis=True), r["st"], am)
                    update(pol_cur, r["sts"], a0, [0] * T)
                ks = [s.k for s in r["sts"]]
                assert r["st"][:, 0].cpu().tolist() == ks, (est, t)
                out = nc.new_counts(T)
                nc.nc_cast_tensor(xd, r["codes"], "e5m2", r["st"], out, ws=ws)
                nc.nc_scale_update(r["pol_d"], r["st"], out, r["hist"])
                torch.cuda.synchronize()
                got = nc.counts_list(out)
                amaxes = []
                for i, x in enumerate(xs):
                    want = _oracle_counts(pool, E5M2, x, ks[i])
                    for f in ("n_finite", "n_clip", "n_underflow", "n_nonfinite"):
                        assert got[i][f] == want[f], (est, t, i, f)
                    assert got[i]["amax"] == want["amax"], (est, t, i)
                    assert np.array_equal(host_u8(r["codes"][i]), _oracle_codes(pool, E5M2, x, ks[i])), (est, t, i)
                    if est == EST_MAX_WINDOW and r["past"][i] and want["amax"] <= max(r["past"][i][-W:]):
                        assert got[i]["n_clip"] == 0, (t, i)     # the window guarantee
                    r["past"][i].append(want["amax"])
                    amaxes.append(Fraction(want["amax"]))
                update(r["pol_o"], r["sts"], amaxes, [0] * T)
            if t % 8 == 7:
                _progress(capsys, f"gradient steps: {t + 1}/{gen.steps} ({time.time() - t_start:.0f} s)")
    for est in ests:
        _assert_states(run[est]["st"], run[est]["hist"], run[est]["sts"], W)


# -- loss-scaled Llama-7B-shaped gradients, full size ------------------------------

def test_llama_full_size_1024_steps(capsys):
    """All 225 tensors (6.6 G fp32 elements, one nc_cast_tensor call per step
    in the benchmark's launch shape) for 1024 steps: fused 2^-16 unscale,
    1e-7 of the elements Inf or NaN, E4M3 with a 16-step window and
    hysteresis, step 0 by current scaling from the oracle's own amax.  Every
    step: the injected count equals each tensor's non-finite count, and the
    scale of every tensor equals the oracle's state machine replayed from the
    step's amaxes and flags (the oracle's own at the sampled steps, where
    they are checked bit for bit).  At steps 0, 1, 2, 512 and 1023: every
    count and the amax of all 225 tensors against the oracle's counts on the
    whole tensor, and every code of tensors 0 (4096 x 4096), 4 (4096 x
    11008) and 224 (the 32000 x 4096 embedding).  After the last step, the
    whole state and history."""
    steps, W = 1024, 16
    sampled = (0, 1, 2, 512, 1023)
    full_codes = (0, 4, 224)
    g = workloads.LlamaGrads(layers=32)
    T = len(g.sizes)
    assert g.shapes[0] == (4096, 4096) and g.shapes[4] == (4096, 11008) and g.shapes[224] == (32000, 4096)
    s_log2 = g.S_LOG2
    ls = nc.new_loss_scale(s_log2)
    st = nc.new_state(T)
    hist = nc.new_history(T, W)
    codes = [torch.empty(m, dtype=torch.uint8, device="cuda") for m in g.sizes]
    desc, cnt = nc.tensors(g.bufs, codes)
    ws = nc.new_workspace(desc, cnt)
    pol_d = nc.policy("e4m3", "max_window", W, hysteresis=True)
    all_counts = torch.zeros((steps, T, 5), dtype=torch.int64, device="cuda")
    all_k = torch.zeros((steps, T), dtype=torch.int32, device="cuda")
    n_inj = np.zeros((steps, T), dtype=np.int64)
    host = torch.empty(max(g.sizes), dtype=torch.float32, pin_memory=True)
    host_c = torch.empty(max(g.sizes), dtype=torch.uint8, pin_memory=True)
    oracle_amax = {}
    t_start = time.time()
    with ThreadPoolExecutor(_procs()) as pool:
        for t in range(steps):
            tens, _, _ = g.fill(t)
            n_inj[t] = np.bincount(tens, minlength=T)
            if t == 0:
                am = nc.new_counts(T)
                nc.nc_amax(g.bufs, am, ls=ls, ws=ws)
                nc.nc_scale_update(nc.policy("e4m3", "current", W, hysteresis=True), st, am)
            all_k[t] = st[:, 0]
            nc.nc_cast_tensor(g.bufs, codes, "e4m3", st, all_counts[t], ls=ls, ws=ws)
            nc.nc_scale_update(pol_d, st, all_counts[t], hist)
            if t not in sampled:
                if t % 128 == 127:
                    torch.cuda.synchronize()
                    _progress(capsys, f"llama: step {t + 1}/{steps} ({time.time() - t_start:.0f} s)")
                continue
            torch.cuda.synchronize()
            k_t = all_k[t].cpu().tolist()
            c_t = all_counts[t].cpu().numpy()
            amaxes = []
            for i in range(T):
                n = g.sizes[i]
                x = host[:n]
                x.copy_(g.bufs[i])
                xn = x.numpy()
                K = k_t[i] - s_log2
                want = _oracle_counts(pool, E4M3, xn, K)
                assert (c_t[i, 0], c_t[i, 1], c_t[i, 2], c_t[i, 3]) == (
                    want["n_finite"], want["n_clip"], want["n_underflow"], want["n_nonfinite"]), (t, i)
                a_u = float(np.float32(np.ldexp(want["amax"], -s_log2)))   # exact: a normal fp32 result
                assert _f32(int(c_t[i, 4]) & 0xFFFFFFFF) == a_u, (t, i)
                if t == 0:
                    assert c_t[i, 1] == 0, i                               # current scaling never clips
                amaxes.append(Fraction(a_u))
                if i in full_codes:
                    cc = host_c[:n]
                    cc.copy_(codes[i])
                    assert np.array_equal(cc.numpy(), _oracle_codes(pool, E4M3, xn, K)), (t, i)
            oracle_amax[t] = amaxes
            _progress(capsys, f"llama: step {t} checked in full ({time.time() - t_start:.0f} s)")
    torch.cuda.synchronize()
    counts = all_counts.cpu().numpy()
    ks = all_k.cpu().numpy()
    assert np.array_equal(counts[:, :, 3], n_inj)
    # the state machine, replayed on every step; step 0 from the oracle's own
    # amax (the amax pass read the same data as the step-0 cast)
    pol_o = Policy(fmt=E4M3, est=EST_MAX_WINDOW, window=W, hysteresis=True)
    sts = [ScaleState() for _ in range(T)]
    update(Policy(fmt=E4M3, est=EST_CURRENT, window=W, hysteresis=True), sts, oracle_amax[0], [0] * T)
    for t in range(steps):
        assert list(ks[t]) == [s.k for s in sts], t
        amaxes = oracle_amax.get(t) or [Fraction(_f32(int(v) & 0xFFFFFFFF)) for v in counts[t, :, 4]]
        update(pol_o, sts, amaxes, list(counts[t, :, 3]))
    _assert_states(st, hist, sts, W)
