"""GPU parity of the update/step-ratio ("swamping") monitor against the
oracle: per-element flags and per-tensor counts bit for bit, at every narrow
weight pattern and its ties, over batches and ragged sizes, the promotion
window step by step, and the full-size workload."""

import numpy as np
import pytest
import torch

import scaled_fp8_casting_amd as nc
from oracle import bulk, swamp
from oracle.formats import BF16, FP16
import workloads
from tests._gpu import dev_f32, host_u8

pytestmark = pytest.mark.gpu
WF = [("bf16", BF16), ("fp16", FP16)]


def _watch(ws, ds, fmt, flags=True):
    wd = [dev_f32(w) for w in ws]
    dd = [dev_f32(d) for d in ds]
    fl = [torch.full((w.size,), 0xEE, dtype=torch.uint8, device="cuda") for w in ws] if flags else None
    out = nc.new_swamp_counts(len(ws))
    nc.nc_swamp_watch(wd, dd, fmt, out, flags=fl)
    torch.cuda.synchronize()
    return ([host_u8(f) for f in fl] if flags else None), nc.swamp_counts_list(out)


def _random_pairs(n, seed):
    r = np.random.default_rng(seed)
    w = (r.standard_normal(n) * np.exp2(r.integers(-40, 40, n))).astype(np.float32)
    d = (w.astype(np.float64) * np.exp2(r.uniform(-30, 4, n)) * r.choice([-1.0, 1.0], n)).astype(np.float32)
    d[r.random(n) < 0.03] = 0.0
    w[:10] = [0.0, -0.0, np.inf, np.nan, 3.4e38, 65504.0, 65520.0, 1e-40, 2.0 ** -24, 2.0 ** -25]
    d[10:14] = [np.inf, -np.inf, np.nan, 1e-45]
    return w, d


def _grid_and_ties(fmt):
    """Every finite narrow-format pattern as a weight (and the fp32 midpoints
    between neighbours, where the rounding of w itself ties, with their fp32
    neighbours, where it must not), each with updates of half a gap up, half
    (or a quarter) a gap down, and just around them."""
    if fmt is FP16:
        g = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    else:
        g = bulk.bf16_bits_to_f64(np.arange(0, 0x7F80, dtype=np.uint16))
    mids = ((g[:-1] + g[1:]) / 2).astype(np.float32)
    near = np.concatenate([np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(np.inf))])
    mids = np.concatenate([mids, near]).astype(np.float64)
    w = np.concatenate([g, -g, mids, -mids]).astype(np.float32)
    wf = swamp._round_to(fmt, w.astype(np.float64))
    a = np.abs(wf)
    _, ex = np.frexp(a)
    e = np.where(a == 0, fmt.emin, ex - 1)
    step = np.ldexp(1.0, np.maximum(e, fmt.emin) - fmt.mbits)
    sgn = np.where(np.signbit(wf), -1.0, 1.0)
    ds = [sgn * step / 2, -sgn * step / 2, -sgn * step / 4, sgn * step, -sgn * step * 0.75]
    ws, dd = [], []
    for d in ds:
        d32 = d.astype(np.float32)
        for t in (d32, np.nextafter(d32, np.float32(np.inf)), np.nextafter(d32, np.float32(-np.inf))):
            ws.append(w)
            dd.append(t)
    return np.concatenate(ws), np.concatenate(dd)


@pytest.mark.parametrize("name,fmt", WF)
def test_flags_every_pattern_and_tie(name, fmt):
    w, d = _grid_and_ties(fmt)
    flags, counts = _watch([w], [d], name)
    want, wc = swamp.watch_f64(fmt, w.astype(np.float64), d.astype(np.float64))
    bad = np.flatnonzero(flags[0] != want)
    assert bad.size == 0, [(w[i], d[i], int(flags[0][i]), int(want[i])) for i in bad[:6]]
    assert counts[0] == wc
    assert 0 < wc["n_noop"] < wc["n_considered"] and wc["n_below"] > wc["n_noop"]


@pytest.mark.parametrize("name,fmt", WF)
def test_batches_ragged_and_without_flags(name, fmt):
    """70 tensors (two launches) of ragged sizes, one empty; the counts with
    and without the flag output are the same."""
    r = np.random.default_rng(5)
    sizes = [int(v) for v in r.integers(1, 40000, 70)]
    sizes[7] = 0
    sizes[8] = 8192 * 3
    pairs = [_random_pairs(m, 10 + j) if m else (np.zeros(0, np.float32), np.zeros(0, np.float32))
             for j, m in enumerate(sizes)]
    flags, counts = _watch([p[0] for p in pairs], [p[1] for p in pairs], name)
    _, counts2 = _watch([p[0] for p in pairs], [p[1] for p in pairs], name, flags=False)
    assert counts == counts2
    for j, (w, d) in enumerate(pairs):
        want, wc = swamp.watch_f64(fmt, w.astype(np.float64), d.astype(np.float64))
        assert np.array_equal(flags[j], want), j
        assert counts[j] == wc, j


def test_counts_add_into_out_and_flags_stop_at_the_end():
    w, d = _random_pairs(8192 * 2 + 5, 3)
    big = torch.full((w.size + 64,), 0xEE, dtype=torch.uint8, device="cuda")
    out = nc.new_swamp_counts(1)
    for _ in range(3):
        nc.nc_swamp_watch([dev_f32(w)], [dev_f32(d)], "bf16", out, flags=[big[:w.size]])
    torch.cuda.synchronize()
    _, wc = swamp.watch_f64(BF16, w.astype(np.float64), d.astype(np.float64))
    assert nc.swamp_counts_list(out)[0] == {k: 3 * v for k, v in wc.items()}
    assert np.all(host_u8(big)[w.size:] == 0xEE)


def test_window_steps_against_the_oracle():
    """24 steps of 6 tensors, three of whose update scales drift down: the
    promotion state after every step, from the counts of that step."""
    r = np.random.default_rng(9)
    T, steps = 6, 24
    pol = nc.swamp_policy(window=4, num=1, den=2)
    opol = swamp.WindowPolicy(window=4, num=1, den=2)
    st = nc.new_swamp_state(T)
    ost = [swamp.WindowState() for _ in range(T)]
    w = [(r.standard_normal(5000) * 0.5).astype(np.float32) for _ in range(T)]
    for t in range(steps):
        # tensors 0-2 drift below their step at different speeds; 3-5 stay far above it
        ds = [(r.standard_normal(5000) * 10.0 ** ((-1 - t / (4 + j) if j < 3 else -0.5) + r.uniform(-1, 1)))
              .astype(np.float32) for j in range(T)]
        out = nc.new_swamp_counts(T)
        nc.nc_swamp_watch([dev_f32(x) for x in w], [dev_f32(x) for x in ds], "bf16", out)
        nc.nc_swamp_window(pol, st, out)
        torch.cuda.synchronize()
        got = st.cpu().numpy()
        for j in range(T):
            _, c = swamp.watch_f64(BF16, w[j].astype(np.float64), ds[j].astype(np.float64))
            ost[j] = swamp.window_step(opol, ost[j], c)
            assert got[j].tolist()[:3] == [ost[j].run, ost[j].promoted, ost[j].steps], (t, j)
    assert 0 < sum(s.promoted for s in ost) < T


def test_full_size_update_step():
    """2^30 fp32 weights and updates (the benchmark's monitor workload):
    2^20 sampled flags against the oracle, and the counts against a
    histogram of all the flags the kernel wrote."""
    u = workloads.UpdateStep(rows=262144)
    fl = torch.empty(u.n, dtype=torch.uint8, device="cuda")
    out = nc.new_swamp_counts(1)
    nc.nc_swamp_watch([u.w], [u.d], "bf16", out, flags=[fl])
    torch.cuda.synchronize()
    idx = torch.from_numpy(np.random.default_rng(4).choice(u.n, 1 << 20, replace=False)).cuda()
    w = u.w[idx].cpu().numpy().astype(np.float64)
    d = u.d[idx].cpu().numpy().astype(np.float64)
    want, _ = swamp.watch_f64(BF16, w, d)
    assert np.array_equal(fl[idx].cpu().numpy(), want)
    h = torch.bincount(fl.to(torch.int32), minlength=16).cpu().numpy()
    b = np.arange(16)
    c = nc.swamp_counts_list(out)[0]
    assert c["n_below"] == int(h[(b & 1) == 1].sum()) and c["n_noop"] == int(h[(b & 2) == 2].sum())
    assert c["n_zero"] == int(h[(b & 4) == 4].sum()) and c["n_excluded"] == int(h[(b & 8) == 8].sum())
    assert c["n_considered"] == u.n - c["n_zero"] - c["n_excluded"]
    frac = c["n_below"] / c["n_considered"]
    assert 0.2 < frac < 0.95, frac
