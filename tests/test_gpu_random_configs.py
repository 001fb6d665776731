"""Seeded random configurations across the whole call surface, every output
against the oracle.

Each case draws a call and its arguments: tensor counts on both sides of one
launch's 64-tensor limit, sizes from empty through ragged tails to a few
hundred tiles (both sides of the direct-count limit of 64 workgroups), both
input dtypes and formats, scale exponents including the clamp values, the
loss-scale unscale on and off, statistics fused and separate, row and
column MX blocks under every rule, stochastic rounding, and dequant.  The
values mix magnitudes over many binades with zeros, fp32 subnormals, huge
finite values, infinities and NaNs."""

import numpy as np
import pytest
import torch

import scaled_fp8_casting_amd as nc
from oracle import E4M3, E5M2, bulk
import workloads
from tests._gpu import assert_counts, codes_like, dev_bf16, dev_f32, host_u8, host_u16, state_with_k, stats_close

pytestmark = pytest.mark.gpu
FMTS = {"e4m3": E4M3, "e5m2": E5M2}
OPS = ("amax", "cast", "cast_sr", "mx_rows", "mx_cols", "dequant", "stats")
N_CASES = 300


def _values(r, n, dtype):
    """n values over many binades with specials; (device tensor, binary64 host values)."""
    x = r.standard_normal(n) * 10.0 ** r.uniform(-6, 6)
    if n:
        k = max(1, n // 97)
        for v in (0.0, -0.0, 1e-40, -3e-42, 3e38, np.inf, -np.inf, np.nan):
            if r.random() < 0.6:
                x[r.integers(0, n, k)] = v
    x32 = x.astype(np.float32)
    if dtype == "bf16":
        bits = workloads.to_bf16_bits(x32.astype(np.float64))
        return dev_bf16(bits), bulk.bf16_bits_to_f64(bits)
    return dev_f32(x32), x32.astype(np.float64)


def _sizes(r, T, unit):
    """Sizes at and around tile multiples; in a call of many tensors most are
    small and three at most are large, which keeps the oracle's work to
    seconds while a launch still spans both sides of the direct-count limit."""
    small = [0, 1, 31, unit - 1, unit, unit + 5, 3 * unit + 17]
    large = [40 * unit, 64 * unit, 64 * unit + 3, 150 * unit + 9]
    out = []
    for i in range(T):
        if (T <= 3 or i < 3) and r.random() < 0.5:
            out.append(int(large[r.integers(0, len(large))]))
        elif r.random() < 0.8:
            out.append(int(small[r.integers(0, len(small))]))
        else:
            out.append(int(r.integers(0, 4 * unit)))
    return out


def _ks(r, T):
    return [int(r.choice([-127, 127])) if r.random() < 0.1 else int(r.integers(-30, 31)) for _ in range(T)]


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_configuration(case):
    r = np.random.default_rng(7000 + case)
    op = OPS[case % len(OPS)]
    dtype = ("f32", "bf16")[int(r.integers(0, 2))]
    fname = ("e4m3", "e5m2")[int(r.integers(0, 2))]
    fmt = FMTS[fname]
    unit = 2048 if dtype == "f32" else 4096          # elements of one cast tile
    T = int(r.choice([1, 3, 64, 65, 70]))
    s = int(r.choice([0, 16]))
    ls = nc.new_loss_scale(s) if s else None
    print(f"[case] {case} op={op} dtype={dtype} fmt={fname} T={T} s={s}", flush=True)

    if op in ("amax", "cast", "cast_sr", "stats"):
        sizes = _sizes(r, T, unit)
        data = [_values(r, m, dtype) for m in sizes]
        xd = [d[0] for d in data]
        x64 = [d[1] for d in data]
        ks = _ks(r, T)
        st = state_with_k(ks)
        codes = [codes_like(m) for m in sizes]
        desc, cnt = nc.tensors(xd, codes)
        ws = nc.new_workspace(desc, cnt)
        out = nc.new_counts(T)
        if op == "amax":
            nc.nc_amax(xd, out, ls=ls, ws=ws)
            got = nc.counts_list(out)
            for j in range(T):
                want = bulk.counts_of(np.zeros(1), np.zeros(1), ~np.isfinite(x64[j]), bulk.amax_f64(x64[j], s),
                                      sizes[j])
                assert_counts(got[j], want, keys=("n_finite", "n_nonfinite"))
            return
        if op == "cast_sr":
            seed, offset = int(r.integers(0, 2 ** 63)), int(r.integers(0, 2 ** 40))
            nc.nc_cast_tensor_sr(xd, codes, fname, st, out, seed, offset, ls=ls, ws=ws)
            got = nc.counts_list(out)
            for j in range(T):
                wc, wn = bulk.cast_tensor_sr_f64(fmt, x64[j], ks[j], s, seed, offset, j)
                assert np.array_equal(host_u8(codes[j]), wc), j
                assert_counts(got[j], wn)
            return
        fused = r.random() < 0.5 or op == "stats"
        stats = nc.new_stats(T)
        nc.nc_cast_tensor(xd, codes, fname, st, out, ls=ls, stats=stats if fused and op == "cast" else None, ws=ws)
        if op == "stats":
            nc.nc_cast_stats(xd, codes, fname, stats, ws, st=st, ls=ls)
        got = nc.counts_list(out)
        sg = stats.cpu().tolist()
        for j in range(T):
            wc, wn = bulk.cast_tensor_f64(fmt, x64[j], ks[j], s)
            assert np.array_equal(host_u8(codes[j]), wc), j
            assert_counts(got[j], wn)
            if fused:
                stats_close(sg[j], bulk.stats_f64(fmt, np.ldexp(x64[j], -s), wc, ks[j]))
        return

    # MX: row or column blocks, or dequant of either layout or of per-tensor codes
    axis = "cols" if op == "mx_cols" or (op == "dequant" and r.random() < 0.4) else "rows"
    per_tensor = op == "dequant" and r.random() < 0.3
    rule = ("ocp", "plus1", "ceil")[int(r.integers(0, 3))]
    shapes = []
    for _ in range(T):
        cols = 32 * int(r.integers(1, 17))
        rows = 32 * int(r.integers(0, 5)) if axis == "cols" else int(r.integers(0, 60))
        shapes.append((rows, cols))
    sizes = [a * b for a, b in shapes]
    data = [_values(r, m, dtype) for m in sizes]
    xd = [d[0] for d in data]
    x64 = [d[1] for d in data]
    colv = [c for _, c in shapes]
    want = [bulk.cast_mx_f64(fmt, x64[j], colv[j], rule, axis=axis) for j in range(T)]
    if op == "dequant":
        ys = [torch.empty(m, dtype=torch.bfloat16, device="cuda") for m in sizes]
        if per_tensor:
            ks = _ks(r, T)
            cs = [bulk.cast_tensor_f64(fmt, x64[j], ks[j])[0] for j in range(T)]
            nc.nc_dequant([torch.from_numpy(c).cuda() for c in cs], ys, fname, st=state_with_k(ks))
            for j in range(T):
                assert np.array_equal(host_u16(ys[j]), bulk.dequant_bf16_f64(fmt, cs[j], ks[j])), j
        else:
            nc.nc_dequant([torch.from_numpy(w[0]).cuda() for w in want], ys, fname,
                          scales=[torch.from_numpy(w[1]).cuda() for w in want], cols=colv, axis=axis)
            for j in range(T):
                K = -bulk.mx_element_exponents(want[j][1].astype(np.int64) - 127, sizes[j], colv[j], axis)
                assert np.array_equal(host_u16(ys[j]), bulk.dequant_bf16_f64(fmt, want[j][0], K)), j
        return
    codes = [codes_like(m) for m in sizes]
    scales = [torch.empty(m // 32, dtype=torch.uint8, device="cuda") for m in sizes]
    desc, cnt = nc.tensors(xd, codes)
    ws = nc.new_workspace(desc, cnt)
    out = nc.new_counts(T)
    fused = r.random() < 0.5
    stats = nc.new_stats(T)
    nc.nc_cast_mx(xd, codes, scales, colv, fname, rule, out, stats=stats if fused else None, ws=ws, axis=axis)
    sep = nc.new_stats(T)
    nc.nc_cast_stats(xd, codes, fname, sep, ws, scales=scales, cols=colv, axis=axis)
    got = nc.counts_list(out)
    sg, sp = stats.cpu().tolist(), sep.cpu().tolist()
    for j in range(T):
        wc, wsc, wn = want[j]
        assert np.array_equal(host_u8(scales[j]), wsc), j
        assert np.array_equal(host_u8(codes[j]), wc), j
        assert_counts(got[j], wn)
        K = -bulk.mx_element_exponents(wsc.astype(np.int64) - 127, sizes[j], colv[j], axis)
        ex = bulk.stats_f64(fmt, x64[j], wc, K)
        stats_close(sp[j], ex)
        if fused:
            stats_close(sg[j], ex)
