"""GPU parity of the stochastic-rounding cast against the oracle: bit-exact
codes and counts for the same generator draws, the tensor index in the
counter, reproducibility, unbiasedness, and the full-size workload."""

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import scaled_fp8_casting_amd as nc
from oracle import E4M3, E5M2, bulk, rng
from oracle.cast import scale_exponent
import workloads
from tests._gpu import assert_counts, codes_like, dev_bf16, dev_f32, host_u8, state_with_k

pytestmark = pytest.mark.gpu
FMTS = [("e4m3", E4M3), ("e5m2", E5M2)]


def _input(dtype, n, seed):
    r = np.random.default_rng(seed)
    x = (r.standard_t(3, n) * 10.0 ** r.uniform(-4, 4, n)).astype(np.float32)
    x[:8] = [0.0, -0.0, np.inf, -np.inf, np.nan, 1e-45, -3e38, 448.0]
    if dtype == "bf16":
        bits = workloads.to_bf16_bits(x.astype(np.float64))
        return dev_bf16(bits), bulk.bf16_bits_to_f64(bits)
    return dev_f32(x), x.astype(np.float64)


def _sr(xds, fmt, ks, seed, offset, ls=None):
    codes = [codes_like(x.numel()) for x in xds]
    out = nc.new_counts(len(xds))
    nc.nc_cast_tensor_sr(xds, codes, fmt, state_with_k(ks), out, seed, offset, ls=ls)
    torch.cuda.synchronize()
    return [host_u8(c) for c in codes], nc.counts_list(out)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name,fmt", FMTS)
@pytest.mark.parametrize("k,s", [(0, 0), (9, 0), (-20, 0), (30, 16), (127, 0)])
def test_sr_parity(dtype, name, fmt, k, s):
    """Several tiles and a ragged tail; seeds and offsets with high words."""
    n = 3 * 8192 + 77
    xd, x64 = _input(dtype, n, 100 + k)
    seed, offset = 0x9E3779B97F4A7C15, (k & 0xFF) << 40 | 3
    ls = nc.new_loss_scale(s) if s else None
    codes, counts = _sr([xd], name, [k], seed, offset, ls=ls)
    want, wn = bulk.cast_tensor_sr_f64(fmt, x64, k, s, seed, offset, 0)
    bad = np.flatnonzero(codes[0] != want)
    assert bad.size == 0, [(int(i), x64[i], hex(codes[0][i]), hex(want[i])) for i in bad[:5]]
    assert_counts(counts[0], wn)
    assert counts[0]["amax"] == wn["amax"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name,fmt", FMTS)
@pytest.mark.parametrize("k", [0, -12])
def test_sr_zero_inputs_in_some_waves(dtype, name, fmt, k):
    """Exact zeros, which the underflow count takes off the zero codes, in
    some waves only: scattered +-0, one lane's whole vector, a whole wave's
    vector, and a tile with none; beside them values far below the grid
    (where fp32 inputs take the exact rule)."""
    vec = 4 if dtype == "f32" else 8              # elements per 16-byte vector
    tile = 256 * vec * 8                          # full tile of the stochastic-rounding cast
    n = 3 * tile + 1000
    r = np.random.default_rng(4242 - k)
    x = (r.standard_t(3, n) * 10.0 ** r.uniform(-7, 3, n)).astype(np.float32)
    x[r.integers(0, n, n // 300)] = 0.0
    x[r.integers(0, n, n // 300)] = -0.0
    x[2 * tile: 3 * tile][x[2 * tile: 3 * tile] == 0] = 1.0     # tile 2: no zero at all
    x[5 * vec: 6 * vec] = 0.0                                   # lane 5's first vector (tile 0)
    x[tile + 64 * vec: tile + 128 * vec] = -0.0                 # wave 1's first vector (tile 1)
    if dtype == "bf16":
        bits = workloads.to_bf16_bits(x.astype(np.float64))
        xd, x64 = dev_bf16(bits), bulk.bf16_bits_to_f64(bits)
    else:
        xd, x64 = dev_f32(x), x.astype(np.float64)
    seed, offset = 0x243F6A8885A308D3, 17
    codes, counts = _sr([xd], name, [k], seed, offset)
    want, wn = bulk.cast_tensor_sr_f64(fmt, x64, k, 0, seed, offset, 0)
    bad = np.flatnonzero(codes[0] != want)
    assert bad.size == 0, [(int(i), x64[i], hex(codes[0][i]), hex(want[i])) for i in bad[:5]]
    assert_counts(counts[0], wn)
    assert wn["n_underflow"] > 0 and np.count_nonzero(x64 == 0) > 64 * vec


def _round_up_to_bits(v: int, bits: int) -> int:
    """The least integer >= v with at most `bits` significant bits."""
    e = max(v.bit_length() - bits, 0)
    return -(-v >> e) << e if v % (1 << e) else v


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name,fmt", FMTS)
@pytest.mark.parametrize("k", [0, -40, 60])
def test_sr_fraction_finer_than_the_converts_resolve(dtype, name, fmt, k):
    """Values placed where the rule rounds up by less than the hardware
    converts resolve.  For a fixed seed and offset every element's uniform u
    is known (oracle.rng); element i gets y = |x| 2^k = t q below the smallest
    subnormal q with t 2^32 the least value above u that x's format holds
    (24 significant bits for fp32, 8 for bf16), so the rule rounds it up to
    q, while t has more fractional bits than the converts keep.  bf16 values
    this small exist only where u < 2^(MB + 16); the other elements get
    ordinary values.  Every code and count against the oracle."""
    n = 1 << 21 if dtype == "bf16" else 1 << 18
    seed, offset = 0x5EED5EED12345678, 0x9ABCDEF012
    u = rng.sr_uniforms(seed, offset, 0, n).astype(np.int64)
    qe = fmt.emin - fmt.mbits                      # log2 of the smallest subnormal
    bits = 8 if dtype == "bf16" else 24
    r = np.random.default_rng(61)
    x = (r.standard_normal(n) * 10.0 ** r.uniform(-3, 3, n)) * 2.0 ** -k
    pick = np.nonzero(u < (1 << (fmt.mbits + 16)))[0] if dtype == "bf16" else np.arange(n)
    tv = np.array([_round_up_to_bits(int(v) + 1, bits) for v in u[pick]], dtype=np.float64)
    sign = np.where(r.random(pick.size) < 0.5, -1.0, 1.0)
    x[pick] = sign * np.ldexp(tv, qe - 32 - k)
    if dtype == "bf16":
        hb = workloads.to_bf16_bits(x)
        assert np.array_equal(bulk.bf16_bits_to_f64(hb)[pick], x[pick])   # placed values are exact
        xd, x64 = dev_bf16(hb), bulk.bf16_bits_to_f64(hb)
    else:
        x32 = x.astype(np.float32)
        assert np.array_equal(x32[pick].astype(np.float64), x[pick])
        xd, x64 = dev_f32(x32), x32.astype(np.float64)
    codes, counts = _sr([xd], name, [k], seed, offset)
    wc, wn = bulk.cast_tensor_sr_f64(fmt, x64, k, 0, seed, offset, 0)
    assert pick.size > 100
    assert np.all(wc[pick] & 0x7F == 1)            # the rule rounds every placed value up to q
    assert np.array_equal(codes[0], wc)
    assert_counts(counts[0], wn)


@pytest.mark.parametrize("name,fmt", FMTS)
@pytest.mark.parametrize("k,s", [(127, 0), (120, 0), (64, 0), (0, 0), (-60, 0), (-127, 0), (-120, 16)])
def test_sr_every_bf16_pattern(name, fmt, k, s):
    """All 65,536 bf16 patterns (subnormals, both zeros, Inf, NaN) at scale
    exponents from 127 down to -136: at the top, subnormal inputs land in
    the format's normal and subnormal ranges; at the bottom, most values
    fall far below the smallest subnormal and round up only on the rarest
    draws."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    xd, x64 = dev_bf16(bits), bulk.bf16_bits_to_f64(bits)
    ls = nc.new_loss_scale(s) if s else None
    codes, counts = _sr([xd], name, [k], 0xC0FFEE, 9, ls=ls)
    want, wn = bulk.cast_tensor_sr_f64(fmt, x64, k, s, 0xC0FFEE, 9, 0)
    bad = np.flatnonzero(codes[0] != want)
    assert bad.size == 0, [(int(i), x64[i], hex(codes[0][i]), hex(want[i])) for i in bad[:5]]
    assert_counts(counts[0], wn)


@pytest.mark.parametrize("name,fmt", FMTS)
@pytest.mark.parametrize("k", [127, 126, 100, 30])
def test_sr_fp32_subnormal_inputs(name, fmt, k):
    """fp32 patterns with every exponent field, a quarter of them subnormal
    (and 2^-149 itself), at large scale exponents, where a subnormal input
    scales into the format's range."""
    r = np.random.default_rng(500 + k)
    n = 4 * 8192 + 5
    e = r.integers(0, 255, n).astype(np.uint32)
    e[: n // 4] = 0
    bits = e << 23 | r.integers(0, 1 << 23, n).astype(np.uint32) | r.integers(0, 2, n).astype(np.uint32) << 31
    bits[:4] = [1, 0x80000001, 0x7FFFFF, 0x400000]
    x = bits.view(np.float32)
    xd = dev_f32(x)
    codes, counts = _sr([xd], name, [k], 31, 1 << 33)
    want, wn = bulk.cast_tensor_sr_f64(fmt, x.astype(np.float64), k, 0, 31, 1 << 33, 0)
    bad = np.flatnonzero(codes[0] != want)
    assert bad.size == 0, [(int(i), hex(bits[i]), hex(codes[0][i]), hex(want[i])) for i in bad[:5]]
    assert_counts(counts[0], wn)


def test_sr_tensor_index_and_launches():
    """70 tensors (two launches; tensor j draws with counter word j, its
    index in the call), ragged sizes, one empty."""
    r = np.random.default_rng(3)
    sizes = [int(v) for v in r.integers(1, 30000, 70)]
    sizes[5] = 0
    ins = [_input("f32", m, 7 + j) if m else (dev_f32(np.zeros(0, np.float32)), np.zeros(0)) for j, m in
           enumerate(sizes)]
    ks = [int(v) for v in r.integers(-10, 20, 70)]
    codes, counts = _sr([d for d, _ in ins], "e4m3", ks, 77, 5)
    for j, ((_, x64), k) in enumerate(zip(ins, ks)):
        want, wn = bulk.cast_tensor_sr_f64(E4M3, x64, k, 0, 77, 5, j)
        assert np.array_equal(codes[j], want), j
        if sizes[j]:
            assert_counts(counts[j], wn)


def test_sr_reproducible_and_fresh():
    xd, x64 = _input("bf16", 50000, 4)
    a, _ = _sr([xd], "e4m3", [3], 1, 10)
    b, _ = _sr([xd], "e4m3", [3], 1, 10)
    c, _ = _sr([xd], "e4m3", [3], 1, 11)
    d, _ = _sr([xd, xd], "e4m3", [3, 3], 1, 10)
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(d[0], a[0]) and not np.array_equal(d[1], a[0])    # tensor index matters
    moved = np.count_nonzero(a[0] != c[0])
    assert moved > 1000                                                      # a new offset redraws
    assert np.array_equal(c[0], bulk.cast_tensor_sr_f64(E4M3, x64, 3, 0, 1, 11, 0)[0])


@pytest.mark.parametrize("name,fmt", FMTS)
def test_sr_unbiased_on_device(name, fmt):
    """[Drift, "The part I would rather not write"]: unbiased at any single
    step.  64 draws (offsets) of 2^16 copies of each value: the mean decoded
    value is within 5 standard errors of the value; every draw matches the
    oracle."""
    vals = np.array([1.0 + 3 * 2 ** -8, 0.0173, 1.7 * 2.0 ** -11, 200.3], dtype=np.float32)
    n = 1 << 16
    x = np.repeat(vals, n)
    xd = dev_f32(x)
    tab = bulk.decode_table(fmt)
    sums = np.zeros(vals.size)
    for off in range(64):
        codes, _ = _sr([xd], name, [0], 12345, off)
        if off < 4:
            assert np.array_equal(codes[0], bulk.cast_tensor_sr_f64(fmt, x.astype(np.float64), 0, 0, 12345, off, 0)[0])
        sums += tab[codes[0]].reshape(vals.size, n).sum(axis=1)
    mean = sums / (64 * n)
    for v, m in zip(vals.astype(np.float64), mean):
        lo = tab[bulk.cast_sr_f64(fmt, np.array([v]), 0, np.array([2 ** 32 - 1], np.uint32))[0]][0]
        hi = tab[bulk.cast_sr_f64(fmt, np.array([v]), 0, np.array([0], np.uint32))[0]][0]
        t = (v - lo) / (hi - lo)
        se = (hi - lo) * np.sqrt(t * (1 - t) / (64 * n))
        assert abs(m - v) < 5 * se, (v, m, se)


def _procs():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def test_sr_full_size_sampled():
    """The 2^30-element heavy-tailed bf16 workload in the benchmark's launch
    shape: 2^20 sampled codes against the oracle (their own draws); the
    deterministic counts exactly (clip, finite, non-finite, amax); the
    underflow count within 6 standard deviations of its exact expectation
    (a sum of independent Bernoulli draws)."""
    rows, cols = 262144, 4096
    n = rows * cols
    bits = workloads.heavy_tailed_parallel(rows, cols, procs=_procs(), context="spawn").reshape(-1)
    x = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    vals = bulk.bf16_bits_to_f64(np.arange(65536, dtype=np.uint16))
    hist = np.bincount(bits, minlength=65536)
    fin = np.isfinite(vals)
    amax = float(np.max(np.abs(vals[(hist > 0) & fin])))
    k = scale_exponent(E4M3, Fraction(amax))
    codes = torch.empty(n, dtype=torch.uint8, device="cuda")
    out = nc.new_counts(1)
    seed, offset = 2024, 7
    nc.nc_cast_tensor_sr([x], [codes], "e4m3", state_with_k([k]), out, seed, offset)
    torch.cuda.synchronize()
    idx = np.random.default_rng(9).choice(n, 1 << 20, replace=False)
    u = rng.sr_uniforms_at(seed, offset, 0, idx)
    want = bulk.cast_sr_f64(E4M3, vals[bits[idx]], k, u)[0]
    got = codes.cpu().numpy()[idx]
    assert np.array_equal(got, want)
    c = nc.counts_list(out)[0]
    _, clip, _, nf = bulk.cast_f64(E4M3, vals, k)
    assert c["n_clip"] == int(hist[clip].sum()) and c["n_nonfinite"] == int(hist[nf].sum())
    assert c["n_finite"] == n - c["n_nonfinite"] and c["amax"] == amax
    # P(code 0) per pattern: y below the smallest subnormal q rounds up with
    # probability ceil(t 2^32) / 2^32, t = y / q
    y = np.ldexp(np.where(fin, np.abs(vals), 0.0), k)
    q = 2.0 ** (E4M3.emin - E4M3.mbits)
    small = fin & (y > 0) & (y < q)
    p_up = np.ceil(np.ldexp(y / q, 32)) / 2.0 ** 32
    p0 = np.where(small, 1 - p_up, 0.0)
    mean = float((hist * p0).sum())
    sd = float(np.sqrt((hist * p0 * (1 - p0)).sum()))
    assert abs(c["n_underflow"] - mean) <= 6 * sd + 1, (c["n_underflow"], mean, sd)
