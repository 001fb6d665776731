"""Tier 1 (vectorised binary64) against tier 0 (exact rationals), and the
exact summation against a library routine (math.fsum, which returns the
correctly rounded sum)."""

import math
import random

import numpy as np
import pytest

from oracle import E4M3, E5M2, Val
from oracle import bulk
from oracle import cast as t0

FMTS = [E4M3, E5M2]


def _tier0_codes(fmt, x64, K):
    vals = bulk.to_vals(x64)
    Ks = np.broadcast_to(np.asarray(K), x64.shape).ravel().tolist()
    return [t0.cast_element(fmt, v, int(k)) for v, k in zip(vals, Ks)]


def _compare(fmt, x64, K):
    ref = _tier0_codes(fmt, x64, K)
    codes, clip, uf, nf = bulk.cast_f64(fmt, x64, K)
    for i, (c, cl, u, n) in enumerate(ref):
        assert (int(codes.ravel()[i]), bool(clip.ravel()[i]), bool(uf.ravel()[i]),
                bool(nf.ravel()[i])) == (c, cl, u, n), (float(x64.ravel()[i]), K)


@pytest.mark.parametrize("fmt", FMTS, ids=["e4m3", "e5m2"])
@pytest.mark.parametrize("K", [0, 7, -9, 21, -40, 127, -127])
def test_all_bf16_patterns(fmt, K):
    x = bulk.bf16_bits_to_f64(np.arange(65536, dtype=np.uint32).astype(np.uint16))
    _compare(fmt, x, K)


def _fp32_boundary_set(fmt, K):
    """Every code's value and every midpoint between neighbouring codes,
    moved to the input scale (times 2^-K), with their fp32 neighbours."""
    mags = sorted({fmt.decode(c).mag for c in range(128) if fmt.decode(c).kind == "num"})
    pts = list(mags) + [(a + b) / 2 for a, b in zip(mags, mags[1:])]
    pts += [fmt.maxval * 2, fmt.maxval + fmt.maxval / 64]
    xs = []
    for p in pts:
        v = np.float32(math.ldexp(float(p), -K))
        if not np.isfinite(v):
            continue
        xs += [np.nextafter(v, np.float32(0)), v, np.nextafter(v, np.float32(np.inf))]
    xs = np.array(xs, dtype=np.float32)
    return np.concatenate([xs, -xs]).astype(np.float64)


@pytest.mark.parametrize("fmt", FMTS, ids=["e4m3", "e5m2"])
@pytest.mark.parametrize("K", [0, 3, -17, 60, -100, 140, 127])
def test_fp32_boundaries(fmt, K):
    _compare(fmt, _fp32_boundary_set(fmt, K), K)


@pytest.mark.parametrize("fmt", FMTS, ids=["e4m3", "e5m2"])
def test_random_fp32_bits_including_specials(fmt):
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=4000, dtype=np.uint64).astype(np.uint32)
    bits[:8] = [0, 0x80000000, 1, 0x80000001, 0x7F800000, 0xFF800000, 0x7FC00001, 0x007FFFFF]
    x = bulk.f32_bits_to_f64(bits)
    for K in (0, 90, -90, 149 + 6):
        _compare(fmt, x, K)


@pytest.mark.parametrize("fmt", FMTS, ids=["e4m3", "e5m2"])
@pytest.mark.parametrize("rule", ["ocp", "plus1", "ceil"])
def test_mx_tier0_vs_tier1(fmt, rule):
    rng = np.random.default_rng(11)
    rows, cols = 6, 64
    x = (np.tanh(rng.normal(0, 1.5, rows * cols)) * 2.0 ** rng.integers(-30, 30, rows * cols))
    x = x.astype(np.float32).astype(np.float64)
    x[5] = np.inf
    x[64:96] = 0.0                       # an all-zero block (block 2)
    x[100] = np.nan
    x[192:224] = np.nan                  # an all-NaN block (block 6)
    codes, scales, counts = bulk.cast_mx_f64(fmt, x, cols, rule)
    c0, s0, n0 = t0.cast_mx(fmt, bulk.to_vals(x), cols, rule)
    assert codes.tolist() == c0 and scales.tolist() == s0
    for key in ("n_finite", "n_clip", "n_underflow", "n_nonfinite"):
        assert counts[key] == n0[key]
    assert counts["amax"] == float(n0["amax"])
    assert scales[2] == 0 and scales[6] == 0    # X = -127 for empty blocks


def _col_input(rows, cols, seed):
    rng = np.random.default_rng(seed)
    x = (np.tanh(rng.normal(0, 1.5, (rows, cols))) * 2.0 ** rng.integers(-30, 30, (rows, cols)))
    x = x.astype(np.float32).astype(np.float64)
    x[3, 1] = np.inf
    x[32:64, 2] = 0.0                    # an all-zero column block
    x[0:32, 5] = np.nan                  # an all-NaN column block
    x[40, 7] = -np.inf
    return x


@pytest.mark.parametrize("fmt", FMTS, ids=["e4m3", "e5m2"])
@pytest.mark.parametrize("rule", ["ocp", "plus1", "ceil"])
def test_mx_column_blocks_tier0_vs_tier1(fmt, rule):
    rows, cols = 64, 32
    x = _col_input(rows, cols, 12).ravel()
    codes, scales, counts = bulk.cast_mx_f64(fmt, x, cols, rule, axis="cols")
    c0, s0, n0 = t0.cast_mx(fmt, bulk.to_vals(x), cols, rule, axis="cols")
    assert codes.tolist() == c0 and scales.tolist() == s0
    for key in ("n_finite", "n_clip", "n_underflow", "n_nonfinite"):
        assert counts[key] == n0[key]
    assert scales[cols + 2] == 0 and scales[5] == 0     # X = -127 for empty blocks


@pytest.mark.parametrize("fmt", FMTS, ids=["e4m3", "e5m2"])
def test_mx_column_blocks_are_row_blocks_of_the_transpose(fmt):
    """Blocks down the columns of A are the row blocks of A^T: codes are the
    transpose of A^T's codes, and the (rows/32) x cols scale matrix is the
    transpose of A^T's cols x (rows/32) one.  Pins the column layout to the
    row layout, which the worked MX cases pin."""
    rows, cols = 96, 64
    x = _col_input(rows, cols, 13)
    for rule in ("ocp", "plus1", "ceil"):
        codes, scales, counts = bulk.cast_mx_f64(fmt, x.ravel(), cols, rule, axis="cols")
        ct, st_, nt = bulk.cast_mx_f64(fmt, x.T.ravel(), rows, rule)
        assert np.array_equal(codes.reshape(rows, cols), ct.reshape(cols, rows).T)
        assert np.array_equal(scales.reshape(rows // 32, cols), st_.reshape(cols, rows // 32).T)
        assert counts == nt


def test_mx_column_block_exponent_closed_form():
    """OCP E4M3 takes X = floor(log2 amax) - 8.  A 32 x 32 diagonal with
    2^(c - 10) at (c, c): column block c has amax 2^(c - 10), X = c - 18.
    Every row equal to [2^-10 .. 2^21]: column blocks are unchanged, while
    each row block sees amax 2^21, X = 13 -- the two layouts differ."""
    n = 32
    x = np.zeros((n, n))
    for c in range(n):
        x[c, c] = 2.0 ** (c - 10)
    _, sc, _ = bulk.cast_mx_f64(E4M3, x.ravel(), n, "ocp", axis="cols")
    assert (sc.astype(int) - 127).tolist() == [c - 18 for c in range(n)]
    y = np.tile(np.exp2(np.arange(n) - 10.0), (n, 1))          # row r = [2^-10 .. 2^21]
    _, sc_c, _ = bulk.cast_mx_f64(E4M3, y.ravel(), n, "ocp", axis="cols")
    _, sc_r, _ = bulk.cast_mx_f64(E4M3, y.ravel(), n, "ocp")
    assert (sc_c.astype(int) - 127).tolist() == [c - 18 for c in range(n)]
    assert (sc_r.astype(int) - 127).tolist() == [21 - 8] * n


def test_mx_element_exponents_layouts():
    rows, cols = 64, 96
    X = np.arange((rows // 32) * cols)
    got = bulk.mx_element_exponents(X, rows * cols, cols, "cols").reshape(rows, cols)
    for r in range(rows):
        for c in range(cols):
            assert got[r, c] == X[(r // 32) * cols + c]
    Xr = np.arange(rows * cols // 32)
    got = bulk.mx_element_exponents(Xr, rows * cols, cols, "rows").reshape(rows, cols)
    for r in range(rows):
        for c in range(cols):
            assert got[r, c] == Xr[r * (cols // 32) + c // 32]
    with pytest.raises(ValueError):
        bulk.mx_element_exponents(X, 48 * cols, cols, "cols")


@pytest.mark.parametrize("fmt", FMTS, ids=["e4m3", "e5m2"])
def test_stats_tier0_vs_tier1(fmt):
    rng = np.random.default_rng(5)
    x = (rng.standard_t(3, 3000) * 10.0 ** rng.uniform(-3, 3, 3000)).astype(np.float32).astype(np.float64)
    x[7] = np.inf
    x[8] = -0.0
    for K in (4, -3, 20):
        codes = bulk.cast_f64(fmt, x, K)[0]
        s1 = bulk.stats_f64(fmt, x, codes, K)
        s0 = t0.stats(fmt, bulk.to_vals(x), codes.tolist(), K)
        assert s1 == s0


def test_stats_clipped_far_outside_range_is_exact():
    """An element far above the clip point has an error needing more than
    53 bits; tier 1 must fall back to exact rationals for it."""
    x = np.array([2.0 ** 100 + 2.0 ** 77, 1.0, 3.0], dtype=np.float64)
    assert np.float32(x[0]) == x[0]
    codes = bulk.cast_f64(E4M3, x, 0)[0]
    assert bulk.stats_f64(E4M3, x, codes, 0) == t0.stats(E4M3, bulk.to_vals(x), codes.tolist(), 0)


def test_stats_from_histogram_matches_elementwise():
    rng = np.random.default_rng(9)
    bits = rng.integers(0, 65536, 20000).astype(np.uint16)
    x = bulk.bf16_bits_to_f64(bits)
    codes = bulk.cast_f64(E4M3, x, 3)[0]
    direct = bulk.stats_f64(E4M3, x, codes, 3)
    hist = np.bincount(bits, minlength=65536)
    allx = bulk.bf16_bits_to_f64(np.arange(65536).astype(np.uint16))
    allc = bulk.cast_f64(E4M3, allx, 3)[0]
    assert bulk.stats_from_histogram(E4M3, allx, allc, 3, hist) == direct


def test_exact_sum_matches_fsum():
    rng = np.random.default_rng(3)
    for _ in range(5):
        t = rng.standard_normal(20000) * 10.0 ** rng.uniform(-30, 30, 20000)
        t[::7] *= -1e12
        assert float(bulk.exact_sum(t)) == math.fsum(t.tolist())
    w = rng.integers(0, 1 << 30, 3000)
    t = rng.standard_normal(3000)
    rep = np.repeat(t[:40], w[:40] % 50)
    assert float(bulk.exact_sum(t[:40], w[:40] % 50)) == math.fsum(rep.tolist())


@pytest.mark.parametrize("fmt", FMTS, ids=["e4m3", "e5m2"])
def test_dequant_tier0_vs_tier1(fmt):
    codes = np.arange(256, dtype=np.uint8)
    for K in (0, 5, -127, 127, -120, 126, 140):
        t1 = bulk.dequant_bf16_f64(fmt, codes, K)
        for c in range(256):
            assert int(t1[c]) == t0.dequant_bf16(fmt, c, K), (c, K)


def test_amax_with_unscale():
    x = np.array([3.0, -7.5, np.inf, np.nan, 2.0 ** -140], dtype=np.float64)
    assert bulk.amax_f64(x) == 7.5 == float(t0.amax(bulk.to_vals(x)))
    assert bulk.amax_f64(x, 16) == 7.5 * 2 ** -16 == float(t0.amax(bulk.to_vals(x), 16))
    tiny = np.array([2.0 ** -126 * 1.5], dtype=np.float64)         # unscale rounds (subnormal)
    assert bulk.amax_f64(tiny, 24) == float(t0.amax(bulk.to_vals(tiny), 24))
    random.seed(1)
    assert bulk.amax_f64(np.array([np.nan, np.inf])) == 0.0
    assert t0.count_nonfinite([Val.of(math.nan), Val.of(1.0)]) == 1


@pytest.mark.parametrize("fmt", [E4M3, E5M2], ids=["e4m3", "e5m2"])
def test_counts_threshold_agrees_with_the_element_cast(fmt):
    """counts_threshold (interval tests) against the counts of cast_f64
    (codes formed element by element): random values across the whole fp32
    range, values at and next to both decision points at several K, Inf and
    NaN, and a per-element K array; chunk boundaries inside the input."""
    rng = np.random.default_rng(41)
    x = (rng.standard_normal(30000) * 10.0 ** rng.uniform(-40, 38, 30000)).astype(np.float32).astype(np.float64)
    edges = []
    for K in (-20, -3, 0, 5, 30):
        M = float(fmt.maxval)
        hs = 2.0 ** (fmt.emin - fmt.mbits - 1)
        for v in (M, hs):
            b = np.float32(np.ldexp(v, -K))
            edges += [float(b), float(np.nextafter(b, np.float32(np.inf))), float(np.nextafter(b, np.float32(0)))]
    x = np.concatenate([x, edges, [-e for e in edges], [np.inf, -np.inf, np.nan, 0.0, -0.0]])
    for K in (-20, -3, 0, 5, 30):
        _, clip, uf, nf = bulk.cast_f64(fmt, x, K)
        # binary64 holding fp32 values, and the fp32 array itself (the
        # scalar-exponent path that compares fp32 magnitudes with the bounds)
        for xin in (x, x.astype(np.float32)):
            got = bulk.counts_threshold(fmt, xin, K, chunk=4097)
            assert got["n_clip"] == int(clip.sum()) and got["n_underflow"] == int(uf.sum())
            assert got["n_nonfinite"] == int(nf.sum()) and got["n_finite"] == x.size - int(nf.sum())
            assert got["amax"] == float(np.max(np.abs(x[np.isfinite(x)])))
    Ks = rng.integers(-30, 30, x.size)
    _, clip, uf, nf = bulk.cast_f64(fmt, x, Ks)
    got = bulk.counts_threshold(fmt, x, Ks, chunk=1000)
    assert (got["n_clip"], got["n_underflow"]) == (int(clip.sum()), int(uf.sum()))
