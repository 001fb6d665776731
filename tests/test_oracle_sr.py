"""Pins of the stochastic-rounding cast's oracle: its generator against an
independent Philox4x32-10 implementation, its rounding law against brute
force over the format's grid, tier 0 against tier 1, and unbiasedness."""

import os
import shutil
import subprocess
from fractions import Fraction

import numpy as np
import pytest

from oracle import E4M3, E5M2, bulk, rng
from oracle import cast as t0
from oracle.formats import Val, pow2

FMTS = [E4M3, E5M2]
HERE = os.path.dirname(os.path.abspath(__file__))


def _hipcc():
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return None


@pytest.fixture(scope="module")
def rocrand_philox(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None or not os.path.exists("/opt/rocm/include/rocrand/rocrand_kernel.h"):
        pytest.skip("hipcc or rocRAND headers not available")
    exe = str(tmp_path_factory.mktemp("philox") / "philox_rocrand")
    subprocess.run([hipcc, "-O1", "-x", "hip", "--offload-arch=gfx950", os.path.join(HERE, "philox_rocrand.cpp"),
                    "-o", exe], check=True, capture_output=True)

    def run(triples):
        inp = "".join(f"{s} {u} {b}\n" for s, u, b in triples)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
        return [tuple(int(v) for v in line.split()) for line in out.strip().splitlines()]
    return run


def test_philox_matches_rocrand(rocrand_philox):
    """rocRAND's Philox4x32-10: key = seed, counter = (block, subsequence) as
    two 64-bit halves.  The oracle's generator, written from the published
    definition, must give the same words for every block, both tiers."""
    r = np.random.default_rng(3)
    # (rocrand_init takes the position in words, 4 per block: blocks below 2^62)
    triples = [(0, 0, 0), (2 ** 64 - 1, 2 ** 64 - 1, 2 ** 62 - 1), (0x0123456789ABCDEF, 5, 7)]
    triples += [(int(r.integers(0, 2 ** 63)) * 2 + 1, int(r.integers(0, 2 ** 63)) * 2, int(r.integers(0, 2 ** 62)))
                for _ in range(200)]
    want = rocrand_philox(triples)
    M = 0xFFFFFFFF
    for (s, u, b), w in zip(triples, want):
        got = rng.philox4x32((b & M, b >> 32, u & M, u >> 32), (s & M, s >> 32))
        assert got == w, (s, u, b)
    c = [np.array([b & M for _, u, b in triples], dtype=np.uint64),
         np.array([b >> 32 for _, u, b in triples], dtype=np.uint64),
         np.array([u & M for _, u, b in triples], dtype=np.uint64),
         np.array([u >> 32 for _, u, b in triples], dtype=np.uint64)]
    for i, (s, u, b) in enumerate(triples[:20]):
        words = rng.philox4x32_np(*(x[i:i + 1] for x in c), s & M, s >> 32)
        assert tuple(int(wd[0]) for wd in words) == want[i]


def test_element_uniforms_layout(rocrand_philox):
    """Element i of tensor j under (seed, offset) takes word i % 4 of the
    block with counter (floor(i / 4), j, offset lo, offset hi): in rocRAND's
    terms block floor(i / 4) + j 2^32 of subsequence `offset`."""
    seed, offset, j = 0xDEADBEEF12345678, 0x0000000300000007, 5
    u = rng.sr_uniforms(seed, offset, j, 103)
    # rocRAND block index b (64-bit) = counter words 0, 1; subsequence = words 2, 3
    want = rocrand_philox([(seed, offset, (j << 32) | bi) for bi in range(26)])
    flat = [w for block in want for w in block][:103]
    assert u.tolist() == flat
    assert [rng.sr_uniform(seed, offset, j, i) for i in range(103)] == flat


def _grid(fmt):
    """Every finite magnitude of the format, ascending (brute force over codes)."""
    vals = sorted({fmt.decode(c).mag for c in range(128) if fmt.decode(c).kind == "num"})
    return vals


def _sr_values(seed):
    r = np.random.default_rng(seed)
    bits = r.integers(0, 2 ** 32, 3000, dtype=np.uint64).astype(np.uint32)
    bits &= np.uint32(0x7FFFFFFF)
    x = bulk.f32_bits_to_f64(bits)
    x = x[np.isfinite(x)]
    return x


@pytest.mark.parametrize("fmt", FMTS, ids=["e4m3", "e5m2"])
def test_rounding_law_brute_force(fmt):
    """For |y| between grid neighbours lo < hi (found by scanning the grid),
    the magnitude is hi exactly for u < ceil((|y| - lo) / (hi - lo) 2^32) and
    lo otherwise; grid points never move; above max saturates."""
    grid = _grid(fmt)
    r = np.random.default_rng(1)
    cases = 0
    for K in (0, 5, -7, 40, -40):
        e = r.uniform(fmt.emin - fmt.mbits - 3, fmt.emax + 1.2, 300)
        ys = [Fraction(float(np.float32(np.exp2(v) * (1 + r.uniform(0, 1))))) * pow2(K) for v in e]
        ys += [g * pow2(0) for g in grid[::7]]
        for y in ys:
            x = Val.num(False, y * pow2(-K))
            if y > fmt.maxval:
                assert t0.sr_element(fmt, x, K, 0)[1] is True
                continue
            lo = max(g for g in grid if g <= y)
            if lo == y:
                for u in (0, 1, 2 ** 31, 2 ** 32 - 1):
                    assert fmt.decode(t0.sr_element(fmt, x, K, u)[0]).mag == y
                continue
            hi = min(g for g in grid if g > y)
            thr = -((-(y - lo) * 2 ** 32) // (hi - lo))          # ceil
            for u in {0, max(thr - 1, 0), thr, min(thr + 1, 2 ** 32 - 1), 2 ** 32 - 1}:
                got = fmt.decode(t0.sr_element(fmt, x, K, u)[0]).mag
                assert got == (hi if u < thr else lo), (y, u, thr)
            cases += 1
    assert cases > 1000


@pytest.mark.parametrize("fmt", FMTS, ids=["e4m3", "e5m2"])
def test_sr_tier0_vs_tier1(fmt):
    x = _sr_values(2)
    x = np.concatenate([x, -x[:500], [0.0, -0.0, np.inf, -np.inf, np.nan, 1e-45, -1e-45]])
    x = x.astype(np.float32).astype(np.float64)
    for k, s, seed, off in ((0, 0, 1, 0), (30, 0, 2 ** 40 + 3, 9), (-20, 3, 7, 2 ** 33), (120, 16, 5, 1)):
        c1, n1 = bulk.cast_tensor_sr_f64(fmt, x, k, s, seed, off, 3)
        c0, n0 = t0.cast_tensor_sr(fmt, bulk.to_vals(x), k, s, seed, off, 3)
        assert c1.tolist() == c0
        for key in ("n_finite", "n_clip", "n_underflow", "n_nonfinite"):
            assert n1[key] == n0[key]
    # u = 0 and u = 2^32 - 1 everywhere
    for u in (0, 2 ** 32 - 1):
        c1 = bulk.cast_sr_f64(fmt, x, 9, np.full(x.size, u, np.uint32))[0]
        c0 = [t0.sr_element(fmt, v, 9, u)[0] for v in bulk.to_vals(x)]
        assert c1.tolist() == c0


@pytest.mark.parametrize("fmt", FMTS, ids=["e4m3", "e5m2"])
def test_unbiased_at_a_single_step(fmt):
    """[Drift, "The part I would rather not write"]: stochastic rounding
    carries no bias within one step.  Over 40,000 draws of the generator the mean
    decoded value of each y is within 5 standard errors of y, while round to
    nearest is off by more than that."""
    tab = bulk.decode_table(fmt)
    n = 40000
    for y in (1.03125 + 2 ** -9, 0.0173, 300.1 if fmt is E4M3 else 3001.7, 1.7 * 2.0 ** -11):
        x = np.full(n, np.float32(y), dtype=np.float64)
        codes, _ = bulk.cast_tensor_sr_f64(fmt, x, 0, 0, 17, 4, 0)
        v = tab[codes]
        yy = float(np.float32(y))
        q = float(np.abs(np.diff(np.sort(np.unique(v))))[0]) if np.unique(v).size > 1 else 1.0
        t = (yy - v.min()) / q
        se = q * np.sqrt(t * (1 - t) / n)
        assert abs(v.mean() - yy) < 5 * se + 1e-300, (y, v.mean(), yy, se)
        rne = tab[bulk.cast_f64(fmt, x[:1], 0)[0]][0]
        assert abs(rne - yy) > 5 * se, y


def test_uniform_words():
    """Top-nibble frequencies of 2^16 generator words: chi-square, 15 dof."""
    u = rng.sr_uniforms(99, 0, 0, 1 << 16)
    h = np.bincount(u >> 28, minlength=16)
    chi2 = float(((h - 4096.0) ** 2 / 4096.0).sum())
    assert chi2 < 45.0


def test_sampled_uniforms_match_the_full_draw():
    u = rng.sr_uniforms(11, 2 ** 35 + 1, 4, 1001)
    idx = np.array([0, 1, 2, 3, 4, 999, 1000, 517, 518])
    assert np.array_equal(rng.sr_uniforms_at(11, 2 ** 35 + 1, 4, idx), u[idx])
