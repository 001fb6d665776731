"""GPU parity of the per-tensor cast, the amax pass and the MX cast against
the oracle (bit-exact codes, scale bytes, counts and amax)."""

import numpy as np
import pytest
import torch

import scaled_fp8_casting_amd as nc
from oracle import E4M3, E5M2
from oracle import bulk
from oracle import cast as t0
import workloads
from tests._gpu import (assert_counts, codes_like, dev_bf16, dev_f32, host_u8, state_with_k, stats_close)

pytestmark = pytest.mark.gpu
FMTS = [("e4m3", E4M3), ("e5m2", E5M2)]


def _cast_pt(xs_dev, ks, fmt, ls=None):
    codes = [codes_like(x.numel()) for x in xs_dev]
    out = nc.new_counts(len(xs_dev))
    nc.nc_cast_tensor(xs_dev, codes, fmt, state_with_k(ks), out, ls=ls)
    torch.cuda.synchronize()
    return [host_u8(c) for c in codes], nc.counts_list(out)


def _expect_pt(fmt, x64, k, s=0):
    codes, clip, uf, nf = bulk.cast_f64(fmt, x64, k - s)
    return codes, bulk.counts_of(clip, uf, nf, bulk.amax_f64(x64, s), x64.size)


@pytest.mark.parametrize("name,fmt", FMTS)
def test_all_bf16_patterns_every_K(name, fmt):
    """All 65,536 bf16 patterns at every exponent K in [-191, 127] (every
    k in [-127, 127] with unscales up to 2^64), one tensor per K in a single
    batched call (several launches of 64)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x64 = bulk.bf16_bits_to_f64(bits)
    Ks = list(range(-191, 128))
    xd = dev_bf16(bits)
    codes, counts = _cast_pt([xd] * len(Ks), Ks, name)
    for K, c, n in zip(Ks, codes, counts):
        want_c, want_n = _expect_pt(fmt, x64, K)
        bad = np.flatnonzero(c != want_c)
        assert bad.size == 0, (K, [(hex(bits[i]), hex(c[i]), hex(want_c[i])) for i in bad[:5]])
        assert_counts(n, want_n)


@pytest.mark.parametrize("name,fmt", FMTS)
def test_fp32_boundaries_and_random_patterns(name, fmt):
    """Every code value and midpoint (+-1 fp32 ulp) moved to the input scale,
    plus uniform 32-bit patterns (subnormals, Inf, NaN), at many K."""
    mags = sorted({float(fmt.decode(c).mag) for c in range(128) if fmt.decode(c).kind == "num"})
    pts = np.array(mags + [(a + b) / 2 for a, b in zip(mags, mags[1:])] + [float(fmt.maxval) * 1.01])
    rnd = bulk.f32_bits_to_f64(workloads.random_fp32_bits(50000, 3))
    xs, Ks = [], []
    for K in (-150, -127, -60, -9, 0, 1, 7, 33, 100, 127, 140, 180):
        with np.errstate(over="ignore"):
            v = np.ldexp(pts, -K).astype(np.float32)
        v = v[np.isfinite(v)]
        nb = np.concatenate([np.nextafter(v, np.float32(0)), v, np.nextafter(v, np.float32(np.inf))])
        xs.append(np.concatenate([nb, -nb, rnd.astype(np.float32)]))
        Ks.append(K)
    codes, counts = _cast_pt([dev_f32(x) for x in xs], Ks, name)
    for K, x, c, n in zip(Ks, xs, codes, counts):
        x64 = x.astype(np.float64)
        want_c, want_n = _expect_pt(fmt, x64, K)
        bad = np.flatnonzero(c != want_c)
        assert bad.size == 0, (K, [(x[i], hex(c[i]), hex(want_c[i])) for i in bad[:5]])
        assert_counts(n, want_n)


def _near_ties(fmt):
    """Every code magnitude and every midpoint between neighbours, each with
    its fp32 neighbours at the unit scale: the values a rounding that keeps
    too few fraction bits would get wrong (a tie moved by the last fp32 bit)."""
    mags = sorted({float(fmt.decode(c).mag) for c in range(128) if fmt.decode(c).kind == "num"})
    return np.array(mags + [(a + b) / 2 for a, b in zip(mags, mags[1:])])


@pytest.mark.parametrize("name,fmt", FMTS)
def test_fp32_near_ties_at_every_third_scale(name, fmt):
    """The per-tensor cast of fp32 values one last bit either side of every
    tie and grid point, at every third exponent K from -130 to 130 (one
    tensor per K, in batches of 64): the scaled converts must round on the
    exact product, the last bit included."""
    pts = _near_ties(fmt)
    xs, Ks = [], []
    for K in range(-130, 131, 3):
        with np.errstate(over="ignore", under="ignore"):
            v = np.ldexp(pts, -K).astype(np.float32)
        v = v[np.isfinite(v) & (v > 0)]
        nb = np.concatenate([np.nextafter(v, np.float32(0)), v, np.nextafter(v, np.float32(np.inf))])
        xs.append(np.concatenate([nb, -nb]))
        Ks.append(K)
    codes, counts = _cast_pt([dev_f32(x) for x in xs], Ks, name)
    for K, x, c, n in zip(Ks, xs, codes, counts):
        want_c, want_n = _expect_pt(fmt, x.astype(np.float64), K)
        bad = np.flatnonzero(c != want_c)
        assert bad.size == 0, (K, [(x[i], hex(c[i]), hex(want_c[i])) for i in bad[:5]])
        assert_counts(n, want_n)


@pytest.mark.parametrize("rule", ["ocp", "plus1", "ceil"])
@pytest.mark.parametrize("name,fmt", FMTS)
def test_mx_fp32_near_ties_at_every_block_exponent(name, fmt, rule):
    """MX blocks of fp32 values one last bit either side of every tie and
    grid point of the block's scale, one block exponent per block over
    X = -120 .. 126 - emax: the first element of each block fixes X (its amax
    1.5 2^(X + emax), which every rule maps to X or X + 1), the other 31
    are near-ties below it (X up to 126 - emax keeps the amax finite);
    codes, scale bytes and counts against the oracle."""
    pts = _near_ties(fmt)
    r = np.random.default_rng(5)
    blocks = []
    for X in range(-120, 127 - fmt.emax):
        a = np.float32(np.ldexp(1.5, X + fmt.emax))
        with np.errstate(over="ignore", under="ignore"):
            v = np.ldexp(pts, X).astype(np.float32)
        nb = np.concatenate([np.nextafter(v, np.float32(0)), v, np.nextafter(v, np.float32(np.inf))])
        nb = nb[(nb > 0) & (nb < a)]
        for i in range(0, nb.size, 31):
            chunk = nb[i:i + 31]
            blk = np.concatenate([[a], chunk, np.zeros(31 - chunk.size, np.float32)]).astype(np.float32)
            blk[1:] *= np.where(r.random(31) < 0.5, -1, 1).astype(np.float32)
            blocks.append(blk)
    x = np.concatenate(blocks).astype(np.float32)
    cols = 32 * 64
    x = np.concatenate([x, np.zeros((-x.size) % cols, np.float32)])
    codes, scales, counts = _cast_mx(dev_f32(x), cols, name, rule)
    wc, ws, wn = bulk.cast_mx_f64(fmt, x.astype(np.float64), cols, rule)
    assert np.array_equal(scales, ws)
    bad = np.flatnonzero(codes != wc)
    assert bad.size == 0, [(x[i], hex(codes[i]), hex(wc[i])) for i in bad[:5]]
    assert_counts(counts, wn)


@pytest.mark.parametrize("name,fmt", FMTS)
def test_all_code_pairs_products_and_sums(name, fmt, consts):
    """The exhaustive 65,536-pair self-check on the GPU: every exact product
    and sum of two codes that is an fp32 value, cast at k = 0."""
    d = bulk.decode_table(fmt)
    a, b = np.meshgrid(d, d, indexing="ij")
    for op in (np.multiply, np.add):
        with np.errstate(invalid="ignore", over="ignore"):
            r = op(a, b).ravel()
        r32 = r.astype(np.float32)
        ok = (r32.astype(np.float64) == r) | np.isnan(r)
        codes, counts = _cast_pt([dev_f32(r32[ok])], [0], name)
        want_c, want_n = _expect_pt(fmt, r32[ok].astype(np.float64), 0)
        assert np.array_equal(codes[0], want_c)
        assert_counts(counts[0], want_n)
        assert ok.sum() >= 57024 if (fmt is E5M2 and op is np.add) else ok.sum() == 65536


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n", [0, 1, 3, 17, 4095, 4096, 4097, 8191, 8192, 8193, 3 * 8192 + 5, 100003])
def test_ragged_sizes(dtype, n):
    rng = np.random.default_rng(n)
    x = (rng.standard_normal(n) * 10.0 ** rng.uniform(-6, 6, n)).astype(np.float32)
    if n > 10:
        x[n // 2] = np.inf
        x[n - 1] = np.nan
    if dtype == "bf16":
        bits = workloads.to_bf16_bits(x.astype(np.float64))
        xd, x64 = dev_bf16(bits), bulk.bf16_bits_to_f64(bits)
    else:
        xd, x64 = dev_f32(x), x.astype(np.float64)
    for name, fmt in FMTS:
        codes, counts = _cast_pt([xd], [5], name)
        want_c, want_n = _expect_pt(fmt, x64, 5)
        assert np.array_equal(codes[0], want_c)
        assert_counts(counts[0], want_n)


def test_per_tensor_small_current_scaling():
    """65,536 fp32 N(0, 1): amax pass -> scale update (current) -> cast.
    k comes from the GPU's own amax; the oracle derives its own."""
    x = workloads.per_tensor_small()
    x64 = x.astype(np.float64)
    xd = dev_f32(x)
    am = nc.new_counts(1)
    nc.nc_amax([xd], am)
    st = nc.new_state(1)
    nc.nc_scale_update(nc.policy("e4m3", "current", hysteresis=False), st, am)
    codes = codes_like(x.size)
    out = nc.new_counts(1)
    nc.nc_cast_tensor([xd], [codes], "e4m3", st, out)
    torch.cuda.synchronize()
    from fractions import Fraction
    a = bulk.amax_f64(x64)
    k = t0.scale_exponent(E4M3, Fraction(a))
    assert nc.counts_list(am)[0]["amax"] == a
    assert int(st[0, 0]) == k == 6
    want_c, want_n = _expect_pt(E4M3, x64, k)
    assert np.array_equal(host_u8(codes), want_c)
    assert_counts(nc.counts_list(out)[0], want_n)
    assert want_n["n_clip"] == 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_amax_pass_and_unscale(dtype):
    rng = np.random.default_rng(8)
    x = (rng.standard_normal(70001) * 3e-3).astype(np.float32)
    x[5], x[77], x[900] = np.inf, -np.inf, np.nan
    x[1000] = -2.0 ** -126 * 1.5   # rounds when unscaled by 2^24
    if dtype == "bf16":
        bits = workloads.to_bf16_bits(x.astype(np.float64))
        xd, x64 = dev_bf16(bits), bulk.bf16_bits_to_f64(bits)
    else:
        xd, x64 = dev_f32(x), x.astype(np.float64)
    for s in (0, 16, 24, 64):
        am = nc.new_counts(1)
        nc.nc_amax([xd], am, ls=nc.new_loss_scale(s))
        torch.cuda.synchronize()
        got = nc.counts_list(am)[0]
        assert got["amax"] == bulk.amax_f64(x64, s)
        assert got["n_nonfinite"] == 3 and got["n_finite"] == x.size - 3 and got["n_clip"] == 0
    # tiny tensor whose amax becomes subnormal after the unscale
    t = np.array([2.0 ** -120 * 1.75, -(2.0 ** -125) * 1.25], dtype=np.float32)
    am = nc.new_counts(1)
    nc.nc_amax([dev_f32(t)], am, ls=nc.new_loss_scale(17))
    torch.cuda.synchronize()
    assert nc.counts_list(am)[0]["amax"] == bulk.amax_f64(t.astype(np.float64), 17)


@pytest.mark.parametrize("name,fmt", FMTS)
def test_fused_unscale_cast(name, fmt):
    """x * 2^-s then the cast at k, in one pass, with non-finite counting."""
    rng = np.random.default_rng(4)
    x = (2.0 ** 16 * rng.normal(0, 1e-6, 300000)).astype(np.float32)
    idx = rng.choice(x.size, 40, replace=False)
    x[idx[:20]] = np.inf
    x[idx[20:]] = np.nan
    x64 = x.astype(np.float64)
    ls = nc.new_loss_scale(16)
    from fractions import Fraction
    k = t0.scale_exponent(fmt, Fraction(bulk.amax_f64(x64, 16)))
    codes, counts = _cast_pt([dev_f32(x)], [k], name, ls=ls)
    want_c, want_n = _expect_pt(fmt, x64, k, 16)
    assert np.array_equal(codes[0], want_c)
    assert_counts(counts[0], want_n)
    assert counts[0]["n_nonfinite"] == 40 and counts[0]["n_clip"] == 0


def test_determinism_and_accumulation():
    x = workloads.mixed_magnitude_fp32(1 << 20, 12, -30, 30)
    xd = dev_f32(x)
    a = _cast_pt([xd], [3], "e4m3")
    b = _cast_pt([xd], [3], "e4m3")
    assert np.array_equal(a[0][0], b[0][0]) and a[1] == b[1]
    # counts accumulate over two calls into the same buffer
    out = nc.new_counts(1)
    st = state_with_k([3])
    c = codes_like(x.size)
    nc.nc_cast_tensor([xd], [c], "e4m3", st, out)
    nc.nc_cast_tensor([xd], [c], "e4m3", st, out)
    torch.cuda.synchronize()
    got = nc.counts_list(out)[0]
    for key in ("n_finite", "n_clip", "n_underflow"):
        assert got[key] == 2 * a[1][0][key]
    assert got["amax"] == a[1][0]["amax"]


# -- MX ----------------------------------------------------------------------------

def _cast_mx(xd, cols, fmt, rule):
    n = xd.numel()
    codes = codes_like(n)
    scales = torch.empty(n // 32, dtype=torch.uint8, device="cuda")
    out = nc.new_counts(1)
    nc.nc_cast_mx([xd], [codes], [scales], [cols], fmt, rule, out)
    torch.cuda.synchronize()
    return host_u8(codes), host_u8(scales), nc.counts_list(out)[0]


def _mx_input(rows, cols, seed):
    rng = np.random.default_rng(seed)
    x = np.tanh(rng.normal(0, 1.5, rows * cols)) * np.repeat(np.exp2(rng.integers(-40, 40, rows * cols // 32)), 32)
    x = x.astype(np.float32)
    x[0:32] = 0.0                                   # all-zero block
    x[32:64] = np.nan                               # all-NaN block
    x[70] = np.inf
    x[96:128] = (np.arange(32) * 2.0 ** -140).astype(np.float32)   # subnormal block
    x[128:160] = np.float32(2.0 ** 127) * 1.5       # huge block
    return x


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rule", ["ocp", "plus1", "ceil"])
@pytest.mark.parametrize("name,fmt", FMTS)
@pytest.mark.parametrize("rows,cols", [(3, 64), (37, 96), (129, 512)])
def test_mx_parity(dtype, rule, name, fmt, rows, cols):
    x = _mx_input(rows, cols, rows * cols)
    if dtype == "bf16":
        bits = workloads.to_bf16_bits(x.astype(np.float64))
        xd, x64 = dev_bf16(bits), bulk.bf16_bits_to_f64(bits)
    else:
        xd, x64 = dev_f32(x), x.astype(np.float64)
    codes, scales, counts = _cast_mx(xd, cols, name, rule)
    wc, ws, wn = bulk.cast_mx_f64(fmt, x64, cols, rule)
    assert np.array_equal(scales, ws)
    bad = np.flatnonzero(codes != wc)
    assert bad.size == 0, [(i, x64[i], hex(codes[i]), hex(wc[i])) for i in bad[:5]]
    assert_counts(counts, wn)
    if rule != "ocp":
        assert counts["n_clip"] == 0


def test_tanh_activations_mx_full_size():
    """4096 x 4096 bf16 tanh(N(0, 1.5)) under the OCP, +1 and ceil rules, in
    full: codes, scales, counts, and the statistics the workload reports per
    rule -- the clipped fraction, the mean signed error, the sign-aligned bias
    and the kept fraction ([Drift, "What the measurements said"]: how much,
    and which way; "The part I would rather not write": the scale rounded
    up) -- against the oracle, then against the values derived for this input
    in closed form (tests/test_oracle_stats_pins.py: scipy's normal
    distribution per bf16 value, torch's float8 rounding), with bands wide
    enough for the 16.8M-element sample: OCP clips 17.8% with a sign-aligned
    bias of -1.32e-2; +1 and ceil clip nothing with +1.17e-3."""
    from tests.test_oracle_stats_pins import tanh_expected
    bits = workloads.tanh_activations()
    x64 = bulk.bf16_bits_to_f64(bits.ravel())
    xd = dev_bf16(bits.ravel())
    n = x64.size
    for rule in ("ocp", "plus1", "ceil"):
        codes, scales, counts = _cast_mx(xd, 4096, "e4m3", rule)
        wc, ws, wn = bulk.cast_mx_f64(E4M3, x64, 4096, rule)
        assert np.array_equal(scales, ws) and np.array_equal(codes, wc)
        assert_counts(counts, wn)
        frac = counts["n_clip"] / n
        assert (0.175 < frac < 0.181) if rule == "ocp" else frac == 0
        st = nc.new_stats(1)
        cd = torch.from_numpy(codes).cuda()
        sd = torch.from_numpy(scales).cuda()
        nc.nc_cast_stats([xd], [cd], "e4m3", st, scales=[sd], cols=[4096])
        torch.cuda.synchronize()
        got = st[0].cpu().tolist()
        want = bulk.stats_f64(E4M3, x64, wc, np.repeat(127 - ws.astype(np.int64), 32))
        stats_close(got, want)
        mean_e, aligned, kept = got[0] / n, got[3] / n, 1 + got[4] / got[5]
        assert abs(mean_e) < 1e-4, (rule, mean_e)
        exp = tanh_expected(rule)
        tol_b, tol_k = (3e-4, 4e-4) if rule == "ocp" else (3e-5, 3e-5)
        assert abs(aligned - exp["sign_aligned"]) < tol_b, (rule, aligned, exp)
        assert abs(kept - exp["kept"]) < tol_k, (rule, kept, exp)


def test_argument_errors_on_device():
    x = dev_f32(np.ones(64, np.float32))
    with pytest.raises(nc.NarrowcastError) as e:
        nc.nc_cast_mx([x], [codes_like(64)], [torch.empty(2, dtype=torch.uint8, device="cuda")], [48],
                      "e4m3", "ocp", nc.new_counts(1))
    assert e.value.status == 3
    with pytest.raises(nc.NarrowcastError) as e:
        nc.nc_cast_tensor([x[1:]], [codes_like(63)], "e4m3", state_with_k([0]), nc.new_counts(1))
    assert e.value.status == 2


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_no_writes_past_the_end(dtype):
    """Every output (codes, MX scales, dequantised values, statistics
    workspace) sits at the head of a larger buffer filled with a sentinel;
    no call may change a byte past its tensor's end (ragged last tiles,
    tail-only tensors, several tensors per launch)."""
    rng = np.random.default_rng(21)
    sizes = [77, 32 * 3, 8192 + 77, 3 * 8192 + 77, 4096 * 5 + 32]
    guard = 1 << 15
    xs = [(rng.standard_normal(n) * 50).astype(np.float32) for n in sizes]
    if dtype == "bf16":
        xd = [dev_bf16(workloads.to_bf16_bits(x.astype(np.float64))) for x in xs]
    else:
        xd = [dev_f32(x) for x in xs]
    fill = 0xA5

    def guarded(nbytes):
        t = torch.full((nbytes + guard,), fill, dtype=torch.uint8, device="cuda")
        return t, t[:nbytes]

    cbufs = [guarded(n) for n in sizes]
    codes = [c for _, c in cbufs]
    desc, cnt = nc.tensors(xd, codes)
    wsz = nc.workspace_bytes(desc, cnt)
    wbig, ws = guarded(wsz)
    out = nc.new_counts(len(sizes))
    stats = nc.new_stats(len(sizes))
    nc.nc_cast_tensor(xd, codes, "e4m3", state_with_k([3] * len(sizes)), out, stats=stats, ws=ws)
    nc.nc_cast_stats(xd, codes, "e4m3", nc.new_stats(len(sizes)), ws, st=state_with_k([3] * len(sizes)))
    ybufs = [guarded(2 * n) for n in sizes]
    ys = [y.view(torch.bfloat16) for _, y in ybufs]
    nc.nc_dequant(codes, ys, "e4m3", st=state_with_k([3] * len(sizes)))
    mx_sizes = [n for n in sizes if n % 32 == 0]
    mx_x = [xd[sizes.index(n)] for n in mx_sizes]
    mbufs = [guarded(n) for n in mx_sizes]
    sbufs = [guarded(n // 32) for n in mx_sizes]
    nc.nc_cast_mx(mx_x, [c for _, c in mbufs], [s for _, s in sbufs], [32] * len(mx_sizes), "e5m2", "ocp",
                  nc.new_counts(len(mx_sizes)), stats=nc.new_stats(len(mx_sizes)), ws=ws)
    torch.cuda.synchronize()
    for name, bufs, lens in (("codes", cbufs, sizes), ("dequant", ybufs, [2 * n for n in sizes]),
                             ("mx codes", mbufs, mx_sizes), ("mx scales", sbufs, [n // 32 for n in mx_sizes]),
                             ("workspace", [(wbig, ws)], [wsz])):
        for (big, _), m in zip(bufs, lens):
            tail = big[m:].cpu().numpy()
            assert np.all(tail == fill), (name, m, int(np.argmax(tail != fill)))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mx_scales_at_any_alignment(dtype):
    """Scale bytes are written a row's worth at a time when the scale array is
    aligned for it, byte by byte otherwise: both give the same bytes (scale
    arrays at offsets 0..3 of an allocation), and nothing around them
    changes."""
    rows, cols = 96, 4096
    x = _mx_input(rows, cols, 17)
    if dtype == "bf16":
        bits = workloads.to_bf16_bits(x.astype(np.float64))
        xd, x64 = dev_bf16(bits), bulk.bf16_bits_to_f64(bits)
    else:
        xd, x64 = dev_f32(x), x.astype(np.float64)
    n = rows * cols
    wc, wsc, _ = bulk.cast_mx_f64(E4M3, x64, cols, "ocp")
    for off in range(4):
        big = torch.full((n // 32 + 8,), 0xA5, dtype=torch.uint8, device="cuda")
        sc = big[off:off + n // 32]
        codes = codes_like(n)
        nc.nc_cast_mx([xd], [codes], [sc], [cols], "e4m3", "ocp", nc.new_counts(1))
        torch.cuda.synchronize()
        assert np.array_equal(host_u8(codes), wc), off
        b = host_u8(big)
        assert np.array_equal(b[off:off + n // 32], wsc), off
        assert np.all(b[:off] == 0xA5) and np.all(b[off + n // 32:] == 0xA5), off


# -- MX, blocks down the columns ---------------------------------------------------

def _col_input(rows, cols, seed, dtype):
    """tanh-shaped values with a per-column-block power-of-two spread, and
    column blocks that are all zero, all NaN, subnormal or huge."""
    rng = np.random.default_rng(seed)
    spread = np.exp2(rng.integers(-40, 40, (rows // 32, 1, cols)))
    x = (np.tanh(rng.normal(0, 1.5, (rows // 32, 32, cols))) * spread).reshape(rows, cols).astype(np.float32)
    x[0:32, 0] = 0.0
    x[0:32, 1] = np.nan
    x[5, 2] = np.inf
    x[7, 3] = -np.inf
    x[0:32, 4] = (np.arange(32) * 2.0 ** -140).astype(np.float32)
    x[0:32, 5] = np.float32(2.0 ** 127) * 1.5
    x = x.ravel()
    if dtype == "bf16":
        bits = workloads.to_bf16_bits(x.astype(np.float64))
        return dev_bf16(bits), bulk.bf16_bits_to_f64(bits)
    return dev_f32(x), x.astype(np.float64)


def _cast_mx_cols(xds, shapes, fmt, rule, stats=None):
    codes = [codes_like(r * c) for r, c in shapes]
    scales = [torch.empty(r * c // 32, dtype=torch.uint8, device="cuda") for r, c in shapes]
    out = nc.new_counts(len(shapes))
    nc.nc_cast_mx(xds, codes, scales, [c for _, c in shapes], fmt, rule, out, stats=stats, axis="cols")
    torch.cuda.synchronize()
    return [host_u8(c) for c in codes], [host_u8(s) for s in scales], nc.counts_list(out)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rule", ["ocp", "plus1", "ceil"])
@pytest.mark.parametrize("name,fmt", FMTS)
@pytest.mark.parametrize("rows,cols", [(32, 32), (64, 96), (96, 4096), (160, 2080)])
def test_mx_column_blocks_parity(dtype, rule, name, fmt, rows, cols):
    """Column blocks: one 32-row band in a partial tile, several bands per
    tile (small cols), whole tiles, and bands that straddle tiles with a
    ragged last tile."""
    xd, x64 = _col_input(rows, cols, rows + cols, dtype)
    codes, scales, counts = _cast_mx_cols([xd], [(rows, cols)], name, rule)
    wc, ws, wn = bulk.cast_mx_f64(fmt, x64, cols, rule, axis="cols")
    assert np.array_equal(scales[0], ws)
    bad = np.flatnonzero(codes[0] != wc)
    assert bad.size == 0, [(i, x64[i], hex(codes[0][i]), hex(wc[i])) for i in bad[:5]]
    assert_counts(counts[0], wn)
    assert counts[0]["amax"] == wn["amax"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mx_column_blocks_batch_of_tensors(dtype):
    """Several shapes in one call (one launch), then 70 tensors (two
    launches): each tensor's codes, scales and counts."""
    for shapes in ([(32, 32), (64, 1024), (96, 160), (32, 8192)], [(32, 64 * (1 + i % 5)) for i in range(70)]):
        ins = [_col_input(r, c, 7 * i + r, dtype) for i, (r, c) in enumerate(shapes)]
        codes, scales, counts = _cast_mx_cols([d for d, _ in ins], shapes, "e4m3", "ocp")
        for (r, c), (_, x64), cg, sg, ng in zip(shapes, ins, codes, scales, counts):
            wc, ws, wn = bulk.cast_mx_f64(E4M3, x64, c, "ocp", axis="cols")
            assert np.array_equal(cg, wc) and np.array_equal(sg, ws), (r, c)
            assert_counts(ng, wn)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mx_column_scales_at_any_alignment_and_no_writes_past_the_end(dtype):
    """Scale arrays at offsets 0..7 of an allocation (word stores when
    aligned, bytes otherwise) give the same bytes; nothing after the codes,
    or around the scales, changes (a ragged last tile)."""
    rows, cols = 96, 2080
    n = rows * cols
    xd, x64 = _col_input(rows, cols, 23, dtype)
    wc, wsc, _ = bulk.cast_mx_f64(E5M2, x64, cols, "plus1", axis="cols")
    guard = 4096
    for off in range(8):
        big = torch.full((n // 32 + 16,), 0xA5, dtype=torch.uint8, device="cuda")
        sc = big[off:off + n // 32]
        cbig = torch.full((n + guard,), 0xA5, dtype=torch.uint8, device="cuda")
        nc.nc_cast_mx([xd], [cbig[:n]], [sc], [cols], "e5m2", "plus1", nc.new_counts(1), axis="cols")
        torch.cuda.synchronize()
        c = host_u8(cbig)
        assert np.array_equal(c[:n], wc) and np.all(c[n:] == 0xA5), off
        b = host_u8(big)
        assert np.array_equal(b[off:off + n // 32], wsc), off
        assert np.all(b[:off] == 0xA5) and np.all(b[off + n // 32:] == 0xA5), off


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_direct_counts_at_the_launch_threshold(dtype):
    """Launches of at most 64 workgroups that form counts only add each
    workgroup's counts straight into the caller's; larger ones, and every
    call with statistics, go through the slots and the reduction kernels.
    At 64 tiles (direct) and 65 (slots), one tensor and several: amax and
    counts against the oracle, and equal to the slot path's (the same call
    with statistics), for the per-tensor cast and the amax pass."""
    per = 2048 if dtype == "f32" else 4096                  # elements per cast tile
    rng = np.random.default_rng(31)
    for sizes in ([64 * per], [64 * per + 1], [per * 20, per * 40 + 3, 100], [per * 30, per * 35]):
        xs = [(rng.standard_normal(m) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32) for m in sizes]
        for x in xs:
            x[rng.integers(0, x.size, 3)] = np.array([np.inf, -np.inf, np.nan], np.float32)
        if dtype == "bf16":
            bits = [workloads.to_bf16_bits(x.astype(np.float64)) for x in xs]
            xd = [dev_bf16(b) for b in bits]
            x64 = [bulk.bf16_bits_to_f64(b) for b in bits]
        else:
            xd = [dev_f32(x) for x in xs]
            x64 = [x.astype(np.float64) for x in xs]
        ks = [int(v) for v in rng.integers(-4, 12, len(sizes))]
        codes = [codes_like(m) for m in sizes]
        plain, with_stats, am = nc.new_counts(len(sizes)), nc.new_counts(len(sizes)), nc.new_counts(len(sizes))
        nc.nc_cast_tensor(xd, codes, "e4m3", state_with_k(ks), plain)
        nc.nc_cast_tensor(xd, codes, "e4m3", state_with_k(ks), with_stats, stats=nc.new_stats(len(sizes)))
        nc.nc_amax(xd, am)
        torch.cuda.synchronize()
        assert torch.equal(plain, with_stats), sizes
        got, got_am = nc.counts_list(plain), nc.counts_list(am)
        for i, x in enumerate(x64):
            want = bulk.cast_tensor_f64(E4M3, x, ks[i])[1]
            assert_counts(got[i], want)
            assert got_am[i]["amax"] == want["amax"] and got_am[i]["n_nonfinite"] == want["n_nonfinite"], (sizes, i)
            assert got_am[i]["n_finite"] == want["n_finite"] and got_am[i]["n_clip"] == 0, (sizes, i)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("layout", ["tensor", "mx_rows", "mx_cols"])
def test_fused_statistics_equal_the_separate_pass(dtype, layout):
    """The casts' fused statistics and nc_cast_stats over the same codes sum
    the same terms in the same order (one tile shape, the same per-lane
    element order, the same workgroup and chunk reductions), so they agree
    bit for bit: several tensors, ragged last tiles, zeros, subnormals,
    huge values, Inf and NaN, a tensor of several reduction chunks."""
    r = np.random.default_rng(911)
    cols = 96 if layout == "mx_cols" else 4096
    rows_list = [1, 37, 64, 640] if layout == "mx_cols" else [1, 37, 300, 4200]
    xs, codes, scales = [], [], []
    for rows in rows_list:
        if layout == "mx_cols":
            rows = max(32, rows // 32 * 32)
        n = rows * cols
        x = (r.standard_t(3, n) * 10.0 ** r.uniform(-8, 4, n)).astype(np.float32)
        for v in (0.0, -0.0, 1e-40, 3e38, np.inf, -np.inf, np.nan):
            x[r.integers(0, n, max(1, n // 5000))] = v
        if dtype == "bf16":
            xs.append(dev_bf16(workloads.to_bf16_bits(x.astype(np.float64))))
        else:
            xs.append(dev_f32(x))
        codes.append(codes_like(n))
        scales.append(torch.empty(n // 32, dtype=torch.uint8, device="cuda"))
    T = len(xs)
    desc, cnt = nc.tensors(xs, codes)
    ws = nc.new_workspace(desc, cnt)
    fused, sep = nc.new_stats(T), nc.new_stats(T)
    out = nc.new_counts(T)
    colv = [cols] * T
    if layout == "tensor":
        st = state_with_k([-9, 3, 0, 12])
        nc.nc_cast_tensor(xs, codes, "e4m3", st, out, stats=fused, ws=ws)
        nc.nc_cast_stats(xs, codes, "e4m3", sep, ws, st=st)
    else:
        axis = "cols" if layout == "mx_cols" else "rows"
        nc.nc_cast_mx(xs, codes, scales, colv, "e4m3", "ocp", out, stats=fused, ws=ws, axis=axis)
        nc.nc_cast_stats(xs, codes, "e4m3", sep, ws, scales=scales, cols=colv, axis=axis)
    torch.cuda.synchronize()
    f, s = fused.cpu().numpy(), sep.cpu().numpy()
    assert np.isfinite(s).all()
    assert np.array_equal(f.view(np.uint64), s.view(np.uint64)), (f, s)
