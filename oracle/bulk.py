"""Tier 1: the tier-0 definitions vectorised with numpy, for large inputs.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Every step is the plain definition of ``oracle.cast`` carried out in binary64
where the operation is exact for the values it meets:

* fp32 and bf16 inputs convert to binary64 exactly;
* multiplying by 2^K (|K| <= 191 here) is exact in binary64 for them;
* frexp gives the binade exactly; dividing by a power of two is exact;
* ``np.rint`` rounds a binary64 value to an integer, ties to even;
* the element error e = xhat - x is exact when it has at most 26 significant
  bits, which holds for every element that does not clip (xhat is then a
  multiple of ulp_fp32(x) with |e| <= |x|); elements that fail the check are
  redone in exact rationals.  e^2, |e|, x e, x^2 are then exact in binary64;
* sums are formed exactly (integer accumulation) and rounded once.

Tier 1 is checked against tier 0 by the tests, over exhaustive and boundary
sets.
"""

from fractions import Fraction

import numpy as np

from .formats import BF16, Fmt, Val, pow2

K_MIN, K_MAX = -127, 127


# -- input decoding -----------------------------------------------------------

def f32_bits_to_f64(bits) -> np.ndarray:
    with np.errstate(invalid="ignore"):
        return np.asarray(bits, dtype=np.uint32).view(np.float32).astype(np.float64)


def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def fmt_consts(fmt: Fmt):
    return dict(M=float(fmt.maxval), emin=fmt.emin, emax=fmt.emax, mbits=fmt.mbits,
                bias=fmt.bias, sign=fmt.sign_bit, maxcode=fmt.max_code(False),
                qnan=fmt.qnan)


# -- the element cast ---------------------------------------------------------

def cast_f64(fmt: Fmt, x: np.ndarray, K):
    """Vectorised ``oracle.cast.cast_element``: x (binary64 holding fp32/bf16
    values, NaN/Inf allowed), K an int or an int array broadcastable to x.

    Returns (codes uint8, clip, underflow, nonfinite) as arrays.
    """
    c = fmt_consts(fmt)
    x = np.asarray(x, dtype=np.float64)
    K = np.asarray(K, dtype=np.int64)
    nan = np.isnan(x)
    finite = np.isfinite(x)
    neg = np.signbit(x) & ~nan
    ax = np.where(finite, np.abs(x), 0.0)
    y = np.ldexp(ax, K)                               # exact
    clip = finite & (y > c["M"])
    _, ex = np.frexp(y)
    e = ex.astype(np.int64) - 1                       # binade of y (y > 0)
    qexp = np.maximum(e, c["emin"]) - c["mbits"]      # exponent of the grid spacing
    r = np.rint(np.ldexp(y, -qexp))                   # ties to even
    rv = np.minimum(np.ldexp(r, qexp), c["M"])        # saturate
    code = _encode(c, rv, neg, finite, nan)
    underflow = finite & (ax > 0) & (rv == 0)
    return code, clip, underflow, ~finite


def _encode(c, rv, neg, finite, nan):
    """Codes of magnitudes rv that lie on the format's grid (<= max), with
    the sign, +-Inf -> +-max and NaN -> the NaN code."""
    _, ex2 = np.frexp(rv)
    er = ex2.astype(np.int64) - 1
    normal = rv >= 2.0 ** c["emin"]
    e_field = np.where(normal, er + c["bias"], 0)
    mant = np.where(normal, np.ldexp(rv, -er) - 1.0, np.ldexp(rv, -c["emin"]))
    mant = np.ldexp(mant, c["mbits"])
    assert np.all(mant == np.floor(mant))
    code = (e_field << c["mbits"]) | mant.astype(np.int64)
    code = np.where(finite, code, c["maxcode"])       # +-Inf saturate
    code = np.where(neg, code | c["sign"], code)
    code = np.where(nan, c["qnan"], code)
    return code.astype(np.uint8)


def cast_sr_f64(fmt: Fmt, x: np.ndarray, K, u: np.ndarray):
    """Vectorised ``oracle.cast.sr_element``: u holds each element's uniform
    32-bit integer.  y = |x| 2^K, y / q, its floor and the fraction t times
    2^32 are all exact in binary64 (y has at most 24 significant bits), and
    so is the comparison with u."""
    c = fmt_consts(fmt)
    x = np.asarray(x, dtype=np.float64)
    K = np.asarray(K, dtype=np.int64)
    nan = np.isnan(x)
    finite = np.isfinite(x)
    neg = np.signbit(x) & ~nan
    ax = np.where(finite, np.abs(x), 0.0)
    y = np.ldexp(ax, K)
    clip = finite & (y > c["M"])
    _, ex = np.frexp(y)
    qexp = np.maximum(ex.astype(np.int64) - 1, c["emin"]) - c["mbits"]
    s = np.ldexp(y, -qexp)
    lo = np.floor(s)
    up = np.asarray(u, dtype=np.float64) < np.ldexp(s - lo, 32)
    rv = np.where(clip, c["M"], np.ldexp(lo + up, qexp))
    code = _encode(c, rv, neg, finite, nan)
    underflow = finite & (ax > 0) & (rv == 0)
    return code, clip, underflow, ~finite


def cast_tensor_sr_f64(fmt: Fmt, x: np.ndarray, k: int, unscale_log2: int, seed: int, offset: int,
                       tensor: int):
    from .rng import sr_uniforms
    u = sr_uniforms(seed, offset, tensor, np.asarray(x).size)
    codes, clip, uf, nf = cast_sr_f64(fmt, x, k - unscale_log2, u)
    return codes, counts_of(clip, uf, nf, amax_f64(x, unscale_log2), np.asarray(x).size)


def amax_f64(x: np.ndarray, unscale_log2: int = 0) -> float:
    """Finite amax after unscale, as an fp32 value (binary64 -> binary32
    conversion rounds to nearest even)."""
    x = np.asarray(x, dtype=np.float64)
    fin = np.isfinite(x)
    a = float(np.max(np.abs(x[fin]))) if fin.any() else 0.0
    return float(np.float32(np.ldexp(a, -unscale_log2)))


def counts_of(clip, uf, nf, amax_value, n):
    n_nf = int(np.count_nonzero(nf))
    return dict(n_finite=n - n_nf, n_clip=int(np.count_nonzero(clip)),
                n_underflow=int(np.count_nonzero(uf)), n_nonfinite=n_nf,
                amax=amax_value)


def cast_tensor_f64(fmt: Fmt, x: np.ndarray, k: int, unscale_log2: int = 0):
    codes, clip, uf, nf = cast_f64(fmt, x, k - unscale_log2)
    return codes, counts_of(clip, uf, nf, amax_f64(x, unscale_log2), x.size)


def counts_threshold(fmt: Fmt, x: np.ndarray, K, chunk: int = 1 << 22):
    """The counts of ``cast_f64`` without forming codes, for large tensors:
    clip <=> finite and |x| 2^K > max (the clip reading, on the exact
    product); underflow <=> finite, nonzero and |x| 2^K <= half the smallest
    subnormal (round to nearest even sends exactly that interval, its upper
    end a tie with even code 0, to zero); non-finite <=> Inf or NaN.  Also
    the finite amax (binary64).  K: an int, or an array like x.  Processed
    in chunks so that a tensor of 2^30 elements needs little memory."""
    c = fmt_consts(fmt)
    x = np.asarray(x).ravel()
    Ka = np.asarray(K)
    half_sub = 2.0 ** (c["emin"] - c["mbits"] - 1)
    n_clip = n_uf = n_nf = 0
    amax = 0.0
    if Ka.ndim == 0 and x.dtype == np.float32:
        # One K for the whole tensor: |x| 2^K > max <=> |x| > max 2^-K, and
        # |x| 2^K <= half_sub <=> |x| <= half_sub 2^-K, the bounds scaled
        # exactly in binary64 and compared as binary64 scalars (the fp32
        # magnitudes widen exactly inside the comparison).  NaN compares
        # false; +-Inf exceeds the clip bound and is taken back out.
        t_clip = np.float64(np.ldexp(c["M"], -int(Ka)))
        t_uf = np.float64(np.ldexp(half_sub, -int(Ka)))
        for i in range(0, x.size, chunk):
            ax = np.abs(x[i:i + chunk])
            fin = np.isfinite(ax)
            n_inf = int(np.count_nonzero(ax == np.inf))
            n_nf += int(ax.size - np.count_nonzero(fin))
            n_clip += int(np.count_nonzero(ax > t_clip)) - n_inf
            n_uf += int(np.count_nonzero((ax > 0) & (ax <= t_uf)))
            if ax.size:
                amax = max(amax, float(np.max(ax, where=fin, initial=np.float32(0))))
        return dict(n_finite=x.size - n_nf, n_clip=n_clip, n_underflow=n_uf, n_nonfinite=n_nf, amax=amax)
    for i in range(0, x.size, chunk):
        xc = np.asarray(x[i:i + chunk], dtype=np.float64)
        Kc = Ka if Ka.ndim == 0 else np.asarray(Ka.ravel()[i:i + chunk], dtype=np.int64)
        fin = np.isfinite(xc)
        ax = np.where(fin, np.abs(xc), 0.0)
        y = np.ldexp(ax, Kc)                           # exact
        n_clip += int(np.count_nonzero(y > c["M"]))
        n_uf += int(np.count_nonzero((ax > 0) & (y <= half_sub)))
        n_nf += int(np.count_nonzero(~fin))
        if ax.size:
            amax = max(amax, float(ax.max()))
    return dict(n_finite=x.size - n_nf, n_clip=n_clip, n_underflow=n_uf, n_nonfinite=n_nf, amax=amax)


# -- MX -----------------------------------------------------------------------

def mx_exponents(fmt: Fmt, x: np.ndarray, rule: str) -> np.ndarray:
    """Vectorised ``oracle.cast.mx_exponent`` over consecutive 32-element
    blocks of x (x.size a multiple of 32)."""
    c = fmt_consts(fmt)
    blocks = np.asarray(x, dtype=np.float64).reshape(-1, 32)
    a = np.where(np.isfinite(blocks), np.abs(blocks), 0.0).max(axis=1)
    _, ex = np.frexp(a)
    floor_rule = ex.astype(np.int64) - 1 - c["emax"]
    if rule == "ocp":
        X = floor_rule
    elif rule == "plus1":
        X = floor_rule + 1
    elif rule == "ceil":
        X = floor_rule + (np.ldexp(a, -floor_rule) > c["M"])
    else:
        raise ValueError(rule)
    X = np.clip(X, K_MIN, K_MAX)
    return np.where(a == 0, K_MIN, X)


def _check_mx_shape(n: int, cols: int, axis: str):
    if cols <= 0 or cols % 32 or n % cols:
        raise ValueError("cols must be a positive multiple of 32 and divide n")
    if axis == "cols" and (n // cols) % 32:
        raise ValueError("column blocks need a multiple of 32 rows")
    if axis not in ("rows", "cols"):
        raise ValueError(axis)


def mx_element_exponents(X: np.ndarray, n: int, cols: int, axis: str = "rows") -> np.ndarray:
    """Each element's block exponent, from the block exponents in scale-byte
    order (``oracle.cast.mx_blocks``)."""
    _check_mx_shape(n, cols, axis)
    X = np.asarray(X, dtype=np.int64)
    if axis == "rows":
        return np.repeat(X, 32)
    bands = n // cols // 32
    return np.broadcast_to(X.reshape(bands, 1, cols), (bands, 32, cols)).ravel()


def cast_mx_f64(fmt: Fmt, x: np.ndarray, cols: int, rule: str, axis: str = "rows"):
    """Vectorised ``oracle.cast.cast_mx``.  Column blocks are gathered by
    viewing the matrix as (bands, 32, cols) and moving the 32 rows of each
    band last, so that each block's elements are consecutive."""
    x = np.asarray(x, dtype=np.float64).ravel()
    _check_mx_shape(x.size, cols, axis)
    if axis == "rows":
        blocks = x
    else:
        blocks = x.reshape(-1, 32, cols).transpose(0, 2, 1).ravel()
    X = mx_exponents(fmt, blocks, rule)
    K = -mx_element_exponents(X, x.size, cols, axis)
    codes, clip, uf, nf = cast_f64(fmt, x, K)
    return codes, (X + 127).astype(np.uint8), counts_of(clip, uf, nf, amax_f64(x), x.size)


# -- decode, dequant, statistics ----------------------------------------------

def decode_table(fmt: Fmt) -> np.ndarray:
    """binary64 value of every code (NaN for NaN codes, +-inf for Inf)."""
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        v = fmt.decode(code)
        if v.kind == "nan":
            out[code] = np.nan
        elif v.kind == "inf":
            out[code] = -np.inf if v.neg else np.inf
        else:
            out[code] = -float(v.mag) if v.neg else float(v.mag)
    return out


def represented_f64(fmt: Fmt, codes: np.ndarray, K) -> np.ndarray:
    """decode(q) * 2^-K, exact in binary64."""
    return np.ldexp(decode_table(fmt)[np.asarray(codes, dtype=np.uint8)],
                    -np.asarray(K, dtype=np.int64))


def round_bf16_bits(v: np.ndarray) -> np.ndarray:
    """bf16 bit pattern of round-to-nearest-even of binary64 values, with
    IEEE overflow to +-Inf and NaN -> 0x7FC0."""
    v = np.asarray(v, dtype=np.float64)
    nan = np.isnan(v)
    inf = np.isinf(v)
    neg = np.signbit(v) & ~nan
    a = np.where(nan | inf, 0.0, np.abs(v))
    _, ex = np.frexp(a)
    e = ex.astype(np.int64) - 1
    qexp = np.maximum(e, BF16.emin) - BF16.mbits
    r = np.ldexp(np.rint(np.ldexp(a, -qexp)), qexp)
    over = r > float(BF16.maxval)
    r32 = np.where(over, 0.0, r).astype(np.float32)   # exact: r is on the bf16 grid
    bits = (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint32)
    bits = np.where(over | inf, 0x7F80, bits)
    bits = np.where(neg, bits | 0x8000, bits)
    bits = np.where(nan, 0x7FC0, bits)
    return bits.astype(np.uint16)


def dequant_bf16_f64(fmt: Fmt, codes: np.ndarray, K) -> np.ndarray:
    return round_bf16_bits(represented_f64(fmt, codes, K))


def exact_sum(terms: np.ndarray, weights: np.ndarray = None) -> Fraction:
    """The exact sum of finite binary64 terms (optionally times integer
    weights), as a rational."""
    t = np.asarray(terms, dtype=np.float64).ravel()
    if t.size == 0:
        return Fraction(0)
    if not np.all(np.isfinite(t)):
        raise ValueError("non-finite term")
    m, ex = np.frexp(t)
    M = np.ldexp(m, 53).astype(np.int64)               # t = M * 2^(ex - 53), exact
    ex = ex.astype(np.int64) - 53
    if weights is not None:
        w = np.asarray(weights, dtype=np.int64).ravel()
        total = Fraction(0)
        acc = {}
        for Mi, ei, wi in zip(M.tolist(), ex.tolist(), w.tolist()):
            acc[ei] = acc.get(ei, 0) + Mi * wi
        for ei, s in acc.items():
            total += s * pow2(ei)
        return total
    total = Fraction(0)
    order = np.argsort(ex, kind="stable")
    M, ex = M[order], ex[order]
    hi = M >> 26                                       # floor division: M = hi*2^26 + lo
    lo = M - (hi << 26)
    CH = 1 << 30                                       # |hi| < 2^27, lo < 2^26: no int64 overflow
    for s in range(0, M.size, CH):
        e_c, hi_c, lo_c = ex[s:s + CH], hi[s:s + CH], lo[s:s + CH]
        starts = np.flatnonzero(np.r_[True, e_c[1:] != e_c[:-1]])
        shi = np.add.reduceat(hi_c, starts)
        slo = np.add.reduceat(lo_c, starts)
        for ei, a, b in zip(e_c[starts].tolist(), shi.tolist(), slo.tolist()):
            total += ((a << 26) + b) * pow2(ei)
    return total


STAT_KEYS = ("sum_e", "sum_abs_e", "sum_e2", "sum_dir_e", "sum_xe", "sum_x2")


def stats_terms_f64(x: np.ndarray, xh: np.ndarray):
    """Vectorised ``oracle.cast.stats_terms``: e = xh - x, then e, |e|, e^2,
    sign(x) e, x e, x^2 in binary64 (exact where e is, see _exact_stats)."""
    e = xh - x
    return [e, np.abs(e), e * e, np.sign(x) * e, x * e, x * x]


def _exact_stats(x: np.ndarray, xh: np.ndarray, w: np.ndarray = None):
    """Exact sums of the six terms for finite x with represented values xh,
    optionally weighted by integer multiplicities w."""
    from .cast import stats_terms
    e = xh - x
    # exactness of e: the TwoSum error of xh + (-x) is zero and e fits 26 bits
    bb = e - xh
    err = (xh - (e - bb)) + (-x - bb)
    m, _ = np.frexp(e)
    safe = (err == 0) & (np.ldexp(m, 26) == np.floor(np.ldexp(m, 26)))
    terms = stats_terms_f64(x, xh)
    ws = None if w is None else w[safe]
    sums = [exact_sum(t[safe], ws) for t in terms]
    for i in np.flatnonzero(~safe):                    # rare: redo exactly
        wi = 1 if w is None else int(w[i])
        for j, tv in enumerate(stats_terms(Fraction(float(x[i])), Fraction(float(xh[i])))):
            sums[j] += wi * tv
    return {k: float(s) for k, s in zip(STAT_KEYS, sums)}


def stats_f64(fmt: Fmt, x: np.ndarray, codes: np.ndarray, K):
    """Vectorised ``oracle.cast.stats``: exact sums of e, |e|, e^2, sign(x) e,
    x e, x^2 over the finite elements, each rounded once to binary64."""
    x = np.asarray(x, dtype=np.float64).ravel()
    codes = np.asarray(codes, dtype=np.uint8).ravel()
    K = np.broadcast_to(np.asarray(K, dtype=np.int64), x.shape)
    fin = np.isfinite(x)
    x, codes, K = x[fin], codes[fin], K[fin]
    return _exact_stats(x, represented_f64(fmt, codes, K))


def stats_from_histogram(fmt: Fmt, values: np.ndarray, codes: np.ndarray,
                         K, counts: np.ndarray):
    """Exact statistics of a tensor given as distinct (value, code, K) triples
    with multiplicities (used for bf16 tensors, whose elements take at most
    65536 distinct values per K)."""
    values = np.asarray(values, dtype=np.float64).ravel()
    counts = np.asarray(counts, dtype=np.int64).ravel()
    K = np.broadcast_to(np.asarray(K, dtype=np.int64), values.shape)
    keep = np.isfinite(values) & (counts > 0)
    x, q, Kk, w = values[keep], np.asarray(codes, dtype=np.uint8).ravel()[keep], K[keep], counts[keep]
    return _exact_stats(x, represented_f64(fmt, q, Kk), w)


def to_vals(x: np.ndarray):
    """binary64 array -> list of tier-0 values (for cross-checks)."""
    return [Val.of(float(v)) for v in np.asarray(x, dtype=np.float64).ravel()]
