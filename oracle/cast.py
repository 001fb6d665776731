"""Tier 0: the scaled cast, its scale rules, flags, statistics and dequant.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Notation.  F is an FP8 format with largest finite value M_F.  A per-tensor
scale is a power of two 2^k: the cast quantises x * 2^k and the value a code
q stands for is decode(q) * 2^-k.  An MX block shares an exponent X: its
elements are quantised as x * 2^-X and stand for decode(q) * 2^X; the block's
scale byte is X + 127.  Both are "quantise x * 2^K" with K = k or K = -X.

Readings of the pages adopted here (they are silent or loose on these points):

* A finite input is never a clip because of fp32 range: x * 2^K is formed
  exactly, and an element clips when |x * 2^K| > M_F (strictly).  Under the
  per-tensor rule below this makes "amax * scale <= M_F" mean zero clips.
* NaN inputs become the canonical NaN code 0x7F (sign dropped) in both FP8
  formats; +-Inf inputs saturate to +-M_F.  Non-finite inputs are counted on
  their own and are left out of amax, clip, underflow and the statistics.
* Scale exponents k and block exponents X are clamped to [-127, 127] so that
  2^k, 2^-k and the X + 127 byte are all representable.  amax = 0 gives
  k = 127 and X = -127.
* The margin is an integer number of binades, so the scale stays a power of
  two ([E3, "Worked solution"]: any other scale would round the values a
  second time).
"""

from fractions import Fraction

from .formats import BF16, FP32, Fmt, Val, floor_log2, pow2  # noqa: F401

K_MIN, K_MAX = -127, 127


def clamp_k(k: int) -> int:
    return max(K_MIN, min(K_MAX, k))


# -- amax ---------------------------------------------------------------------

def amax(values, unscale_log2: int = 0) -> Fraction:
    """Largest finite magnitude of a tensor, after the optional loss-scale
    unscale x -> x * 2^-s, returned as an fp32 value (round-to-nearest-even
    of the exact result; exact unless it falls below the fp32 normal range).

    [E3, "Worked solution"]: the quantity watched is each tensor's largest
    magnitude.  Non-finite elements are excluded (they are counted apart).
    The maximum of no finite elements is 0.
    """
    best = Fraction(0)
    for v in values:
        if v.kind == "num" and v.mag > best:
            best = v.mag
    exact = best * pow2(-unscale_log2)
    return FP32.round_mag(exact)


def count_nonfinite(values) -> int:
    return sum(1 for v in values if v.kind != "num")


# -- scale rules --------------------------------------------------------------

def scale_exponent(fmt: Fmt, a: Fraction, margin: int = 0) -> int:
    """The per-tensor scale rule: the largest power of two 2^k that keeps the
    estimate a at or below M_F with a margin, a * 2^k <= M_F * 2^-margin,
    searched over k in [-127, 127] ([E3, "Worked solution"]: the biggest
    power-of-two scale under which the watched maximum, with a margin, still
    fits the format).  a = 0 satisfies every k and gives 127; an a too large
    for any k gives -127.
    """
    bound = fmt.maxval * pow2(-margin)
    # The search may start at any k known to be at or above the answer: for
    # a > 0, a * 2^(emax - e(a) + 1 - margin) >= 2^(emax + 1 - margin) > bound,
    # since M_F < 2^(emax + 1).
    start = K_MAX if a == 0 else min(K_MAX, fmt.emax - floor_log2(a) + 1 - margin)
    for k in range(start, K_MIN - 1, -1):
        if a * pow2(k) <= bound:
            return k
    return K_MIN


MX_RULES = ("ocp", "plus1", "ceil")


def mx_exponent(fmt: Fmt, a: Fraction, rule: str) -> int:
    """The shared block exponent X for a block whose finite amax is a.

    [Drift, "What the measurements said"] and ["The part I would rather not
    write"]: the OCP specification's rule is floor based -- X is the binade of
    the block's largest magnitude minus the largest exponent of the element
    format, which can put that magnitude above M_F (so it clips); raising the
    exponent by one (X + 1) took the clipping away; the alternative
    recipe rounds the shared scale up, i.e. takes the smallest X for which the
    block's largest magnitude fits (a * 2^-X <= M_F).
    An all-zero (or all-non-finite) block gives X = -127.
    """
    if a == 0:
        return K_MIN
    floor_rule = floor_log2(a) - fmt.emax
    if rule == "ocp":
        x = floor_rule
    elif rule == "plus1":
        x = floor_rule + 1
    elif rule == "ceil":
        x = floor_rule - 2
        while a * pow2(-x) > fmt.maxval:
            x += 1
    else:
        raise ValueError(rule)
    return clamp_k(x)


# -- the element cast ---------------------------------------------------------

def cast_element(fmt: Fmt, v: Val, K: int):
    """Quantise one input value at exponent K (the value cast is v * 2^K).

    Returns (code, clip, underflow, nonfinite).  Round to nearest, ties to
    even, saturating at M_F ([MP-card, item (3)] for the formats; the rounding
    mode and saturation are the cast's definition).  clip: finite and
    |v * 2^K| > M_F.  underflow: finite, nonzero, and rounded to zero.
    A zero keeps its sign; a nonzero value that rounds to zero gets the signed
    zero of its own sign.
    """
    if v.kind == "nan":
        return fmt.qnan, False, False, True
    if v.kind == "inf":
        return fmt.max_code(v.neg), False, False, True
    y = v.mag * pow2(K)
    clip = y > fmt.maxval
    code = fmt.encode(Val.num(v.neg, y), saturate=True)
    mag_code = code & ~fmt.sign_bit
    underflow = v.mag != 0 and mag_code == 0
    return code, clip, underflow, False


def sr_element(fmt: Fmt, v: Val, K: int, u: int):
    """Stochastic rounding of one input value at exponent K (the value cast is
    y = v * 2^K, exact), with u a uniform 32-bit integer.

    Reading: the pages only say the rounding carries no bias within one step
    ([Drift, "The part I would rather not write"]) and that its damage sits in
    the backward matmuls ([Drift, "What the measurements said"]).  Taken
    here as the textbook rule: with lo <= |y| < lo + q the two neighbouring
    grid points (q the grid spacing in |y|'s binade, or the subnormal spacing
    below the normal range), t = (|y| - lo) / q, the magnitude rounds up to
    lo + q iff u < t 2^32 -- probability ceil(t 2^32) / 2^32, which is t
    whenever t has at most 32 fractional bits, so the expected value is y.
    Above the largest finite value the result saturates (a clip, as in
    ``cast_element``); non-finite inputs are coded as there.  Returns (code,
    clip, underflow, nonfinite); underflow: nonzero and the drawn code is a
    zero.
    """
    if v.kind == "nan":
        return fmt.qnan, False, False, True
    if v.kind == "inf":
        return fmt.max_code(v.neg), False, False, True
    y = v.mag * pow2(K)
    if y > fmt.maxval:
        return fmt.max_code(v.neg), True, False, False
    if y == 0:
        return fmt.encode(Val.num(v.neg, Fraction(0)), saturate=True), False, False, False
    q = pow2(max(floor_log2(y), fmt.emin) - fmt.mbits)
    lo = (y // q) * q
    t = (y - lo) / q
    mag = lo + q if u < t * 2 ** 32 else lo
    code = fmt.encode(Val.num(v.neg, mag), saturate=True)
    return code, False, mag == 0, False


def cast_tensor_sr(fmt: Fmt, values, k: int, unscale_log2: int, seed: int, offset: int, tensor: int):
    """Per-tensor stochastic-rounding cast of x * 2^-s at scale 2^k, element i
    drawing ``oracle.rng.sr_uniform(seed, offset, tensor, i)``.  Returns
    (codes, counts) as ``cast_tensor``."""
    from .rng import sr_uniform
    K = k - unscale_log2
    codes, n_clip, n_uf, n_nf = [], 0, 0, 0
    for i, v in enumerate(values):
        c, cl, uf, nf = sr_element(fmt, v, K, sr_uniform(seed, offset, tensor, i))
        codes.append(c)
        n_clip += cl
        n_uf += uf
        n_nf += nf
    counts = dict(n_finite=len(codes) - n_nf, n_clip=n_clip, n_underflow=n_uf,
                  n_nonfinite=n_nf, amax=amax(values, unscale_log2))
    return codes, counts


def cast_tensor(fmt: Fmt, values, k: int, unscale_log2: int = 0):
    """Per-tensor cast with scale 2^k of the unscaled tensor x * 2^-s.

    The element cast is v * 2^(k - s), formed exactly ([MP-card, item (1)]:
    the gradients are divided back by the loss scale S = 2^s).
    Returns (codes, counts) with counts a dict of n_finite, n_clip,
    n_underflow, n_nonfinite and amax (an fp32 value, see ``amax``).
    """
    K = k - unscale_log2
    codes, n_clip, n_uf, n_nf = [], 0, 0, 0
    for v in values:
        c, cl, uf, nf = cast_element(fmt, v, K)
        codes.append(c)
        n_clip += cl
        n_uf += uf
        n_nf += nf
    counts = dict(n_finite=len(codes) - n_nf, n_clip=n_clip, n_underflow=n_uf,
                  n_nonfinite=n_nf, amax=amax(values, unscale_log2))
    return codes, counts


def mx_blocks(n: int, cols: int, axis: str = "rows"):
    """Element indices of each MX block of a row-major (n / cols) x cols
    matrix, in scale-byte order.  axis "rows": 32 consecutive elements of a
    row, scales row-major rows x (cols / 32).  axis "cols": 32 consecutive
    rows of one column, scales row-major (rows / 32) x cols -- the blocks of
    the transposed matrix, with the scales kept in the matrix's own
    orientation."""
    if cols <= 0 or cols % 32 or n % cols:
        raise ValueError("cols must be a positive multiple of 32 and divide n")
    rows = n // cols
    if axis == "rows":
        return [list(range(b, b + 32)) for b in range(0, n, 32)]
    if axis != "cols":
        raise ValueError(axis)
    if rows % 32:
        raise ValueError("column blocks need a multiple of 32 rows")
    return [[(32 * band + r) * cols + c for r in range(32)]
            for band in range(rows // 32) for c in range(cols)]


def cast_mx(fmt: Fmt, values, cols: int, rule: str, axis: str = "rows"):
    """MX cast: each block of 32 elements (``mx_blocks``: along a row, or down
    a column) shares the exponent X given by ``mx_exponent`` from the block's
    finite amax ([Drift, "What the measurements said"]: blocks of 32, one
    shared power of two per block).  Returns (codes, scale_bytes, counts);
    the scale byte is X + 127.  counts['amax'] is the finite amax of the
    whole tensor.
    """
    n = len(values)
    codes, scales = [0] * n, []
    n_clip = n_uf = n_nf = 0
    for idx in mx_blocks(n, cols, axis):
        block = [values[i] for i in idx]
        a = max((v.mag for v in block if v.kind == "num"), default=Fraction(0))
        X = mx_exponent(fmt, a, rule)
        scales.append(X + 127)
        for i, v in zip(idx, block):
            c, cl, uf, nf = cast_element(fmt, v, -X)
            codes[i] = c
            n_clip += cl
            n_uf += uf
            n_nf += nf
    counts = dict(n_finite=n - n_nf, n_clip=n_clip, n_underflow=n_uf,
                  n_nonfinite=n_nf, amax=amax(values))
    return codes, scales, counts


# -- dequant and statistics ---------------------------------------------------

def represented(fmt: Fmt, code: int, K: int) -> Val:
    """The exact value a code stands for at cast exponent K: decode(q) * 2^-K."""
    v = fmt.decode(code)
    if v.kind != "num":
        return v
    return Val.num(v.neg, v.mag * pow2(-K))


def dequant_bf16(fmt: Fmt, code: int, K: int) -> int:
    """The bf16 pattern of decode(q) * 2^-K: round-to-nearest-even with IEEE
    overflow to +-Inf; a NaN code gives the quiet NaN 0x7FC0; a signed zero
    keeps its sign."""
    return BF16.encode(represented(fmt, code, K), saturate=False)


STAT_KEYS = ("sum_e", "sum_abs_e", "sum_e2", "sum_dir_e", "sum_xe", "sum_x2")


def stats_terms(x: Fraction, xhat: Fraction):
    """The six per-element terms for a finite element x with represented value
    xhat, e = xhat - x: e, |e|, e^2, sign(x) e, x e, x^2.

    [Drift, "What the measurements said"]: the size of the change the cast
    makes is measured apart from its direction; sign(x) e is the
    component of the error along the element (negative when the cast shrinks
    magnitudes, as clipping does), x e / x^2 gives the fraction of the tensor
    kept along itself.
    """
    e = xhat - x
    sgn = (x > 0) - (x < 0)
    return (e, abs(e), e * e, sgn * e, x * e, x * x)


def stats(fmt: Fmt, values, codes, Ks):
    """Exact sums of the six terms over the finite elements, each rounded
    once to binary64 (round to nearest even, via Fraction -> float).

    Ks gives the cast exponent per element (a single int for per-tensor).
    The reference value of an element is x itself (after any unscale, which
    the caller applies to ``values``).
    """
    if isinstance(Ks, int):
        Ks = [Ks] * len(values)
    sums = [Fraction(0)] * 6
    for v, c, K in zip(values, codes, Ks):
        if v.kind != "num":
            continue
        xhat = represented(fmt, c, K)
        t = stats_terms(v.signed, xhat.signed)
        sums = [s + ti for s, ti in zip(sums, t)]
    return {k: float(s) for k, s in zip(STAT_KEYS, sums)}


def unscaled(values, unscale_log2: int):
    """x * 2^-s for every finite element (exact rationals; non-finite kept)."""
    f = pow2(-unscale_log2)
    return [Val.num(v.neg, v.mag * f) if v.kind == "num" else v for v in values]
