"""Number-format codecs for the oracle (TEST INFRASTRUCTURE ONLY).

Written from the formats' published definitions, not from any library:

* bfloat16: the upper 16 bits of an IEEE-754 binary32; encoding rounds to
  nearest, ties to even (RNE).
* OCP 8-bit floating point, E4M3 ("FN" variant, the one gfx950's fp8 MFMA
  reads): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent
  field 0 holds subnormals m/8 * 2^-6; no infinities; S.1111.111 is NaN, so the
  largest finite magnitude is 1.75 * 2^8 = 448.  The encoder rounds to nearest
  even and saturates finite magnitudes above 448 to 448 (the page names FP8 in
  section "The cost of laziness in large-model training" but fixes no format;
  saturation is this build's reading).

All decoders return float64.  Pins: tests/test_oracle_codecs.py.
"""

import numpy as np

E4M3_MAX = 448.0


def bf16_decode(bits):
    """uint16 bf16 bit patterns -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # NaN payloads convert to NaN
        return b.view(np.float32).astype(np.float64)


def bf16_encode(x):
    """float64 -> uint16 bf16 bit patterns, round to nearest even, directly
    from the float64 value (no intermediate float32 rounding)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    flat = x.ravel()
    res = out.ravel()
    for idx in range(flat.size):
        res[idx] = _bf16_encode_scalar(float(flat[idx]))
    return out


def _bf16_encode_scalar(v):
    if v != v:
        return 0x7FC0
    sign = 0x8000 if (v < 0 or (v == 0 and np.signbit(v))) else 0
    a = abs(v)
    if a == 0.0:
        return sign
    if a == float("inf"):
        return sign | 0x7F80
    m, e = np.frexp(a)  # a = m * 2**e, m in [0.5, 1)
    e = int(e) - 1      # a = (2m) * 2**e, 2m in [1, 2)
    if e < -126:        # subnormal: quantum is 2**-133
        q = _round_half_even(a / 2.0 ** -133)
        if q >= 128:    # rounded up into the normal range
            return sign | (1 << 7)
        return sign | q
    frac = 2.0 * float(m) - 1.0
    q = _round_half_even(frac * 128.0)
    if q == 128:
        q = 0
        e += 1
    if e > 127:
        return sign | 0x7F80
    return sign | ((e + 127) << 7) | q


def _round_half_even(t):
    """Round a non-negative float64 to the nearest integer, ties to even.
    The inputs here are exact multiples of powers of two, so the float64
    arithmetic below is exact."""
    f = np.floor(t)
    d = t - f
    q = int(f)
    if d > 0.5 or (d == 0.5 and (q & 1)):
        q += 1
    return q


def e4m3_decode(codes):
    """uint8 E4M3FN codes -> float64 values (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    sub = m / 8.0 * 2.0 ** -6
    nrm = (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64))
    v = np.where(e == 0, sub, nrm)
    v = np.where((e == 15) & ((c & 7) == 7), np.nan, v)
    return sign * v


def e4m3_encode(x):
    """float64 -> uint8 E4M3FN codes, RNE, saturating to +-448."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint8)
    flat = x.ravel()
    res = out.ravel()
    for idx in range(flat.size):
        res[idx] = _e4m3_encode_scalar(float(flat[idx]))
    return out


def _e4m3_encode_scalar(v):
    if v != v:
        return 0x7F
    sign = 0x80 if (v < 0 or (v == 0 and np.signbit(v))) else 0
    a = abs(v)
    if a >= E4M3_MAX:
        return sign | 0x7E
    if a < 2.0 ** -6:   # subnormal range, quantum 2**-9
        q = _round_half_even(a * 512.0)
        return sign | q  # q == 8 encodes 2**-6, the smallest normal
    m, e = np.frexp(a)
    e = int(e) - 1
    q = _round_half_even((2.0 * float(m) - 1.0) * 8.0)
    if q == 8:
        q = 0
        e += 1
    code = ((e + 7) << 3) | q
    if code > 0x7E:     # cannot happen below 448, kept as a guard
        code = 0x7E
    return sign | code


def e4m3_encode_fast(x):
    """Vectorised form of e4m3_encode for large arrays (same rounding).

    Works on exact float64 arithmetic: the quantum of the target binade is a
    power of two, so x / quantum is exact and np.rint rounds half to even."""
    x = np.asarray(x, dtype=np.float64)
    a_full = np.abs(x)
    # magnitudes at or past 448 (and NaN) are decided at the end; clamp them
    # here so the exact arithmetic below stays in range
    a = np.where(np.isnan(a_full), 0.0, np.minimum(a_full, E4M3_MAX))
    sign = np.where(np.signbit(x), 0x80, 0).astype(np.int64)
    # binade exponent, clamped to the normal range [-6, 8]
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0))).astype(np.int64)
    # guard against log2 rounding at exact powers of two
    e = np.where(np.exp2(e.astype(np.float64)) > a, e - 1, e)
    e = np.where(np.exp2((e + 1).astype(np.float64)) <= a, e + 1, e)
    e = np.clip(e, -6, 8)
    quantum = np.exp2((e - 3).astype(np.float64))
    q = np.rint(a / quantum).astype(np.int64)  # multiple count of the quantum
    # q in [8, 16] for normals (16 means carry into the next binade),
    # q in [0, 8] for subnormals (e == -6 and a < 2**-6)
    val = q.astype(np.float64) * quantum
    val = np.minimum(val, E4M3_MAX)
    code = _e4m3_code_of_exact(val)
    code = np.where(a_full >= E4M3_MAX, 0x7E, code)
    code = np.where(np.isnan(x), 0x7F, code | sign)
    return code.astype(np.uint8)


def _e4m3_code_of_exact(val):
    """Code of a non-negative float64 that is exactly representable."""
    out = np.zeros(val.shape, dtype=np.int64)
    sub = val < 2.0 ** -6
    out = np.where(sub, np.rint(val * 512.0).astype(np.int64), out)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(val > 0, val, 1.0))).astype(np.int64)
    e = np.where(np.exp2(e.astype(np.float64)) > val, e - 1, e)
    mant = np.rint((val / np.exp2(e.astype(np.float64)) - 1.0) * 8.0).astype(np.int64)
    nrm = ((e + 7) << 3) | mant
    return np.where(sub, out, nrm)
