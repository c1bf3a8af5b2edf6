"""Storage formats: BF16 and OCP FP8 E4M3 (E4M3FN), decoded to and rounded from fp64.

Page A, "Why does dynamic scheduling matter in attention?": the backend runs
in BF16 and in FP8.  Page B, intro: the FP8 type is E4M3.  The bit layout is
the OCP OFP8 rev. 1.0 E4M3 format: 1 sign bit, 4 exponent bits with bias 7,
3 mantissa bits, subnormals, no infinities, and S.1111.111 as NaN, so the
largest finite magnitude is 448.

Rounding is round-to-nearest-even, computed exactly in fp64 with rint (which
rounds halves to even) on a value scaled by a power of two, so no step here
rounds twice.  Reading R9: a value is clamped to [-448, 448] *before* it is
rounded to E4M3, i.e. out-of-range values saturate instead of becoming NaN.
"""

import numpy as np

BF16_NAN_BITS = 0x7FC0
E4M3_NAN_CODE = 0x7F
E4M3_MAX = 448.0


def bf16_bits_to_f64(bits):
    """BF16 bit patterns (uint16) -> exact fp64 values.

    A BF16 value is the upper half of an IEEE binary32 word, so the decode is
    a 16-bit shift and a reinterpretation; fp32 -> fp64 is exact.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):          # NaN payloads convert to NaN
        return b.view(np.float32).astype(np.float64)


def _round_to_quantum(x, quantum):
    """RNE of x to a multiple of ``quantum`` (a power of two): exact in fp64."""
    return np.rint(x / quantum) * quantum


def f64_to_bf16_bits(x):
    """fp64 -> BF16 bit patterns with one round-to-nearest-even step.

    BF16 keeps 8 significant bits (7 stored), exponent range of binary32:
    normal numbers have quantum 2**(e-7) for |x| in [2**e, 2**(e+1)), the
    subnormal quantum is 2**-133.  Results that round past the largest finite
    value become +-inf; NaN becomes the canonical quiet NaN 0x7FC0.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_x = x.reshape(-1)
    flat_o = out.reshape(-1)
    nan = np.isnan(flat_x)
    ax = np.abs(flat_x)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
        # log2 of a value just below a power of two can round up: fix the binade.
        e = np.where(np.ldexp(1.0, e.astype(np.int64)) > ax, e - 1, e)
        e = np.where(np.ldexp(1.0, (e + 1).astype(np.int64)) <= ax, e + 1, e)
        e = np.maximum(e, -126.0)               # below 2**-126: subnormal quantum
        quantum = np.ldexp(1.0, (e - 7).astype(np.int64))
        r = np.where(np.isfinite(flat_x), _round_to_quantum(flat_x, quantum), flat_x)
    # r is exactly representable in binary32 unless it overflowed BF16's range.
    big = np.abs(r) >= 2.0 ** 128
    r = np.where(big, np.copysign(np.inf, flat_x), r)
    r32 = r.astype(np.float32)
    bits = (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits[nan] = BF16_NAN_BITS
    flat_o[:] = bits
    return out


def e4m3_to_f64(codes):
    """E4M3FN codes (uint8) -> fp64 values (NaN for 0x7F and 0xFF).

    Exponent field E and mantissa M: E = 0 gives M * 2**-9 (subnormal);
    otherwise (1 + M/8) * 2**(E-7).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp_field = (c >> 3) & 0xF
    mant = c & 0x7
    sub = mant * 2.0 ** -9
    norm = (1.0 + mant / 8.0) * np.ldexp(1.0, exp_field - 7)
    mag = np.where(exp_field == 0, sub, norm)
    mag = np.where((exp_field == 15) & (mant == 7), np.nan, mag)
    return sign * mag


def f64_to_e4m3(x):
    """fp64 -> E4M3FN codes: clamp to +-448 (R9), then one RNE step.

    Normal binades [2**e, 2**(e+1)) for e in [-6, 8] have quantum 2**(e-3);
    below 2**-6 the subnormal quantum is 2**-9.  A value that rounds up into
    the next binade is still encoded exactly (its new exponent is recomputed).
    NaN -> 0x7F.  The sign of zero is kept.
    """
    x = np.asarray(x, dtype=np.float64)
    nan = np.isnan(x)
    xc = np.clip(np.where(nan, 0.0, x), -E4M3_MAX, E4M3_MAX)
    ax = np.abs(xc)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.where(np.ldexp(1.0, e.astype(np.int64)) > ax, e - 1, e)
    e = np.where(np.ldexp(1.0, (e + 1).astype(np.int64)) <= ax, e + 1, e)
    e = np.maximum(e, -6.0)
    quantum = np.ldexp(1.0, (e - 3).astype(np.int64))
    r = np.abs(_round_to_quantum(xc, quantum))          # exact multiple of quantum
    # encode the rounded magnitude
    with np.errstate(divide="ignore"):
        re = np.floor(np.log2(np.where(r > 0, r, 1.0)))
    re = np.where(np.ldexp(1.0, re.astype(np.int64)) > r, re - 1, re)
    is_sub = r < 2.0 ** -6
    exp_field = np.where(is_sub, 0, re + 7).astype(np.int64)
    mant = np.where(is_sub, np.rint(r / 2.0 ** -9),
                    np.rint((r / np.ldexp(1.0, re.astype(np.int64)) - 1.0) * 8.0)).astype(np.int64)
    code = (exp_field << 3) | mant
    code = np.where(np.signbit(xc), code | 0x80, code)
    code = np.where(nan, E4M3_NAN_CODE, code)
    return code.astype(np.uint8)
