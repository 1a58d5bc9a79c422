"""Bit-level number formats used by NVFP4, from their definitions.

Test infrastructure (see the package docstring); not part of the product path.

E2M1 (the element format): 4 bits ``s e e m``.  Bit 3 is the sign.  The low
three bits index the magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}: exponent field 0
is subnormal (m * 0.5), exponent fields 1..3 give 2**(e-1) * (1 + m/2).
Rounding to E2M1 is round-to-nearest with ties to the even code (the code
whose mantissa bit is 0), saturating at 6: the format has no Inf or NaN.

E4M3 (the block-scale format, the "FN" variant): bias 7, 3 mantissa bits,
subnormals in steps of 2**-9, largest finite value 448, codes 0x7F/0xFF are
NaN, no Inf.  Block scales are non-negative, so the sign bit is always 0.
Encoding is round-to-nearest-even on the mantissa, then saturation to 448.

bf16: the top 16 bits of an IEEE binary32; rounding is to nearest, ties to
even mantissa.
"""
import numpy as np

# --- E2M1 -----------------------------------------------------------------

E2M1_MAGNITUDE = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
# Rounding boundaries between consecutive magnitudes (exact in binary).
_E2M1_MID = (E2M1_MAGNITUDE[:-1] + E2M1_MAGNITUDE[1:]) / 2.0


def e2m1_decode(codes):
    """Code (uint8, 0..15) -> value (float64).  Code 0x8 is -0.0."""
    c = np.asarray(codes, dtype=np.uint8)
    mag = E2M1_MAGNITUDE[c & 0x7]
    return np.where((c & 0x8) != 0, -mag, mag)


def e2m1_magnitude_index(a):
    """|v| (float, >= 0) -> magnitude index 0..7: nearest, ties to even index.

    ``searchsorted(..., 'left')`` counts the boundaries strictly below a,
    which is the nearest index whenever a is not itself a boundary.  On a
    boundary between indices i and i+1 the even one of the two is taken.
    Values above 6 land on index 7 (saturation)."""
    a = np.asarray(a, dtype=np.float64)
    idx = np.searchsorted(_E2M1_MID, a, side="left")
    on_mid = (idx < _E2M1_MID.size) & (a == _E2M1_MID[np.minimum(idx, _E2M1_MID.size - 1)])
    idx = np.where(on_mid & (idx % 2 == 1), idx + 1, idx)
    return idx.astype(np.uint8)


# --- E4M3 (FN) --------------------------------------------------------------

def e4m3_decode(codes):
    """Code (uint8) -> value (float64); 0x7F and 0xFF decode to NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c & 0x80) != 0, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = m * 2.0 ** -9
    nor = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    val = sign * np.where(e == 0, sub, nor)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


# Non-negative finite E4M3 values, indexed by their code 0x00..0x7E.  They
# increase with the code, which the searches below rely on.
E4M3_POS_VALUES = e4m3_decode(np.arange(0x7F, dtype=np.uint8))
assert np.all(np.diff(E4M3_POS_VALUES) > 0)


def e4m3_encode_nonneg(s):
    """Non-negative finite s -> E4M3 code: nearest value, ties to the even
    code, anything above 448 saturating to 448 (code 0x7E), never NaN."""
    s = np.minimum(np.asarray(s, dtype=np.float64), 448.0)
    if np.any(~(s >= 0.0)):
        raise ValueError("e4m3_encode_nonneg needs finite non-negative input")
    v = E4M3_POS_VALUES
    hi = np.searchsorted(v, s, side="left")          # first value >= s
    hi = np.minimum(hi, v.size - 1)
    lo = np.maximum(hi - 1, 0)
    exact = v[hi] == s
    d_lo = s - v[lo]
    d_hi = v[hi] - s
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(exact, hi, np.where(pick_hi, hi, lo))
    return code.astype(np.uint8)


# --- bf16 -------------------------------------------------------------------

def bf16_round(x):
    """float32 values -> float32 values rounded to bf16 (nearest, ties even).

    Written with float64 arithmetic on the value, not with the bit trick:
    the unit in the last place of a bf16 number of binade 2**E is 2**(E-7)
    for normal numbers and 2**-133 below 2**-126.  Finite input only; a
    result beyond the largest bf16 becomes +-Inf as IEEE rounding would."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16_round needs finite input")
    ax = np.abs(x)
    _, e = np.frexp(ax)                      # ax = f * 2**e, f in [0.5, 1)
    e = e.astype(np.int64) - 1               # ax in [2**e, 2**(e+1))
    ulp_exp = np.maximum(e, -126) - 7
    ulp = np.exp2(ulp_exp.astype(np.float64))
    q = np.rint(ax / ulp) * ulp              # np.rint: ties to even integer
    q = np.where(ax == 0.0, 0.0, q)
    out = np.copysign(q, x)
    with np.errstate(over="ignore"):
        return out.astype(np.float32)


def bf16_bits(x):
    """float32 values already representable in bf16 -> their uint16 bits."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("value not representable in bf16")
    return (u >> 16).astype(np.uint16)


def bf16_from_bits(b):
    """uint16 bf16 bits -> float32 values."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
