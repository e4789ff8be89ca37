"""Element and scale codecs of NVFP4 and MXFP8.

Source: "End-to-End 4-Bit Training", section "Low-precision formats on
Blackwell" and its interactive NVFP4 figure (Figure 1):
  * FP4 (E2M1) values are +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}; the figure shows
    bits ``0 11 1`` = 6 (sign, 2 exponent bits, 1 mantissa bit, bias 1).
  * E4M3 scale: sign, 4 exponent bits, 3 mantissa bits; the figure shows
    bits ``0 1101 100`` = 2^(13-7) * 1.5 = 96 (bias 7).  The printed range
    of NVFP4 magnitudes [2^-10, 2688] fixes the largest E4M3 value at
    2688 / 6 = 448 and the smallest subnormal at 2^-10 / 0.5 = 2^-9, i.e.
    the OCP "E4M3FN" variant (no infinities, S.1111.111 is NaN).
  * E8M0 scale: 8 exponent bits, no sign, no mantissa: 2^(c-127), c = 255 NaN.

Encoders work on exact values: a float32 input is widened to float64 (exact)
and compared against the float64 grid (exact), so the only rounding decisions
are the ones stated here.
"""
import numpy as np

# ---------------------------------------------------------------- E2M1 (FP4)
# code layout: bit3 sign, bits2..1 exponent, bit0 mantissa
E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_MAX = 6.0


def e2m1_decode(codes):
    """FP4 code(s) 0..15 -> float64 value."""
    c = np.asarray(codes).astype(np.int64)
    mag = E2M1_MAG[c & 7]
    return np.where((c & 8) != 0, -mag, mag)


def _nearest_even(grid, v):
    """Index into an ascending, non-negative ``grid`` of the value nearest to
    ``v >= 0``; exact ties go to the even index; values past either end clamp
    to that end (saturation)."""
    v = np.asarray(v, dtype=np.float64)
    hi = np.searchsorted(grid, v, side="left")          # grid[hi-1] < v <= grid[hi]
    hi = np.clip(hi, 1, len(grid) - 1)
    lo = hi - 1
    dlo = v - grid[lo]
    dhi = grid[hi] - v
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(v <= grid[0], 0, idx)
    idx = np.where(v >= grid[-1], len(grid) - 1, idx)
    return idx


def e2m1_encode_rne_sat(y):
    """float32 y -> FP4 code: nearest magnitude, ties to the even code,
    magnitudes >= 6 saturate to 6, the sign bit is copied from y (also when
    the magnitude rounds to 0)."""
    y = np.asarray(y, dtype=np.float32)
    mag_idx = _nearest_even(E2M1_MAG, np.abs(y.astype(np.float64)))
    sign = np.signbit(y).astype(np.int64)
    return (mag_idx | (sign << 3)).astype(np.uint8)


# ---------------------------------------------------------------- E4M3 (FN)
def _e4m3_table():
    vals = []
    for c in range(0x7F):            # 0x00 .. 0x7E, positive finite codes
        e, m = c >> 3, c & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals, dtype=np.float64)


E4M3_VAL = _e4m3_table()             # index = code, ascending
E4M3_MAX = 448.0


def e4m3_decode(codes):
    """E4M3 code(s) -> float64 value (0x7F / 0xFF decode to NaN)."""
    c = np.asarray(codes).astype(np.int64)
    mag = np.where((c & 0x7F) == 0x7F, np.nan, E4M3_VAL[np.minimum(c & 0x7F, 0x7E)])
    return np.where((c & 0x80) != 0, -mag, mag)


def e4m3_encode_rne_sat(v):
    """Non-negative value -> E4M3 code, round to nearest, ties to even,
    saturating at 448."""
    return _nearest_even(E4M3_VAL, v).astype(np.uint8)


def e4m3_encode_ru_cap(v):
    """Non-negative value -> smallest E4M3 code whose value is >= v; values
    above 448 give 448."""
    v = np.asarray(v, dtype=np.float64)
    idx = np.searchsorted(E4M3_VAL, v, side="left")
    return np.minimum(idx, 0x7E).astype(np.uint8)


def e4m3_encode_exact(v):
    """Signed value that lies exactly on the E4M3 grid -> code. Raises if not."""
    v = np.asarray(v, dtype=np.float64)
    idx = np.searchsorted(E4M3_VAL, np.abs(v), side="left")
    idx = np.minimum(idx, 0x7E)
    if not np.all(E4M3_VAL[idx] == np.abs(v)):
        raise ValueError("value not on the E4M3 grid")
    return (idx | (np.signbit(v).astype(np.int64) << 7)).astype(np.uint8)


def e2m1_encode_exact(v):
    """Signed value that lies exactly on the FP4 grid -> code. Raises if not."""
    v = np.asarray(v, dtype=np.float64)
    idx = np.searchsorted(E2M1_MAG, np.abs(v), side="left")
    idx = np.minimum(idx, 7)
    if not np.all(E2M1_MAG[idx] == np.abs(v)):
        raise ValueError("value not on the FP4 grid")
    return (idx | (np.signbit(v).astype(np.int64) << 3)).astype(np.uint8)


# ---------------------------------------------------------------- E8M0
def e8m0_decode(codes):
    """E8M0 code(s) -> float64 2^(c-127); 255 -> NaN."""
    c = np.asarray(codes).astype(np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - 127))


# ---------------------------------------------------------------- packing
def pack_fp4(codes):
    """[..., 2n] FP4 codes -> [..., n] bytes; element 2k in the low nibble."""
    c = np.asarray(codes).astype(np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_fp4(packed):
    """[..., n] bytes -> [..., 2n] FP4 codes; low nibble first."""
    p = np.asarray(packed).astype(np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out
