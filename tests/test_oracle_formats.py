"""Pins of the oracle's codecs: printed values of the pages, closed forms and
brute force over every code."""
import json
import os

import numpy as np
import pytest

from oracle import formats as F

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def test_fp4_value_set_matches_page():
    mags = GOLD["fp4_value_set"]["magnitudes"]
    vals = F.e2m1_decode(np.arange(16))
    assert sorted(set(np.abs(vals).tolist())) == mags
    assert list(vals[:8]) == mags and list(-vals[8:]) == mags


def test_fp4_closed_form():
    # E2M1: 1 sign, 2 exponent, 1 mantissa bit, bias 1; exponent 0 is subnormal (m * 0.5)
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        v = (m * 0.5) if e == 0 else (1 + m / 2) * 2.0 ** (e - 1)
        assert F.e2m1_decode(c) == (-v if s else v)


def test_figure1_bits():
    g = GOLD["figure1_593_7"]
    assert F.e4m3_decode(int(g["scale_bits"], 2)) == g["scale"]
    assert F.e2m1_decode(int(g["value_bits"], 2)) == g["value"]


def test_e4m3_closed_form_and_range():
    # OCP E4M3FN: bias 7, subnormals m*2^-9, max 448, S.1111.111 NaN
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        got = F.e4m3_decode(c)
        if e == 15 and m == 7:
            assert np.isnan(got)
            continue
        v = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        assert got == (-v if s else v)
    rng = GOLD["range"]["outer_1"]
    # largest NVFP4 magnitude 6 * 448, smallest 0.5 * 2^-9
    assert 6 * F.E4M3_VAL.max() == rng[1]
    assert 0.5 * F.E4M3_VAL[1] == rng[0]


def test_e8m0_closed_form():
    assert F.e8m0_decode(127) == 1.0
    assert F.e8m0_decode(0) == 2.0 ** -127
    assert F.e8m0_decode(254) == 2.0 ** 127
    assert np.isnan(F.e8m0_decode(255))


def _brute_nearest_even(grid, v):
    d = np.abs(v[:, None] - grid[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    idx = np.argmax(cand, axis=1)                    # first (lowest) candidate
    two = cand.sum(axis=1) == 2
    # on a tie of two neighbours keep the even index
    idx = np.where(two & (idx % 2 == 1), idx + 1, idx)
    return idx


def _patterns(lo, hi, stride, midpoints):
    """float32 values: every ``stride``-th pattern in [lo, hi] plus +-2048
    patterns around each midpoint (where rounding decisions live)."""
    b_lo = np.float32(lo).view(np.uint32)
    b_hi = np.float32(hi).view(np.uint32)
    bits = [np.arange(b_lo, b_hi + 1, stride, dtype=np.uint32)]
    for m in midpoints:
        mb = np.float32(m).view(np.uint32)
        bits.append(np.arange(max(int(mb) - 2048, 0), int(mb) + 2049, dtype=np.uint32))
    return np.concatenate(bits).view(np.float32)


def test_e2m1_encoder_brute_force():
    g = F.E2M1_MAG
    mids = (g[1:] + g[:-1]) / 2
    v = _patterns(0.0, 8.0, 4093, list(mids) + [6.0])
    got = F.e2m1_encode_rne_sat(v)
    want = _brute_nearest_even(g, v.astype(np.float64))
    assert np.array_equal(got, want)
    # sign copied, also for magnitudes that round to zero
    got_n = F.e2m1_encode_rne_sat(-v)
    assert np.array_equal(got_n, want | 8)
    assert F.e2m1_encode_rne_sat(np.float32(-0.0)) == 8
    # saturation
    assert F.e2m1_encode_rne_sat(np.float32(1e30)) == 7


def test_e4m3_encoders_brute_force():
    g = F.E4M3_VAL
    mids = (g[1:] + g[:-1]) / 2
    v = _patterns(0.0, 480.0, 1021, list(mids[::3]) + [448.0, 2.0 ** -10])
    vd = v.astype(np.float64)
    assert np.array_equal(F.e4m3_encode_rne_sat(v), _brute_nearest_even(g, vd))
    # round-up capped: smallest code with value >= v
    ge = g[None, :] >= vd[:, None]
    want_ru = np.where(ge.any(axis=1), np.argmax(ge, axis=1), 0x7E)
    assert np.array_equal(F.e4m3_encode_ru_cap(v), want_ru)


def test_pack_nibble_order_and_bits_per_value():
    codes = np.arange(16, dtype=np.uint8)
    p = F.pack_fp4(codes)
    assert p[0] == 0x10 and p[7] == 0xFE
    assert np.array_equal(F.unpack_fp4(p), codes)
    b = GOLD["bits_per_value"]
    C = 4096
    assert (C / 2 + C / 16) * 8 / C == b["nvfp4"]          # codes + one E4M3 per 16
    assert (C + C / 32) * 8 / C == b["mxfp8"]              # codes + one E8M0 per 32
