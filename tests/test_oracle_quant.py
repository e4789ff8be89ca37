"""Pins of the oracle's quantizers: the pages' worked examples, brute force
over every 16x16 tile of small inputs, and the SR unbiasedness test."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F
from oracle import quant as Q
from oracle.rng import sr_bits16

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))
f32 = np.float32


def q1(row, outer=1.0):
    """Quantize one row with a given outer scale; return (codes, scale values)."""
    x = np.asarray(row, dtype=f32)[None, None, :]
    p, s, _ = Q.quantize_nvfp4(x, Q.OUTER_GIVEN, np.array([outer], f32))
    return F.unpack_fp4(p)[0, 0], F.e4m3_decode(s[0, 0])


def test_minus_54_block():
    g = GOLD["block_max_minus_54"]
    row = np.zeros(16, f32)
    row[3] = g["block_max"]
    row[5] = 10.0
    codes, sc = q1(row, g["outer"])
    assert sc[0] == g["scale"]
    assert F.e2m1_decode(codes[3]) == g["value"]


def test_figure1_593_7():
    g = GOLD["figure1_593_7"]
    row = np.zeros(16, f32)
    row[0] = g["input"]
    codes, sc = q1(row, g["outer"])
    assert sc[0] == g["scale"]
    assert F.e2m1_decode(codes[0]) == g["value"]
    rec = F.e2m1_decode(codes[0]) * sc[0]
    assert rec == g["reconstructed"]
    assert abs((rec - g["input"]) - g["error"]) < 1e-3


def test_5_4_forward_value():
    g = GOLD["sr_5_4"]
    row = np.zeros(16, f32)
    row[0] = g["forward_block_max"]
    row[1] = g["input"]
    codes, sc = q1(row)
    assert sc[0] == g["forward_scale"]
    assert F.e2m1_decode(codes[1]) * sc[0] == g["forward_value"]


@pytest.mark.parametrize("key,outer", [("outer_1", 1.0), ("outer_2", 2.0), ("outer_0_5", 0.5)])
def test_range_shifts_with_outer_scale(key, outer):
    lo, hi = GOLD["range"][key]
    # the largest magnitude is representable exactly
    codes, sc = q1(np.r_[hi, np.zeros(15)], outer)
    assert F.e2m1_decode(codes[0]) * sc[0] * outer == hi
    # the smallest: a block whose max is 6 * 2^-9 * outer has the smallest scale 2^-9
    blk = np.zeros(16, f32)
    blk[0] = 6 * 2.0 ** -9 * outer
    blk[1] = lo
    codes, sc = q1(blk, outer)
    assert sc[0] == 2.0 ** -9
    assert F.e2m1_decode(codes[1]) * sc[0] * outer == lo
    # half of it is a tie between 0 and the smallest value and rounds to even (0)
    blk[1] = lo / 2
    codes, sc = q1(blk, outer)
    assert F.e2m1_decode(codes[1]) == 0


def test_outer_scale_per_tensor_row_expert():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 8, 64)).astype(f32) * np.array([1, 100, 1e-3], f32)[:, None, None]
    for mode in (Q.OUTER_TENSOR, Q.OUTER_ROW):
        p, s, st = Q.quantize_nvfp4(x, mode)
        amax = np.abs(x).max(axis=(1, 2)) if mode == Q.OUTER_TENSOR else np.abs(x).max(axis=2)
        assert np.array_equal(st, (amax / f32(2688)).astype(f32))
        xh = Q.dequantize_nvfp4_f64(p, s, st, mode)
        # the group maximum is reproduced to within one FP4/E4M3 step of the top of the range
        top = np.abs(xh).max(axis=(1, 2)) if mode == Q.OUTER_TENSOR else np.abs(xh).max(axis=2)
        assert np.all(np.abs(top - amax) <= amax * 2e-3)
    # all-zero group -> outer scale 1 and zero codes
    z = np.zeros((1, 2, 32), f32)
    p, s, st = Q.quantize_nvfp4(z, Q.OUTER_TENSOR)
    assert st[0] == 1.0 and not p.any() and not s.any()


def _near_tie(v, grid, rel=1e-6):
    mids = (grid[1:] + grid[:-1]) / 2
    return np.min(np.abs(v[:, None] - mids[None, :]), axis=1) <= rel * np.maximum(np.abs(v), 1e-30)


@pytest.mark.parametrize("shape,dist,seed", [((32, 32), "normal", 0), ((64, 64), "normal", 1),
                                             ((64, 64), "t3", 2), ((32, 32), "outlier", 3),
                                             ((32, 32), "zeros", 4), ((64, 64), "wide", 5)])
def test_brute_force_every_16x16_tile(shape, dist, seed):
    rng = np.random.default_rng(seed)
    if dist == "normal":
        x = rng.standard_normal(shape)
    elif dist == "t3":
        x = rng.standard_t(3, shape)
    elif dist == "outlier":
        x = rng.uniform(1, 2, shape)
        x[rng.integers(0, shape[0]), rng.integers(0, shape[1])] = 1000.0
    elif dist == "zeros":
        x = rng.standard_normal(shape)
        x[:16, :16] = 0.0
        x[16:, 16:] = -0.0
    else:
        x = rng.standard_normal(shape) * np.exp(rng.uniform(-20, 20, shape))
    x = x.astype(f32)
    for mode, outer in ((Q.OUTER_TENSOR, None), (Q.OUTER_GIVEN, np.array([0.37], f32))):
        p, s, st = Q.quantize_nvfp4(x[None], mode, outer)
        codes = F.unpack_fp4(p)[0]
        st = float(np.asarray(st).reshape(-1)[0])
        R, C = shape
        for ti in range(R // 16):
            for tj in range(C // 16):
                blk = x[ti * 16:(ti + 1) * 16, tj * 16:(tj + 1) * 16].astype(np.float64)   # 16 row blocks
                ab = np.abs(blk).max(axis=1)
                ratio = ab / (6 * st)
                got_s = s[0, ti * 16:(ti + 1) * 16, tj]
                want_s = np.argmin(np.abs(F.E4M3_VAL[None, :] - ratio[:, None]), axis=1)
                bad = (got_s != want_s) & ~_near_tie(ratio, F.E4M3_VAL)
                assert not bad.any(), (ti, tj)
                D = F.e4m3_decode(got_s) * st
                live = D >= 2.0 ** -126
                yv = np.where(live[:, None], blk / np.where(live, D, 1)[:, None], 0.0)
                want_c = np.argmin(np.abs(F.E2M1_MAG[None, :] - np.abs(yv).reshape(-1)[:, None]), axis=1).reshape(16, 16)
                got_c = codes[ti * 16:(ti + 1) * 16, tj * 16:(tj + 1) * 16]
                nt = _near_tie(np.abs(yv).reshape(-1), F.E2M1_MAG).reshape(16, 16)
                assert not (((got_c & 7) != want_c) & ~nt).any(), (ti, tj)
                assert np.array_equal(got_c >> 3, np.signbit(blk.astype(f32)).astype(np.uint8))


def test_figure3_outlier_tile():
    g = GOLD["figure3_outlier_tile"]
    rng = np.random.default_rng(11)
    x = rng.uniform(1.0, 2.0, (16, 16)).astype(f32)
    x[15, 7] = 100.0                                         # one outlier in the last row
    p, s, _ = Q.quantize_nvfp4(x[None], Q.OUTER_GIVEN, np.array([1.0], f32))
    assert int(np.count_nonzero(F.unpack_fp4(p)[0] & 7)) == g["survive_1x16"]
    codes, _ = Q.quantize_nvfp4_tile16(x, 1.0)
    assert int(np.count_nonzero(codes & 7)) == g["survive_16x16"]


def test_figure2_row_vs_column_scaling():
    g = GOLD["figure2_row_tile"]
    rng = np.random.default_rng(12)
    x = rng.uniform(0.5, 2.0, (16, 16)).astype(f32)
    x[0] = rng.uniform(40.0, 64.0, 16).astype(f32)           # first row large
    p, s, _ = Q.quantize_nvfp4(x[None], Q.OUTER_GIVEN, np.array([1.0], f32))
    assert int(np.count_nonzero(F.unpack_fp4(p)[0] & 7)) == g["survive_rows"]
    # 16x1 column blocks = 1x16 blocks of the transpose
    p, s, _ = Q.quantize_nvfp4(x.T.copy()[None], Q.OUTER_GIVEN, np.array([1.0], f32))
    c = F.unpack_fp4(p)[0].T
    assert np.all(c[0] & 7)                                   # the large row survives
    assert int(np.count_nonzero(c[1:] & 7)) < 240 // 2        # most small values flush


# ------------------------------------------------------------------ SR
def sr_example_tile():
    """16x32 tile whose transposed block 0 holds the dequantized 4.5 next to a
    12 (new scale 12/6 = 2) and a 2688 elsewhere so the new outer scale is 1."""
    g = GOLD["sr_5_4"]
    x = np.full((16, 32), 0.125, f32)
    x[0, 0] = g["input"]
    x[0, 1] = g["forward_block_max"]
    x[1, 0] = 12.0
    x[2, 20] = 2688.0
    return x


def test_sr_worked_example_rn_and_counts():
    g = GOLD["sr_5_4"]
    x = sr_example_tile()
    p, s, st = Q.quantize_nvfp4(x[None], Q.OUTER_GIVEN, np.array([1.0], f32))
    xh = Q.dequantize_nvfp4(p, s, st, Q.OUTER_GIVEN)[0]
    assert xh[0, 0] == g["forward_value"] and xh[1, 0] == 12.0 and xh[2, 20] == 2688.0
    # deterministic rounding of the transposed value
    pr, sr, str_ = Q.requant_transpose_sr(p, s, st, Q.OUTER_GIVEN, Q.NVFP4, 0, 0, rnd=Q.RN)
    assert str_[0] == 1.0 and F.e4m3_decode(sr[0, 0, 0]) == g["new_scale"]
    assert F.e2m1_decode(F.unpack_fp4(pr)[0, 0, 0]) == g["rn_code_value"]
    # stochastic rounding over 10^4 seeds: 2 w.p. 3/4, 3 w.p. 1/4
    n = 10_000
    highs = 0
    for seed in range(n):
        pr, sr, _ = Q.requant_transpose_sr(p, s, st, Q.OUTER_GIVEN, Q.NVFP4, seed, 0)
        v = F.e2m1_decode(F.unpack_fp4(pr)[0, 0, 0])
        assert v in (g["sr_low"], g["sr_high"])
        highs += v == g["sr_high"]
    mean = n * g["p_high"]
    sd = np.sqrt(n * g["p_high"] * (1 - g["p_high"]))
    assert abs(highs - mean) <= 4 * sd
    # and the 16-bit draw gives exactly p = 1/4: 16384 of the 65536 values satisfy (r + 1/2)/2^16 < 1/4
    assert np.count_nonzero((np.arange(65536) + 0.5) / 65536 < 0.25) == 16384


def _sr_stats(vals, z, step, n):
    """Fraction of elements whose mean over n draws lies outside
    4 sigma/sqrt(n) (+ one draw and the 2^-17 resolution) of z, and the pooled z-score."""
    mean = vals.mean(axis=0)
    frac = np.clip((np.abs(z) - np.floor(np.abs(z) / step) * step) / step, 0, 1)
    sigma = step * np.sqrt(frac * (1 - frac))
    dev = np.abs(mean - z)
    bad = dev > 4 * sigma / np.sqrt(n) + step / n + step * 2.0 ** -17
    pooled = np.sum(mean - z) / np.sqrt(np.sum(sigma ** 2) / n + 1e-300)
    return int(bad.sum()), float(pooled)


@pytest.mark.parametrize("fmt", [Q.NVFP4, Q.MXFP8])
def test_sr_unbiased_over_10k_seeds(fmt):
    """Mean of the SR requantization over 10^4 seeds vs the dequantized input
    (E[w_q] = E[(w_q^T)^T])."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((64, 64)).astype(f32)
    x[3, 5] = 40.0
    p, s, st = Q.quantize_nvfp4(x[None], Q.OUTER_TENSOR)
    z = Q.dequantize_nvfp4(p, s, st, Q.OUTER_TENSOR)[0].T.astype(np.float64)   # [C, R]
    n = 10_000
    vals = np.empty((n, 64, 64))
    for seed in range(n):
        out = Q.requant_transpose_sr(p, s, st, Q.OUTER_TENSOR, fmt, seed, 5)
        if fmt == Q.NVFP4:
            pc, sc, st2 = out
            vals[seed] = F.e2m1_decode(F.unpack_fp4(pc)[0]) * np.repeat(F.e4m3_decode(sc[0]), 16, axis=1) * float(st2[0])
            if seed == 0:
                step = np.repeat(F.e4m3_decode(sc[0]), 16, axis=1) * float(st2[0])
                y = z / step
                step = step * np.where(np.abs(y) < 2, 0.5, np.where(np.abs(y) < 4, 1.0, 2.0))
        else:
            pc, sc = out
            vals[seed] = Q.dequantize_mxfp8_f64(pc[0], sc[0])
            if seed == 0:
                scale = np.repeat(F.e8m0_decode(sc[0]), 32, axis=1)
                y = np.abs(z) / scale
                e = np.floor(np.log2(np.maximum(y, 2.0 ** -6)))
                step = 2.0 ** (e - 3) * scale
    # scales do not depend on the seed
    bad, pooled = _sr_stats(vals, z, step, n)
    assert bad <= 3, bad
    assert abs(pooled) <= 4, pooled


def test_requant_scales_seed_independent_and_brute_force():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((64, 96)) * np.exp(rng.uniform(-4, 4, (64, 96)))).astype(f32)
    p, s, st = Q.quantize_nvfp4(x[None], Q.OUTER_ROW)
    z = Q.dequantize_nvfp4(p, s, st, Q.OUTER_ROW)[0].T.astype(np.float64)      # [96, 64]
    c1, s1 = Q.requant_transpose_sr(p, s, st, Q.OUTER_ROW, Q.MXFP8, 1, 3)
    c2, s2 = Q.requant_transpose_sr(p, s, st, Q.OUTER_ROW, Q.MXFP8, 2, 3)
    assert np.array_equal(s1, s2) and not np.array_equal(c1, c2)
    ab = np.abs(z).reshape(96, 2, 32).max(axis=2)
    # smallest E8M0 code c with a_b <= 448 * 2^(c-127), by trying every code
    cand = ab[..., None] <= 448.0 * np.ldexp(1.0, np.arange(255) - 127)
    assert np.array_equal(s1[0], np.argmax(cand, axis=-1))
    # every SR code is one of the two grid neighbours of y = z / scale
    y = z / np.repeat(F.e8m0_decode(s1[0]), 32, axis=1)
    v = np.abs(F.e4m3_decode(c1[0]))
    lo_idx = np.searchsorted(F.E4M3_VAL, np.abs(y), side="right") - 1
    assert np.all((v == F.E4M3_VAL[lo_idx]) | (v == F.E4M3_VAL[np.minimum(lo_idx + 1, 126)]))
    # NVFP4 target: round-up scale is the smallest code >= exact a_b / (6 s_t')
    c3, s3, st3 = Q.requant_transpose_sr(p, s, st, Q.OUTER_ROW, Q.NVFP4, 1, 3)
    assert st3[0] == np.float32(np.float32(np.abs(z).max()) / np.float32(2688))
    ab16 = np.abs(z).reshape(96, 4, 16).max(axis=2)
    ratio = ab16 / (6 * float(st3[0]))
    ge = F.E4M3_VAL[None, None, :] >= ratio[..., None]
    want = np.where(ge.any(-1), np.argmax(ge, axis=-1), 0x7E)
    # exempt ratios within float32 rounding of a grid value (the spec divides in float32)
    near = np.min(np.abs(F.E4M3_VAL[None, None, :] - ratio[..., None]), axis=-1) <= 1e-6 * ratio
    assert not ((s3[0] != want) & ~near).any()
    assert np.count_nonzero(near) < ratio.size // 50


def test_sr_decision_matches_definition_on_random_elements():
    """Independent exact check of a sample of SR decisions with rationals."""
    rng = np.random.default_rng(13)
    x = rng.standard_normal((32, 64)).astype(f32)
    p, s, st = Q.quantize_nvfp4(x[None], Q.OUTER_TENSOR)
    codes, sc = Q.requant_transpose_sr(p, s, st, Q.OUTER_TENSOR, Q.MXFP8, 1234, 9)
    z = Q.dequantize_nvfp4(p, s, st, Q.OUTER_TENSOR)[0].T
    idx = np.arange(64 * 32, dtype=np.uint64).reshape(64, 32)
    r = sr_bits16(1234, 9, idx)
    for (i, j) in [(a, b) for a in range(0, 64, 7) for b in range(0, 32, 3)]:
        e = int(sc[0, i, j // 32]) - 127
        y = Fraction(float(z[i, j])) / Fraction(2) ** e
        m = abs(y)
        grid = [Fraction(float(g)) for g in F.E4M3_VAL]
        lo = max(g for g in grid if g <= m)
        hi = min([g for g in grid if g > m], default=lo)
        delta = (m - lo) / (hi - lo) if hi != lo else Fraction(0)
        up = Fraction(2 * int(r[i, j]) + 1, 1 << 17) < delta
        want = hi if up else lo
        assert Fraction(float(abs(F.e4m3_decode(codes[0, i, j])))) == want


def test_mxfp8_rn_and_zero_block():
    x = np.zeros((2, 64), f32)
    x[0, :32] = np.linspace(-3, 500, 32)
    c, s = Q.quantize_mxfp8(x, Q.RN)
    # block max 500 -> smallest 2^e with 500 <= 448 * 2^e is 2^1
    assert s[0, 0] == 128 and s[0, 1] == 0 and s[1, 0] == 0
    assert not c[1].any() and not c[0, 32:].any()
    assert np.all(np.abs(F.e4m3_decode(c[0, :32]) * 2 - x[0, :32]) <= np.abs(x[0, :32]) / 16 + 1e-9)


def test_segmented_transposed_layout_and_padding():
    rng = np.random.default_rng(3)
    seg = np.array([0, 5, 5, 40, 72], dtype=np.int64)          # includes an empty and a ragged segment
    x = rng.standard_normal((72, 64)).astype(f32)
    codes, scales = Q.quantize_mxfp8_transposed(x, seg, Q.SR, 4, 2)
    mp, base = Q.segmented_layout(seg, 64)
    assert mp == [32, 0, 64, 32] and codes.size == 64 * 128 and scales.size == 64 * 4
    # segment 2 = rows 5..39 (35 rows) padded to 64 tokens; the padding is code 0
    blk = codes[base[2]:base[2] + 64 * 64].reshape(64, 64)
    assert not blk[:, 35:].any()
    # same values as the plain transposed quantizer applied to the padded segment
    Z = np.zeros((64, 64), f32)
    Z[:, :35] = x[5:40].T
    idx = (np.uint64(base[2]) + np.arange(64 * 64, dtype=np.uint64)).reshape(64, 64)
    c2, s2 = Q.mxfp8_quantize(Z, idx, Q.SR, 4, 2)
    assert np.array_equal(blk, c2)


def _token_table(rng, T, C):
    """NVFP4 token rows with per-row outer scales over a wide range."""
    x = rng.standard_normal((T, C)).astype(f32) * np.exp2(rng.integers(-6, 7, (T, 1))).astype(f32)
    p, s, o = Q.quantize_nvfp4(x[None], Q.OUTER_ROW)
    return p[0], s[0], o[0]


@pytest.mark.parametrize("rnd", [Q.RN, Q.SR])
def test_requant_segmented_gather_equals_pregathered_batch(rnd):
    """Dispatched row m reads token row_gather[m] with that token's outer
    scale. Segments of equal length R (a multiple of 32) start at element
    e*C*R of the output, so segment e must equal the batch requantizer (item
    e) applied to the table gathered here with NumPy indexing: a swapped or
    shifted gather index, or an outer scale taken from the wrong row, breaks
    the equality (SR draws included)."""
    rng = np.random.default_rng(21)
    T, C, R, nseg = 50, 64, 32, 3
    p, s, o = _token_table(rng, T, C)
    gather = rng.integers(0, T, nseg * R)                    # repeats and any order
    seg = np.arange(nseg + 1, dtype=np.int64) * R
    codes, scales = Q.requant_transpose_sr_segmented(p, s, o, Q.OUTER_ROW, gather, seg, 7, 3, rnd=rnd)
    for e in range(nseg):
        g = gather[e * R:(e + 1) * R]
        c2, s2 = Q.requant_transpose_sr(p[g][None], s[g][None], o[g][None], Q.OUTER_ROW, Q.MXFP8, 7, 3, rnd=rnd,
                                        item0=e)
        assert np.array_equal(codes[e * C * R:(e + 1) * C * R], c2.reshape(-1))
        assert np.array_equal(scales[e * C * R // 32:(e + 1) * C * R // 32], s2.reshape(-1))


def test_requant_segmented_gather_ragged_equals_dequantize_then_gather():
    """Ragged and empty segments: the result equals the transposed MXFP8
    quantizer applied to the rows of the dequantized token table taken in
    gather order (the whole table dequantized first, then indexed)."""
    rng = np.random.default_rng(22)
    T, C = 40, 64
    p, s, o = _token_table(rng, T, C)
    seg = np.array([0, 7, 7, 70, 101], dtype=np.int64)
    gather = rng.integers(0, T, 101)
    codes, scales = Q.requant_transpose_sr_segmented(p, s, o, Q.OUTER_ROW, gather, seg, 9, 3)
    table = Q.dequantize_nvfp4(p[None], s[None], o[None], Q.OUTER_ROW)[0]
    c2, s2 = Q.quantize_mxfp8_transposed(table[gather], seg, Q.SR, 9, 3)
    assert np.array_equal(codes, c2) and np.array_equal(scales, s2)
    # a shifted gather gives a different result (the check can fail)
    c3, _ = Q.quantize_mxfp8_transposed(table[np.roll(gather, 1)], seg, Q.SR, 9, 3)
    assert not np.array_equal(codes, c3)


# ---------------------------------------------------------------- Four Over Six
def _given(x):
    return Q.quantize_nvfp4(np.asarray(x, np.float32).reshape(1, 1, -1), Q.OUTER_GIVEN,
                            np.ones(1, np.float32), four_over_six=True)


def test_four_over_six_worked_blocks():
    """A block of 5.0 (outer scale 1): the 6 scale 5/6 rounds to E4M3 0.8125,
    so 5 -> 6.15 -> 6 -> 4.875; the 4 scale 5/4 = 1.25 is exact and gives 5
    exactly, so 4/6 keeps it. A block [6, 1, ..., 1]: the 6 scale (1.0) is
    exact; the 4 scale 1.5 sends 1 to 1/1.5 -> 0.5 -> 0.75, so 6 is kept."""
    plain = Q.quantize_nvfp4(np.full((1, 1, 16), 5.0, np.float32), Q.OUTER_GIVEN, np.ones(1, np.float32))
    assert int(plain[1][0, 0, 0]) == 0x35  # 0.8125
    assert np.all(Q.dequantize_nvfp4(*plain, Q.OUTER_GIVEN) == np.float32(4.875))
    fs = _given(np.full(16, 5.0))
    assert int(fs[1][0, 0, 0]) == 0x3A     # 1.25
    assert np.all(Q.dequantize_nvfp4(*fs, Q.OUTER_GIVEN) == np.float32(5.0))
    blk = np.ones(16, np.float32)
    blk[0] = 6.0
    fs = _given(blk)
    assert int(fs[1][0, 0, 0]) == 0x38     # 1.0: the 6 scale
    assert np.array_equal(Q.dequantize_nvfp4(*fs, Q.OUTER_GIVEN).reshape(-1), blk)


def _f64_block_errors(x, packed, scales, outer):
    xh = Q.dequantize_nvfp4_f64(packed, scales, outer, Q.OUTER_GIVEN)
    d = x.astype(np.float64) - xh
    return (d * d).reshape(x.shape[0], x.shape[1], -1, 16).sum(-1)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_four_over_six_choice_matches_exact_errors(seed):
    """Independent of the float32 error sum: compute both candidates' block
    errors in float64 from their dequantized values; wherever they differ by
    more than float32 rounding could explain, 4/6 must have taken the smaller."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((1, 64, 512)) * np.exp(rng.standard_normal((1, 64, 1)))).astype(np.float32)
    outer = np.ones(1, np.float32)
    six = Q.quantize_nvfp4(x, Q.OUTER_GIVEN, outer)
    fs = Q.quantize_nvfp4(x, Q.OUTER_GIVEN, outer, four_over_six=True)
    # the 4 candidate alone: scales from r4, codes as RTN
    a_b = np.abs(x.reshape(1, 64, 32, 16)).max(-1)
    s4 = F.e4m3_encode_rne_sat((a_b / np.float32(4.0)).astype(np.float32))
    e6 = _f64_block_errors(x, *six[:2], outer)
    took4 = fs[1] != six[1]
    assert np.all(fs[1][took4] == s4[took4])
    # float64 errors of what 4/6 produced vs of the plain 6 choice
    efs = _f64_block_errors(x, *fs[:2], outer)
    clear = np.abs(efs - e6) > 1e-5 * np.maximum(e6, 1e-30)
    assert np.all(efs[clear & took4] < e6[clear & took4])
    assert took4.mean() > 0.1 and (~took4).mean() > 0.1


def test_four_over_six_never_worse_and_off_by_default():
    rng = np.random.default_rng(5)
    x = rng.standard_t(3, (2, 32, 256)).astype(np.float32)
    for mode in (Q.OUTER_TENSOR, Q.OUTER_ROW):
        plain = Q.quantize_nvfp4(x, mode)
        fs = Q.quantize_nvfp4(x, mode, four_over_six=True)
        assert np.array_equal(plain[2], fs[2])            # outer scales unchanged
        d_plain = x.astype(np.float64) - Q.dequantize_nvfp4_f64(*plain, mode)
        d_fs = x.astype(np.float64) - Q.dequantize_nvfp4_f64(*fs, mode)
        e_plain = (d_plain ** 2).reshape(2, 32, 16, 16).sum(-1)
        e_fs = (d_fs ** 2).reshape(2, 32, 16, 16).sum(-1)
        assert np.all(e_fs <= e_plain * (1 + 1e-5) + 1e-30)
        assert e_fs.sum() < 0.95 * e_plain.sum()


def _square_inputs(dist, shape, seed):
    rng = np.random.default_rng(seed)
    if dist == "normal":
        x = rng.standard_normal(shape)
    elif dist == "outlier":
        x = rng.uniform(1, 2, shape)
        x[..., rng.integers(0, shape[-2]), rng.integers(0, shape[-1])] = 1000.0
    elif dist == "zeros":
        x = rng.standard_normal(shape)
        x[..., :16, :16] = 0.0
        x[..., 16:32, 16:32] = -0.0
    else:
        x = rng.standard_normal(shape) * np.exp(rng.uniform(-20, 20, shape))
    return x.astype(f32)


@pytest.mark.parametrize("dist,seed", [("normal", 0), ("outlier", 1), ("zeros", 2), ("wide", 3)])
def test_square_tile_brute_force(dist, seed):
    """Every 16x16 tile against a float64 nearest-value search: the tile scale is
    the E4M3 value nearest to (tile max)/(6 s_t), each element the E2M1 value
    nearest to x/(s_b s_t); near-ties are skipped."""
    x = _square_inputs(dist, (2, 48, 64), seed)
    for mode, outer in ((Q.OUTER_TENSOR, None), (Q.OUTER_GIVEN, np.array([0.37, 2.5], f32))):
        p, s, st = Q.quantize_nvfp4_square(x, mode, outer)
        codes = F.unpack_fp4(p)
        for b in range(2):
            stb = float(st[b])
            if mode == Q.OUTER_TENSOR:
                amax = float(np.abs(x[b]).max())
                assert stb == (f32(amax) / f32(2688.0) if amax > 0 else 1.0)
            for ti in range(3):
                for tj in range(4):
                    blk = x[b, ti * 16:(ti + 1) * 16, tj * 16:(tj + 1) * 16].astype(np.float64)
                    ratio = np.abs(blk).max() / (6 * stb)
                    got = s[b, ti * 16:(ti + 1) * 16, tj]
                    assert (got == got[0]).all()                  # one scale for the 16 rows
                    want = int(np.argmin(np.abs(F.E4M3_VAL - ratio)))
                    if not _near_tie(np.array([ratio]), F.E4M3_VAL)[0]:
                        assert got[0] == want, (b, ti, tj)
                    D = F.e4m3_decode(got[0]) * stb
                    yv = blk / D if D >= 2.0 ** -126 else np.zeros_like(blk)
                    want_c = np.argmin(np.abs(F.E2M1_MAG[None, :] - np.abs(yv).reshape(-1)[:, None]), axis=1)
                    got_c = codes[b, ti * 16:(ti + 1) * 16, tj * 16:(tj + 1) * 16]
                    nt = _near_tie(np.abs(yv).reshape(-1), F.E2M1_MAG).reshape(16, 16)
                    assert not (((got_c & 7) != want_c.reshape(16, 16)) & ~nt).any(), (b, ti, tj)
                    assert np.array_equal(got_c >> 3, np.signbit(blk.astype(f32)).astype(np.uint8))


@pytest.mark.parametrize("dist,seed", [("normal", 4), ("outlier", 5), ("wide", 6)])
def test_square_tile_transpose_is_bitwise(dist, seed):
    """The property the pages give the square tile: quantizing the transpose
    yields the transpose of the codes and of the tile scales, bit for bit."""
    x = _square_inputs(dist, (3, 32, 80), seed)
    p, s, st = Q.quantize_nvfp4_square(x, Q.OUTER_TENSOR)
    pt, s_t, st_t = Q.quantize_nvfp4_square(np.ascontiguousarray(x.transpose(0, 2, 1)), Q.OUTER_TENSOR)
    assert np.array_equal(st, st_t)
    assert np.array_equal(F.unpack_fp4(pt), F.unpack_fp4(p).transpose(0, 2, 1))
    assert np.array_equal(s_t[:, ::16, :], s[:, ::16, :].transpose(0, 2, 1))


def test_square_tile_equals_row_blocks_when_row_maxima_agree():
    """When every 1x16 block of a tile has the tile's largest magnitude, the
    square variant reduces to the pinned 1x16 quantizer bit for bit; otherwise
    its scale is never below the row block's (E4M3 codes order like values)."""
    rng = np.random.default_rng(7)
    x = rng.uniform(-1, 1, (2, 32, 48)).astype(f32)
    tiles = x.reshape(2, 2, 16, 3, 16)
    m = rng.uniform(0.5, 40, (2, 2, 1, 3, 1)).astype(f32)
    tiles *= m
    tiles[..., 5] = np.where(rng.integers(0, 2, (2, 2, 16, 3)) == 1, m[..., 0], -m[..., 0])
    outer = np.array([0.25, 1.5], f32)
    p, s, _ = Q.quantize_nvfp4_square(x, Q.OUTER_GIVEN, outer)
    p1, s1, _ = Q.quantize_nvfp4(x, Q.OUTER_GIVEN, outer)
    assert np.array_equal(p, p1) and np.array_equal(s, s1)
    y = rng.standard_t(3, (2, 32, 48)).astype(f32)
    _, s, _ = Q.quantize_nvfp4_square(y, Q.OUTER_TENSOR)
    _, s1, _ = Q.quantize_nvfp4(y, Q.OUTER_TENSOR)
    assert (s >= s1).all() and (s > s1).any()
