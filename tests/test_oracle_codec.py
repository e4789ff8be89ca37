"""Pins of the combine codec oracle (RHT-32 + block-scaled S2F6) against
closed forms, exact special cases and brute force."""
import numpy as np
import pytest

from oracle import codec as C

f32 = np.float32


def test_hadamard_closed_form():
    """Sylvester's matrix has entries (-1)^popcount(i & j); it is symmetric
    and H H = 32 I (so H / sqrt(32) is orthonormal and its own inverse)."""
    h = C.hadamard32()
    i, j = np.meshgrid(np.arange(32), np.arange(32), indexing="ij")
    pc = np.vectorize(lambda v: bin(v).count("1"))(i & j)
    assert np.array_equal(h, np.where(pc % 2, -1.0, 1.0))
    assert np.array_equal(h, h.T)
    assert np.array_equal(h @ h, 32 * np.eye(32))


def test_sign_mask():
    s = C.sign_vector(0x80000005)
    assert s[0] == -1 and s[1] == 1 and s[2] == -1 and s[31] == -1 and (s[3:31] == 1).all()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_butterfly_equals_matrix_exactly_on_integers(seed):
    """Integer inputs below 2^18 keep every butterfly sum exact in float32, so
    the float32 transform must equal the matrix product exactly: a wrong
    stage span, sign or index fails here."""
    rng = np.random.default_rng(seed)
    x = rng.integers(-2 ** 18, 2 ** 18, size=(64, 32)).astype(f32)
    assert np.array_equal(C.fwht32_f32(x).astype(np.float64), x.astype(np.float64) @ C.hadamard32())
    one_hot = np.eye(32, dtype=f32)
    assert np.array_equal(C.fwht32_f32(one_hot), C.hadamard32().astype(f32))


@pytest.mark.parametrize("mask", [0, 0xDEADBEEF, 0xFFFFFFFF])
def test_float32_transform_within_rounding_of_definition(mask):
    """rht_f32 against the float64 definition H D x / sqrt(32): five rounded
    butterfly stages and one rounded multiply, so the error is below
    6 * 2^-24 * sum|x| / sqrt(32) per element (each stage's partial sums are
    bounded by sum|x|)."""
    rng = np.random.default_rng(mask & 0xFF)
    x = (rng.standard_normal((256, 32)) * np.exp(rng.uniform(-8, 8, (256, 1)))).astype(f32)
    z32 = C.rht_f32(x, mask).astype(np.float64)
    z64 = C.rht_f64(x, mask)
    bound = 6 * 2.0 ** -24 * np.abs(x.astype(np.float64)).sum(axis=1, keepdims=True) / np.sqrt(32) * 1.01
    assert (np.abs(z32 - z64) <= bound).all()
    x2 = C.irht_f32(C.rht_f32(x, mask), mask).astype(np.float64)
    assert (np.abs(x2 - x) <= 2 * bound * np.sqrt(32)).all()


def test_energy_preserved_and_inverse_exact_in_float64():
    """The section's figure: the transform keeps the block's sum of squares and
    is inverted exactly (float64, up to rounding of 1e-12)."""
    rng = np.random.default_rng(3)
    x = rng.uniform(-60, 60, (40, 32))
    x[:, [3, 11, 20, 29]] = rng.choice([-1, 1], (40, 4)) * rng.uniform(200, 310, (40, 4))  # 4 outliers per block
    z = C.rht_f64(x, 0x12345678)
    assert np.allclose((z ** 2).sum(axis=1), (x ** 2).sum(axis=1), rtol=1e-12)
    assert np.allclose(C.irht_f64(z, 0x12345678), x, rtol=0, atol=1e-9)
    # the rotation spreads the outliers: the block maximum drops for these blocks
    assert (np.abs(z).max(axis=1) < np.abs(x).max(axis=1)).mean() > 0.9


def test_s2f6_grid_range_and_bits_per_value():
    """S2F6 codes are the two's-complement bytes k, value k/64 in
    [-128/64, 127/64]; one UE8M0 byte per 32 codes is 8.25 bits per value."""
    codes = np.arange(256, dtype=np.uint8).reshape(8, 32)
    scales = np.full((8, 1), 127, np.uint8)                        # 2^0
    v = C.s2f6_dequantize(codes, scales).reshape(-1)
    k = np.arange(256).astype(np.uint8).astype(np.int8).astype(np.float64)
    assert np.array_equal(v, (k / 64).astype(f32))
    assert v.min() == -2.0 and v.max() == 127 / 64
    c, s = C.s2f6_quantize(np.ones((3, 64), f32))
    assert (c.nbytes * 8 + s.nbytes * 8) / (3 * 64) == 8.25


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_s2f6_brute_force(seed):
    """Every block: the scale is the smallest power of two keeping the block
    maximum within 127/64 of it (checked against e - 1), and every code is the
    nearest of the 256 grid values (near-ties skipped); the error is at most
    half a step."""
    rng = np.random.default_rng(seed)
    z = (rng.standard_normal((300, 32)) * np.exp2(rng.integers(-140, 120, (300, 1)))).astype(f32)
    z[0] = 0.0
    z[1, :] = 0.0
    z[1, 7] = f32(127 / 64)           # exactly the top of the grid at e = 0
    z[2, :] = 0.0
    z[2, 5] = -f32(2.0)               # 2 > 127/64: needs e = 1
    codes, scales = C.s2f6_quantize(z)
    e = scales.astype(np.int64).reshape(-1) - 127
    zz = z.astype(np.float64)
    amax = np.abs(zz).max(axis=1)
    assert e[0] == -127 and (codes[0] == 0).all()
    assert e[1] == 0 and codes[1, 7] == 127
    assert e[2] == 1 and codes[2, 5].astype(np.int8) == -64
    for b in range(3, 300):
        step = 2.0 ** (e[b] - 6)
        if -127 < e[b] < 127:
            assert amax[b] <= 127 * step and amax[b] > 127 * step / 2
        grid = np.arange(-128, 128) * step
        d = np.abs(zz[b][:, None] - grid[None, :])
        want = np.argmin(d, axis=1) - 128
        srt = np.sort(d, axis=1)
        tie = (srt[:, 1] - srt[:, 0]) <= 1e-9 * step
        got = codes[b].astype(np.int8).astype(np.int64)
        assert np.array_equal(got[~tie], want[~tie]), b
        if -127 < e[b]:
            assert (np.abs(got * step - zz[b]) <= step / 2).all()


def test_combine_against_float64_definition():
    """The receiver: the sum over a token's copies of the dequantized rows,
    inverse-transformed; against the float64 definition on the same codes,
    and the round trip against the inputs within the quantization error
    (half a step per rotated value, so at most sqrt(32)/2 steps in L2 per
    block and copy)."""
    rng = np.random.default_rng(9)
    T, k, cols, mask = 24, 4, 96, 0xA5A5F00F
    rows = rng.standard_normal((T * k, cols)).astype(f32)
    rows[rng.integers(0, T * k, 10), rng.integers(0, cols, 10)] = 80.0
    pair_row = rng.permutation(T * k)
    codes, scales = C.encode(rows, mask)
    out = C.combine(codes, scales, pair_row, k, mask)
    deq = C.s2f6_dequantize(codes, scales).astype(np.float64)
    want = C.irht_f64(deq[pair_row.reshape(T, k)].sum(axis=1), mask)
    assert np.allclose(out, want, rtol=0, atol=1e-5 * np.abs(want).max())
    exact = rows.astype(np.float64)[pair_row.reshape(T, k)].sum(axis=1)
    step = np.exp2(scales.astype(np.float64) - 127 - 6)            # [T*k, cols/32]
    err_blocks = np.sqrt(((out.astype(np.float64) - exact) ** 2).reshape(T, cols // 32, 32).sum(axis=2))
    bound = (np.sqrt(32) / 2 * step[pair_row.reshape(T, k)]).sum(axis=1) * 1.001 + 1e-5
    assert (err_blocks <= bound).all()
