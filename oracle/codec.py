"""The combine codec: 32-point random Hadamard transform (RHT) followed by
block-scaled S2F6, and its inverse after aggregation. Test infrastructure
only (tests, smoke and the benchmark's CPU baseline use it).

Page: "End-to-End 4-Bit Training" (Thinking Machines Lab), section
"Quantized communications":
  * before the combine exchange each expert output row is rotated by a
    32-dimensional random Hadamard transform and quantized to block-scaled
    S2F6 with one scale factor per 32 values (8.25 bits per value);
  * S2F6 is fixed point with two signed integer bits and six fractional bits:
    the values k/64 for integers k in [-128, 127];
  * the scale factors are UE8M0 (the PTX conversions it names scale by
    ue8m0 factors);
  * the receiver dequantizes and aggregates the copies of a token, then
    inverts the RHT; the transform is orthonormal, keeps the energy of the
    block (its figure: 32 values, peak 310 -> 227, sum of squares 319,030
    unchanged) and is inverted exactly.

Readings (where the section leaves a step open):
  * RHT = H D / sqrt(32): D = diag of 32 random signs (one sign vector for all
    blocks, given as a 32-bit mask, bit i set = element i negated), H the
    Sylvester Hadamard matrix of order 32 (H_1 = [1], H_2n = [[H, H], [H, -H]]).
    Its inverse is D H / sqrt(32) (H is symmetric and H H = 32 I).
  * Scale: the smallest power of two 2^e with max|z| <= (127/64) 2^e, e in
    [-127, 127] (a zero block takes e = -127), code e + 127; the element code
    is k = round-half-even(z / 2^e * 64) saturated to [-128, 127], stored as a
    two's-complement byte.
  * Aggregation is the plain sum of the k dequantized copies of a token, in
    the order of its (token, slot) pairs (routing weights, being linear, are
    applied by the sender before the transform).
  * Precision: the transform runs in float32 as the fast Walsh-Hadamard
    butterfly (stages of span 1, 2, 4, 8, 16; each butterfly (a, b) ->
    (a + b, a - b)), then one float32 multiply by f32(1/sqrt(32)); the code
    decision uses that float32 value, the precision of the GPU kernel (the
    pages fix none). The float64 matrix definition (rht_f64) pins it.
"""
import numpy as np

F32 = np.float32
BLOCK = 32
INV_SQRT32 = F32(1.0 / np.sqrt(32.0))   # f32 of 1/sqrt(32)
S2F6_MAX_CODE = 127


def hadamard32():
    """Sylvester Hadamard matrix of order 32 (entries +-1), float64."""
    h = np.ones((1, 1))
    while h.shape[0] < BLOCK:
        h = np.block([[h, h], [h, -h]])
    return h


def sign_vector(signs_mask):
    """32-bit mask -> float64 vector of +-1 (bit i set: element i negated)."""
    m = int(signs_mask) & 0xFFFFFFFF
    return np.array([-1.0 if (m >> i) & 1 else 1.0 for i in range(BLOCK)])


def rht_f64(x, signs_mask):
    """The definition: z = H D x / sqrt(32) per block of 32 along the last axis, float64."""
    x = np.asarray(x, dtype=np.float64)
    blocks = x.reshape(-1, BLOCK) * sign_vector(signs_mask)
    z = blocks @ hadamard32().T / np.sqrt(32.0)
    return z.reshape(x.shape)


def irht_f64(z, signs_mask):
    """Inverse of rht_f64: x = D H z / sqrt(32)."""
    z = np.asarray(z, dtype=np.float64)
    x = (z.reshape(-1, BLOCK) @ hadamard32().T / np.sqrt(32.0)) * sign_vector(signs_mask)
    return x.reshape(z.shape)


def fwht32_f32(v):
    """Unnormalized Walsh-Hadamard transform of each block of 32 (last axis) in
    float32, butterfly stages of span 1, 2, 4, 8, 16; equals v @ H."""
    v = np.asarray(v, dtype=F32).reshape(-1, BLOCK).copy()
    h = 1
    while h < BLOCK:
        w = v.reshape(-1, BLOCK // (2 * h), 2, h)
        a = w[:, :, 0, :].copy()
        b = w[:, :, 1, :].copy()
        w[:, :, 0, :] = (a + b).astype(F32)
        w[:, :, 1, :] = (a - b).astype(F32)
        h *= 2
    return v


def rht_f32(x, signs_mask):
    """Forward transform in float32: signs (exact), butterfly, times f32(1/sqrt(32))."""
    x = np.asarray(x, dtype=F32)
    s = sign_vector(signs_mask).astype(F32)
    u = (x.reshape(-1, BLOCK) * s).astype(F32)
    return (fwht32_f32(u) * INV_SQRT32).astype(F32).reshape(x.shape)


def irht_f32(z, signs_mask):
    """Inverse transform in float32: butterfly, times f32(1/sqrt(32)), signs."""
    z = np.asarray(z, dtype=F32)
    s = sign_vector(signs_mask).astype(F32)
    u = (fwht32_f32(z) * INV_SQRT32).astype(F32)
    return (u * s).astype(F32).reshape(z.shape)


def s2f6_exponent(amax):
    """Smallest e with amax <= (127/64) 2^e, clamped to [-127, 127]; -127 for
    a zero block. amax float32; exact in float64: with amax = f 2^p,
    f in [1, 2), e = p when f <= 127/64, else p + 1."""
    a = np.asarray(amax, dtype=np.float64)
    m, p = np.frexp(a)                        # a = m 2^p, m in [0.5, 1)
    f, p = m * 2.0, p.astype(np.int64) - 1    # a = f 2^p, f in [1, 2)
    e = np.where(f <= 127.0 / 64.0, p, p + 1)
    e = np.where(a > 0, e, -127)
    return np.clip(e, -127, 127)


def s2f6_quantize(z):
    """Block-scaled S2F6 of z (float32, last axis a multiple of 32).
    Returns (codes uint8 [..., n] two's complement, scales uint8 [..., n/32])."""
    z = np.asarray(z, dtype=F32)
    blocks = z.reshape(-1, BLOCK).astype(np.float64)            # exact
    e = s2f6_exponent(np.max(np.abs(blocks), axis=1))
    y = blocks * np.exp2(-e.astype(np.float64))[:, None] * 64.0  # exact (powers of two)
    k = np.clip(np.rint(y), -128, 127).astype(np.int64)          # rint: half to even
    codes = (k & 0xFF).astype(np.uint8).reshape(z.shape)
    scales = (e + 127).astype(np.uint8).reshape(z.shape[:-1] + (z.shape[-1] // BLOCK,))
    return codes, scales


def s2f6_dequantize(codes, scales):
    """k/64 * 2^(s-127), exact in float32 for |k| <= 128, s in [0, 254]."""
    c = np.asarray(codes).astype(np.int8).astype(np.float64)
    s = np.asarray(scales).astype(np.int64)
    v = c.reshape(-1, BLOCK) / 64.0 * np.exp2((s.reshape(-1) - 127).astype(np.float64))[:, None]
    return v.astype(F32).reshape(np.asarray(codes).shape)


def encode(x, signs_mask):
    """Sender: x [rows, cols] (float32 values) -> (codes, scales) of the
    rotated rows."""
    return s2f6_quantize(rht_f32(x, signs_mask))


def combine(codes, scales, pair_row, k, signs_mask):
    """Receiver: token t sums the dequantized rows pair_row[t*k + j],
    j = 0..k-1, in float32 in that order, then inverts the transform.
    Returns float32 [T, cols]."""
    pair_row = np.asarray(pair_row).reshape(-1, k)
    deq = s2f6_dequantize(codes, scales)
    agg = deq[pair_row[:, 0]].astype(F32)
    for j in range(1, k):
        agg = (agg + deq[pair_row[:, j]]).astype(F32)
    return irht_f32(agg, signs_mask)
