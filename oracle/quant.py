"""Block-scaled quantization, written step by step from the pages.

Page: "End-to-End 4-Bit Training" (Thinking Machines Lab).
  * Section "Low-precision formats on Blackwell": a 1x16 block is scaled
    from its largest magnitude (-54 -> -6 with scale 9), values round to the
    nearest FP4 value, an FP32 outer scale covers a large group, and each value
    is reconstructed as x_i = q_i * s_{i//16} * s_t.
  * Section "Block-scaled backward passes": the backward operands are the
    transposes of the forward ones, so their blocks run along the other axis.
  * Section "Re-quantization with stochastic rounding": dequantize the forward
    tensor, transpose it in higher precision, requantize with stochastic
    rounding so that E[w_q] = E[(w_q^T)^T]; MXFP8 (E4M3 values, one E8M0 scale
    per 32) is the backward format; the quantized linear layer figure
    (Figure 4) quantizes the BF16 output gradient to MXFP8 with SR, both
    row-wise and transposed.
  * Section "Recipe details": per-token outer scales for activations,
    per-expert outer scales for weights.

Where the pages leave a step open the reading taken is stated at the step.
Floating-point steps that decide a code are done in float32 (NumPy float32
arithmetic is IEEE round-to-nearest-even), in the order written.
"""
import numpy as np

from .formats import (E2M1_MAG, E4M3_VAL, e2m1_decode, e2m1_encode_rne_sat,
                      e4m3_decode, e4m3_encode_rne_sat, e4m3_encode_ru_cap,
                      pack_fp4, unpack_fp4)
from .rng import sr_uniform

F32 = np.float32
OUTER_TENSOR, OUTER_ROW, OUTER_GIVEN = 0, 1, 2
RN, SR = 0, 1
NVFP4, MXFP8 = 0, 1
NVFP4_BLOCK = 16
MXFP8_BLOCK = 32
FP32_MIN_NORMAL = 2.0 ** -126


def _f32(x):
    return np.asarray(x, dtype=F32)


# ----------------------------------------------------------------- outer scale
def outer_scale_from_amax(amax):
    """Reading: the FP32 outer scale maps the group's largest magnitude to the
    top of the NVFP4 range [2^-10, 2688]: s_t = f32(amax / 2688); a group of
    zeros gets s_t = 1."""
    a = _f32(amax)
    s = (a / F32(2688.0)).astype(F32)
    return np.where(a > 0, s, F32(1.0)).astype(F32)


# ----------------------------------------------------------------- NVFP4 block
def _nvfp4_block_codes(blocks, d_scale_codes, st_blk):
    """Element step shared by RTN: D = f32(dec(s_b) * s_t); a block whose D is
    below the smallest normal float32 (zero, or a subnormal scale product) has
    all magnitudes 0 (reading: avoids dividing by zero); otherwise
    y = f32(x * f32(1/D)) and each y rounds to the nearest FP4 value."""
    s_val = _f32(e4m3_decode(d_scale_codes))
    D = (s_val * st_blk).astype(F32)
    live = D >= F32(FP32_MIN_NORMAL)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        inv = (F32(1.0) / np.where(live, D, F32(1.0))).astype(F32)
        y = (blocks * inv[..., None]).astype(F32)
    codes = e2m1_encode_rne_sat(y)
    sign_only = (np.signbit(blocks).astype(np.uint8) << 3)
    return np.where(live[..., None], codes, sign_only).astype(np.uint8)


def _block_sq_error(blocks, codes, s_code, st_blk):
    """Squared quantization error of each 1x16 block, the measure Four Over
    Six compares (reading: the pages name the technique, not its error
    measure). In float32, in a fixed order: x^_i = f32(f32(q_i * s_b) * s_t)
    (the dequantized value), e_i = f32(x_i - x^_i), and
    err = f32(...f32(f32(e_0^2 + e_1^2) + e_2^2)... + e_15^2), each square and
    each partial sum rounded to float32 in element order."""
    q = e2m1_decode(codes).astype(F32)
    s = _f32(e4m3_decode(s_code))[..., None]
    xh = ((q * s).astype(F32) * st_blk[..., None]).astype(F32)
    e = (blocks - xh).astype(F32)
    sq = (e * e).astype(F32)
    err = sq[..., 0]
    for i in range(1, NVFP4_BLOCK):
        err = (err + sq[..., i]).astype(F32)
    return err


def quantize_nvfp4(x, mode, outer_in=None, four_over_six=False):
    """Round-to-nearest NVFP4 quantization of x (float32, shape [B, R, C],
    C % 16 == 0); blocks of 16 run along C.

    mode OUTER_TENSOR: one outer scale per batch item b (a tensor or an
    expert's weight matrix); OUTER_ROW: one per row (a token); OUTER_GIVEN:
    ``outer_in`` holds one per batch item.

    Steps per 1x16 block (section "Low-precision formats on Blackwell"):
      a_b = max |x| over the block
      d   = f32(6 * s_t)
      r   = f32(a_b / d)                 scale that maps a_b to 6
      s_b = E4M3 round-to-nearest-even of r, saturating at 448
            (reading pinned by the 593.7 example: 98.95 -> 96, error -17.7)
      codes: see _nvfp4_block_codes; two codes per byte, element 2k in the
      low nibble (reading).
    four_over_six (section "Recipe details": the activation quantizer chooses
    between two scale factors per block to reduce quantization error;
    Figure 4 applies it to the per-token activation quantize): each block
    also tries r4 = f32(a_b / f32(4 * s_t)), the scale that maps a_b to 4, and
    keeps it when its squared error (_block_sq_error) is strictly smaller
    than that of the 6 scale (reading: ties keep 6).
    Returns (packed [B,R,C/2] u8, scales [B,R,C/16] u8, outer f32 [B] or [B,R]).
    """
    x = _f32(x)
    B, R, C = x.shape
    assert C % NVFP4_BLOCK == 0
    if mode == OUTER_TENSOR:
        st = outer_scale_from_amax(np.max(np.abs(x), axis=(1, 2)) if R * C else np.zeros(B, F32))
        st_b = st[:, None, None]
    elif mode == OUTER_ROW:
        st = outer_scale_from_amax(np.max(np.abs(x), axis=2) if C else np.zeros((B, R), F32))
        st_b = st[:, :, None]
    elif mode == OUTER_GIVEN:
        st = _f32(outer_in).reshape(B)
        st_b = st[:, None, None]
    else:
        raise ValueError("mode")
    blocks = x.reshape(B, R, C // NVFP4_BLOCK, NVFP4_BLOCK)
    a_b = np.max(np.abs(blocks), axis=-1)
    d = (F32(6.0) * st_b).astype(F32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = (a_b / d).astype(F32)
    s_code = e4m3_encode_rne_sat(r)
    codes = _nvfp4_block_codes(blocks, s_code, st_b)
    if four_over_six:
        d4 = (F32(4.0) * st_b).astype(F32)
        with np.errstate(divide="ignore", invalid="ignore"):
            r4 = (a_b / d4).astype(F32)
        s4 = e4m3_encode_rne_sat(r4)
        codes4 = _nvfp4_block_codes(blocks, s4, st_b)
        st_full = np.broadcast_to(st_b, a_b.shape)
        use4 = _block_sq_error(blocks, codes4, s4, st_full) < _block_sq_error(blocks, codes, s_code, st_full)
        s_code = np.where(use4, s4, s_code).astype(np.uint8)
        codes = np.where(use4[..., None], codes4, codes).astype(np.uint8)
    return pack_fp4(codes.reshape(B, R, C)), s_code, st


def quantize_nvfp4_square(x, mode, outer_in=None):
    """The square-tile NVFP4 variant the pages compare against (section
    "Block-scaled backward passes", the row-vs-column and outlier figures):
    one E4M3 scale per 16x16 tile instead of per 1x16 block, so that the
    quantization of the transpose is the transpose of the quantization.

    x float32 [B, R, C], R % 16 == 0 and C % 16 == 0. mode OUTER_TENSOR (one
    outer scale per item from its amax, as in quantize_nvfp4) or OUTER_GIVEN
    (``outer_in`` [B]). Per 16x16 tile:
      a_t = max |x| over the tile
      s_b = E4M3 round-to-nearest-even of f32(a_t / f32(6 * s_t)), saturating
      every element then rounds exactly as in a 1x16 block with scale s_b
      (_nvfp4_block_codes).
    Returns (packed [B,R,C/2] u8, scales [B,R,C/16] u8, outer f32 [B]); the
    scales use the layout of the 1x16 quantizer (one byte per row block), each
    tile's byte repeated in its 16 rows, so any consumer of 1x16 blocks reads
    the result unchanged (reading: the pages do not fix a storage layout)."""
    x = _f32(x)
    B, R, C = x.shape
    assert R % 16 == 0 and C % 16 == 0
    if mode == OUTER_TENSOR:
        st = outer_scale_from_amax(np.max(np.abs(x), axis=(1, 2)) if R * C else np.zeros(B, F32))
    elif mode == OUTER_GIVEN:
        st = _f32(outer_in).reshape(B)
    else:
        raise ValueError("mode")
    st_b = st[:, None, None]
    tiles = x.reshape(B, R // 16, 16, C // 16, 16)
    a_t = np.max(np.abs(tiles), axis=(2, 4))                      # [B, R/16, C/16]
    d = (F32(6.0) * st_b).astype(F32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = (a_t / d).astype(F32)
    s_tile = e4m3_encode_rne_sat(r)
    s_code = np.repeat(s_tile, 16, axis=1)                         # [B, R, C/16]
    codes = _nvfp4_block_codes(x.reshape(B, R, C // 16, 16), s_code, st_b)
    return pack_fp4(codes.reshape(B, R, C)), s_code.astype(np.uint8), st


def quantize_nvfp4_tile16(x, outer):
    """One item of quantize_nvfp4_square with a given outer scale: x float32
    [R, C]; returns unpacked codes [R, C] and the tile scales [R/16, C/16]."""
    packed, s_code, _ = quantize_nvfp4_square(_f32(x)[None], OUTER_GIVEN, np.array([outer], F32))
    return unpack_fp4(packed)[0], s_code[0, ::16, :]


def _outer_broadcast(outer, mode, B, R):
    o = _f32(outer)
    if mode == OUTER_ROW:
        return o.reshape(B, R)[:, :, None]
    return o.reshape(B)[:, None, None]


def dequantize_nvfp4(packed, scales, outer, mode):
    """x^ = f32(f32(q * s_b) * s_t) -- the higher-precision value that the
    requantization transposes (reading: float32; q * s_b is exact)."""
    packed = np.asarray(packed)
    B, R, C2 = packed.shape
    q = e2m1_decode(unpack_fp4(packed))
    s = np.repeat(e4m3_decode(scales), NVFP4_BLOCK, axis=-1)
    qs = (q * s).astype(F32)                                    # exact
    return (qs * _outer_broadcast(outer, mode, B, R)).astype(F32)


def dequantize_nvfp4_f64(packed, scales, outer, mode):
    """x_i = q_i * s_{i//16} * s_t evaluated in float64 (exact: at most 30
    significant bits)."""
    packed = np.asarray(packed)
    B, R, C2 = packed.shape
    q = e2m1_decode(unpack_fp4(packed))
    s = np.repeat(e4m3_decode(scales), NVFP4_BLOCK, axis=-1)
    return q * s * _outer_broadcast(outer, mode, B, R).astype(np.float64)


# ----------------------------------------------------------------- rounding
def sr_to_grid(y, grid, u):
    """Stochastic rounding of float32 y onto the symmetric grid +-``grid``
    (section "Re-quantization with stochastic rounding": round up or down with
    probability inversely proportional to the distance to each neighbour).
    Reading: lo <= |y| < hi are the two neighbouring grid magnitudes,
    delta = (|y| - lo) / (hi - lo) (exact in float64: the step is a power of
    two), and the magnitude rounds up iff u < delta for the uniform draw u.
    Magnitudes at or above the largest grid value give the largest value.
    Returns (magnitude index into grid, sign bit)."""
    m = np.abs(_f32(y).astype(np.float64))
    n = len(grid)
    hi_idx = np.clip(np.searchsorted(grid, m, side="right"), 1, n - 1)
    lo_idx = hi_idx - 1
    lo = grid[lo_idx]
    hi = grid[hi_idx]
    delta = (m - lo) / (hi - lo)
    up = np.asarray(u, dtype=np.float64) < delta
    idx = np.where(up, hi_idx, lo_idx)
    idx = np.where(m >= grid[-1], n - 1, idx)
    return idx, np.signbit(_f32(y)).astype(np.int64)


# ----------------------------------------------------------------- MXFP8
def e8m0_exponent(a_b):
    """Reading: the smallest integer e with a_b <= 448 * 2^e, clamped to
    [-127, 127] (a block of zeros gets -127, code 0). With this choice no
    element exceeds 448 after scaling, so SR never saturates."""
    a = np.asarray(a_b, dtype=np.float64)
    pos = a > 0
    with np.errstate(divide="ignore"):
        e = np.where(pos, np.ceil(np.log2(np.where(pos, a, 1.0) / 448.0)), -127.0)
    e = np.clip(e, -200, 200).astype(np.int64)
    for _ in range(3):            # exact correction of the float64 estimate
        e = np.where(pos & (a > 448.0 * np.ldexp(1.0, e)), e + 1, e)
        e = np.where(pos & (a <= 448.0 * np.ldexp(1.0, e - 1)), e - 1, e)
    return np.clip(e, -127, 127)


def mxfp8_quantize(z, idx, rnd, seed=0, stream=0):
    """MXFP8 quantization of float32 z [..., L] (L % 32 == 0) along the last
    axis: one E8M0 scale per 32 values, E4M3 values.
    y = f32(z * 2^-e) (exact unless float32 underflow); RN: E4M3 nearest-even;
    SR: sr_to_grid with u drawn for each element's output index ``idx``.
    Returns (codes u8 same shape as z, scale codes u8 [..., L/32])."""
    z = _f32(z)
    L = z.shape[-1]
    assert L % MXFP8_BLOCK == 0
    blocks = z.reshape(z.shape[:-1] + (L // MXFP8_BLOCK, MXFP8_BLOCK))
    a_b = np.max(np.abs(blocks), axis=-1) if blocks.size else np.zeros(blocks.shape[:-1], F32)
    e = e8m0_exponent(a_b)
    pw = np.ldexp(1.0, -e).astype(F32)                           # exact, 2^127 .. 2^-127
    y = (blocks * pw[..., None]).astype(F32).reshape(z.shape)
    if rnd == RN:
        mag = e4m3_encode_rne_sat(np.abs(y.astype(np.float64))).astype(np.int64)
        sign = np.signbit(y).astype(np.int64)
    else:
        u = sr_uniform(seed, stream, idx)
        mag, sign = sr_to_grid(y, E4M3_VAL, u)
    codes = (mag | (sign << 7)).astype(np.uint8)
    return codes, (e + 127).astype(np.uint8)


def dequantize_mxfp8_f64(codes, scales):
    """x = q * 2^(s - 127) in float64 (exact)."""
    codes = np.asarray(codes)
    L = codes.shape[-1]
    s = np.repeat(np.ldexp(1.0, np.asarray(scales).astype(np.int64) - 127), MXFP8_BLOCK, axis=-1)
    return e4m3_decode(codes) * s.reshape(codes.shape[:-1] + (L,))


def quantize_mxfp8(x, rnd, seed=0, stream=0):
    """Row-wise MXFP8 of x [R, C] (blocks along C), as for the DGRAD operand
    g in the quantized linear layer figure. Output index idx = r*C + c."""
    x = _f32(x)
    R, C = x.shape
    idx = np.arange(R * C, dtype=np.uint64).reshape(R, C)
    return mxfp8_quantize(x, idx, rnd, seed, stream)


def pad32(n):
    return (int(n) + 31) // 32 * 32


def segmented_layout(seg_offsets, C):
    """Per-segment transposed layout: segment e of length M_e becomes a
    [C, Mp_e] block (Mp_e = M_e rounded up to 32), stored one after another.
    Returns (Mp list, element base offset of each segment)."""
    seg = np.asarray(seg_offsets, dtype=np.int64)
    mp = [pad32(seg[e + 1] - seg[e]) for e in range(len(seg) - 1)]
    base = np.concatenate([[0], np.cumsum(np.asarray(mp, dtype=np.int64) * C)]).astype(np.int64)
    return mp, base


def _transposed_segments_to_mxfp8(rows_f32, seg_offsets, rnd, seed, stream, segments=None):
    """rows_f32 [M_total, C] in segment order -> for each segment e the
    transpose [C, Mp_e] zero-padded along the token axis, quantized to MXFP8
    with blocks of 32 along tokens starting at the segment start (reading:
    padding zeros do not change a block's largest magnitude).
    Output index of element (e, c, m) = base_e + c * Mp_e + m.
    ``segments`` (optional) limits the output to those segments, concatenated
    in the given order; ``rows_f32`` may then be a callable returning the rows
    of a segment's range [start, stop)."""
    C = rows_f32(0, 0).shape[1] if callable(rows_f32) else rows_f32.shape[1]
    mp, base = segmented_layout(seg_offsets, C)
    seg = np.asarray(seg_offsets, dtype=np.int64)
    codes_out, scales_out = [], []
    for e in (range(len(seg) - 1) if segments is None else segments):
        Me = int(seg[e + 1] - seg[e])
        Z = np.zeros((C, mp[e]), dtype=F32)
        rows = rows_f32(seg[e], seg[e + 1]) if callable(rows_f32) else rows_f32[seg[e]:seg[e + 1]]
        Z[:, :Me] = rows.T
        idx = (np.uint64(base[e]) + np.arange(C * mp[e], dtype=np.uint64)).reshape(C, mp[e])
        c, s = mxfp8_quantize(Z, idx, rnd, seed, stream)
        codes_out.append(c.reshape(-1))
        scales_out.append(s.reshape(-1))
    cat = lambda parts, dt: np.concatenate(parts).astype(dt) if parts else np.zeros(0, dt)
    return cat(codes_out, np.uint8), cat(scales_out, np.uint8)


def quantize_mxfp8_transposed(x, seg_offsets, rnd, seed=0, stream=0, segments=None):
    """The WGRAD operand g^T: x [M_total, C] holds the dispatched rows in
    expert order; each expert's segment is transposed and quantized along the
    token axis (see _transposed_segments_to_mxfp8)."""
    x = np.asarray(x)
    return _transposed_segments_to_mxfp8(lambda a, b: _f32(x[a:b]), seg_offsets, rnd, seed, stream, segments)


# ----------------------------------------------------------------- requant
def requant_transpose_sr(packed, scales, outer, in_mode, out_fmt, seed, stream, rnd=SR, item0=0):
    """Dequantize -> transpose -> requantize with stochastic rounding
    (section "Re-quantization with stochastic rounding").
    Input NVFP4 [B, R, C] (blocks along C); output [B, C, R] with blocks along
    R, the old column axis.  Output index idx = b*C*R + c*R + r, where b
    counts from ``item0`` (so a slice of the batch can be checked on its own).

    out_fmt MXFP8: mxfp8_quantize of Z = x^T.
    out_fmt NVFP4 (reading): a new outer scale s_t' = f32(max|Z| / 2688) per
      batch item, then per 1x16 block r = f32(a_b / f32(6 s_t')) and the block
      scale is r rounded UP to E4M3 (capped at 448) so that no element of the
      block exceeds 6 and SR stays unbiased; D, 1/D and y as in the RTN
      quantizer; y rounds stochastically onto the FP4 grid.
    Returns (codes, scales[, outer']) in the output layout."""
    packed = np.asarray(packed)
    B, R, C2 = packed.shape
    C = 2 * C2
    xh = dequantize_nvfp4(packed, scales, outer, in_mode)
    Z = np.ascontiguousarray(np.transpose(xh, (0, 2, 1)))         # [B, C, R] float32
    idx = (np.uint64(int(item0) * C * R) + np.arange(B * C * R, dtype=np.uint64)).reshape(B, C, R)
    if out_fmt == MXFP8:
        assert R % MXFP8_BLOCK == 0
        return mxfp8_quantize(Z, idx, rnd, seed, stream)
    assert R % NVFP4_BLOCK == 0
    st = outer_scale_from_amax(np.max(np.abs(Z), axis=(1, 2)) if C * R else np.zeros(B, F32))
    st_b = st[:, None, None]
    blocks = Z.reshape(B, C, R // NVFP4_BLOCK, NVFP4_BLOCK)
    a_b = np.max(np.abs(blocks), axis=-1)
    d = (F32(6.0) * st_b).astype(F32)
    r = (a_b / d).astype(F32)
    s_code = e4m3_encode_ru_cap(r)
    s_val = _f32(e4m3_decode(s_code))
    D = (s_val * st_b).astype(F32)
    live = D >= F32(FP32_MIN_NORMAL)
    inv = (F32(1.0) / np.where(live, D, F32(1.0))).astype(F32)
    y = (blocks * inv[..., None]).astype(F32).reshape(B, C, R)
    if rnd == SR:
        mag, sign = sr_to_grid(y, E2M1_MAG, sr_uniform(seed, stream, idx))
        codes = (mag | (sign << 3)).astype(np.uint8)
    else:
        codes = e2m1_encode_rne_sat(y)
    live_e = np.repeat(live, NVFP4_BLOCK, axis=-1).reshape(B, C, R)
    codes = np.where(live_e, codes, (np.signbit(Z).astype(np.uint8) << 3)).astype(np.uint8)
    return pack_fp4(codes), s_code, st


def requant_transpose_sr_segmented(packed, scales, outer, in_mode, row_gather, seg_offsets,
                                   seed, stream, rnd=SR, segments=None):
    """The WGRAD operand x_q^T: input NVFP4 [T, C] (one row per token, per-row
    or per-tensor outer scale); dispatched row m of the output is token
    row_gather[m]; rows are grouped into expert segments by seg_offsets; each
    segment is dequantized, transposed and requantized to MXFP8 along the
    token axis as in _transposed_segments_to_mxfp8."""
    packed = np.asarray(packed)
    scales = np.asarray(scales)
    outer = np.asarray(outer)
    gather = np.asarray(row_gather, dtype=np.int64)

    def rows(a, b):
        tok = gather[a:b]
        o = outer[tok].reshape(1, -1) if in_mode == OUTER_ROW else outer.reshape(1)
        return dequantize_nvfp4(packed[tok][None], scales[tok][None], o, in_mode)[0]
    return _transposed_segments_to_mxfp8(rows, seg_offsets, rnd, seed, stream, segments)
