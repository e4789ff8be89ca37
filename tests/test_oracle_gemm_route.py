"""Pins of the GEMM references (closed forms, brute force with rationals)
and of the routing (hand-worked example, invariants)."""
from fractions import Fraction

import numpy as np

from oracle import formats as F
from oracle import gemm as G
from oracle import quant as Q
from oracle.route import route

f32 = np.float32


def _nvfp4_operands(rng, T, E, N, K, scale=1.0):
    x = (rng.standard_normal((T, K)) * scale).astype(f32)
    w = (rng.standard_normal((E, N, K)) * 0.02).astype(f32)
    ap, as_, ao = Q.quantize_nvfp4(x[None], Q.OUTER_ROW)
    bp, bs, bo = Q.quantize_nvfp4(w, Q.OUTER_TENSOR)
    return ap[0], as_[0], ao[0], bp, bs, bo


def test_single_block_closed_form():
    """K = 16: y = s_t,x * s_t,w * s_a * s_w * sum q_a q_w, with the integer sum exact."""
    rng = np.random.default_rng(1)
    ap, as_, ao, bp, bs, bo = _nvfp4_operands(rng, 4, 1, 3, 16)
    seg = np.array([0, 4])
    y, ya = G.grouped_gemm_nvfp4_ref(ap, as_, ao, None, bp, bs, bo, seg)
    qa = F.e2m1_decode(F.unpack_fp4(ap))
    qw = F.e2m1_decode(F.unpack_fp4(bp[0]))
    for r in range(4):
        for n in range(3):
            isum = int(np.sum((2 * qa[r]).astype(int) * (2 * qw[n]).astype(int)))   # 4 * sum q q, exact
            want = (Fraction(float(ao[r])) * Fraction(float(bo[0])) * Fraction(float(F.e4m3_decode(as_[r, 0])))
                    * Fraction(float(F.e4m3_decode(bs[0, n, 0]))) * Fraction(isum, 4))
            # exact up to float64 rounding of the product of two 30-bit operands
            assert abs(Fraction(float(y[r, n])) - want) <= abs(want) * Fraction(1, 1 << 50)


def test_diagonal_weights_reproduce_dequantized_rows():
    rng = np.random.default_rng(2)
    K = 64
    x = rng.standard_normal((5, K)).astype(f32)
    ap, as_, ao = Q.quantize_nvfp4(x[None], Q.OUTER_ROW)
    w = np.eye(K, dtype=f32)[None] * f32(3.0)
    bp, bs, bo = Q.quantize_nvfp4(w, Q.OUTER_TENSOR)
    y, _ = G.grouped_gemm_nvfp4_ref(ap[0], as_[0], ao[0], None, bp, bs, bo, np.array([0, 5]))
    xh = Q.dequantize_nvfp4_f64(ap, as_, ao, Q.OUTER_ROW)[0]
    wd = np.diag(Q.dequantize_nvfp4_f64(bp, bs, bo, Q.OUTER_TENSOR)[0])
    assert np.array_equal(y, xh * wd[None, :])


def test_grouped_gather_brute_force_rationals():
    """Tiny grouped GEMM with a row gather, summed exactly with rationals."""
    rng = np.random.default_rng(3)
    T, E, N, K = 6, 3, 4, 32
    ap, as_, ao, bp, bs, bo = _nvfp4_operands(rng, T, E, N, K)
    row_index = np.array([5, 0, 2, 2, 1, 4, 3, 0], dtype=np.int32)
    seg = np.array([0, 3, 3, 8])                                  # expert 1 empty
    y, ya = G.grouped_gemm_nvfp4_ref(ap, as_, ao, row_index, bp, bs, bo, seg)
    qa = F.e2m1_decode(F.unpack_fp4(ap)); sa = F.e4m3_decode(as_)
    qw = F.e2m1_decode(F.unpack_fp4(bp)); sw = F.e4m3_decode(bs)
    for r in range(8):
        e = 0 if r < 3 else 2
        t = row_index[r]
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += (Fraction(float(qa[t, k])) * Fraction(float(sa[t, k // 16])) * Fraction(float(ao[t]))
                        * Fraction(float(qw[e, n, k])) * Fraction(float(sw[e, n, k // 16])) * Fraction(float(bo[e])))
            assert abs(Fraction(float(y[r, n])) - acc) <= abs(acc) * Fraction(1, 1 << 50)
    ok, _ = G.within_tolerance(y, y, ya)
    assert ok


def test_mxfp8_dgrad_wgrad_brute_force():
    rng = np.random.default_rng(4)
    M_total, K, N, E = 40, 64, 8, 2
    seg = np.array([0, 13, 40])
    g = rng.standard_normal((M_total, K)).astype(f32)
    wt = rng.standard_normal((E, N, K)).astype(f32)
    gc, gs = Q.quantize_mxfp8(g, Q.RN)
    wc, ws = Q.mxfp8_quantize(wt, np.zeros(wt.shape, np.uint64), Q.RN)
    y, _ = G.mxfp8_dgrad_ref(gc, gs, wc, ws, seg)
    gh = Q.dequantize_mxfp8_f64(gc, gs)
    wh = Q.dequantize_mxfp8_f64(wc, ws)
    for r in (0, 12, 13, 39):
        e = 0 if r < 13 else 1
        for n in range(N):
            acc = sum(Fraction(float(gh[r, k])) * Fraction(float(wh[e, n, k])) for k in range(K))
            assert abs(Fraction(float(y[r, n])) - acc) <= abs(acc) * Fraction(1, 1 << 50)
    # WGRAD: dw_e = g_e^T x_e with both operands transposed per segment
    M, Nw = 8, 16
    ga = rng.standard_normal((M_total, M)).astype(f32)
    xb = rng.standard_normal((M_total, Nw)).astype(f32)
    ac, as_ = Q.quantize_mxfp8_transposed(ga, seg, Q.RN)
    bc, bs = Q.quantize_mxfp8_transposed(xb, seg, Q.RN)
    dw, _ = G.mxfp8_wgrad_ref(ac, as_, bc, bs, seg, M, Nw)
    mp, base = Q.segmented_layout(seg, M)
    for e in range(E):
        A = Q.dequantize_mxfp8_f64(ac[base[e]:base[e] + M * mp[e]].reshape(M, mp[e]),
                                   as_[base[e] // 32:(base[e] + M * mp[e]) // 32].reshape(M, -1))
        # the transposed operand holds the segment's rows (quantized along tokens), zero padded
        assert not A[:, seg[e + 1] - seg[e]:].any()
        for m in (0, M - 1):
            for n in (0, Nw - 1):
                mpb, baseb = Q.segmented_layout(seg, Nw)
                B = Q.dequantize_mxfp8_f64(bc[baseb[e]:baseb[e] + Nw * mpb[e]].reshape(Nw, mpb[e]),
                                           bs[baseb[e] // 32:(baseb[e] + Nw * mpb[e]) // 32].reshape(Nw, -1))
                acc = sum(Fraction(float(A[m, t])) * Fraction(float(B[n, t])) for t in range(mp[e]))
                assert abs(Fraction(float(dw[e, m, n])) - acc) <= abs(acc) * Fraction(1, 1 << 50)


def test_dequantize_mxfp8_every_code_and_scale_against_torch():
    """x = q * 2^(s - 127) for all 256 E4M3 codes under all 255 finite E8M0
    scales, against torch's own float8_e4m3fn and float8_e8m0fnu decoders (a
    library decode of both formats, independent of the oracle's tables); the
    two NaN codes stay NaN."""
    import torch
    codes = np.tile(np.arange(256, dtype=np.uint8), (255, 1))                  # [scale, code]
    scales = np.repeat(np.arange(255, dtype=np.uint8)[:, None], 256 // 32, axis=1)
    got = Q.dequantize_mxfp8_f64(codes, scales)
    q = torch.from_numpy(np.arange(256, dtype=np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    sv = torch.from_numpy(np.arange(255, dtype=np.uint8)).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    want = sv[:, None] * q[None, :]             # exact: a 4-bit significand times a power of two
    nan = np.isnan(want)
    assert nan.sum() == 2 * 255 and np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # the smallest and largest magnitudes: 2^-9 * 2^-127 and 448 * 2^127
    assert got[0, 1] == 2.0 ** -136 and got[254, 0x7E] == 448.0 * 2.0 ** 127


def test_tolerance_rule():
    y_ref = np.array([1.0, -2.0, 1e-9])
    ya = np.array([1.0, 2.0, 1.0])
    ok, _ = G.within_tolerance(y_ref * (1 + 1.9e-3), y_ref, ya)
    assert ok
    ok, _ = G.within_tolerance(y_ref * (1 + 2.1e-3), y_ref, ya)
    assert not ok
    # near-cancellation element: floor 2^-20 * sum|x w|
    ok, _ = G.within_tolerance(np.array([1.0, -2.0, 5e-7]), y_ref, ya)
    assert ok


def test_route_hand_example():
    ids = np.array([[2, 0], [0, 1], [2, 1]])
    row_index, seg, pair_row = route(ids, 3)
    assert row_index.tolist() == [0, 1, 1, 2, 0, 2]
    assert seg.tolist() == [0, 2, 4, 6]
    assert pair_row.tolist() == [4, 0, 1, 2, 5, 3]


def test_route_invariants():
    rng = np.random.default_rng(5)
    T, E, k = 1000, 16, 4
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :k]
    row_index, seg, pair_row = route(ids, E)
    assert seg[-1] == T * k and np.all(np.diff(seg) == np.bincount(ids.ravel(), minlength=E))
    for e in range(E):
        toks = row_index[seg[e]:seg[e + 1]]
        assert np.all(np.diff(toks) > 0)                             # strictly ascending tokens
        assert set(toks.tolist()) == set(np.nonzero((ids == e).any(axis=1))[0].tolist())
    flat = ids.ravel()
    assert np.all(row_index[pair_row] == np.arange(T * k) // k)
    assert np.all(np.searchsorted(seg, pair_row, side="right") - 1 == flat)
