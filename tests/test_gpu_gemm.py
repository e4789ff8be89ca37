"""GPU parity of the expert grouped GEMMs against the oracle's float64
product of the same dequantized operands (accept rule of oracle.gemm), at
small sizes with ragged and empty segments and at the workloads' full sizes on
sampled output rows. Full-size operands hold oracle-quantized data wherever an
output is checked and valid random bytes elsewhere."""
import numpy as np
import pytest
import torch

import block_scaled_bit_quantize_amd as bsq
import synth
from oracle import formats as F
from oracle import gemm as G
from oracle import quant as Q
from oracle.route import route as oroute

from _gpu_util import DEV, bf16_t, filler_mxfp8, filler_nvfp4, h, log, t

pytestmark = pytest.mark.gpu
f32 = np.float32


def _check(y, yref, yabs, what, floor=G.ABS_FLOOR):
    """y: the float32 GEMM result (before output rounding) vs the float64 reference."""
    ok, ratio = G.within_tolerance(y, yref, yabs, floor)
    rel = G.max_rel_error(y, yref)
    print(f"[{what}] worst bound ratio {ratio:.3f}, max rel err {rel:.2e}", flush=True)
    assert ok, f"{what}: outside tolerance (ratio {ratio})"


def _check_bf16(y16, y32, what):
    """The bf16 output is the round-to-nearest-even of the float32 result."""
    want = synth.bf16_bits(np.asarray(y32, dtype=f32))
    got = np.asarray(y16).view(np.uint16)
    assert np.array_equal(got, want), f"{what}: bf16 output differs from RNE(float32 output)"


def _nvfp4(*args, **kw):
    """Run the NVFP4 GEMM twice (float32 and bf16 outputs)."""
    y32 = bsq.grouped_gemm_nvfp4(*args, out_dtype=torch.float32, **kw)
    y16 = bsq.grouped_gemm_nvfp4(*args, out_dtype=torch.bfloat16, **kw)
    return y32, y16


@pytest.mark.parametrize("per_row", [True, False])
def test_gemm_nvfp4_small_ragged(per_row):
    log(f"gemm nvfp4 small per_row={per_row}")
    rng = np.random.default_rng(5)
    T, E, N, K = 400, 5, 512, 384
    seg = np.array([0, 0, 300, 317, 830, 831], dtype=np.int64)
    row_index = rng.integers(0, T, size=831).astype(np.int32)
    x = rng.standard_t(3, (T, K)).astype(f32)
    w = (rng.standard_normal((E, N, K)) * 0.02).astype(f32)
    if per_row:
        ap, as_, ao = Q.quantize_nvfp4(x[None], Q.OUTER_ROW)
        ao = ao[0]
    else:
        ap, as_, ao = Q.quantize_nvfp4(x[None], Q.OUTER_TENSOR)
    bp, bs, bo = Q.quantize_nvfp4(w, Q.OUTER_TENSOR)
    y32, y16 = _nvfp4(t(ap[0]), t(as_[0]), t(ao), t(bp), t(bs), t(bo), t(seg), 831, row_index=t(row_index))
    yref, yabs = G.grouped_gemm_nvfp4_ref(ap[0], as_[0], ao, row_index, bp, bs, bo, seg)
    _check(h(y32), yref, yabs, "nvfp4 small")
    _check_bf16(h(y16.view(torch.int16)), h(y32), "nvfp4 small")


def test_gemm_nvfp4_workload1():
    """256x256x256: A = the SR-requantized X^T (NVFP4, seed 0), B = W RTN."""
    log("gemm nvfp4 workload1")
    X, W = synth.workload1()
    p, s, o = Q.quantize_nvfp4(X[None], Q.OUTER_TENSOR)
    ac, as_, ao = Q.requant_transpose_sr(p, s, o, Q.OUTER_TENSOR, Q.NVFP4, 0, 0)
    bp, bs, bo = Q.quantize_nvfp4(W[None], Q.OUTER_TENSOR)
    seg = np.array([0, 256], dtype=np.int64)
    y32, y16 = _nvfp4(t(ac[0]), t(as_[0]), t(ao), t(bp), t(bs), t(bo), t(seg), 256)
    yref, yabs = G.grouped_gemm_nvfp4_ref(ac[0], as_[0], ao, None, bp, bs, bo, seg)
    _check(h(y32), yref, yabs, "nvfp4 workload1 (X^T_sr W^T)")
    _check_bf16(h(y16.view(torch.int16)), h(y32), "nvfp4 workload1")
    # the forward product X_q W_q^T as well
    y32, y16 = _nvfp4(t(p[0]), t(s[0]), t(o), t(bp), t(bs), t(bo), t(seg), 256)
    yref, yabs = G.grouped_gemm_nvfp4_ref(p[0], s[0], o, None, bp, bs, bo, seg)
    _check(h(y32), yref, yabs, "nvfp4 workload1 (X_q W_q^T)")
    _check_bf16(h(y16.view(torch.int16)), h(y32), "nvfp4 workload1 forward")


def _moe_full(wl, sample_experts, four_over_six=False):
    """Full-size NVFP4 grouped GEMM of workload 2 or 5 with sampled rows. The
    activations are quantized per token with Four Over Six block scales when
    four_over_six is set (the forward's activation quantizer, as timed)."""
    p = synth.WORKLOADS[wl]
    T, K, E, N = p["tokens"], p["hidden"], p["experts"], p["ffn"]
    log(f"gemm nvfp4 workload{wl}: generate inputs")
    ids = synth.moe_routing(wl)
    row_index, seg, _ = oroute(ids, E)
    x = synth.moe_activations(wl)
    w = synth.moe_weights(wl)
    rng = np.random.default_rng(wl)
    ac, as_ = filler_nvfp4(rng, (T,), K)
    ao = np.full(T, 2e-3, f32)
    bc, bs = filler_nvfp4(rng, (E, N), K)
    bo = np.full(E, 1e-5, f32)
    lens = np.diff(seg)
    experts = sorted(set(sample_experts) | {int(np.argmax(lens)), int(np.argmin(np.where(lens > 0, lens, 1 << 30)))})
    rows = []
    for e in experts:
        if lens[e] == 0:
            continue
        cand = np.r_[seg[e], seg[e + 1] - 1, rng.integers(seg[e], seg[e + 1], size=14)]
        rows.extend(cand.tolist())
    rows = np.unique(np.array(rows, dtype=np.int64))
    toks = np.unique(row_index[rows])
    fos = dict(four_over_six=four_over_six)
    qa, qs, qo = Q.quantize_nvfp4(synth.bf16_to_f32(x[toks])[None], Q.OUTER_ROW, **fos)
    ac[toks], as_[toks], ao[toks] = qa[0], qs[0], qo[0]
    # the quantizers at this workload's full size (per token; per expert in one pass): sampled tokens and
    # experts against the oracle
    log(f"quantize workload{wl} activations (four_over_six={four_over_six}) and weights")
    gxc, gxs, gxo = bsq.quantize_nvfp4(bf16_t(x), "row", **fos)
    tt = t(toks)
    assert np.array_equal(h(gxc[tt]), qa[0]) and np.array_equal(h(gxs[tt]), qs[0])
    assert np.array_equal(h(gxo[tt]), np.asarray(qo).reshape(-1))
    more = np.unique(np.r_[rng.choice(T, 256, replace=False), 0, T - 1])   # and 256 more tokens
    ma, ms, mo = Q.quantize_nvfp4(synth.bf16_to_f32(x[more])[None], Q.OUTER_ROW, **fos)
    tm = t(more)
    assert np.array_equal(h(gxc[tm]), ma[0]) and np.array_equal(h(gxs[tm]), ms[0])
    assert np.array_equal(h(gxo[tm]), np.asarray(mo).reshape(-1))
    del gxc, gxs, gxo
    gwc, gws, gwo = bsq.quantize_nvfp4(bf16_t(w), "tensor")
    for e in experts:
        qb, qbs, qbo = Q.quantize_nvfp4(synth.bf16_to_f32(w[e])[None], Q.OUTER_TENSOR)
        bc[e], bs[e], bo[e] = qb[0], qbs[0], qbo[0]
        assert np.array_equal(h(gwc[e]), qb[0]) and np.array_equal(h(gws[e]), qbs[0]), e
        assert h(gwo)[e] == np.asarray(qbo).reshape(-1)[0]
    del gwc, gws, gwo, x, w
    torch.cuda.empty_cache()
    log(f"gemm nvfp4 workload{wl}: run (M_total={seg[-1]}, N={N}, K={K}, E={E})")
    y32, y16 = _nvfp4(t(ac), t(as_), t(ao), t(bc), t(bs), t(bo), t(seg), int(seg[-1]), row_index=t(row_index))
    ys = h(y32[t(rows)])
    yref, yabs = G.grouped_gemm_nvfp4_ref(ac, as_, ao, row_index, bc, bs, bo, seg, rows=rows)
    _check(ys, yref, yabs, f"nvfp4 workload{wl} sampled {len(rows)} rows")
    # bf16 output of the whole launch vs the float32 one, compared on the GPU
    assert torch.equal(y16, y32.to(torch.bfloat16)), "bf16 output differs from RNE(float32 output)"


def test_gemm_nvfp4_workload2_full():
    _moe_full(2, [0, 5, 11, 21, 28, 34, 40, 47, 55, 63])


def test_gemm_nvfp4_workload5_full():
    _moe_full(5, [0, 9, 33, 64, 90, 101, 116, 127], four_over_six=True)


@pytest.mark.parametrize("M,N,K", [(128, 128, 64), (256, 384, 192), (384, 512, 320)])
def test_gemm_nvfp4_inreg_scale(M, N, K):
    """The in-register scale variant (FP8 MFMA per 16-value block, fp32 scale
    products) against the float64 oracle (accept rule) and against the exact
    16-bit decode kernel on the same operands (both within the rule)."""
    log(f"gemm nvfp4 inreg-scale M={M} N={N} K={K}")
    rng = np.random.default_rng(M + N + K)
    x = rng.standard_t(3, (M, K)).astype(f32)
    w = (rng.standard_normal((1, N, K)) * 0.02).astype(f32)
    ap, as_, ao = Q.quantize_nvfp4(x[None], Q.OUTER_ROW, four_over_six=True)
    bp, bs, bo = Q.quantize_nvfp4(w, Q.OUTER_TENSOR)
    ao = np.asarray(ao).reshape(-1)
    seg = np.array([0, M], dtype=np.int64)
    yref, yabs = G.grouped_gemm_nvfp4_ref(ap[0], as_[0], ao, None, bp, bs, bo, seg)
    y = bsq.gemm_nvfp4_inreg_scale(t(ap[0]), t(as_[0]), t(ao), t(bp[0]), t(bs[0]), t(np.asarray(bo).reshape(-1)))
    _check(h(y), yref, yabs, f"nvfp4 inreg-scale {M}x{N}x{K}")
    if N % 256:  # the grouped kernel's tiles are 256 wide
        return
    y16 = bsq.grouped_gemm_nvfp4(t(ap[0]), t(as_[0]), t(ao), t(bp), t(bs), t(np.asarray(bo).reshape(-1)), t(seg), M,
                                 out_dtype=torch.float32)
    _check(h(y16), yref, yabs, f"nvfp4 decode16 {M}x{N}x{K}")


def _mxfp8_from(rng, x, rnd=Q.SR):
    return Q.quantize_mxfp8(x, rnd, int(rng.integers(1 << 30)), 1)


@pytest.mark.parametrize("K", [64, 192, 320])
def test_gemm_short_k(K):
    """1, 3 and 5 K steps of 64: the block scales come in groups of four K
    steps, so these cover a group cut short, a single partial group and a
    full group followed by a partial one, for the NVFP4 forward (gathered
    rows) and the MXFP8 DGRAD (odd row count: its scale array ends off a
    4-byte boundary when K % 128 == 64)."""
    log(f"gemm short K={K}")
    rng = np.random.default_rng(K)
    T, E, N = 97, 3, 256
    seg = np.array([0, 40, 41, 195], dtype=np.int64)
    row_index = rng.integers(0, T, size=195).astype(np.int32)
    x = rng.standard_t(3, (T, K)).astype(f32)
    w = (rng.standard_normal((E, N, K)) * 0.02).astype(f32)
    ap, as_, ao = Q.quantize_nvfp4(x[None], Q.OUTER_ROW, four_over_six=True)
    bp, bs, bo = Q.quantize_nvfp4(w, Q.OUTER_TENSOR)
    ao, bo = np.asarray(ao).reshape(-1), np.asarray(bo).reshape(-1)
    y32, y16 = _nvfp4(t(ap[0]), t(as_[0]), t(ao), t(bp), t(bs), t(bo), t(seg), 195, row_index=t(row_index))
    yref, yabs = G.grouped_gemm_nvfp4_ref(ap[0], as_[0], ao, row_index, bp, bs, bo, seg)
    _check(h(y32), yref, yabs, f"nvfp4 short K={K}")
    assert torch.equal(y16, y32.to(torch.bfloat16))
    g = (rng.standard_normal((195, K)) * 1e-3).astype(f32)
    ac, as2 = _mxfp8_from(rng, g)
    wt = (rng.standard_normal((E * N, K)) * 0.02).astype(f32)
    bc, bs2 = _mxfp8_from(rng, wt)
    bc, bs2 = bc.reshape(E, N, K), bs2.reshape(E, N, K // 32)
    y = bsq.grouped_gemm_mxfp8(False, t(ac), t(as2), t(bc), t(bs2), t(seg), 195, N, K, out_dtype=torch.float32)
    yref, yabs = G.mxfp8_dgrad_ref(ac, as2, bc, bs2, seg)
    _check(h(y), yref, yabs, f"mxfp8 dgrad short K={K}")


@pytest.mark.parametrize("K", [128, 192])
def test_gemm_tail_tiles(K):
    """Segments whose last 256-row tile holds 1, 127, 128 or 129..255 rows:
    a last tile with at most 128 rows runs as a tail tile (both halves of the
    workgroup on its first 128 rows, each over half of every K step, partial
    sums added at the end); 129 rows and more run as a full tile. NVFP4
    forward (gathered rows, bf16 = RNE of the float32 result) and MXFP8 DGRAD,
    with an even and an odd number of K steps."""
    log(f"gemm tail tiles K={K}")
    rng = np.random.default_rng(900 + K)
    lens = [128, 129, 1, 255, 256, 384, 385, 127, 0, 640]
    seg = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    M, E, N, T = int(seg[-1]), len(lens), 256, 700
    row_index = rng.integers(0, T, size=M).astype(np.int32)
    x = rng.standard_t(3, (T, K)).astype(f32)
    w = (rng.standard_normal((E, N, K)) * 0.02).astype(f32)
    ap, as_, ao = Q.quantize_nvfp4(x[None], Q.OUTER_ROW, four_over_six=True)
    bp, bs, bo = Q.quantize_nvfp4(w, Q.OUTER_TENSOR)
    ao, bo = np.asarray(ao).reshape(-1), np.asarray(bo).reshape(-1)
    y32, y16 = _nvfp4(t(ap[0]), t(as_[0]), t(ao), t(bp), t(bs), t(bo), t(seg), M, row_index=t(row_index))
    yref, yabs = G.grouped_gemm_nvfp4_ref(ap[0], as_[0], ao, row_index, bp, bs, bo, seg)
    _check(h(y32), yref, yabs, f"nvfp4 tail tiles K={K}")
    _check_bf16(h(y16.view(torch.int16)), h(y32), f"nvfp4 tail tiles K={K}")
    g = (rng.standard_normal((M, K)) * 1e-3).astype(f32)
    ac, as2 = _mxfp8_from(rng, g)
    wt = (rng.standard_normal((E * N, K)) * 0.02).astype(f32)
    bc, bs2 = _mxfp8_from(rng, wt)
    bc, bs2 = bc.reshape(E, N, K), bs2.reshape(E, N, K // 32)
    y = bsq.grouped_gemm_mxfp8(False, t(ac), t(as2), t(bc), t(bs2), t(seg), M, N, K, out_dtype=torch.float32)
    y16 = bsq.grouped_gemm_mxfp8(False, t(ac), t(as2), t(bc), t(bs2), t(seg), M, N, K)
    yref, yabs = G.mxfp8_dgrad_ref(ac, as2, bc, bs2, seg)
    _check(h(y), yref, yabs, f"mxfp8 dgrad tail tiles K={K}")
    _check_bf16(h(y16.view(torch.int16)), h(y), f"mxfp8 dgrad tail tiles K={K}")


def test_gemm_mxfp8_scale_code_range():
    """The bf16 decode of MXFP8 operands over the whole E8M0 range: row r of A
    holds 32 copies of one E4M3 value q under scale code c_r (block 0; block 1
    is zero) and B is all ones, so y[r, n] = 32 * dec(q, c_r) with dec the
    bf16 value of q * 2^(c - 127). Codes 3..246: dec is exact, so y equals the
    float64 product. Codes 0..2: dec is the round-to-nearest-even of the exact
    value onto bf16's subnormal grid (multiples of 2^-133). Codes 247..254:
    magnitudes of 2^128 and more decode to infinity."""
    log("gemm mxfp8 scale code range")
    codes = list(range(0, 13)) + list(range(240, 255))
    M, N, K = 256, 256, 64
    seg = np.array([0, M], dtype=np.int64)
    bc = np.full((1, N, K), 0x38, np.uint8)                 # 1.0
    bs = np.full((1, N, K // 32), 127, np.uint8)
    for q in (0x01, 0x07, 0x38, 0x3F, 0x77, 0x7E, 0xB9):
        ac = np.zeros((M, K), np.uint8)
        ac[:, :32] = q
        asc = np.full((M, K // 32), 127, np.uint8)
        asc[:len(codes), 0] = codes
        y = h(bsq.grouped_gemm_mxfp8(False, t(ac), t(asc), t(bc), t(bs), t(seg), M, N, K, out_dtype=torch.float32))
        qv = float(F.e4m3_decode(np.array([q], np.uint8))[0])
        for r, c in enumerate(codes):
            exact = qv * 2.0 ** (c - 127)
            dec = float(torch.tensor(exact, dtype=torch.float64).to(torch.bfloat16).to(torch.float64))
            with np.errstate(over="ignore"):
                want = np.float32(32.0 * dec)              # a power-of-two multiple: exact unless it overflows
            assert np.all(y[r] == want), (hex(q), c, y[r, 0], want)
            if 3 <= c <= 246:
                assert dec == exact, (hex(q), c)
            if c < 3:
                assert abs(dec - exact) <= 2.0 ** -134
            if c >= 247 and abs(exact) >= 2.0 ** 128:
                assert np.isinf(want)


def test_gemm_mxfp8_dgrad_small():
    log("gemm mxfp8 dgrad small")
    rng = np.random.default_rng(6)
    E, N, K = 4, 512, 384
    seg = np.array([0, 100, 100, 357, 613], dtype=np.int64)
    g = (rng.standard_normal((613, K)) * 1e-3).astype(f32)
    wt = (rng.standard_normal((E * N, K)) * 0.02).astype(f32)
    ac, as_ = _mxfp8_from(rng, g)
    bc, bs = _mxfp8_from(rng, wt)
    bc, bs = bc.reshape(E, N, K), bs.reshape(E, N, K // 32)
    y = bsq.grouped_gemm_mxfp8(False, t(ac), t(as_), t(bc), t(bs), t(seg), 613, N, K, out_dtype=torch.float32)
    y16 = bsq.grouped_gemm_mxfp8(False, t(ac), t(as_), t(bc), t(bs), t(seg), 613, N, K)
    yref, yabs = G.mxfp8_dgrad_ref(ac, as_, bc, bs, seg)
    _check(h(y), yref, yabs, "mxfp8 dgrad small")
    _check_bf16(h(y16.view(torch.int16)), h(y), "mxfp8 dgrad small")


def test_gemm_mxfp8_wgrad_small():
    log("gemm mxfp8 wgrad small")
    rng = np.random.default_rng(7)
    M, N = 256, 512
    seg = np.array([0, 0, 45, 245, 245, 374], dtype=np.int64)       # Kp = 0, 64, 224, 0, 160
    ga = (rng.standard_normal((374, M)) * 1e-3).astype(f32)
    xb = rng.standard_normal((374, N)).astype(f32)
    ac, as_ = Q.quantize_mxfp8_transposed(ga, seg, Q.SR, 1, 2)
    bc, bs = Q.quantize_mxfp8_transposed(xb, seg, Q.SR, 1, 3)
    y = bsq.grouped_gemm_mxfp8(True, t(ac), t(as_), t(bc), t(bs), t(seg), M, N)
    yref, yabs = G.mxfp8_wgrad_ref(ac, as_, bc, bs, seg, M, N)
    _check(h(y), yref, yabs, "mxfp8 wgrad small")
    y16 = bsq.grouped_gemm_mxfp8(True, t(ac), t(as_), t(bc), t(bs), t(seg), M, N,
                                 out_dtype=torch.bfloat16)
    assert torch.equal(y16, y.to(torch.bfloat16))


def test_gemm_mxfp8_workload4_full():
    """DGRAD dx[131072, 4096] = g w_q and WGRAD dw[64, 1536, 4096] = g^T x_q at
    full size with workload 2's routing; sampled rows / experts."""
    log("gemm mxfp8 workload4: setup")
    E, T, Kx, Ng = 64, 16384, 4096, 1536
    ids = synth.moe_routing(2)
    row_index, seg, _ = oroute(ids, E)
    M_total = int(seg[-1])
    rng = np.random.default_rng(44)
    lens = np.diff(seg)
    experts = [0, 33, 63]
    # DGRAD: A = g rows [M_total, 1536], B = w_q^T [E, 4096, 1536]
    ac, as_ = filler_mxfp8(rng, M_total * Ng)
    ac, as_ = ac.reshape(M_total, Ng), as_.reshape(M_total, Ng // 32)
    bc, bs = filler_mxfp8(rng, E * Kx * Ng)
    bc, bs = bc.reshape(E, Kx, Ng), bs.reshape(E, Kx, Ng // 32)
    rows = np.unique(np.concatenate([np.r_[seg[e], seg[e + 1] - 1, rng.integers(seg[e], seg[e + 1], size=14)]
                                     for e in experts]))
    g = synth.output_grad(M_total, Ng)
    gq, gs = Q.quantize_mxfp8(synth.bf16_to_f32(g[rows]), Q.SR, 42, 1)
    ac[rows], as_[rows] = gq, gs
    W = synth.moe_weights(2)
    for e in experts:
        p, s, o = Q.quantize_nvfp4(synth.bf16_to_f32(W[e])[None], Q.OUTER_TENSOR)
        c, sc = Q.requant_transpose_sr(p, s, o, Q.OUTER_TENSOR, Q.MXFP8, 42, 0, item0=e)
        bc[e], bs[e] = c[0], sc[0]
    log("gemm mxfp8 workload4: dgrad")
    y = bsq.grouped_gemm_mxfp8(False, t(ac), t(as_), t(bc), t(bs), t(seg), M_total, Kx, Ng, out_dtype=torch.float32)
    ys = h(y[t(rows)])
    del y
    yref, yabs = G.mxfp8_dgrad_ref(ac, as_, bc, bs, seg, rows=rows)
    _check(ys, yref, yabs, "mxfp8 dgrad workload4")
    # WGRAD: A = g^T per expert [1536, Kp_e], B = x_q^T per expert [4096, Kp_e]
    log("gemm mxfp8 workload4: wgrad setup")
    mpa, na = bsq.padded_segment_layout(seg, Ng)
    mpb, nb = bsq.padded_segment_layout(seg, Kx)
    A, As = filler_mxfp8(rng, na)
    B, Bs = filler_mxfp8(rng, nb)
    _, basea = Q.segmented_layout(seg, Ng)
    _, baseb = Q.segmented_layout(seg, Kx)
    gf = synth.bf16_to_f32(g).reshape(M_total, Ng)
    x = synth.moe_activations(2)
    for e in experts:
        c, sc = Q.quantize_mxfp8_transposed(gf, seg, Q.SR, 42, 2, segments=[e])
        A[basea[e]:basea[e] + c.size], As[basea[e] // 32:basea[e] // 32 + sc.size] = c, sc
        toks = row_index[seg[e]:seg[e + 1]]
        p, s, o = Q.quantize_nvfp4(synth.bf16_to_f32(x[toks])[None], Q.OUTER_ROW)
        # the gathered rows of expert e as their own token table
        c, sc = Q.requant_transpose_sr_segmented(p[0], s[0], o[0], Q.OUTER_ROW,
                                                 np.arange(len(toks)), np.array([0, len(toks)]), 42, 3)
        B[baseb[e]:baseb[e] + c.size], Bs[baseb[e] // 32:baseb[e] // 32 + sc.size] = c, sc
    del gf, x, g
    log("gemm mxfp8 workload4: wgrad")
    dw = bsq.grouped_gemm_mxfp8(True, t(A), t(As), t(B), t(Bs), t(seg), Ng, Kx)
    for e in experts:
        ys = h(dw[e])
        yref, yabs = G.mxfp8_wgrad_ref(A, As, B, Bs, seg, Ng, Kx, experts=[e])
        _check(ys, yref[0], yabs[0], f"mxfp8 wgrad workload4 expert {e}")


@pytest.mark.parametrize("kind", [0, 1, 2, 3, 4])
def test_mfma_rate_probe_runs(kind):
    """The throughput probe's launches complete and keep every accumulator:
    zero operands give exactly zero, the other data kinds finite values."""
    log(f"mfma rate probe kind={kind}")
    z = h(bsq.mfma_rate_probe(kind, 1, 8, 4))
    assert z.shape == (1024,) and np.all(z == 0.0)
    for data in (0, 2):
        r = h(bsq.mfma_rate_probe(kind, data, 8, 4))
        assert np.all(np.isfinite(r)) and np.any(r != 0.0)
