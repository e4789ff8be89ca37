"""Every output of the step's three expert grouped GEMMs at full size under the
accept rule of oracle.gemm: FPROP y[131072, 1536] (NVFP4, gathered token
rows), DGRAD dx[131072, 4096] and WGRAD dw[64, 1536, 4096] (MXFP8), with the
step's routing and random valid operand bytes. The operands are dequantized
by the oracle (exact float64 values); the float64 reference products of each
expert's blocks and of their magnitudes are taken with torch's float64
matmul on the device (a library product in float64, as the oracle's own
reference uses one; error far below the rule's bound) and compared expert by
expert on the host. The oracle's own products are compared on sampled rows
and experts in test_gpu_gemm.py."""
import numpy as np
import pytest
import torch

import block_scaled_bit_quantize_amd as bsq
import synth
from oracle import gemm as G
from oracle import quant as Q
from oracle.route import route as oroute

from _gpu_util import filler_mxfp8, filler_nvfp4, h, log, t

pytestmark = pytest.mark.gpu


class _Worst:
    def __init__(self, what):
        self.what, self.ratio, self.n = what, 0.0, 0

    def add(self, y, a, b):
        """y: the kernel's float32 block (device); a [m, k], b [n, k] float64 (device)."""
        yref = h(a @ b.T)
        yabs = h(a.abs() @ b.abs().T)
        ok, ratio = G.within_tolerance(h(y), yref, yabs)
        assert ok, (self.what, ratio)
        self.ratio = max(self.ratio, ratio)
        self.n += yref.size

    def report(self):
        log(f"{self.what}: {self.n} outputs within the rule, worst bound ratio {self.ratio:.3f}")


def _routing():
    ids = synth.moe_routing(2)
    row_index, seg, _ = oroute(ids, 64)
    return row_index, seg


@pytest.mark.parametrize("N", [1536, 3072])
def test_fprop_nvfp4_every_output(N):
    """N = 1536: the layer's forward; N = 3072: the expert chain's w13 product."""
    E, T, K = 64, 16384, 4096
    row_index, seg = _routing()
    M = int(seg[-1])
    rng = np.random.default_rng(71)
    ac, as_ = filler_nvfp4(rng, (T,), K)
    ao = rng.uniform(1e-3, 4e-3, T).astype(np.float32)
    bc, bs = filler_nvfp4(rng, (E, N), K)
    bo = rng.uniform(5e-6, 2e-5, E).astype(np.float32)
    log(f"fullsize fprop N={N}: run")
    y = bsq.grouped_gemm_nvfp4(t(ac), t(as_), t(ao), t(bc), t(bs), t(bo), t(seg), M, row_index=t(row_index),
                               out_dtype=torch.float32)
    xa = t(Q.dequantize_nvfp4_f64(ac[None], as_[None], ao.reshape(1, -1), Q.OUTER_ROW)[0])
    ri = t(row_index.astype(np.int64))
    w = _Worst(f"fprop (nvfp4, N={N})")
    for e in range(E):
        if seg[e + 1] == seg[e]:
            continue
        we = t(Q.dequantize_nvfp4_f64(bc[e:e + 1], bs[e:e + 1], bo[e:e + 1], Q.OUTER_TENSOR)[0])
        w.add(y[seg[e]:seg[e + 1]], xa[ri[seg[e]:seg[e + 1]]], we)
    w.report()


def test_dgrad_wgrad_mxfp8_every_output():
    E, Kx, Ng = 64, 4096, 1536
    row_index, seg = _routing()
    M = int(seg[-1])
    rng = np.random.default_rng(72)
    ac, as_ = filler_mxfp8(rng, M * Ng)
    bc, bs = filler_mxfp8(rng, E * Kx * Ng)
    log("fullsize dgrad: run")
    y = bsq.grouped_gemm_mxfp8(False, t(ac.reshape(M, Ng)), t(as_.reshape(M, Ng // 32)),
                               t(bc.reshape(E, Kx, Ng)), t(bs.reshape(E, Kx, Ng // 32)), t(seg), M, Kx, Ng,
                               out_dtype=torch.float32)
    ga = t(Q.dequantize_mxfp8_f64(ac, as_).reshape(M, Ng))
    w = _Worst("dgrad (mxfp8)")
    for e in range(E):
        if seg[e + 1] == seg[e]:
            continue
        wt = t(Q.dequantize_mxfp8_f64(bc[e * Kx * Ng:(e + 1) * Kx * Ng], bs[e * Kx * Ng // 32:(e + 1) * Kx * Ng // 32])
               .reshape(Kx, Ng))
        w.add(y[seg[e]:seg[e + 1]], ga[seg[e]:seg[e + 1]], wt)
    w.report()
    del y, ga

    log("fullsize wgrad: run")
    _, na = bsq.padded_segment_layout(seg, Ng)
    _, nb = bsq.padded_segment_layout(seg, Kx)
    A, As = filler_mxfp8(rng, na)
    B, Bs = filler_mxfp8(rng, nb)
    mpa, basea = Q.segmented_layout(seg, Ng)
    mpb, baseb = Q.segmented_layout(seg, Kx)
    for e in range(E):  # the layout's padding tokens hold zeros
        Me = int(seg[e + 1] - seg[e])
        A[basea[e]:basea[e] + Ng * mpa[e]].reshape(Ng, mpa[e])[:, Me:] = 0
        B[baseb[e]:baseb[e] + Kx * mpb[e]].reshape(Kx, mpb[e])[:, Me:] = 0
    dw = bsq.grouped_gemm_mxfp8(True, t(A), t(As), t(B), t(Bs), t(seg), Ng, Kx)
    A64 = t(Q.dequantize_mxfp8_f64(A, As))
    B64 = t(Q.dequantize_mxfp8_f64(B, Bs))
    w = _Worst("wgrad (mxfp8)")
    for e in range(E):
        a = A64[basea[e]:basea[e] + Ng * mpa[e]].reshape(Ng, mpa[e])
        b = B64[baseb[e]:baseb[e] + Kx * mpb[e]].reshape(Kx, mpb[e])
        w.add(dw[e], a, b)
    w.report()


def test_fprop_nvfp4_workload5_every_output():
    """Workload 5's NVFP4 forward at full size (65536 tokens, hidden 7168, 128
    experts of 2048 x 7168, top-8 Zipf routing: segments of 717 to 59174
    rows), every output under the accept rule. The operands are decoded on the
    device with the oracle's E2M1 and E4M3 tables (q * s_b * s_t, exact in
    float64) and the rule is applied there with the oracle's constants."""
    from oracle import formats as F
    p = synth.WORKLOADS[5]
    T, K, E, N = p["tokens"], p["hidden"], p["experts"], p["ffn"]
    row_index, seg, _ = oroute(synth.moe_routing(5), E)
    M = int(seg[-1])
    rng = np.random.default_rng(75)
    ac, as_ = filler_nvfp4(rng, (T,), K)
    ao = rng.uniform(1e-3, 4e-3, T).astype(np.float32)
    bc, bs = filler_nvfp4(rng, (E, N), K)
    bo = rng.uniform(5e-6, 2e-5, E).astype(np.float32)
    log("fullsize fprop workload 5: run")
    y = bsq.grouped_gemm_nvfp4(t(ac), t(as_), t(ao), t(bc), t(bs), t(bo), t(seg), M, row_index=t(row_index),
                               out_dtype=torch.float32)
    q_lut = t(F.e2m1_decode(np.arange(16)).astype(np.float64))
    s_lut = t(F.e4m3_decode(np.arange(256)).astype(np.float64))

    def decode(codes, scales, outer):  # codes u8 [R, K/2] (low nibble first), scales u8 [R, K/16], outer [R, 1]
        c = codes.long()
        q = torch.stack((q_lut[c & 15], q_lut[c >> 4]), dim=-1).reshape(codes.shape[0], -1)
        return q * s_lut[scales.long()].repeat_interleave(16, dim=1) * outer

    xa = decode(t(ac), t(as_), t(ao.astype(np.float64)).reshape(-1, 1))
    ri = t(row_index.astype(np.int64))
    worst, count = 0.0, 0
    for e in range(E):
        a, b = int(seg[e]), int(seg[e + 1])
        if a == b:
            continue
        we = decode(t(bc[e]), t(bs[e]), float(bo[e]))
        xe = xa[ri[a:b]]
        yref = xe @ we.T
        yabs = xe.abs() @ we.abs().T
        bound = G.REL_TOL * yref.abs() + G.ABS_FLOOR * yabs
        err = (y[a:b].double() - yref).abs()
        worst = max(worst, float((err / bound.clamp_min(1e-300)).max()))
        count += err.numel()
        assert bool((err <= bound).all()), (e, worst)
    log(f"fprop workload 5: {count} outputs within the rule, worst bound ratio {worst:.3f}")
