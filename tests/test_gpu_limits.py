"""The segment-count limit of the segmented entry points on the GPU: 1024
experts (the largest count the routing, the segmented quantizers and the
grouped GEMMs accept), with a routing that leaves segments empty, short and
longer than a tile, against the oracle: routing and quantizers bit-exact, the
GEMMs under the accept rule of oracle.gemm."""
import numpy as np
import pytest
import torch

import block_scaled_bit_quantize_amd as bsq
from oracle import gemm as G
from oracle import quant as Q
from oracle.route import route as oroute

from _gpu_util import h, log, t

pytestmark = pytest.mark.gpu
E = 1024
f32 = np.float32


@pytest.fixture(scope="module")
def routing():
    """3000 tokens, top-8 over 1024 experts; experts 0..99 are never picked and
    experts 1000..1023 take a tenth of the picks (segments over 32 rows)."""
    rng = np.random.default_rng(1024)
    T, k = 3000, 8
    ids = np.empty((T, k), np.int32)
    for i in range(T):
        hot = rng.random() < 0.8
        pool = np.arange(1000, 1024) if hot else np.arange(100, 1000)
        ids[i] = rng.choice(pool if len(pool) >= k else np.arange(100, 1024), k, replace=False)
    log("limits: route 1024 experts")
    ri, seg, pr = bsq.route(t(ids), E)
    want_ri, want_seg, want_pr = oroute(ids, E)
    assert np.array_equal(h(seg), want_seg) and np.array_equal(h(ri), want_ri) and np.array_equal(h(pr), want_pr)
    lens = np.diff(want_seg)
    assert (lens == 0).sum() >= 100 and lens.max() > 32 and ((lens > 0) & (lens < 32)).any()
    return ids, want_ri, want_seg


def test_route_and_transposed_quantizers_1024_segments(routing):
    ids, ri, seg = routing
    M = int(seg[-1])
    rng = np.random.default_rng(5)
    C = 64
    x = rng.standard_normal((M, C)).astype(f32)
    log("limits: transposed mxfp8, 1024 segments")
    _, n = bsq.padded_segment_layout(seg, C)
    tc, ts = bsq.quantize_mxfp8(t(x), "sr", seed=9, stream_id=2, transpose=True, seg_offsets=t(seg), out_elems=n)
    oc, os_ = Q.quantize_mxfp8_transposed(x, seg, Q.SR, 9, 2)
    assert np.array_equal(h(tc), oc) and np.array_equal(h(ts), os_)
    log("limits: gathered nvfp4 -> mxfp8 requant, 1024 segments")
    T, Cx = ids.shape[0], 128
    xt = rng.standard_t(3, (T, Cx)).astype(f32)
    p, s, o = Q.quantize_nvfp4(xt[None], Q.OUTER_ROW)
    _, nx = bsq.padded_segment_layout(seg, Cx)
    rc, rs = bsq.requant_transpose_sr(t(p[0]), t(s[0]), t(np.asarray(o).reshape(-1)), "row", "mxfp8", seed=9,
                                      stream_id=3, rnd="sr", row_gather=t(ri), seg_offsets=t(seg), out_elems=nx)
    wc, ws = Q.requant_transpose_sr_segmented(p[0], s[0], np.asarray(o).reshape(-1), Q.OUTER_ROW, ri, seg, 9, 3)
    assert np.array_equal(h(rc), wc) and np.array_equal(h(rs), ws)


def test_grouped_gemms_1024_experts(routing):
    ids, ri, seg = routing
    M = int(seg[-1])
    T = ids.shape[0]
    rng = np.random.default_rng(6)
    N, K = 256, 128
    log("limits: nvfp4 grouped gemm, 1024 experts")
    x = rng.standard_t(3, (T, K)).astype(f32)
    w = (rng.standard_normal((E, N, K)) * 0.02).astype(f32)
    ap, as_, ao = Q.quantize_nvfp4(x[None], Q.OUTER_ROW)
    bp, bs, bo = Q.quantize_nvfp4(w, Q.OUTER_TENSOR)
    ao, bo = np.asarray(ao).reshape(-1), np.asarray(bo).reshape(-1)
    y = bsq.grouped_gemm_nvfp4(t(ap[0]), t(as_[0]), t(ao), t(bp), t(bs), t(bo), t(seg), M, row_index=t(ri),
                               out_dtype=torch.float32)
    yref, yabs = G.grouped_gemm_nvfp4_ref(ap[0], as_[0], ao, ri, bp, bs, bo, seg)
    ok, ratio = G.within_tolerance(h(y), yref, yabs)
    assert ok, ratio
    log("limits: mxfp8 dgrad, 1024 experts")
    g = (rng.standard_normal((M, K)) * 1e-3).astype(f32)
    gc, gs = Q.quantize_mxfp8(g, Q.SR, 11, 1)
    wt = (rng.standard_normal((E * N, K)) * 0.02).astype(f32)
    wc, wsc = Q.quantize_mxfp8(wt, Q.SR, 12, 1)
    wc, wsc = wc.reshape(E, N, K), wsc.reshape(E, N, K // 32)
    dx = bsq.grouped_gemm_mxfp8(False, t(gc), t(gs), t(wc), t(wsc), t(seg), M, N, K, out_dtype=torch.float32)
    yref, yabs = G.mxfp8_dgrad_ref(gc, gs, wc, wsc, seg)
    ok, ratio = G.within_tolerance(h(dx), yref, yabs)
    assert ok, ratio
    log("limits: mxfp8 wgrad, 1024 experts")
    Mg, Nx = 256, 256
    gg = (rng.standard_normal((M, Mg)) * 1e-3).astype(f32)
    xx = rng.standard_normal((M, Nx)).astype(f32)
    A, As = Q.quantize_mxfp8_transposed(gg, seg, Q.SR, 13, 2)
    B, Bs = Q.quantize_mxfp8_transposed(xx, seg, Q.SR, 14, 3)
    dw = bsq.grouped_gemm_mxfp8(True, t(A), t(As), t(B), t(Bs), t(seg), Mg, Nx)
    yref, yabs = G.mxfp8_wgrad_ref(A, As, B, Bs, seg, Mg, Nx)
    ok, ratio = G.within_tolerance(h(dw), yref, yabs)
    assert ok, ratio
