"""Every output byte at full size, bit-exact against the oracle, of the
forward's NVFP4 quantizers (the activations [16384, 4096] per token with Four
Over Six, and the 64 expert weights [1536, 4096] with per-expert outer scales
from the one-pass kernel: round to nearest with two-level scales, section
"Low-precision formats on Blackwell"; Four Over Six, section "Recipe
details"), the same for workload 5's sizes, and of the combine codec. The oracle runs in slices; each slice is
compared as soon as it is done."""
import numpy as np
import pytest
import torch

import block_scaled_bit_quantize_amd as bsq
import synth
from oracle import codec as C
from oracle import quant as Q
from oracle.route import route as oroute

from _gpu_util import bf16_t, h, log, t

pytestmark = pytest.mark.gpu


def test_activations_four_over_six_fullsize_exact():
    x = synth.moe_activations(2)
    log("fullsize exact: activations, four over six")
    gc, gs, go = bsq.quantize_nvfp4(bf16_t(x), "row", four_over_six=True)
    gc, gs, go = h(gc), h(gs), h(go)
    for r0 in range(0, x.shape[0], 2048):
        xf = synth.bf16_to_f32(x[r0:r0 + 2048])
        oc, os_, oo = Q.quantize_nvfp4(xf[None], Q.OUTER_ROW, four_over_six=True)
        assert np.array_equal(go[r0:r0 + 2048], oo[0]), r0
        assert np.array_equal(gs[r0:r0 + 2048], os_[0]), r0
        assert np.array_equal(gc[r0:r0 + 2048], oc[0]), r0
        log(f"activations rows {r0}..{r0 + 2047} equal")


def test_expert_weights_fullsize_exact():
    w = synth.moe_weights(2)
    log("fullsize exact: expert weights, per-expert outer scale (one pass)")
    gc, gs, go = bsq.quantize_nvfp4(bf16_t(w), "tensor")
    gc, gs, go = h(gc), h(gs), h(go)
    for e0 in range(0, w.shape[0], 8):
        we = synth.bf16_to_f32(w[e0:e0 + 8])
        oc, os_, oo = Q.quantize_nvfp4(we, Q.OUTER_TENSOR)
        assert np.array_equal(go[e0:e0 + 8], oo.reshape(-1)), e0
        assert np.array_equal(gs[e0:e0 + 8], os_), e0
        assert np.array_equal(gc[e0:e0 + 8], oc), e0
        log(f"experts {e0}..{e0 + 7} equal")


def test_combine_codec_fullsize_exact():
    """The combine payload (131072 dispatched rows of 4096, the step's
    routing): every encoded byte (RHT-32 + S2F6, section "Quantized
    communications") and every combined token, bit-exact against the oracle."""
    T, k, H = 16384, 8, 4096
    mask = 0x9E3779B9
    rows = synth.combine_rows(T * k, H)
    _, _, pair_row = oroute(synth.moe_routing(2), 64)
    pair_row = np.asarray(pair_row, np.int64)
    log("fullsize exact: combine codec")
    gc, gs = bsq.rht_s2f6_encode(bf16_t(rows), mask)
    out = bsq.rht_s2f6_combine(gc, gs, t(pair_row.astype(np.int32)), k, mask, out_dtype=torch.float32)
    gc, gs, out = h(gc), h(gs), h(out)
    oc = np.empty_like(gc)
    os_ = np.empty_like(gs)
    for r0 in range(0, T * k, 16384):
        oc[r0:r0 + 16384], os_[r0:r0 + 16384] = C.encode(synth.bf16_to_f32(rows[r0:r0 + 16384]), mask)
        assert np.array_equal(gc[r0:r0 + 16384], oc[r0:r0 + 16384]), r0
        assert np.array_equal(gs[r0:r0 + 16384], os_[r0:r0 + 16384]), r0
    log("encoded rows equal")
    pr = pair_row.reshape(T, k)
    for t0 in range(0, T, 2048):
        sub = pr[t0:t0 + 2048].reshape(-1)
        want = C.combine(oc[sub], os_[sub], np.arange(len(sub)), k, mask)
        assert np.array_equal(out[t0:t0 + 2048].view(np.uint32), want.view(np.uint32)), t0
    log("combined tokens equal")


def test_workload5_quantizers_fullsize_exact():
    """Workload 5 (65536 tokens, hidden 7168; 128 experts of 2048 x 7168):
    every output byte of the per-token Four Over Six activation quantizer and
    of the per-expert one-pass weight quantizer, against the oracle run over
    slices in a pool of worker processes."""
    import _oracle_pool
    x = synth.moe_activations(5)
    log("fullsize exact: workload 5 activations, four over six")
    gc, gs, go = bsq.quantize_nvfp4(bf16_t(x), "row", four_over_six=True)
    gc, gs, go = h(gc), h(gs), h(go)
    R = 4096
    with _oracle_pool.pool() as ex:
        jobs = ((x[r0:r0 + R], "row", True) for r0 in range(0, x.shape[0], R))
        for i, (oc, os_, oo) in enumerate(ex.map(_oracle_pool.nvfp4_slice, jobs)):
            r0 = i * R
            assert np.array_equal(go[r0:r0 + R], oo[0]), r0
            assert np.array_equal(gs[r0:r0 + R], os_[0]), r0
            assert np.array_equal(gc[r0:r0 + R], oc[0]), r0
        log("workload 5 activations equal")
        del x, gc, gs, go
        w = synth.moe_weights(5)
        log("fullsize exact: workload 5 expert weights")
        gc, gs, go = bsq.quantize_nvfp4(bf16_t(w), "tensor")
        gc, gs, go = h(gc), h(gs), h(go)
        jobs = ((w[e0:e0 + 4], "tensor", False) for e0 in range(0, w.shape[0], 4))
        for i, (oc, os_, oo) in enumerate(ex.map(_oracle_pool.nvfp4_slice, jobs)):
            e0 = i * 4
            assert np.array_equal(go[e0:e0 + 4], oo.reshape(-1)), e0
            assert np.array_equal(gs[e0:e0 + 4], os_), e0
            assert np.array_equal(gc[e0:e0 + 4], oc), e0
        log("workload 5 expert weights equal")


def test_swiglu_quantize_fullsize_exact():
    """The expert chain's quantization step at the layer's size: h13 [131072,
    2 x 1536] bf16 -> NVFP4 of silu(gate) * up, per-row outer scale, Four Over
    Six; every output byte against the oracle (worker pool)."""
    import _oracle_pool
    M, F = 131072, 1536
    rng = np.random.default_rng(88)
    h13 = np.empty((M, 2 * F), np.uint16)
    for r0 in range(0, M, 16384):
        h13[r0:r0 + 16384] = synth.bf16_bits((rng.standard_normal((16384, 2 * F), dtype=np.float32) * 2.0))
    log("fullsize exact: swiglu + nvfp4")
    gc, gs, go = bsq.swiglu_quantize_nvfp4(bf16_t(h13))
    gc, gs, go = h(gc), h(gs), h(go)
    R = 8192
    with _oracle_pool.pool() as ex:
        jobs = ((h13[r0:r0 + R], F) for r0 in range(0, M, R))
        for i, (oc, os_, oo) in enumerate(ex.map(_oracle_pool.swiglu_slice, jobs)):
            r0 = i * R
            assert np.array_equal(go[r0:r0 + R], oo), r0
            assert np.array_equal(gs[r0:r0 + R], os_), r0
            assert np.array_equal(gc[r0:r0 + R], oc), r0
    log("swiglu + nvfp4 rows equal")
