"""GPU parity of the combine codec (RHT-32 + block-scaled S2F6) against the
CPU oracle: encoder bytes bit for bit, combine outputs bit for bit (float32)
or as the round-to-nearest-even bf16 of the oracle's float32 result."""
import numpy as np
import pytest
import torch

import block_scaled_bit_quantize_amd as bsq
import synth
from oracle import codec as C
from oracle.route import route as oroute

from _gpu_util import DEV, bf16_t, h, log, t

pytestmark = pytest.mark.gpu
f32 = np.float32


def _rows(rng, shape, kind):
    if kind == "normal":
        return rng.standard_normal(shape).astype(f32)
    if kind == "wide":
        return (rng.standard_normal(shape) * np.exp(rng.uniform(-30, 30, shape))).astype(f32)
    if kind == "outliers":
        x = rng.standard_normal(shape).astype(f32)
        m = rng.random(shape) < 0.01
        x[m] *= f32(300.0)
        return x
    if kind == "tiny":  # float32 subnormals and values near them
        return (rng.standard_normal(shape) * np.exp2(rng.integers(-149, -120, shape).astype(np.float64))).astype(f32)
    if kind == "zeros_mix":
        x = rng.standard_normal(shape).astype(f32)
        x.reshape(-1, 32)[::3] = 0.0
        x.reshape(-1, 32)[1::5] = -0.0
        return x
    if kind == "huge":
        return (rng.standard_normal(shape) * 3e35).astype(f32)
    raise ValueError(kind)


def _dev_input(x, dtype):
    if dtype == "bf16":
        bits = synth.bf16_bits(x)
        return synth.bf16_to_f32(bits).reshape(x.shape), bf16_t(bits.reshape(x.shape))
    return x, t(x)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mask", [0, 0xDEADBEEF, 0xFFFFFFFF])
@pytest.mark.parametrize("shape,kind", [((1, 32), "normal"), ((5, 64), "wide"), ((33, 4096), "outliers"),
                                        ((7, 96), "tiny"), ((3, 160), "zeros_mix"), ((2, 64), "huge"),
                                        ((300, 320), "normal")])
def test_encode_small(dtype, mask, shape, kind):
    log(f"rht_s2f6 encode {dtype} {mask:#x} {shape} {kind}")
    rng = np.random.default_rng(hash((dtype, mask, shape, kind)) % 2**32)
    x, xd = _dev_input(_rows(rng, shape, kind), dtype)
    gc, gs = bsq.rht_s2f6_encode(xd, mask)
    oc, os_ = C.encode(x, mask)
    assert np.array_equal(h(gs), os_)
    assert np.array_equal(h(gc), oc)


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("T,k,cols,kind", [(1, 1, 32, "normal"), (5, 3, 96, "outliers"), (64, 8, 4096, "normal"),
                                           (17, 2, 64, "tiny"), (40, 8, 320, "wide")])
def test_combine_small(out, T, k, cols, kind):
    """Codes from the oracle's encoder, rows gathered through a random
    pair_row table (two entries out of range: clamped)."""
    log(f"rht_s2f6 combine {out} T={T} k={k} cols={cols} {kind}")
    rng = np.random.default_rng(hash((out, T, k, cols, kind)) % 2**32)
    mask = int(rng.integers(0, 2**32))
    R = T * k + 3
    rows = _rows(rng, (R, cols), kind)
    codes, scales = C.encode(rows, mask)
    pair_row = rng.permutation(R)[:T * k].astype(np.int32)
    if T * k >= 4:
        pair_row[1], pair_row[2] = -5, R + 3
    want = C.combine(codes, scales, np.clip(pair_row, 0, R - 1), k, mask)
    od = torch.float32 if out == "f32" else torch.bfloat16
    got = bsq.rht_s2f6_combine(t(codes), t(scales), t(pair_row), k, mask, out_dtype=od)
    if out == "f32":
        assert np.array_equal(h(got).view(np.uint32), want.view(np.uint32))
    else:
        assert np.array_equal(h(got.view(torch.int16)).view(np.uint16), synth.bf16_bits(want))


def test_codec_combine_payload_full():
    """The combine payload of the MoE layer (131072 dispatched rows of 4096,
    workload 2's routing): encoder bytes on sampled rows and combined tokens on
    sampled tokens against the oracle; the round trip of every sampled token
    within the quantization bound of its blocks."""
    log("rht_s2f6 full payload")
    T, k, H = 16384, 8, 4096
    mask = 0x9E3779B9
    rows = synth.combine_rows(T * k, H)
    ids = synth.moe_routing(2)
    _, _, pair_row = oroute(ids, 64)
    xd = bf16_t(rows)
    gc, gs = bsq.rht_s2f6_encode(xd, mask)
    out = bsq.rht_s2f6_combine(gc, gs, t(np.asarray(pair_row, np.int32)), k, mask, out_dtype=torch.float32)
    sample_rows = np.r_[0, 1, 4097, 77777, T * k - 1]
    oc, os_ = C.encode(synth.bf16_to_f32(rows[sample_rows]), mask)
    assert np.array_equal(h(gc[sample_rows]), oc) and np.array_equal(h(gs[sample_rows]), os_)
    toks = np.r_[0, 5, 9999, T - 1]
    pr = np.asarray(pair_row).reshape(T, k)[toks]                   # rows of the sampled tokens
    sub = pr.reshape(-1)
    sc, ss = C.encode(synth.bf16_to_f32(rows[sub]), mask)
    want = C.combine(sc, ss, np.arange(len(sub)), k, mask)
    got = h(out[toks])
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    exact = synth.bf16_to_f32(rows[sub]).astype(np.float64).reshape(len(toks), k, H).sum(axis=1)
    step = np.exp2(ss.astype(np.float64) - 133).reshape(len(toks), k, H // 32).sum(axis=1)
    err = np.sqrt(((got - exact) ** 2).reshape(len(toks), H // 32, 32).sum(axis=2))
    assert (err <= np.sqrt(32) / 2 * step * 1.001 + 1e-4).all()
