"""Pins of the expert-chain oracle: its float32 exp and SwiGLU against float64
closed forms, and the whole quantized chain against an unquantized float64
MoE forward."""
import math

import numpy as np
import pytest

from oracle import chain as CH
from oracle import codec as CODEC
from oracle import quant as Q
from oracle.route import route

f32 = np.float32


def test_exp_constants():
    assert math.log(2.0).hex() == "0x1.62e42fefa39efp-1"          # the double nearest to ln 2
    assert float(CH.LN2_HI) == 0.693145751953125 and (CH.LN2_HI.view(np.uint32) & 0xFF) == 0
    assert abs(float(CH.LN2_HI) + float(CH.LN2_LO) - math.log(2.0)) < 2.0 ** -40
    for k, c in enumerate(CH.EXP_TAYLOR):
        assert c == f32(1.0 / math.factorial(k))


def test_exp_within_two_ulp_of_float64():
    x = np.concatenate([np.linspace(-87.0, 88.0, 300001), np.linspace(-1, 1, 20001)]).astype(f32)
    e = CH.exp_f32(x).astype(np.float64)
    r = np.exp(x.astype(np.float64))
    ulp = np.spacing(r.astype(f32)).astype(np.float64)
    assert (np.abs(e - r) <= 2 * ulp).all()
    assert CH.exp_f32(f32(0.0)) == 1.0
    assert CH.exp_f32(f32(-120.0)) == f32(np.exp(-120.0)) or abs(CH.exp_f32(f32(-120.0)) - np.exp(-120.0)) < 2e-45
    assert np.isinf(CH.exp_f32(f32(100.0))) and CH.exp_f32(f32(-200.0)) == 0.0


def test_silu_closed_form_and_identities():
    g = np.concatenate([np.linspace(-60, 60, 100001), [0.0, 1e-30, -1e-30]]).astype(f32)
    s = CH.silu_f32(g).astype(np.float64)
    gd = g.astype(np.float64)
    want = gd / (1.0 + np.exp(-gd))
    assert (np.abs(s - want) <= 4 * np.spacing(np.abs(want).astype(f32)).astype(np.float64) + 1e-44).all()
    assert CH.silu_f32(f32(0.0)) == 0.0 and CH.silu_f32(f32(40.0)) == 40.0
    assert CH.silu_f32(f32(-200.0)) == 0.0
    # silu(x) - silu(-x) = x
    s2 = CH.silu_f32(-g).astype(np.float64)
    assert np.allclose(s - s2, gd, rtol=1e-6, atol=1e-30)


def test_swiglu_layout_gate_then_up():
    """Columns [0, F) are the gate, [F, 2F) the up projection: a large gate
    passes the up values through (silu(g) ~ g), a zero gate zeroes them."""
    rng = np.random.default_rng(0)
    F = 48
    up = rng.standard_normal((4, F)).astype(f32)
    gate = np.zeros((4, F), f32)
    gate[0] = 30.0
    h = CH.swiglu_f32(np.concatenate([gate, up], axis=1), F)
    assert np.allclose(h[0], 30.0 * up[0], rtol=1e-6)
    assert (h[1:] == 0).all()


def _moe_f64(x, topk_ids, w13, w2):
    """Unquantized float64 MoE forward: out[t] = sum_j w2_e (silu(g) * u)."""
    E, F2, H = w13.shape
    F = F2 // 2
    out = np.zeros((x.shape[0], w2.shape[1]))
    for t in range(x.shape[0]):
        for e in topk_ids[t]:
            h13 = w13[e].astype(np.float64) @ x[t].astype(np.float64)
            g, u = h13[:F], h13[F:]
            out[t] += w2[e].astype(np.float64) @ (g / (1 + np.exp(-g)) * u)
    return out


@pytest.mark.parametrize("seed", [0, 1])
def test_chain_against_float64_moe(seed):
    """The quantized chain against float64 forwards of the same MoE. With the
    chain's own dequantized x, w13 and w2 the remaining error is one NVFP4
    rounding of h (about 8% relative RMS for such data) plus the S2F6 codec:
    below 12%. Against the unquantized MoE it is below 30%, while a reference
    with the gate and up halves exchanged is off by more than 50%."""
    rng = np.random.default_rng(seed)
    T, H, F, E, k = 64, 128, 64, 4, 2
    x = rng.standard_normal((T, H)).astype(f32)
    w13 = (rng.standard_normal((E, 2 * F, H)) * 0.1).astype(f32)
    w2 = (rng.standard_normal((E, H, F)) * 0.1).astype(f32)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    r = CH.expert_forward(x, ids, w13, w2, 0x0F0F1234)
    rel = lambda a, b: np.linalg.norm(a - b) / np.linalg.norm(b)
    xd = Q.dequantize_nvfp4_f64(r["x_q"][0][None], r["x_q"][1][None], r["x_q"][2][None], Q.OUTER_ROW)[0]
    w13d = Q.dequantize_nvfp4_f64(*r["w13_q"], Q.OUTER_TENSOR)
    w2d = Q.dequantize_nvfp4_f64(*r["w2_q"], Q.OUTER_TENSOR)
    assert rel(r["out"], _moe_f64(xd, ids, w13d, w2d)) < 0.12
    assert rel(r["out"], _moe_f64(x, ids, w13, w2)) < 0.30
    swapped = _moe_f64(x, ids, np.concatenate([w13[:, F:], w13[:, :F]], axis=1), w2)
    assert rel(r["out"], swapped) > 0.5
    # the intermediates hang together: the combine of the codec bytes is the output
    row_index, seg, pair_row = route(ids, E)
    assert np.array_equal(r["pair_row"], pair_row)
    assert np.array_equal(CODEC.combine(r["codes"], r["scales"], pair_row, k, 0x0F0F1234), r["out"])
