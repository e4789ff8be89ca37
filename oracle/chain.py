"""The expert forward chain of the MoE layer, composed from the pinned
quantizers, GEMM reference, routing and combine codec. Test infrastructure
only (tests, smoke and the benchmark's CPU baseline use it).

Page: "End-to-End 4-Bit Training", section "Quantized communications" and its
Figure 5: tokens are dispatched to their experts, each expert runs the w13
GEMM, a quantization step and the w2 GEMM, and the outputs are combined; the
RHT and S2F6 quantization run in the w2 GEMM's epilogue and the receiver
dequantizes, aggregates and inverts the RHT. The quantized linear layer
figure (Figure 4): NVFP4 GEMMs in the forward pass, activations quantized per
token (section "Recipe details", with Four Over Six), weights per expert.

Readings (the pages leave these open):
  * w13 holds the gate projection (output columns [0, F)) above the up
    projection (columns [F, 2F)); the activation between w13 and w2 is SwiGLU,
    h = silu(gate) * up, silu(g) = g / (1 + exp(-g)), in float32.
  * exp is evaluated in float32 with Cody and Waite's argument reduction:
    n = round-half-even(f32(x * f32(1/ln 2))) clamped to [-300, 300],
    r = f32(f32(x - n ln2_hi) - f32(n ln2_lo)) (ln2_hi = 0.693145751953125, so
    n ln2_hi is exact), e^r by its degree-7 Taylor polynomial in Horner form with
    every product and sum rounded to float32 (no fused operations), then
    scaled by 2^n; so that the GPU, computing the same steps, reaches the same
    quantization decisions (the precision of the kernel; the pages fix none).
  * The w13 output is rounded to bf16 (the GEMM's output type) before the
    activation; h is quantized to NVFP4 per dispatched row (a token's copy)
    with Four Over Six; w2's float32 output goes straight into the codec.
"""
import math

import numpy as np

from . import codec as CODEC
from .gemm import grouped_gemm_nvfp4_ref
from .quant import OUTER_ROW, OUTER_TENSOR, quantize_nvfp4
from .route import route

F32 = np.float32
LN2 = math.log(2.0)                         # the double nearest to ln 2
LOG2E = F32(1.0 / LN2)
LN2_HI = F32(0.693145751953125)             # ln 2 to 16 significant bits: n * LN2_HI is exact
LN2_LO = F32(LN2 - 0.693145751953125)


def _exp_taylor():
    """e^r = sum_k r^k / k!: c_k = 1/k!, k = 0..7, formed in double precision
    by c_k = c_(k-1) / k, then rounded to float32."""
    c = [1.0]
    for k in range(1, 8):
        c.append(c[-1] / k)
    return [F32(v) for v in c]


EXP_TAYLOR = _exp_taylor()


def exp_f32(x):
    """e^x in float32 by the steps in the module docstring."""
    x = np.asarray(x, dtype=F32)
    n = np.rint((x * LOG2E).astype(F32)).astype(F32)
    n = np.clip(n, F32(-300), F32(300))
    r = (x - (n * LN2_HI).astype(F32)).astype(F32)
    r = (r - (n * LN2_LO).astype(F32)).astype(F32)
    p = np.full(x.shape, EXP_TAYLOR[7], dtype=F32)
    for c in EXP_TAYLOR[6::-1]:
        p = ((p * r).astype(F32) + c).astype(F32)
    with np.errstate(over="ignore", under="ignore"):
        return np.ldexp(p, n.astype(np.int64)).astype(F32)


def silu_f32(g):
    g = np.asarray(g, dtype=F32)
    with np.errstate(over="ignore"):
        d = (F32(1.0) + exp_f32(-g)).astype(F32)
    return (g / d).astype(F32)


def swiglu_f32(h13, F):
    """h13 float32 [M, 2F] -> float32 [M, F]: silu(gate) * up."""
    h13 = np.asarray(h13, dtype=F32)
    return (silu_f32(h13[:, :F]) * h13[:, F:2 * F]).astype(F32)


def bf16_round(v):
    """float32 -> nearest bfloat16 value (ties to even), as float32."""
    b = np.ascontiguousarray(v, dtype=F32).view(np.uint32).astype(np.uint64)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return b.astype(np.uint32).view(F32)


def swiglu_quantize(h13, F):
    """The chain's quantization step: SwiGLU, then per-row NVFP4 with Four
    Over Six. Returns (codes [M, F/2], scales [M, F/16], outer [M])."""
    h = swiglu_f32(h13, F)
    c, s, o = quantize_nvfp4(h[None], OUTER_ROW, four_over_six=True)
    return c[0], s[0], np.asarray(o).reshape(-1)


def expert_forward(x, topk_ids, w13, w2, signs):
    """Figure 5 on one GPU's experts. x float32 [T, H]; topk_ids int [T, k];
    w13 float32 [E, 2F, H]; w2 float32 [E, H, F]. Returns a dict with every
    intermediate: routing, quantized operands, h13 (bf16 values), h_q, the w2
    output y (float64 reference), the codec bytes and the combined output."""
    x = np.asarray(x, dtype=F32)
    E, F2, H = np.asarray(w13).shape
    F = F2 // 2
    k = np.asarray(topk_ids).shape[1]
    row_index, seg, pair_row = route(topk_ids, E)
    xc, xs, xo = quantize_nvfp4(x[None], OUTER_ROW, four_over_six=True)
    w13c, w13s, w13o = quantize_nvfp4(w13, OUTER_TENSOR)
    w2c, w2s, w2o = quantize_nvfp4(w2, OUTER_TENSOR)
    h13, _ = grouped_gemm_nvfp4_ref(xc[0], xs[0], np.asarray(xo).reshape(-1), row_index, w13c, w13s, w13o, seg)
    h13 = bf16_round(h13.astype(F32))
    hc, hs, ho = swiglu_quantize(h13, F)
    y, y_abs = grouped_gemm_nvfp4_ref(hc, hs, ho, None, w2c, w2s, w2o, seg)
    codes, scales = CODEC.encode(y.astype(F32), signs)
    out = CODEC.combine(codes, scales, pair_row, k, signs)
    return dict(row_index=row_index, seg=seg, pair_row=pair_row, x_q=(xc[0], xs[0], np.asarray(xo).reshape(-1)),
                w13_q=(w13c, w13s, w13o), w2_q=(w2c, w2s, w2o), h13=h13, h_q=(hc, hs, ho), y=y, y_abs=y_abs,
                codes=codes, scales=scales, out=out)
