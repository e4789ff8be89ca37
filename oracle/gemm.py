"""float64 references for the expert GEMMs.

Page: "End-to-End 4-Bit Training", section "Block-scaled backward passes":
the forward pass computes y = x_q w_q^T, and an NVFP4 dot product pairs
16-value blocks of a row of x_q and a column of w_q^T, multiplies the pairs
and multiplies each block sum by the two block scales; the backward pass
computes dx = g w_q (DGRAD) and dw = g^T x_q (WGRAD), in MXFP8 (quantized
linear layer figure).  Section "Quantized communications": tokens are routed
to experts, so the forward GEMM runs per expert over that expert's tokens.

The reference is the exact product of the dequantized operands evaluated in
float64 (a library matmul of float64 operands; every operand value is exact
in float64).  The accept rule (reading, because a bf16 output alone can be
off by 2^-9 relative and a literal relative bound fails where the exact
result is near zero):
    |y - y_ref| <= 2e-3 * |y_ref| + 2^-20 * sum_k |x_k w_k|
"""
import numpy as np

from .quant import (OUTER_ROW, OUTER_TENSOR, dequantize_mxfp8_f64,
                    dequantize_nvfp4_f64, segmented_layout)

REL_TOL = 2e-3
ABS_FLOOR = 2.0 ** -20


def grouped_gemm_nvfp4_ref(a_packed, a_scales, a_outer, row_index, b_packed, b_scales, b_outer,
                           seg_offsets, rows=None):
    """y[r, n] = sum_k x^[tok(r), k] * w^_e[n, k] for dispatched row r of expert e.
    a_*: NVFP4 [T, K] with per-token outer scales a_outer [T]; b_*: NVFP4
    [E, N, K] with per-expert outer scales b_outer [E]; row_index [M_total]
    maps a dispatched row to its token (None = identity).  ``rows`` selects
    the output rows to compute (default all).  Returns (y_ref, sum|x w|)."""
    a_packed = np.asarray(a_packed)
    a_scales = np.asarray(a_scales)
    a_outer = np.asarray(a_outer, dtype=np.float32).reshape(-1)
    T = a_packed.shape[0]
    if a_outer.size == 1 and T > 1:                  # one outer scale for the whole activation tensor
        a_outer = np.full(T, a_outer[0], dtype=np.float32)
    seg = np.asarray(seg_offsets, dtype=np.int64)
    M_total = int(seg[-1])
    rows = np.arange(M_total) if rows is None else np.asarray(rows, dtype=np.int64)
    tok = rows if row_index is None else np.asarray(row_index, dtype=np.int64)[rows]
    expert = np.searchsorted(seg, rows, side="right") - 1
    N = np.asarray(b_packed).shape[1]
    y = np.zeros((len(rows), N))
    ya = np.zeros((len(rows), N))
    for e in np.unique(expert):
        sel = expert == e
        t = tok[sel]
        # dequantize only the rows and the expert this output block needs
        xa = dequantize_nvfp4_f64(a_packed[t][None], a_scales[t][None], a_outer[t].reshape(1, -1), OUTER_ROW)[0]
        we = dequantize_nvfp4_f64(np.asarray(b_packed)[e:e + 1], np.asarray(b_scales)[e:e + 1],
                                  np.asarray(b_outer)[e:e + 1], OUTER_TENSOR)[0]
        y[sel] = xa @ we.T
        ya[sel] = np.abs(xa) @ np.abs(we).T
    return y, ya


def mxfp8_dgrad_ref(a_codes, a_scales, b_codes, b_scales, seg_offsets, rows=None):
    """DGRAD dx[r, n] = sum_k g^[r, k] * w^T_e[n, k]: A = g MXFP8 [M_total, K]
    (blocks along K), B = w^T MXFP8 [E, N, K]; row r belongs to expert e by
    seg_offsets."""
    a_codes = np.asarray(a_codes); a_scales = np.asarray(a_scales)
    b_codes = np.asarray(b_codes); b_scales = np.asarray(b_scales)
    seg = np.asarray(seg_offsets, dtype=np.int64)
    rows = np.arange(int(seg[-1])) if rows is None else np.asarray(rows, dtype=np.int64)
    expert = np.searchsorted(seg, rows, side="right") - 1
    y = np.zeros((len(rows), b_codes.shape[1]))
    ya = np.zeros_like(y)
    for e in np.unique(expert):
        sel = expert == e
        ga = dequantize_mxfp8_f64(a_codes[rows[sel]], a_scales[rows[sel]])
        we = dequantize_mxfp8_f64(b_codes[e], b_scales[e])
        y[sel] = ga @ we.T
        ya[sel] = np.abs(ga) @ np.abs(we).T
    return y, ya


def mxfp8_wgrad_ref(a_codes, a_scales, b_codes, b_scales, seg_offsets, M, N, experts=None):
    """WGRAD dw_e[m, n] = sum_t g^T_e[m, t] * x^T_e[n, t] with both operands in
    the per-segment transposed MXFP8 layout (A: [M, Mp_e], B: [N, Mp_e] for
    each expert, blocks along tokens, zero padding).  Returns [E', M, N] for
    the selected experts (default all) and the matching sum|.|."""
    seg = np.asarray(seg_offsets, dtype=np.int64)
    E = len(seg) - 1
    mpa, basea = segmented_layout(seg, M)
    mpb, baseb = segmented_layout(seg, N)
    experts = range(E) if experts is None else experts
    outs, outa = [], []
    a_codes = np.asarray(a_codes); b_codes = np.asarray(b_codes)
    a_scales = np.asarray(a_scales); b_scales = np.asarray(b_scales)
    for e in experts:
        kp = mpa[e]
        A = dequantize_mxfp8_f64(a_codes[basea[e]:basea[e] + M * kp].reshape(M, kp),
                                 a_scales[basea[e] // 32:(basea[e] + M * kp) // 32].reshape(M, kp // 32))
        B = dequantize_mxfp8_f64(b_codes[baseb[e]:baseb[e] + N * kp].reshape(N, kp),
                                 b_scales[baseb[e] // 32:(baseb[e] + N * kp) // 32].reshape(N, kp // 32))
        outs.append(A @ B.T)
        outa.append(np.abs(A) @ np.abs(B).T)
    return np.array(outs).reshape(-1, M, N), np.array(outa).reshape(-1, M, N)


def within_tolerance(y, y_ref, y_abs, abs_floor=ABS_FLOOR):
    """Element-wise accept rule; returns (all_ok, worst excess ratio).
    ``abs_floor`` replaces 2^-20 for a product computed on hardware whose
    accumulation is known to be coarser (stated where it is used)."""
    y = np.asarray(y, dtype=np.float64)
    bound = REL_TOL * np.abs(y_ref) + abs_floor * y_abs
    err = np.abs(y - y_ref)
    ratio = np.max(err / np.maximum(bound, 1e-300)) if err.size else 0.0
    return bool(np.all(err <= bound)), float(ratio)


def max_rel_error(y, y_ref):
    """Largest literal relative error over elements with |y_ref| at least
    2^-10 of the rms of y_ref (reported next to the accept rule)."""
    y = np.asarray(y, dtype=np.float64)
    if y_ref.size == 0:
        return 0.0
    rms = np.sqrt(np.mean(y_ref ** 2))
    sel = np.abs(y_ref) >= rms * 2.0 ** -10
    if not np.any(sel):
        return 0.0
    return float(np.max(np.abs(y[sel] - y_ref[sel]) / np.abs(y_ref[sel])))
