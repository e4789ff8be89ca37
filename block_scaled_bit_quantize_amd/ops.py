"""PyTorch-facing wrappers of the bsq_* entry points (argument marshalling
only: shapes, output allocation, device pointers, the current stream)."""
import torch

from ._lib import BsqError, check, load_library

F32, BF16 = 0, 1
OUTER_TENSOR, OUTER_ROW, OUTER_GIVEN = 0, 1, 2
FOUR_OVER_SIX = 16  # flag OR-ed into the NVFP4 quantize mode
RN, SR = 0, 1
NVFP4, MXFP8 = 0, 1

_OUTER = {"tensor": OUTER_TENSOR, "row": OUTER_ROW, "given": OUTER_GIVEN}
_RND = {"rn": RN, "sr": SR}
_FMT = {"nvfp4": NVFP4, "mxfp8": MXFP8}


def _enum(v, table):
    return table[v] if isinstance(v, str) else int(v)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _dev(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise BsqError("expected contiguous device tensors")


def _ws(nbytes, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def quantize_nvfp4(x, mode="tensor", outer_in=None, four_over_six=False):
    """Round-to-nearest NVFP4 of x [B, R, C] or [R, C] (float32 or bfloat16);
    four_over_six picks each block's scale from the 6- and 4-mapping candidates.
    Returns (codes u8 [..., C/2], scales u8 [..., C/16], outer f32 [B] or [B*R])."""
    lib = load_library()
    _dev(x, outer_in)
    squeeze = x.dim() == 2
    x3 = x.unsqueeze(0) if squeeze else x
    B, R, C = x3.shape
    dt = {torch.float32: F32, torch.bfloat16: BF16}.get(x.dtype)
    if dt is None:
        raise BsqError("x must be float32 or bfloat16")
    m = _enum(mode, _OUTER)
    flags = m | (FOUR_OVER_SIX if four_over_six else 0)
    codes = torch.empty((B, R, C // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((B, R, C // 16), dtype=torch.uint8, device=x.device)
    outer = torch.empty((B * R,) if m == OUTER_ROW else (B,), dtype=torch.float32, device=x.device)
    wsb = lib.bsq_quantize_nvfp4_workspace(B, R, C, flags)
    ws = _ws(wsb, x.device) if wsb else None
    check(lib.bsq_quantize_nvfp4(x3.data_ptr(), dt, B, R, C, flags, _ptr(outer_in), codes.data_ptr(),
                                 scales.data_ptr(), outer.data_ptr(), _ptr(ws), wsb, _stream()),
          "bsq_quantize_nvfp4")
    if squeeze:
        return codes[0], scales[0], outer
    return codes, scales, outer


def swiglu_quantize_nvfp4(h13, four_over_six=True):
    """The expert chain's quantization step: h13 [M, 2F] (float32 or bfloat16,
    gate columns first) -> NVFP4 of silu(gate) * up with per-row outer scales:
    (codes u8 [M, F/2], scales u8 [M, F/16], outer f32 [M])."""
    lib = load_library()
    _dev(h13)
    M, F2 = h13.shape
    F = F2 // 2
    dt = {torch.float32: F32, torch.bfloat16: BF16}.get(h13.dtype)
    if dt is None:
        raise BsqError("h13 must be float32 or bfloat16")
    codes = torch.empty((M, F // 2), dtype=torch.uint8, device=h13.device)
    scales = torch.empty((M, F // 16), dtype=torch.uint8, device=h13.device)
    outer = torch.empty((M,), dtype=torch.float32, device=h13.device)
    check(lib.bsq_swiglu_quantize_nvfp4(h13.data_ptr(), dt, M, F, FOUR_OVER_SIX if four_over_six else 0,
                                        codes.data_ptr(), scales.data_ptr(), outer.data_ptr(), _stream()),
          "bsq_swiglu_quantize_nvfp4")
    return codes, scales, outer


def quantize_nvfp4_square(x, mode="tensor", outer_in=None, transpose=True):
    """Square-tile NVFP4 (one scale per 16x16 tile) of x [B, R, C] or [R, C]
    (float32 or bfloat16; R and C multiples of 16); mode "tensor" or "given".
    Returns (codes [..., R, C/2], scales [..., R, C/16], outer f32 [B],
    codes_t [..., C, R/2], scales_t [..., C, R/16]); the transposed pair is
    None when transpose is False."""
    lib = load_library()
    _dev(x, outer_in)
    squeeze = x.dim() == 2
    x3 = x.unsqueeze(0) if squeeze else x
    B, R, C = x3.shape
    dt = {torch.float32: F32, torch.bfloat16: BF16}.get(x.dtype)
    if dt is None:
        raise BsqError("x must be float32 or bfloat16")
    m = _enum(mode, _OUTER)
    dev = x.device
    codes = torch.empty((B, R, C // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((B, R, C // 16), dtype=torch.uint8, device=dev)
    codes_t = torch.empty((B, C, R // 2), dtype=torch.uint8, device=dev) if transpose else None
    scales_t = torch.empty((B, C, R // 16), dtype=torch.uint8, device=dev) if transpose else None
    outer = torch.empty((B,), dtype=torch.float32, device=dev)
    wsb = lib.bsq_quantize_nvfp4_square_workspace(B, R, C, m)
    ws = _ws(wsb, dev) if wsb else None
    check(lib.bsq_quantize_nvfp4_square(x3.data_ptr(), dt, B, R, C, m, _ptr(outer_in), codes.data_ptr(),
                                        scales.data_ptr(), _ptr(codes_t), _ptr(scales_t), outer.data_ptr(),
                                        _ptr(ws), wsb, _stream()), "bsq_quantize_nvfp4_square")
    if squeeze:
        return (codes[0], scales[0], outer, codes_t[0] if transpose else None,
                scales_t[0] if transpose else None)
    return codes, scales, outer, codes_t, scales_t


def padded_segment_layout(seg_offsets_host, cols):
    """Host helper: (padded length of each segment, total elements) of the padded
    per-segment transposed layout for a host list/array of segment offsets."""
    seg = [int(v) for v in seg_offsets_host]
    mp = [(seg[e + 1] - seg[e] + 31) // 32 * 32 for e in range(len(seg) - 1)]
    return mp, cols * sum(mp)


def _segmented_capacity(rows, nseg, cols):
    # upper bound of cols * sum(pad32(M_e)); the exact size needs the offsets on the host
    return cols * (rows + 31 * nseg)


def quantize_mxfp8(x, rnd="sr", seed=0, stream_id=0, transpose=False, seg_offsets=None, out_elems=None):
    """MXFP8 of x [R, C] (float32 or bfloat16). transpose=False: codes [R, C],
    scales [R, C/32]. transpose=True: flat codes / scales in the padded
    per-segment transposed layout (seg_offsets: int64 device [E+1] or None for
    one segment); out_elems (optional) sets the exact output length."""
    lib = load_library()
    _dev(x, seg_offsets)
    R, C = x.shape
    dt = {torch.float32: F32, torch.bfloat16: BF16}.get(x.dtype)
    if dt is None:
        raise BsqError("x must be float32 or bfloat16")
    r = _enum(rnd, _RND)
    if not transpose:
        codes = torch.empty((R, C), dtype=torch.uint8, device=x.device)
        scales = torch.empty((R, C // 32), dtype=torch.uint8, device=x.device)
        check(lib.bsq_quantize_mxfp8(x.data_ptr(), dt, R, C, 0, None, 0, r, seed, stream_id, codes.data_ptr(),
                                     scales.data_ptr(), None, 0, _stream()), "bsq_quantize_mxfp8")
        return codes, scales
    nseg = seg_offsets.numel() - 1 if seg_offsets is not None else 1
    n = out_elems if out_elems is not None else _segmented_capacity(R, nseg, C)
    codes = torch.empty((n,), dtype=torch.uint8, device=x.device)
    scales = torch.empty((n // 32,), dtype=torch.uint8, device=x.device)
    wsb = lib.bsq_quantize_mxfp8_workspace(R, 1, nseg)
    ws = _ws(wsb, x.device)
    check(lib.bsq_quantize_mxfp8(x.data_ptr(), dt, R, C, 1, _ptr(seg_offsets), nseg if seg_offsets is not None else 0,
                                 r, seed, stream_id, codes.data_ptr(), scales.data_ptr(), ws.data_ptr(), wsb,
                                 _stream()), "bsq_quantize_mxfp8")
    return codes, scales


def quantize_mxfp8_dual(x, rnd="sr", seed=0, stream_rows=0, stream_t=0, seg_offsets=None, out_elems=None):
    """Both MXFP8 quantizations of x [R, C] from one read: ((codes [R, C],
    scales [R, C/32]) as quantize_mxfp8(transpose=False, stream_id=stream_rows),
    (codes_t, scales_t) as quantize_mxfp8(transpose=True, stream_id=stream_t))."""
    lib = load_library()
    _dev(x, seg_offsets)
    R, C = x.shape
    dt = {torch.float32: F32, torch.bfloat16: BF16}.get(x.dtype)
    if dt is None:
        raise BsqError("x must be float32 or bfloat16")
    r = _enum(rnd, _RND)
    nseg = seg_offsets.numel() - 1 if seg_offsets is not None else 1
    n = out_elems if out_elems is not None else _segmented_capacity(R, nseg, C)
    codes = torch.empty((R, C), dtype=torch.uint8, device=x.device)
    scales = torch.empty((R, C // 32), dtype=torch.uint8, device=x.device)
    codes_t = torch.empty((n,), dtype=torch.uint8, device=x.device)
    scales_t = torch.empty((n // 32,), dtype=torch.uint8, device=x.device)
    wsb = lib.bsq_quantize_mxfp8_workspace(R, 1, nseg)
    ws = _ws(wsb, x.device)
    check(lib.bsq_quantize_mxfp8_dual(x.data_ptr(), dt, R, C, _ptr(seg_offsets),
                                      nseg if seg_offsets is not None else 0, r, seed, stream_rows, stream_t,
                                      codes.data_ptr(), scales.data_ptr(), codes_t.data_ptr(), scales_t.data_ptr(),
                                      ws.data_ptr(), wsb, _stream()), "bsq_quantize_mxfp8_dual")
    return (codes, scales), (codes_t, scales_t)


def requant_transpose_sr(codes, scales, outer, in_mode, out_fmt="mxfp8", seed=0, stream_id=0, rnd="sr",
                         row_gather=None, seg_offsets=None, out_elems=None):
    """Dequantize -> transpose -> requantize.
    Batch mode: codes [B, R, C/2] (or [R, C/2]) -> output [B, C, R] codes
    (MXFP8 [B, C, R] bytes, NVFP4 [B, C, R/2]) and scales; NVFP4 also returns
    the new outer scales [B].
    Gather mode (row_gather int32 [rows], seg_offsets int64 [E+1]): input
    [T, C/2], output flat padded per-segment transposed MXFP8."""
    lib = load_library()
    _dev(codes, scales, outer, row_gather, seg_offsets)
    im = _enum(in_mode, _OUTER)
    fmt = _enum(out_fmt, _FMT)
    r = _enum(rnd, _RND)
    dev = codes.device
    if row_gather is not None:
        T, C2 = codes.shape
        C = 2 * C2
        rows = row_gather.numel()
        nseg = seg_offsets.numel() - 1
        n = out_elems if out_elems is not None else _segmented_capacity(rows, nseg, C)
        oc = torch.empty((n,), dtype=torch.uint8, device=dev)
        osc = torch.empty((n // 32,), dtype=torch.uint8, device=dev)
        wsb = lib.bsq_requant_workspace(1, rows, nseg, fmt, 1)
        ws = _ws(wsb, dev)
        check(lib.bsq_requant_transpose_sr(codes.data_ptr(), scales.data_ptr(), outer.data_ptr(), im, 1, rows, C, T,
                                           row_gather.data_ptr(), seg_offsets.data_ptr(), nseg, fmt, r, seed,
                                           stream_id, oc.data_ptr(), osc.data_ptr(), None, ws.data_ptr(), wsb,
                                           _stream()), "bsq_requant_transpose_sr")
        return oc, osc
    squeeze = codes.dim() == 2
    c3 = codes.unsqueeze(0) if squeeze else codes
    B, R, C2 = c3.shape
    C = 2 * C2
    if fmt == MXFP8:
        oc = torch.empty((B, C, R), dtype=torch.uint8, device=dev)
        osc = torch.empty((B, C, R // 32), dtype=torch.uint8, device=dev)
        oo = None
    else:
        oc = torch.empty((B, C, R // 2), dtype=torch.uint8, device=dev)
        osc = torch.empty((B, C, R // 16), dtype=torch.uint8, device=dev)
        oo = torch.empty((B,), dtype=torch.float32, device=dev)
    wsb = lib.bsq_requant_workspace(B, R, 0, fmt, 0)
    ws = _ws(wsb, dev) if wsb else None
    check(lib.bsq_requant_transpose_sr(c3.data_ptr(), scales.data_ptr(), outer.data_ptr(), im, B, R, C, B * R, None,
                                       None, 0, fmt, r, seed, stream_id, oc.data_ptr(), osc.data_ptr(), _ptr(oo),
                                       _ptr(ws), wsb, _stream()), "bsq_requant_transpose_sr")
    if squeeze:
        oc, osc = oc[0], osc[0]
    return (oc, osc) if fmt == MXFP8 else (oc, osc, oo)


_OUT = {torch.bfloat16: BF16, torch.float32: F32}


def grouped_gemm_nvfp4(a_codes, a_scales, a_outer, b_codes, b_scales, b_outer, seg_offsets, M_total,
                       row_index=None, out=None, out_dtype=torch.bfloat16):
    """y [M_total, N] = per expert, gathered x_q rows times w_q^T with both
    outer scales (bf16 or float32 output). a_*: [T, K/2], [T, K/16], a_outer
    [T] (per token) or [1]; b_*: [E, N, K/2], [E, N, K/16], b_outer [E]."""
    lib = load_library()
    _dev(a_codes, a_scales, a_outer, b_codes, b_scales, b_outer, seg_offsets, row_index)
    T, K2 = a_codes.shape
    E, N, _ = b_codes.shape
    per_row = 1 if a_outer.numel() == T and T > 1 else 0
    if out is None:
        out = torch.empty((M_total, N), dtype=out_dtype, device=a_codes.device)
    check(lib.bsq_grouped_gemm_nvfp4(a_codes.data_ptr(), a_scales.data_ptr(), a_outer.data_ptr(), per_row, T,
                                     _ptr(row_index), b_codes.data_ptr(), b_scales.data_ptr(), b_outer.data_ptr(),
                                     seg_offsets.data_ptr(), E, M_total, N, 2 * K2, out.data_ptr(), _OUT[out.dtype],
                                     _stream()), "bsq_grouped_gemm_nvfp4")
    return out


def grouped_gemm_nvfp4_s2f6(a_codes, a_scales, a_outer, b_codes, b_scales, b_outer, seg_offsets, M_total, signs,
                            row_index=None):
    """The w2 GEMM with the combine codec in its epilogue: the product of
    grouped_gemm_nvfp4, RHT-rotated and S2F6-quantized per 32 columns ->
    (codes u8 [M_total, N], scales u8 [M_total, N/32])."""
    lib = load_library()
    _dev(a_codes, a_scales, a_outer, b_codes, b_scales, b_outer, seg_offsets, row_index)
    T, K2 = a_codes.shape
    E, N, _ = b_codes.shape
    per_row = 1 if a_outer.numel() == T and T > 1 else 0
    codes = torch.empty((M_total, N), dtype=torch.uint8, device=a_codes.device)
    scales = torch.empty((M_total, N // 32), dtype=torch.uint8, device=a_codes.device)
    check(lib.bsq_grouped_gemm_nvfp4_s2f6(a_codes.data_ptr(), a_scales.data_ptr(), a_outer.data_ptr(), per_row, T,
                                          _ptr(row_index), b_codes.data_ptr(), b_scales.data_ptr(),
                                          b_outer.data_ptr(), seg_offsets.data_ptr(), E, M_total, N, 2 * K2,
                                          signs & 0xFFFFFFFF, codes.data_ptr(), scales.data_ptr(), _stream()),
          "bsq_grouped_gemm_nvfp4_s2f6")
    return codes, scales


def grouped_gemm_mxfp8(wgrad, a_codes, a_scales, b_codes, b_scales, seg_offsets, M, N, K=0, out=None,
                       out_dtype=None):
    """wgrad=False (DGRAD): a [M_total(=M), K], b [E, N, K] -> [M, N] (bf16
    by default). wgrad=True (WGRAD): a, b flat padded per-segment transposed
    layouts with M and N rows per expert -> [E, M, N] (float32 by default)."""
    lib = load_library()
    _dev(a_codes, a_scales, b_codes, b_scales, seg_offsets)
    E = seg_offsets.numel() - 1
    if out is None:
        dt = out_dtype or (torch.float32 if wgrad else torch.bfloat16)
        shape = (E, M, N) if wgrad else (M, N)
        out = torch.empty(shape, dtype=dt, device=a_codes.device)
    check(lib.bsq_grouped_gemm_mxfp8(1 if wgrad else 0, a_codes.data_ptr(), a_scales.data_ptr(), b_codes.data_ptr(), b_scales.data_ptr(),
             seg_offsets.data_ptr(), E, M, N, K, out.data_ptr(), _OUT[out.dtype], _stream()), "bsq_grouped_gemm_mxfp8")
    return out


def gemm_nvfp4_inreg_scale(a_codes, a_scales, a_outer, b_codes, b_scales, b_outer):
    """Dense NVFP4 product with the block scales applied in registers (FP8
    MFMA per 16-value block, fp32 scaling): a_* [M, K/2], [M, K/16], [M];
    b_* [N, K/2], [N, K/16], [1] -> float32 [M, N]. The alternative to the
    exact 16-bit decode of grouped_gemm_nvfp4, kept for comparison."""
    lib = load_library()
    _dev(a_codes, a_scales, a_outer, b_codes, b_scales, b_outer)
    M, N, K = a_codes.shape[0], b_codes.shape[0], 2 * a_codes.shape[1]
    out = torch.empty((M, N), dtype=torch.float32, device=a_codes.device)
    check(lib.bsq_gemm_nvfp4_inreg_scale(a_codes.data_ptr(), a_scales.data_ptr(), a_outer.data_ptr(),
                                         b_codes.data_ptr(), b_scales.data_ptr(), b_outer.data_ptr(), M, N, K,
                                         out.data_ptr(), _stream()), "bsq_gemm_nvfp4_inreg_scale")
    return out


def route(topk_ids, num_experts):
    """topk_ids int32 [T, k] -> (row_index int32 [T*k], seg_offsets int64 [E+1], pair_row int32 [T*k])."""
    lib = load_library()
    _dev(topk_ids)
    T, k = topk_ids.shape
    dev = topk_ids.device
    row_index = torch.empty((T * k,), dtype=torch.int32, device=dev)
    pair_row = torch.empty((T * k,), dtype=torch.int32, device=dev)
    seg = torch.empty((num_experts + 1,), dtype=torch.int64, device=dev)
    wsb = lib.bsq_route_workspace(T, num_experts)
    ws = _ws(wsb, dev) if wsb else None
    check(lib.bsq_route(topk_ids.data_ptr(), T, k, num_experts, row_index.data_ptr(), seg.data_ptr(),
                        pair_row.data_ptr(), _ptr(ws), wsb, _stream()), "bsq_route")
    return row_index, seg, pair_row


def route_noalloc(topk_ids, num_experts, row_index, seg_offsets, pair_row):
    """route() into caller-provided outputs with no device allocation: the
    library's own per-GPU array holds the per-chunk counts (tokens x E up to
    the 1 MiB limit of BSQ_ROUTE_NOALLOC_MAX_BYTES). Calls on one GPU that
    overlap in time race."""
    lib = load_library()
    _dev(topk_ids, row_index, seg_offsets, pair_row)
    T, k = topk_ids.shape
    if row_index.numel() != T * k or pair_row.numel() != T * k or seg_offsets.numel() != num_experts + 1:
        raise BsqError("route_noalloc: output sizes do not match topk_ids and num_experts")
    check(lib.bsq_route_noalloc(topk_ids.data_ptr(), T, k, num_experts, row_index.data_ptr(), seg_offsets.data_ptr(),
                                pair_row.data_ptr(), _stream()), "bsq_route_noalloc")
    return row_index, seg_offsets, pair_row


def rht_s2f6_encode(x, signs):
    """Combine-codec sender: x [R, C] (float32 or bfloat16, C % 32 == 0) ->
    (codes u8 [R, C] two's-complement S2F6, scales u8 [R, C/32] UE8M0) of the
    rows rotated by the 32-point Hadamard transform with sign mask `signs`."""
    lib = load_library()
    _dev(x)
    R, C = x.shape
    dt = {torch.float32: F32, torch.bfloat16: BF16}.get(x.dtype)
    if dt is None:
        raise BsqError("x must be float32 or bfloat16")
    codes = torch.empty((R, C), dtype=torch.uint8, device=x.device)
    scales = torch.empty((R, C // 32), dtype=torch.uint8, device=x.device)
    check(lib.bsq_rht_s2f6_encode(x.data_ptr(), dt, R, C, signs & 0xFFFFFFFF, codes.data_ptr(), scales.data_ptr(),
                                  _stream()), "bsq_rht_s2f6_encode")
    return codes, scales


def rht_s2f6_combine(codes, scales, pair_row, k, signs, out_dtype=torch.bfloat16):
    """Combine-codec receiver: token t sums the dequantized rows
    pair_row[t*k + j] (int32 [T*k]) and inverts the transform -> [T, C]."""
    lib = load_library()
    _dev(codes, scales, pair_row)
    R, C = codes.shape
    T = pair_row.numel() // k
    od = {torch.float32: F32, torch.bfloat16: BF16}.get(out_dtype)
    if od is None:
        raise BsqError("out_dtype must be float32 or bfloat16")
    out = torch.empty((T, C), dtype=out_dtype, device=codes.device)
    check(lib.bsq_rht_s2f6_combine(codes.data_ptr(), scales.data_ptr(), R, C, pair_row.data_ptr(), T, k,
                                   signs & 0xFFFFFFFF, out.data_ptr(), od, _stream()), "bsq_rht_s2f6_combine")
    return out


def dequantize_nvfp4(codes, scales, outer, mode="tensor"):
    lib = load_library()
    _dev(codes, scales, outer)
    squeeze = codes.dim() == 2
    c3 = codes.unsqueeze(0) if squeeze else codes
    B, R, C2 = c3.shape
    out = torch.empty((B, R, 2 * C2), dtype=torch.float32, device=codes.device)
    check(lib.bsq_dequantize_nvfp4(c3.data_ptr(), scales.data_ptr(), outer.data_ptr(), _enum(mode, _OUTER), B, R,
                                   2 * C2, out.data_ptr(), _stream()), "bsq_dequantize_nvfp4")
    return out[0] if squeeze else out


def dequantize_mxfp8(codes, scales):
    lib = load_library()
    _dev(codes, scales)
    R, C = codes.shape
    out = torch.empty((R, C), dtype=torch.float32, device=codes.device)
    check(lib.bsq_dequantize_mxfp8(codes.data_ptr(), scales.data_ptr(), R, C, out.data_ptr(), _stream()),
          "bsq_dequantize_mxfp8")
    return out


def rng_bits16(seed, stream_id, first, n, device="cuda"):
    lib = load_library()
    out = torch.empty((n,), dtype=torch.int16, device=device)
    check(lib.bsq_rng_bits16(seed, stream_id, first, n, out.data_ptr(), _stream()), "bsq_rng_bits16")
    return out


def mfma_rate_probe(kind, data, iters, workgroups, device="cuda"):
    """Launch the per-instruction MFMA throughput probe (see bsq.h) and
    return its output tensor [workgroups * 256]; the caller times the launch."""
    lib = load_library()
    out = torch.empty((workgroups * 256,), dtype=torch.float32, device=device)
    check(lib.bsq_mfma_rate_probe(kind, data, iters, workgroups, out.data_ptr(), _stream()), "bsq_mfma_rate_probe")
    return out
