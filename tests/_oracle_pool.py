"""Process-pool helper for the full-size comparisons: the oracle's NVFP4
quantizer on slices of bf16 inputs (NumPy only; the workers never touch the
GPU)."""
import os

import synth
from oracle import quant as Q


def nvfp4_slice(args):
    """(bf16 bits [rows, C] or [items, rows, C], 'row' | 'tensor', four_over_six)
    -> the oracle's (codes, scales, outer) of the slice."""
    bits, mode, fos = args
    x = synth.bf16_to_f32(bits)
    if mode == "row":
        return Q.quantize_nvfp4(x[None], Q.OUTER_ROW, four_over_six=fos)
    return Q.quantize_nvfp4(x, Q.OUTER_TENSOR, four_over_six=fos)


def pool():
    """A spawn-context pool sized to the host's CPU share (at most 16)."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    return ProcessPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1)), mp_context=mp.get_context("spawn"))


def swiglu_slice(args):
    """(bf16 bits of h13 [rows, 2F], F) -> the oracle's SwiGLU + NVFP4 (Four
    Over Six) of the slice: (codes, scales, outer)."""
    from oracle import chain as CH
    bits, F = args
    return CH.swiglu_quantize(synth.bf16_to_f32(bits), F)
