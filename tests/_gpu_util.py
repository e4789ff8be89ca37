"""Helpers shared by the GPU parity tests (not collected by pytest)."""
import sys

import numpy as np
import torch

DEV = torch.device("cuda:0")


def log(msg):
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def t(a):
    """numpy -> contiguous device tensor."""
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bf16_t(bits):
    """uint16 bf16 bit patterns -> device bfloat16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def h(x):
    torch.cuda.synchronize()
    return x.cpu().numpy()


def filler_nvfp4(rng, shape_rows, cols):
    """Random valid NVFP4 bytes (codes, E4M3 scales in [2^-3, 15]) used where a
    full-size operand is not checked; the checked parts come from the oracle."""
    codes = rng.integers(0, 256, size=(*shape_rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(0x28, 0x5F, size=(*shape_rows, cols // 16), dtype=np.uint8)
    return codes, scales


def filler_mxfp8(rng, n):
    """Random valid MXFP8 bytes: E4M3 codes without NaN, E8M0 scales near 2^-8."""
    codes = rng.integers(0, 256, size=n, dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x7E
    scales = rng.integers(112, 124, size=n // 32, dtype=np.uint8)
    return codes, scales
