"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the
benchmark. Holds no arithmetic of the quantization method: only random draws
with the shapes and distributions of the five workloads, bf16 rounding of the
draws, and routing draws.

Workloads (data seed 1000 + workload number; tensor t of a workload is drawn in
chunks of 2^24 elements, chunk c from its own PCG64 stream seeded with
[1000 + workload, t, c], so that chunks are generated in parallel threads):
  1 single tensor: X, W float32 [256, 256] ~ N(0,1), 8 distinct seeded
    positions of each scaled by 100.
  2 MoE expert forward: x bf16 [16384, 4096] ~ N(0,1); W bf16 [64, 1536, 4096]
    ~ N(0, 0.02); top-8 of 64 experts, uniform, distinct per token.
  3 weight requantization: workload 2's W quantized to NVFP4.
  4 backward GEMMs: g bf16 [131072, 1536] ~ N(0, 1e-3), 0.1% of entries
    scaled by 50; workload 2's routing and x.
  5 large skewed forward: x bf16 [65536, 7168] ~ Student-t(3);
    W bf16 [128, 2048, 7168] ~ N(0, 0.02); top-8 of 128 experts with Zipf(1.1)
    popularity.
Expert chain (w13 GEMM, SwiGLU, w2 GEMM) at workload 2's sizes: w13 bf16
    [64, 3072, 4096] (gate rows, then up rows) and w2 bf16 [64, 4096, 1536],
    both ~ N(0, 0.02).
Combine payload (the expert output rows that the combine codec carries):
    workload 2's dispatched rows, bf16 [131072, 4096] ~ N(0, 1), 0.1% of
    entries scaled by 20 (outliers).
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

WORKLOADS = {
    1: dict(rows=256, cols=256, outliers=8, outlier_scale=100.0, sr_seed=0),
    2: dict(tokens=16384, hidden=4096, experts=64, topk=8, ffn=1536, w_std=0.02),
    3: dict(experts=64, ffn=1536, hidden=4096, sr_seed=42),
    4: dict(tokens=16384, hidden=4096, experts=64, topk=8, ffn=1536, g_std=1e-3,
            spike_frac=1e-3, spike_scale=50.0, sr_seed=42),
    5: dict(tokens=65536, hidden=7168, experts=128, topk=8, ffn=2048, w_std=0.02, zipf_s=1.1),
}

_CHUNK = 1 << 24


def rng_for(workload, stream):
    """Independent PCG64 stream for tensor ``stream`` of a workload."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([1000 + int(workload), int(stream)])))


def bf16_bits(f32):
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    b = np.ascontiguousarray(f32, dtype=np.float32).view(np.uint32)
    return ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits):
    """bfloat16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _par_bf16(workload, stream, shape, draw):
    """bf16 bits [shape] whose chunk c of 2^24 elements is draw(rng_c, m), rng_c
    seeded with [1000 + workload, stream, c]; chunks run on a thread pool
    (NumPy's fills and ufuncs release the GIL). The result does not depend on
    the number of threads."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)

    def one(c):
        s = c * _CHUNK
        m = min(_CHUNK, n - s)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([1000 + int(workload), int(stream), c])))
        out[s:s + m] = bf16_bits(draw(rng, m))

    chunks = (n + _CHUNK - 1) // _CHUNK
    workers = max(1, min(16, os.cpu_count() or 1, chunks))
    if workers == 1:
        for c in range(chunks):
            one(c)
    else:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(one, range(chunks)))
    return out.reshape(shape)


def normal_bf16(shape, std, rng):
    """bf16 bits of N(0, std^2) draws, generated in chunks."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, _CHUNK):
        m = min(_CHUNK, n - s)
        out[s:s + m] = bf16_bits(rng.standard_normal(m, dtype=np.float32) * np.float32(std))
    return out.reshape(shape)


def student_t_bf16(shape, dof, rng):
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, _CHUNK):
        m = min(_CHUNK, n - s)
        out[s:s + m] = bf16_bits(rng.standard_t(dof, m).astype(np.float32))
    return out.reshape(shape)


def topk_uniform(tokens, experts, k, rng):
    """k distinct experts per token, uniformly at random."""
    out = np.empty((tokens, k), dtype=np.int32)
    for s in range(0, tokens, 8192):
        m = min(8192, tokens - s)
        out[s:s + m] = np.argsort(rng.random((m, experts)), axis=1)[:, :k]
    return out


def topk_zipf(tokens, experts, k, s_exp, rng):
    """k distinct experts per token; expert r-1 has popularity ~ r^-s
    (Gumbel top-k of the log popularities)."""
    logp = -s_exp * np.log(np.arange(1, experts + 1, dtype=np.float64))
    out = np.empty((tokens, k), dtype=np.int32)
    for s in range(0, tokens, 8192):
        m = min(8192, tokens - s)
        g = logp[None, :] - np.log(-np.log(rng.random((m, experts))))
        out[s:s + m] = np.argsort(-g, axis=1)[:, :k]
    return out


def workload1():
    """(X, W) float32 [256, 256] with 8 outliers each."""
    p = WORKLOADS[1]
    out = []
    for stream in (0, 1):
        rng = rng_for(1, stream)
        x = rng.standard_normal((p["rows"], p["cols"]), dtype=np.float32)
        pos = rng.choice(x.size, size=p["outliers"], replace=False)
        x.reshape(-1)[pos] *= np.float32(p["outlier_scale"])
        out.append(x)
    return out[0], out[1]


def moe_activations(workload, tokens=None, hidden=None):
    p = WORKLOADS[workload]
    shape = (tokens or p["tokens"], hidden or p["hidden"])
    if workload == 5:
        return _par_bf16(5, 0, shape, lambda rng, m: rng.standard_t(3, m).astype(np.float32))
    return _par_bf16(workload, 0, shape, lambda rng, m: rng.standard_normal(m, dtype=np.float32))


def moe_weights(workload, experts=None, ffn=None, hidden=None):
    p = WORKLOADS[workload]
    shape = (experts or p["experts"], ffn or p["ffn"], hidden or p["hidden"])
    std = np.float32(p["w_std"])
    return _par_bf16(workload, 1, shape, lambda rng, m: rng.standard_normal(m, dtype=np.float32) * std)


def moe_routing(workload, tokens=None, experts=None):
    p = WORKLOADS[workload]
    t = tokens or p["tokens"]
    e = experts or p["experts"]
    if workload == 5:
        return topk_zipf(t, e, p["topk"], p["zipf_s"], rng_for(5, 2))
    return topk_uniform(t, e, p["topk"], rng_for(workload, 2))


def output_grad(rows, cols, workload=4):
    """g bf16 [rows, cols] ~ N(0, 1e-3) with 0.1% of entries scaled by 50."""
    p = WORKLOADS[4]

    def draw(rng, m):
        v = rng.standard_normal(m, dtype=np.float32) * np.float32(p["g_std"])
        spike = rng.random(m) < p["spike_frac"]
        v[spike] *= np.float32(p["spike_scale"])
        return v
    return _par_bf16(workload, 3, (rows, cols), draw)


def combine_rows(rows, cols, workload=2):
    """Expert output rows bf16 [rows, cols] ~ N(0, 1) with 0.1% of entries
    scaled by 20."""
    def draw(rng, m):
        v = rng.standard_normal(m, dtype=np.float32)
        spike = rng.random(m) < 1e-3
        v[spike] *= np.float32(20.0)
        return v
    return _par_bf16(workload, 4, (rows, cols), draw)


def moe_w13(workload=2):
    """Gate and up projections bf16 [E, 2 * ffn, hidden] ~ N(0, w_std^2)."""
    p = WORKLOADS[workload]
    std = np.float32(p["w_std"])
    return _par_bf16(workload, 5, (p["experts"], 2 * p["ffn"], p["hidden"]),
                     lambda rng, m: rng.standard_normal(m, dtype=np.float32) * std)


def moe_w2(workload=2):
    """Down projections bf16 [E, hidden, ffn] ~ N(0, w_std^2)."""
    p = WORKLOADS[workload]
    std = np.float32(p["w_std"])
    return _par_bf16(workload, 6, (p["experts"], p["hidden"], p["ffn"]),
                     lambda rng, m: rng.standard_normal(m, dtype=np.float32) * std)
