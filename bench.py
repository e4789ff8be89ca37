"""Benchmark of the block-scaled MoE expert hot path on one MI355X.

One step = the whole hot path of a quantized MoE expert up-projection layer
("End-to-End 4-Bit Training": NVFP4 forward, MXFP8 backward with stochastic
requantization) at the sizes of the MoE expert forward workload -- 16384
tokens, hidden 4096, 64 experts of 4096 x 1536, top-8 routing -- and of its
backward (weight requantization and backward GEMMs):

  route          top-8 ids -> expert segments
  quant_x        NVFP4 RTN of x [16384, 4096] bf16, per-token outer scale,
                 Four Over Six block scales (the pages' activation quantizer)
  quant_w        NVFP4 RTN of W [64, 1536, 4096] bf16, per-expert outer scale
  fprop          NVFP4 grouped GEMM y [131072, 1536] (bf16 out)
  requant_w      W_q -> MXFP8 W_q^T [64, 4096, 1536], SR seed 42
  quant_g_rows   g [131072, 1536] bf16 -> MXFP8 rows, SR (stream 1)
  quant_g_t      g -> MXFP8 g^T per expert, SR (stream 2)
  requant_x      x_q gathered per expert -> MXFP8 x_q^T, SR (stream 3)
  dgrad          MXFP8 grouped GEMM dx [131072, 4096] (bf16 out)
  wgrad          MXFP8 grouped GEMM dw [64, 1536, 4096] (fp32 out)

Inputs are seeded synthetic tensors resident in HBM before timing. Prints one
JSON line; `value` is the step's GEMM work (FPROP + DGRAD + WGRAD FLOPs) per
second of the whole step, quantization included.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "quantize/requant GB/s (% HBM peak); NVFP4 expert grouped-GEMM TFLOPS (% MFMA)"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "fp8": 5000.0, "fp4": 10100.0}  # dense, published

# The pages' contraction dtype of each GEMM stage: NVFP4 forward GEMMs against
# the FP4 MFMA peak, MXFP8 backward GEMMs against the FP8 peak. They execute
# on the 16-bit MFMA (exact decode), reported beside as frac_of_mfma16_peak.
GEMM_DTYPE = {"fprop": "fp4", "chain_w13": "fp4", "chain_w2_codec": "fp4", "w5_fprop": "fp4",
              "dgrad": "fp8", "wgrad": "fp8"}


def rate_entry(name, ms, unit, work):
    """ms, achieved, peak and fraction of one stage (HBM or MFMA roofline)."""
    if unit == "GB/s":
        ach = work / (ms * 1e-3) / 1e9
        return {"ms": round(ms, 4), "achieved": round(ach, 2), "unit": unit, "peak": HBM_PEAK_GBS,
                "frac": round(ach / HBM_PEAK_GBS, 4)}
    ach = work / (ms * 1e-3) / 1e12
    dt = GEMM_DTYPE[name]
    peak = MFMA_PEAK_TFLOPS[dt]
    return {"ms": round(ms, 4), "achieved": round(ach, 2), "unit": unit, "peak": peak, "peak_dtype": dt,
            "frac": round(ach / peak, 4), "frac_of_mfma16_peak": round(ach / MFMA_PEAK_TFLOPS["f16"], 4)}


T, H, E, K_TOP, F = 16384, 4096, 64, 8, 1536
M = T * K_TOP


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--stages", default="", help="comma list of stages to run (profiling aid); default all")
    p.add_argument("--scale-handling-only", action="store_true",
                   help="run only the NVFP4 scale-handling comparison (decode16 vs inreg_scale) and print it (profiling aid)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="after timing, run a plain 512 MiB device copy three times (reference for HBM byte counters)")
    return p.parse_args()


def make_inputs(torch, dev):
    import numpy as np

    import synth
    x = synth.moe_activations(2)
    w = synth.moe_weights(2)
    ids = synth.moe_routing(2)
    g = synth.output_grad(M, F)
    to_bf16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    return dict(x=to_bf16(x), w=to_bf16(w), ids=torch.from_numpy(ids).to(dev), g=to_bf16(g))


def algorithmic(seg_host):
    """Algorithmic bytes (each input read once, each output written once) or
    FLOPs of one call of each stage."""
    mp = [(int(seg_host[e + 1] - seg_host[e]) + 31) // 32 * 32 for e in range(E)]
    smp = sum(mp)
    nv = lambda rows, cols: rows * (cols // 2 + cols // 16)          # NVFP4 codes + scales
    mx = lambda elems: elems + elems // 32                            # MXFP8 codes + scales
    gemm = 2.0 * M * F * H
    return {
        "route": ("GB/s", T * K_TOP * 4 + M * 4 * 2 + (E + 1) * 8),
        "quant_x": ("GB/s", T * H * 2 + nv(T, H) + T * 4),
        "quant_w": ("GB/s", E * F * H * 2 + nv(E * F, H) + E * 4),
        "fprop": ("TFLOP/s", gemm),
        "requant_w": ("GB/s", nv(E * F, H) + E * 4 + mx(E * H * F)),
        "quant_g_rows": ("GB/s", M * F * 2 + mx(M * F)),
        "quant_g_t": ("GB/s", M * F * 2 + mx(F * smp)),
        "requant_x": ("GB/s", nv(T, H) + T * 4 + M * 4 + mx(H * smp)),
        "dgrad": ("TFLOP/s", gemm),
        "wgrad": ("TFLOP/s", gemm),
        # not step stages: the square-tile weight quantizer (both layouts from one
        # read) and the combine codec on the dispatched expert output rows [M, H]
        "quant_w_square": ("GB/s", E * F * H * 2 + 2 * nv(E * F, H) + E * 4),
        "quant_g_dual": ("GB/s", M * F * 2 + mx(M * F) + mx(F * smp)),
        "combine_encode": ("GB/s", M * H * 2 + M * H + M * H // 32),
        "combine_decode": ("GB/s", M * H + M * H // 32 + M * 4 + T * H * 2),
        # the expert forward chain (w13 GEMM, SwiGLU + quantize, w2 GEMM + codec)
        "chain_quant_w13": ("GB/s", E * 2 * F * H * 2 + nv(E * 2 * F, H) + E * 4),
        "chain_w13": ("TFLOP/s", 2.0 * M * 2 * F * H),
        "chain_swiglu_quant": ("GB/s", M * 2 * F * 2 + nv(M, F) + M * 4),
        "chain_quant_w2": ("GB/s", E * H * F * 2 + nv(E * H, F) + E * 4),
        "chain_w2_codec": ("TFLOP/s", 2.0 * M * H * F),
        "chain_combine": ("GB/s", M * H + M * H // 32 + M * 4 + T * H * 2),
    }


def stage_sources(stage):
    """HIP sources whose kernels a stage launches (their hash keys the
    committed HBM traffic figures)."""
    if stage in ("chain_w13", "chain_w2_codec"):
        return ("gemm.hip", "bsq_device.h", "bsq_internal.h")
    if stage == "chain_combine":
        return ("codec.hip", "bsq_device.h", "bsq_internal.h")
    if stage in ("fprop", "dgrad", "wgrad", "w5_fprop"):
        return ("gemm.hip", "bsq_device.h", "bsq_internal.h")
    if stage == "route":
        return ("route.hip", "bsq_internal.h")
    if stage.startswith("combine_"):
        return ("codec.hip", "bsq_device.h", "bsq_internal.h")
    return ("quantize.hip", "transpose_quant.hip", "bsq_device.h", "bsq_internal.h")


def kernel_sha(*files):
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, "block_scaled_bit_quantize_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def read_traffic(stage, sha):
    """HBM bytes per launch of `stage` from a committed rocprofv3 counter summary
    (profiles/traffic_<stage>.txt, lines 'key: value'); None when absent or
    taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{stage}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha") != sha:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(seg_host, row_index_host):
    """The oracle on a bounded sample of every stage of the step, timed on this
    host; each stage's time is scaled by (full work / sample work) to a
    CPU-equivalent step time."""
    import numpy as np

    import synth
    from oracle import gemm as G
    from oracle import quant as Q
    from oracle.route import route as oroute

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = os.cpu_count() or 1
    rng = np.random.default_rng(0)
    R = 2048                                     # rows per quantization sample
    G_R, G_N = 512, 512                          # GEMM sample: rows x output columns
    xs = synth.bf16_to_f32(synth.normal_bf16((R, H), 1.0, rng))
    ws = synth.bf16_to_f32(synth.normal_bf16((1, R, H), 0.02, rng))
    gs = synth.bf16_to_f32(synth.normal_bf16((R, F), 1e-3, rng))
    times = {}

    def timed(name, fn, scale):
        t0 = time.perf_counter()
        out = fn()
        times[name] = (time.perf_counter() - t0) * scale
        return out

    ids = synth.moe_routing(2)
    timed("route", lambda: oroute(ids, E), 1.0)
    xq = timed("quant_x", lambda: Q.quantize_nvfp4(xs[None], Q.OUTER_ROW, four_over_six=True), T / R)
    wq = timed("quant_w", lambda: Q.quantize_nvfp4(ws, Q.OUTER_TENSOR), E * F / R)
    seg_g = np.array([0, G_R], dtype=np.int64)
    wsub = (wq[0][:, :G_N], wq[1][:, :G_N], wq[2])
    timed("fprop", lambda: G.grouped_gemm_nvfp4_ref(xq[0][0][:G_R], xq[1][0][:G_R], xq[2][0][:G_R], None, *wsub,
                                                     seg_g), (M * F) / (G_R * G_N))
    timed("requant_w", lambda: Q.requant_transpose_sr(wq[0], wq[1], wq[2], Q.OUTER_TENSOR, Q.MXFP8, 42, 0), E * F / R)
    gq = timed("quant_g_rows", lambda: Q.quantize_mxfp8(gs, Q.SR, 42, 1), M / R)
    seg_r = np.array([0, R], dtype=np.int64)
    gt = timed("quant_g_t", lambda: Q.quantize_mxfp8_transposed(gs, seg_r, Q.SR, 42, 2), M / R)
    xt = timed("requant_x", lambda: Q.requant_transpose_sr_segmented(xq[0][0], xq[1][0], xq[2][0], Q.OUTER_ROW,
                                                                       np.arange(R), seg_r, 42, 3), M / R)
    # DGRAD sample: G_R rows of g times G_N rows of w^T (K = F)
    wt_c, wt_s = Q.quantize_mxfp8(synth.bf16_to_f32(synth.normal_bf16((G_N, F), 0.02, rng)), Q.RN)
    timed("dgrad", lambda: G.mxfp8_dgrad_ref(gq[0][:G_R], gq[1][:G_R], wt_c[None], wt_s[None], seg_g),
          (M * H) / (G_R * G_N))
    # WGRAD sample: dw over R tokens of one expert, all of [F, H]
    timed("wgrad", lambda: G.mxfp8_wgrad_ref(gt[0], gt[1], xt[0], xt[1], seg_r, F, H), M / R)
    step_s = sum(times.values())
    flops = 3 * 2.0 * M * F * H
    return {"value": round(flops / step_s / 1e12, 6), "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": ("extrapolated: each stage timed on a slice of the step (2048 rows/tokens for quantize, "
                       "requant and WGRAD; 512 x 512 outputs for FPROP and DGRAD), NumPy oracle, time scaled by "
                       "full/sample work; GEMM references are float64 BLAS"),
            "step_seconds_equiv": round(step_s, 3),
            "stage_seconds_equiv": {k: round(v, 3) for k, v in times.items()}}


def latency_workload1(torch, bsq, dev, reps=50):
    """Workload 1 (256 x 256, fits in L2: latency-bound): microseconds per call
    of the NVFP4 quantizer (X and W, per tensor), the NVFP4 -> NVFP4 SR
    requantization and the 256^3 grouped GEMM (one expert)."""
    import synth
    X, W = synth.workload1()
    x, w = torch.from_numpy(X).to(dev), torch.from_numpy(W).to(dev)
    xq = bsq.quantize_nvfp4(x, "tensor")
    wq = bsq.quantize_nvfp4(w[None], "tensor")
    seg = torch.tensor([0, 256], dtype=torch.int64, device=dev)
    calls = {
        "quantize_nvfp4_x": lambda: bsq.quantize_nvfp4(x, "tensor"),
        "quantize_nvfp4_w": lambda: bsq.quantize_nvfp4(w, "tensor"),
        "requant_nvfp4_sr": lambda: bsq.requant_transpose_sr(xq[0], xq[1], xq[2], "tensor", "nvfp4", seed=0,
                                                             stream_id=0),
        "gemm_nvfp4_256": lambda: bsq.grouped_gemm_nvfp4(xq[0], xq[1], xq[2], wq[0], wq[1], wq[2], seg, 256),
    }
    out = {}
    for name, fn in calls.items():
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        out[name] = round(a.elapsed_time(b) / reps * 1e3, 2)
    out["unit"] = "us per call (including the binding's output allocation)"
    return out


def workload5(torch, bsq, dev, reps=5):
    """Workload 5 (65536 tokens, hidden 7168, 128 experts of 2048 x 7168, top-8 with Zipf(1.1) expert
    popularity, Student-t(3) activations): per-token Four Over Six activation quantize, per-expert weight
    quantize and the NVFP4 grouped GEMM over the skewed segments, each timed on its own (HIP events,
    mean of `reps` calls), on the seeded inputs the parity tests use (synth). Carries its own roofline
    object for its dominant kernel, the GEMM."""
    import numpy as np

    import synth
    p = synth.WORKLOADS[5]
    T5, H5, E5, F5, k5 = p["tokens"], p["hidden"], p["experts"], p["ffn"], p["topk"]
    to_bf16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    x = to_bf16(synth.moe_activations(5))
    w = to_bf16(synth.moe_weights(5))
    ids = torch.from_numpy(synth.moe_routing(5)).to(dev)
    ri, seg, _ = bsq.route(ids, E5)
    M5 = T5 * k5
    xq = bsq.quantize_nvfp4(x, "row", four_over_six=True)
    wq = bsq.quantize_nvfp4(w, "tensor")
    lens = np.diff(seg.cpu().numpy())
    nv = lambda rows, cols: rows * (cols // 2 + cols // 16)
    calls = {
        "quant_x": (lambda: bsq.quantize_nvfp4(x, "row", four_over_six=True), "GB/s",
                    T5 * H5 * 2 + nv(T5, H5) + T5 * 4),
        "quant_w": (lambda: bsq.quantize_nvfp4(w, "tensor"), "GB/s", E5 * F5 * H5 * 2 + nv(E5 * F5, H5) + E5 * 4),
        "w5_fprop": (lambda: bsq.grouped_gemm_nvfp4(xq[0], xq[1], xq[2], wq[0], wq[1], wq[2], seg, M5, row_index=ri),
                     "TFLOP/s", 2.0 * M5 * F5 * H5),
    }
    out = {}
    for name, (fn, unit, work) in calls.items():
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        out[name] = rate_entry(name, a.elapsed_time(b) / reps, unit, work)
    g = out["w5_fprop"]
    out["roofline"] = {"bound": "mfma", "kernel": "w5_fprop", "achieved": g["achieved"], "peak": g["peak"],
                       "unit": g["unit"], "frac": g["frac"], "frac_of_mfma16_peak": g["frac_of_mfma16_peak"],
                       "traffic": read_traffic("w5_fprop", kernel_sha(*stage_sources("w5_fprop")))}
    out["segments"] = {"experts": int(E5), "min_rows": int(lens.min()), "max_rows": int(lens.max()),
                       "total_rows": int(M5)}
    out["what"] = "workload 5 (Zipf-skewed MoE forward, seeded synth inputs), outside the step"
    del x, w, xq, wq
    torch.cuda.empty_cache()
    return out


def _time(torch, fn, reps):
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def scale_handling(torch, bsq, inp, xq, dev, reps=5):
    """The two ways to handle NVFP4's E4M3 block scales on CDNA4, timed on one
    dense problem with the forward GEMM's work: the step's quantized tokens
    x_q [16384, 4096] against eight experts' weights stacked as one
    [12288, 4096] NVFP4 tensor (2 * 16384 * 12288 * 4096 = 1.649 TFLOP, fp32
    out). decode16: the library's kernel (exact fp16 operands, 16-bit MFMA);
    inreg_scale: one FP8 MFMA per 16-value block with the partial sums scaled
    in fp32 registers."""
    xc, xs, xo = xq
    w = inp["w"][:8].reshape(1, 8 * F, H)
    wc, ws, wo = bsq.quantize_nvfp4(w, "tensor")
    seg = torch.tensor([0, T], dtype=torch.int64, device=dev)
    flops = 2.0 * T * 8 * F * H
    calls = {"decode16": lambda: bsq.grouped_gemm_nvfp4(xc, xs, xo, wc, ws, wo, seg, T, out_dtype=torch.float32),
             "inreg_scale": lambda: bsq.gemm_nvfp4_inreg_scale(xc, xs, xo, wc[0], ws[0], wo)}
    out = {}
    for name, fn in calls.items():
        ms = _time(torch, fn, reps)
        ach = flops / (ms * 1e-3) / 1e12
        out[name] = {"ms": round(ms, 4), "achieved": round(ach, 2), "unit": "TFLOP/s",
                     "frac_of_fp4_peak": round(ach / MFMA_PEAK_TFLOPS["fp4"], 4),
                     "frac_of_fp8_peak": round(ach / MFMA_PEAK_TFLOPS["fp8"], 4),
                     "frac_of_mfma16_peak": round(ach / MFMA_PEAK_TFLOPS["f16"], 4)}
    out["shape"] = "dense M=16384, N=12288, K=4096 (1.649 TFLOP, the forward GEMM's work)"
    del w, wc, ws, wo
    return out


def dense_library_gemm(torch, dev, reps=5):
    """A practical 16-bit reference: torch.matmul (hipBLASLt) on dense bf16
    operands (no decode, no grouping) at the step's three GEMM shapes."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    out = {}
    x = torch.randn((M, H), generator=gen, device=dev).to(torch.bfloat16)
    w = torch.randn((H, F), generator=gen, device=dev).to(torch.bfloat16)
    out["fprop_shape"] = _time(torch, lambda: x @ w, reps)
    g = torch.randn((M, F), generator=gen, device=dev).to(torch.bfloat16)
    wt = torch.randn((F, H), generator=gen, device=dev).to(torch.bfloat16)
    out["dgrad_shape"] = _time(torch, lambda: g @ wt, reps)
    gt = g.t().contiguous()
    out["wgrad_shape"] = _time(torch, lambda: gt @ x, reps)
    del x, w, g, wt, gt
    torch.cuda.empty_cache()
    flops = 2.0 * M * F * H
    res = {k: {"ms": round(v, 4), "achieved": round(flops / (v * 1e-3) / 1e12, 2), "unit": "TFLOP/s"}
           for k, v in out.items()}
    res["what"] = ("torch.matmul bf16 [131072,4096]x[4096,1536], [131072,1536]x[1536,4096], "
                   "[1536,131072]x[131072,4096]: dense, no block scales")
    return res


def gemm_operand_data(torch, bsq, state, seg, ri, reps=5):
    """FPROP and DGRAD launched on the step's operands and on copies whose
    codes are all zero (same shapes, block scales, tiles and instruction
    stream; only the values the MFMAs and decode see differ). The GEMMs run
    at the chip's power limit, so the time depends on the data's switching
    activity: the zero-coded launches show how much of the gap to the
    16-bit peak is the clock, not the kernel."""
    xc, xs, xo = state["xq"]
    wc, ws, wo = state["wq"]
    gc, gs = state["gq"]
    wtc, wts = state["wt"]
    out = {"fprop": _time(torch, lambda: bsq.grouped_gemm_nvfp4(xc, xs, xo, wc, ws, wo, seg, M, row_index=ri), reps)}
    zx, zw = torch.zeros_like(xc), torch.zeros_like(wc)
    out["fprop_zero_codes"] = _time(
        torch, lambda: bsq.grouped_gemm_nvfp4(zx, xs, xo, zw, ws, wo, seg, M, row_index=ri), reps)
    del zx, zw
    out["dgrad"] = _time(torch, lambda: bsq.grouped_gemm_mxfp8(False, gc, gs, wtc, wts, seg, M, H, F), reps)
    zg, zt = torch.zeros_like(gc), torch.zeros_like(wtc)
    out["dgrad_zero_codes"] = _time(torch, lambda: bsq.grouped_gemm_mxfp8(False, zg, gs, zt, wts, seg, M, H, F), reps)
    del zg, zt
    torch.cuda.empty_cache()
    res = {k: round(v, 4) for k, v in out.items()}
    res["unit"] = "ms"
    res["what"] = "the step's FPROP and DGRAD on its operands and on all-zero codes (same scales and launches)"
    return res


def mfma_rates(torch, bsq, reps=3, iters=20000):
    """Per-instruction MFMA throughput (bsq_mfma_rate_probe): two workgroups
    of 4 waves per CU, each wave running only MFMAs on register operands,
    for the 16-bit instructions the GEMMs use, the K = 16 FP8 instruction and
    the block-scaled FP8 / FP4 instructions, on random, two-significant-bit
    and zero operand data. Against the nominal dense peaks (2.5 / 5.0 / 10.1
    PFLOP/s at 2.4 GHz) these give the sustained rate of each instruction on
    this chip and how much of it is power (data dependence)."""
    wg = 2 * torch.cuda.get_device_properties(0).multi_processor_count
    names = {0: ("f16_32x32x16", 32768, 2500.0), 1: ("bf16_32x32x16", 32768, 2500.0),
             2: ("fp8_32x32x16", 32768, 5000.0), 3: ("scaled_fp8_32x32x64", 131072, 5000.0),
             4: ("scaled_fp4_32x32x64", 131072, 10100.0)}
    datas = {0: "random", 2: "two_bit", 1: "zero"}
    out = {}
    for kind, (name, flop, peak) in names.items():
        row = {"nominal_peak_tflops": peak}
        for data, dname in datas.items():
            ms = _time(torch, lambda: bsq.mfma_rate_probe(kind, data, iters, wg), reps)
            tf = wg * 4 * iters * 4 * flop / (ms * 1e-3) / 1e12
            row[dname] = {"ms": round(ms, 4), "tflops": round(tf, 1), "frac": round(tf / peak, 4)}
        out[name] = row
    out["what"] = f"{wg} workgroups x 4 waves x {iters} rounds of 4 independent MFMA chains, register operands"
    return out


def chain_forward(torch, bsq, inp, algo, dev, pair_row, reps=5):
    """The expert forward chain (w13 GEMM, SwiGLU + per-row NVFP4, w2 GEMM with
    the RHT + S2F6 combine codec in its epilogue, combine) on the step's
    tokens and routing with the seeded w13 [E, 2F, H] and w2 [E, H, F]; each
    stage timed with HIP events, median over `reps` passes."""
    import numpy as np

    import synth
    to_bf16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    w13 = to_bf16(synth.moe_w13(2))
    w2 = to_bf16(synth.moe_w2(2))
    ri, seg, _ = bsq.route(inp["ids"], E)
    xc, xs, xo = bsq.quantize_nvfp4(inp["x"], "row", four_over_six=True)
    signs = 0x13579BDF
    names = ["chain_quant_w13", "chain_w13", "chain_swiglu_quant", "chain_quant_w2", "chain_w2_codec",
             "chain_combine"]
    times = {n: [] for n in names}
    for it in range(reps + 1):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
        ev[0].record()
        w13q = bsq.quantize_nvfp4(w13, "tensor")
        ev[1].record()
        h13 = bsq.grouped_gemm_nvfp4(xc, xs, xo, *w13q, seg, M, row_index=ri)
        ev[2].record()
        hq = bsq.swiglu_quantize_nvfp4(h13)
        ev[3].record()
        w2q = bsq.quantize_nvfp4(w2, "tensor")
        ev[4].record()
        codes, scales = bsq.grouped_gemm_nvfp4_s2f6(*hq, *w2q, seg, M, signs)
        ev[5].record()
        bsq.rht_s2f6_combine(codes, scales, pair_row, K_TOP, signs)
        ev[6].record()
        torch.cuda.synchronize()
        if it:  # the first pass is warm-up
            for i, n in enumerate(names):
                times[n].append(ev[i].elapsed_time(ev[i + 1]))
    out = {}
    for n in names:
        unit, work = algo[n]
        out[n] = rate_entry(n, float(np.median(times[n])), unit, work)
        out[n]["traffic"] = read_traffic(n, kernel_sha(*stage_sources(n)))
    out["ms_total"] = round(sum(out[n]["ms"] for n in names), 4)
    out["what"] = ("MoE expert forward (w13 GEMM -> SwiGLU + NVFP4 -> w2 GEMM with RHT-32 + S2F6 epilogue -> "
                   "combine), outside the step")
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (this path runs on a single "
              "MI355X; multi-GPU expert parallelism is design-only).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import block_scaled_bit_quantize_amd as bsq
    from block_scaled_bit_quantize_amd import _lib
    if not os.path.exists(_lib.library_path()):
        from block_scaled_bit_quantize_amd.build import build
        build()
    dev = torch.device("cuda:0")
    inp = make_inputs(torch, dev)
    outer_one = torch.ones(1, dtype=torch.float32, device=dev)

    if args.scale_handling_only:
        xq = bsq.quantize_nvfp4(inp["x"], "row", four_over_six=True)
        print(json.dumps({"nvfp4_scale_handling": scale_handling(torch, bsq, inp, xq, dev)}))
        return
    # routing is deterministic: read the segment sizes once (outside timing) for byte accounting
    ri, seg, _ = bsq.route(inp["ids"], E)
    torch.cuda.synchronize()
    seg_host = seg.cpu().numpy()
    n_gt = F * sum((int(seg_host[e + 1] - seg_host[e]) + 31) // 32 * 32 for e in range(E))
    n_xt = H * (n_gt // F)
    stages = [s for s in args.stages.split(",") if s] or None
    run = lambda name: stages is None or name in stages
    state = {}

    def step(ev):
        def mark(name):
            if ev is not None:
                e = torch.cuda.Event(enable_timing=True)
                e.record()
                ev.append((name, e))
        mark("start")
        if run("route"):
            state["ri"], state["seg"], _ = bsq.route(inp["ids"], E)
            mark("route")
        ri_, seg_ = state.get("ri", ri), state.get("seg", seg)
        if run("quant_x") or "xq" not in state:
            state["xq"] = bsq.quantize_nvfp4(inp["x"], "row", four_over_six=True)
            mark("quant_x")
        if run("quant_w") or "wq" not in state:
            state["wq"] = bsq.quantize_nvfp4(inp["w"], "tensor")
            mark("quant_w")
        xc, xs_, xo = state["xq"]
        wc, ws_, wo = state["wq"]
        if run("fprop"):
            state["y"] = bsq.grouped_gemm_nvfp4(xc, xs_, xo, wc, ws_, wo, seg_, M, row_index=ri_)
            mark("fprop")
        if run("requant_w") or "wt" not in state:
            state["wt"] = bsq.requant_transpose_sr(wc, ws_, wo, "tensor", "mxfp8", seed=42, stream_id=0)
            mark("requant_w")
        if run("quant_g_rows") or "gq" not in state:
            state["gq"] = bsq.quantize_mxfp8(inp["g"], "sr", seed=42, stream_id=1)
            mark("quant_g_rows")
        if run("quant_g_t") or "gt" not in state:
            state["gt"] = bsq.quantize_mxfp8(inp["g"], "sr", seed=42, stream_id=2, transpose=True, seg_offsets=seg_,
                                             out_elems=n_gt)
            mark("quant_g_t")
        if run("requant_x") or "xt" not in state:
            state["xt"] = bsq.requant_transpose_sr(xc, xs_, xo, "row", "mxfp8", seed=42, stream_id=3, row_gather=ri_,
                                                   seg_offsets=seg_, out_elems=n_xt)
            mark("requant_x")
        wtc, wts = state["wt"]
        if run("dgrad"):
            state["dx"] = bsq.grouped_gemm_mxfp8(False, state["gq"][0], state["gq"][1], wtc, wts, seg_, M, H, F)
            mark("dgrad")
        if run("wgrad"):
            state["dw"] = bsq.grouped_gemm_mxfp8(True, state["gt"][0], state["gt"][1], state["xt"][0], state["xt"][1],
                                                 seg_, F, H)
            mark("wgrad")

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    events = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        ev = []
        step(ev)
        events.append(ev)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    per_stage = {}
    for ev in events:
        for (pname, pe), (name, e) in zip(ev[:-1], ev[1:]):
            per_stage.setdefault(name, []).append(pe.elapsed_time(e))
    algo = algorithmic(seg_host)
    kernels = {}
    for name, ts in per_stage.items():
        unit, work = algo[name]
        kernels[name] = rate_entry(name, float(np.median(ts)), unit, work)

    gemm_flops = sum(algo[n][1] for n in ("fprop", "dgrad", "wgrad") if n in kernels)
    value = gemm_flops / (ms_per_step * 1e-3) / 1e12
    dom = max(kernels, key=lambda n: kernels[n]["ms"])
    dk = kernels[dom]
    traffic = read_traffic(dom, kernel_sha(*stage_sources(dom)))
    roofline = {"bound": "hbm" if dk["unit"] == "GB/s" else "mfma", "kernel": dom, "achieved": dk["achieved"],
                "peak": dk["peak"], "unit": dk["unit"], "frac": dk["frac"], "traffic": traffic}
    if "frac_of_mfma16_peak" in dk:
        roofline["peak_dtype"] = dk["peak_dtype"]
        roofline["frac_of_mfma16_peak"] = dk["frac_of_mfma16_peak"]

    # Alternatives to a step stage, timed on their own after the step (not in
    # ms_per_step): the 16x16 square-tile weight quantizer writing W and W^T.
    alternatives = {}
    if stages is None:
        reps = 10
        for _ in range(2):
            bsq.quantize_nvfp4_square(inp["w"], "tensor")
        torch.cuda.synchronize()
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        for _ in range(reps):
            bsq.quantize_nvfp4_square(inp["w"], "tensor")
        a1.record()
        torch.cuda.synchronize()
        ms = a0.elapsed_time(a1) / reps
        ach = algo["quant_w_square"][1] / (ms * 1e-3) / 1e9
        alternatives["quant_w_square"] = {
            "ms": round(ms, 4), "achieved": round(ach, 2), "unit": "GB/s", "peak": HBM_PEAK_GBS,
            "frac": round(ach / HBM_PEAK_GBS, 4),
            "traffic": read_traffic("quant_w_square", kernel_sha(*stage_sources("quant_w_square"))),
            "alternative_to": "quant_w + requant_w where the backward reads W^T in NVFP4 (square tiles) instead of SR MXFP8"}
        # both MXFP8 quantizations of g from one read (the step times them as
        # two stages, quant_g_rows and quant_g_t)
        ms = _time(torch, lambda: bsq.quantize_mxfp8_dual(inp["g"], "sr", seed=42, stream_rows=1, stream_t=2,
                                                           seg_offsets=seg, out_elems=n_gt), reps)
        ach = algo["quant_g_dual"][1] / (ms * 1e-3) / 1e9
        alternatives["quant_g_dual"] = {
            "ms": round(ms, 4), "achieved": round(ach, 2), "unit": "GB/s", "peak": HBM_PEAK_GBS,
            "frac": round(ach / HBM_PEAK_GBS, 4),
            "traffic": read_traffic("quant_g_dual", kernel_sha(*stage_sources("quant_g_dual"))),
            "separate_ms": round(kernels["quant_g_rows"]["ms"] + kernels["quant_g_t"]["ms"], 4),
            "alternative_to": "quant_g_rows + quant_g_t (g read once instead of twice)"}
        # the combine codec (RHT-32 + block-scaled S2F6) on the expert output
        # rows of the layer's combine: [tokens * topk, hidden] bf16, seeded
        import synth
        payload = torch.from_numpy(synth.combine_rows(M, H).view(np.int16)).to(dev).view(torch.bfloat16)
        _, _, pair_row = bsq.route(inp["ids"], E)
        signs = 0x9E3779B9
        enc = bsq.rht_s2f6_encode(payload, signs)
        for name, fn in (("combine_encode", lambda: bsq.rht_s2f6_encode(payload, signs)),
                         ("combine_decode", lambda: bsq.rht_s2f6_combine(enc[0], enc[1], pair_row, K_TOP, signs))):
            for _ in range(2):
                fn()
            torch.cuda.synchronize()
            a0.record()
            for _ in range(reps):
                fn()
            a1.record()
            torch.cuda.synchronize()
            ms = a0.elapsed_time(a1) / reps
            ach = algo[name][1] / (ms * 1e-3) / 1e9
            alternatives[name] = {
                "ms": round(ms, 4), "achieved": round(ach, 2), "unit": "GB/s", "peak": HBM_PEAK_GBS,
                "frac": round(ach / HBM_PEAK_GBS, 4),
                "traffic": read_traffic(name, kernel_sha(*stage_sources(name))),
                "alternative_to": "bf16 combine payload (16 bits per value; the codec carries 8.25)"}
        del payload, enc
        alternatives["expert_chain_fwd"] = chain_forward(torch, bsq, inp, algo, dev, pair_row)
        alternatives["workload1_latency"] = latency_workload1(torch, bsq, dev)
        alternatives["workload5_fwd"] = workload5(torch, bsq, dev)
        alternatives["nvfp4_scale_handling"] = scale_handling(torch, bsq, inp, state["xq"], dev)
        alternatives["dense_bf16_library_gemm"] = dense_library_gemm(torch, dev)
        alternatives["gemm_operand_data"] = gemm_operand_data(torch, bsq, state, seg, ri)
        alternatives["mfma_rate"] = mfma_rates(torch, bsq)

    if args.copy_calibration:
        src_buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst_buf = torch.empty_like(src_buf)
        for _ in range(3):
            dst_buf.copy_(src_buf)
        torch.cuda.synchronize()
        del src_buf, dst_buf

    cpu = None
    if not args.no_cpu_baseline and stages is None:
        cpu = cpu_baseline(seg_host, None)

    line = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 (NVFP4) / bf16 (MXFP8) MFMA on exactly decoded operands, f32 accumulate",
        "data": "synthetic (seeded; bf16 N(0,1) activations, N(0,0.02) weights, N(0,1e-3) gradients with 0.1% x50)",
        "config": {"workload": "moe_expert_fwd_bwd", "tokens": T, "hidden": H, "experts": E, "topk": K_TOP,
                   "ffn": F, "global_batch": T, "parallelism": "none (1 GPU)"},
        "kernels": kernels,
        "roofline": roofline,
        "alternatives": alternatives,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
