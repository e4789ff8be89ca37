"""GPU parity of the quantizers, requantization, RNG and routing against the
CPU oracle (bit-exact bytes), at small sizes spanning several tiles with
ragged tails and at the workloads' full sizes on sampled outputs."""
import json
import os

import numpy as np
import pytest
import torch

import block_scaled_bit_quantize_amd as bsq
from block_scaled_bit_quantize_amd import _lib
import synth
from oracle import formats as F
from oracle import quant as Q
from oracle.rng import sr_bits16
from oracle.route import route as oroute

from _gpu_util import DEV, bf16_t, h, log, t

pytestmark = pytest.mark.gpu
f32 = np.float32


def _data(rng, shape, kind):
    if kind == "normal":
        return rng.standard_normal(shape).astype(f32)
    if kind == "wide":
        return (rng.standard_normal(shape) * np.exp(rng.uniform(-30, 30, shape))).astype(f32)
    if kind == "zeros_mix":
        x = rng.standard_normal(shape).astype(f32)
        x.reshape(-1, 16)[::3] = 0.0
        x.reshape(-1, 16)[1::7] *= f32(1e-38)
        return x
    if kind == "t3":
        return rng.standard_t(3, shape).astype(f32)
    raise ValueError(kind)


def test_rng_bits_match_oracle():
    for seed, stream, first in [(0, 0, 0), (42, 1, 8 * 12345 + 3), (2**63 + 5, 2**40 + 7, 2**35 - 11)]:
        log(f"rng seed={seed} stream={stream} first={first}")
        g = h(bsq.rng_bits16(seed, stream, first, 4099)).astype(np.int64) & 0xFFFF
        o = sr_bits16(seed, stream, np.arange(4099, dtype=np.uint64) + np.uint64(first))
        assert np.array_equal(g, o)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["tensor", "row", "given"])
@pytest.mark.parametrize("shape,kind", [((1, 3, 48), "normal"), ((2, 5, 256), "wide"), ((3, 7, 1040), "zeros_mix"),
                                        ((2, 33, 4096), "t3"), ((1, 2, 8192), "normal"), ((1, 3, 32768), "t3")])
def test_quantize_nvfp4_small(dtype, mode, shape, kind):
    log(f"quantize_nvfp4 {dtype} {mode} {shape} {kind}")
    rng = np.random.default_rng(hash((dtype, mode, shape, kind)) % 2**32)
    x = _data(rng, shape, kind)
    if dtype == "bf16":
        bits = synth.bf16_bits(x)
        x = synth.bf16_to_f32(bits).reshape(shape)
        xd = bf16_t(bits.reshape(shape))
    else:
        xd = t(x)
    outer = (np.abs(rng.standard_normal(shape[0])) * 0.01 + 1e-3).astype(f32) if mode == "given" else None
    m = {"tensor": Q.OUTER_TENSOR, "row": Q.OUTER_ROW, "given": Q.OUTER_GIVEN}[mode]
    gc, gs, go = bsq.quantize_nvfp4(xd, mode, t(outer) if outer is not None else None)
    oc, os_, oo = Q.quantize_nvfp4(x, m, outer)
    assert np.array_equal(h(gc), oc)
    assert np.array_equal(h(gs), os_)
    assert np.array_equal(h(go), np.asarray(oo).reshape(-1))


@pytest.mark.parametrize("dtype,shape", [("bf16", (3, 300, 4096)), ("f32", (2, 257, 1040)), ("bf16", (1, 4100, 1024)),
                                         ("bf16", (3, 3072, 4096)), ("f32", (1, 2048, 4096)),
                                         ("bf16", (5, 1536, 4096)), ("bf16", (2, 1200, 2048)), ("f32", (2, 1200, 2048)),
                                         ("bf16", (2, 2304, 4096)), ("bf16", (2, 2048, 7168)), ("bf16", (2, 4096, 4096)),
                                         ("bf16", (32, 1024, 1536)), ("bf16", (33, 1536, 1024)),
                                         ("bf16", (32, 1536, 2048))])
def test_quantize_nvfp4_tensor_one_pass(dtype, shape):
    """Items of at least 1 MiB take the one-pass grid kernel (shares of blocks
    per workgroup that do not divide evenly, several items in sequence, odd
    and even item counts per group, one and two groups, shares of 1 to 8
    blocks per thread on 256 CUs with two and three register sets, and 32 or
    more items on two halves of the chip); the bytes must equal the oracle's."""
    log(f"quantize_nvfp4 tensor one-pass {dtype} {shape}")
    rng = np.random.default_rng(7 + shape[1])
    x = rng.standard_normal(shape).astype(f32)
    x[0, 1, 5] = 300.0  # an outlier sets item 0's outer scale
    if dtype == "bf16":
        bits = synth.bf16_bits(x)
        x = synth.bf16_to_f32(bits).reshape(shape)
        xd = bf16_t(bits.reshape(shape))
    else:
        xd = t(x)
    gc, gs, go = bsq.quantize_nvfp4(xd, "tensor")
    oc, os_, oo = Q.quantize_nvfp4(x, Q.OUTER_TENSOR)
    assert np.array_equal(h(go), np.asarray(oo).reshape(-1))
    assert np.array_equal(h(gs), os_)
    assert np.array_equal(h(gc), oc)


@pytest.mark.parametrize("shape", [(2, 300, 2048), (7, 1536, 4096), (32, 1024, 1536)])
def test_quantize_nvfp4_tensor_one_pass_wait_fallback(shape):
    """A poll limit of 0 sends every workgroup of the one-pass kernel that
    finds a slot unmarked through its fallback (it reduces the item itself);
    the bytes are unchanged (one block per thread in two groups; three blocks
    per thread in one group with enough items for the steady-state
    pipeline; 32 items on two halves of the chip)."""
    import os
    log(f"quantize_nvfp4 tensor one-pass, fallback {shape}")
    rng = np.random.default_rng(11)
    bits = synth.bf16_bits(rng.standard_normal(shape).astype(f32))
    x = synth.bf16_to_f32(bits).reshape(shape)
    os.environ["BSQ_WAIT_POLLS"] = "0"
    try:
        gc, gs, go = bsq.quantize_nvfp4(bf16_t(bits.reshape(shape)), "tensor")
        torch.cuda.synchronize()
    finally:
        del os.environ["BSQ_WAIT_POLLS"]
    oc, os_, oo = Q.quantize_nvfp4(x, Q.OUTER_TENSOR)
    assert np.array_equal(h(go), np.asarray(oo).reshape(-1))
    assert np.array_equal(h(gs), os_)
    assert np.array_equal(h(gc), oc)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["tensor", "row", "given"])
@pytest.mark.parametrize("shape,kind", [((2, 5, 256), "wide"), ((3, 7, 1040), "zeros_mix"), ((1, 33, 64), "normal")])
def test_quantize_nvfp4_four_over_six_small(dtype, mode, shape, kind):
    log(f"quantize_nvfp4 4/6 {dtype} {mode} {shape} {kind}")
    rng = np.random.default_rng(hash(("46", dtype, mode, shape, kind)) % 2**32)
    x = _data(rng, shape, kind)
    if dtype == "bf16":
        bits = synth.bf16_bits(x)
        x = synth.bf16_to_f32(bits).reshape(shape)
        xd = bf16_t(bits.reshape(shape))
    else:
        xd = t(x)
    outer = (np.abs(rng.standard_normal(shape[0])) * 0.01 + 1e-3).astype(f32) if mode == "given" else None
    m = {"tensor": Q.OUTER_TENSOR, "row": Q.OUTER_ROW, "given": Q.OUTER_GIVEN}[mode]
    gc, gs, go = bsq.quantize_nvfp4(xd, mode, t(outer) if outer is not None else None, four_over_six=True)
    oc, os_, oo = Q.quantize_nvfp4(x, m, outer, four_over_six=True)
    assert np.array_equal(h(gs), os_)
    assert np.array_equal(h(gc), oc)
    assert np.array_equal(h(go), np.asarray(oo).reshape(-1))


def test_quantize_nvfp4_edge_cases():
    # empty tensors, all zeros, largest bf16 values, single block
    log("quantize_nvfp4 edges")
    c, s, o = bsq.quantize_nvfp4(torch.zeros((2, 0, 32), device=DEV), "tensor")
    assert h(o).tolist() == [1.0, 1.0]
    c, s, o = bsq.quantize_nvfp4(torch.zeros((0, 4, 32), device=DEV), "row")
    assert c.numel() == 0
    c, s, o = bsq.quantize_nvfp4(torch.zeros((3, 4, 32), device=DEV), "row")
    assert not h(c).any() and not h(s).any() and np.all(h(o) == 1.0)
    big = np.full((1, 2, 16), 3.3e38, f32)
    big[0, 1, 3] = -1e-30
    gc, gs, go = bsq.quantize_nvfp4(t(big), "row")
    oc, os_, oo = Q.quantize_nvfp4(big, Q.OUTER_ROW)
    assert np.array_equal(h(gc), oc) and np.array_equal(h(gs), os_) and np.array_equal(h(go), oo.reshape(-1))


def test_pages_examples_on_gpu():
    """The worked examples of the pages, through the GPU quantizer."""
    log("pages examples")
    row = np.zeros((1, 1, 32), f32)
    row[0, 0, 0] = 593.7                       # Figure 1: scale 96, value 6
    row[0, 0, 16] = -54.0                      # block max -54 -> -6 with scale 9
    row[0, 0, 17] = 5.4                        # -> 0.6 -> 0.5 -> 4.5
    c, s, o = bsq.quantize_nvfp4(t(row), "given", t(np.ones(1, f32)))
    codes = F.unpack_fp4(h(c))[0, 0]
    sc = F.e4m3_decode(h(s))[0, 0]
    assert sc[0] == 96 and F.e2m1_decode(codes[0]) == 6
    assert sc[1] == 9 and F.e2m1_decode(codes[16]) == -6 and F.e2m1_decode(codes[17]) * 9 == 4.5


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rnd", ["rn", "sr"])
@pytest.mark.parametrize("shape,kind", [((3, 32), "normal"), ((67, 96), "wide"), ((130, 1536), "zeros_mix")])
def test_quantize_mxfp8_rows_small(dtype, rnd, shape, kind):
    log(f"quantize_mxfp8 rows {dtype} {rnd} {shape} {kind}")
    rng = np.random.default_rng(7)
    x = _data(rng, shape, kind)
    if dtype == "bf16":
        bits = synth.bf16_bits(x)
        x = synth.bf16_to_f32(bits).reshape(shape)
        xd = bf16_t(bits.reshape(shape))
    else:
        xd = t(x)
    r = Q.RN if rnd == "rn" else Q.SR
    gc, gs = bsq.quantize_mxfp8(xd, rnd, seed=11, stream_id=1)
    oc, os_ = Q.quantize_mxfp8(x, r, 11, 1)
    assert np.array_equal(h(gs), os_)
    assert np.array_equal(h(gc), oc)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rnd", ["rn", "sr"])
def test_quantize_mxfp8_transposed_small(dtype, rnd):
    log(f"quantize_mxfp8 transposed {dtype} {rnd}")
    rng = np.random.default_rng(8)
    seg = np.array([0, 0, 45, 245, 245, 374, 375, 631], dtype=np.int64)      # empty, ragged, 1-row segments
    x = _data(rng, (631, 192), "wide")
    if dtype == "bf16":
        bits = synth.bf16_bits(x)
        x = synth.bf16_to_f32(bits).reshape(x.shape)
        xd = bf16_t(bits.reshape(x.shape))
    else:
        xd = t(x)
    r = Q.RN if rnd == "rn" else Q.SR
    _, n = bsq.padded_segment_layout(seg, 192)
    gc, gs = bsq.quantize_mxfp8(xd, rnd, seed=5, stream_id=2, transpose=True, seg_offsets=t(seg), out_elems=n)
    oc, os_ = Q.quantize_mxfp8_transposed(x, seg, r, 5, 2)
    assert np.array_equal(h(gs), os_)
    assert np.array_equal(h(gc), oc)
    # no segment table: one segment of all rows
    _, n1 = bsq.padded_segment_layout([0, 631], 192)
    gc, gs = bsq.quantize_mxfp8(xd, rnd, seed=5, stream_id=2, transpose=True, out_elems=n1)
    oc, os_ = Q.quantize_mxfp8_transposed(x, [0, 631], r, 5, 2)
    assert np.array_equal(h(gc), oc) and np.array_equal(h(gs), os_)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rnd", ["rn", "sr"])
def test_quantize_mxfp8_dual_small(dtype, rnd):
    """Both MXFP8 quantizations from one read equal the oracle's row-wise
    (stream 1) and per-segment transposed (stream 2) results bit for bit."""
    log(f"quantize_mxfp8 dual {dtype} {rnd}")
    rng = np.random.default_rng(9)
    seg = np.array([0, 0, 45, 245, 245, 374, 375, 631], dtype=np.int64)      # empty, ragged, 1-row segments
    x = _data(rng, (631, 192), "zeros_mix")
    if dtype == "bf16":
        bits = synth.bf16_bits(x)
        x = synth.bf16_to_f32(bits).reshape(x.shape)
        xd = bf16_t(bits.reshape(x.shape))
    else:
        xd = t(x)
    r = Q.RN if rnd == "rn" else Q.SR
    _, n = bsq.padded_segment_layout(seg, 192)
    (gc, gs), (tc, ts) = bsq.quantize_mxfp8_dual(xd, rnd, seed=5, stream_rows=1, stream_t=2, seg_offsets=t(seg),
                                                 out_elems=n)
    oc, os_ = Q.quantize_mxfp8(x, r, 5, 1)
    assert np.array_equal(h(gc), oc) and np.array_equal(h(gs), os_)
    oc, os_ = Q.quantize_mxfp8_transposed(x, seg, r, 5, 2)
    assert np.array_equal(h(tc), oc) and np.array_equal(h(ts), os_)
    _, n1 = bsq.padded_segment_layout([0, 631], 192)   # no segment table: one segment of all rows
    (gc, gs), (tc, ts) = bsq.quantize_mxfp8_dual(xd, rnd, seed=5, stream_rows=1, stream_t=2, out_elems=n1)
    oc, os_ = Q.quantize_mxfp8(x, r, 5, 1)
    assert np.array_equal(h(gc), oc) and np.array_equal(h(gs), os_)
    oc, os_ = Q.quantize_mxfp8_transposed(x, [0, 631], r, 5, 2)
    assert np.array_equal(h(tc), oc) and np.array_equal(h(ts), os_)


def test_quantize_mxfp8_dual_uncovered_rows():
    """Offsets [-10, 100, 50, 200] over 256 rows read as [0, 100, 100, 200]:
    rows 0..199 get the row-wise codes and scales, rows 200..255 (in no
    segment) keep their contents, and the transposed output is the oracle's
    on the normalized table."""
    log("quantize_mxfp8 dual uncovered rows")
    rng = np.random.default_rng(12)
    R, C = 256, 64
    x = _data(rng, (R, C), "normal")
    seg = np.array([-10, 100, 50, 200], np.int64)
    norm = np.maximum.accumulate(np.clip(seg, 0, R))
    lib = _lib.load_library()
    codes = torch.full((R, C), 0xA5, dtype=torch.uint8, device=DEV)
    scales = torch.full((R, C // 32), 0xA5, dtype=torch.uint8, device=DEV)
    cap = C * (R + 31 * 3)
    codes_t = torch.full((cap,), 0xA5, dtype=torch.uint8, device=DEV)
    scales_t = torch.full((cap // 32,), 0xA5, dtype=torch.uint8, device=DEV)
    wsb = lib.bsq_quantize_mxfp8_workspace(R, 1, 3)
    ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device=DEV)
    xd, segd = t(x), t(seg)
    st = lib.bsq_quantize_mxfp8_dual(xd.data_ptr(), 0, R, C, segd.data_ptr(), 3, 1, 5, 1, 2, codes.data_ptr(),
                                     scales.data_ptr(), codes_t.data_ptr(), scales_t.data_ptr(), ws.data_ptr(), wsb,
                                     None)
    assert st == 0
    oc, os_ = Q.quantize_mxfp8(x, Q.SR, 5, 1)
    gc, gs = h(codes), h(scales)
    assert np.array_equal(gc[:200], oc[:200]) and np.array_equal(gs[:200], os_[:200])
    assert np.all(gc[200:] == 0xA5) and np.all(gs[200:] == 0xA5)
    tc_o, ts_o = Q.quantize_mxfp8_transposed(x, norm, Q.SR, 5, 2)
    assert np.array_equal(h(codes_t)[:tc_o.size], tc_o) and np.array_equal(h(scales_t)[:ts_o.size], ts_o)


@pytest.mark.parametrize("seg", [[0, 256, 0, 256], [-10, 100, 50, 400], [0, 300, 200, 100, 256]])
def test_segmented_malformed_offsets_stay_in_bounds(seg):
    """Decreasing or out-of-range offsets are read as clamped to [0, rows]
    and replaced by their running maximum: the result equals the oracle on
    that table, and nothing is written past the documented output bound
    cols * (rows + 31 * num_segments) (a guard region after it keeps its fill)."""
    log(f"segmented malformed offsets {seg}")
    rng = np.random.default_rng(31)
    R, C = 256, 64
    nseg = len(seg) - 1
    x = _data(rng, (R, C), "normal")
    norm = np.maximum.accumulate(np.clip(np.asarray(seg, np.int64), 0, R))
    lib = _lib.load_library()
    cap = C * (R + 31 * nseg)
    guard = 4096
    codes = torch.full((cap + guard,), 0xA5, dtype=torch.uint8, device=DEV)
    scales = torch.full((cap // 32 + guard,), 0xA5, dtype=torch.uint8, device=DEV)
    wsb = lib.bsq_quantize_mxfp8_workspace(R, 1, nseg)
    ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device=DEV)
    xd, segd = t(x), t(np.asarray(seg, np.int64))
    st = lib.bsq_quantize_mxfp8(xd.data_ptr(), 0, R, C, 1, segd.data_ptr(), nseg, 1, 5, 2, codes.data_ptr(),
                                scales.data_ptr(), ws.data_ptr(), wsb, None)
    assert st == 0
    oc, os_ = Q.quantize_mxfp8_transposed(x, norm, Q.SR, 5, 2)
    gc, gs = h(codes), h(scales)
    assert np.array_equal(gc[:oc.size], oc) and np.array_equal(gs[:os_.size], os_)
    assert np.all(gc[cap:] == 0xA5) and np.all(gs[cap // 32:] == 0xA5)
    # the gathered NVFP4 -> MXFP8 requant shares the plan
    p, s_, o = Q.quantize_nvfp4(x[None], Q.OUTER_ROW)
    gather = rng.integers(0, R, R).astype(np.int32)
    codes.fill_(0xA5)
    scales.fill_(0xA5)
    wsb = lib.bsq_requant_workspace(1, R, nseg, Q.MXFP8, 1)
    ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device=DEV)
    pd, sd, od, gd = t(p[0]), t(s_[0]), t(o.reshape(-1)), t(gather)
    st = lib.bsq_requant_transpose_sr(pd.data_ptr(), sd.data_ptr(), od.data_ptr(), 1, 1, R, C, R, gd.data_ptr(),
                                      segd.data_ptr(), nseg, 1, 1, 3, 3, codes.data_ptr(), scales.data_ptr(), None,
                                      ws.data_ptr(), wsb, None)
    assert st == 0
    wc, wsc = Q.requant_transpose_sr_segmented(p[0], s_[0], o.reshape(-1), Q.OUTER_ROW, gather, norm, 3, 3)
    gc, gs = h(codes), h(scales)
    assert np.array_equal(gc[:wc.size], wc) and np.array_equal(gs[:wsc.size], wsc)
    assert np.all(gc[cap:] == 0xA5) and np.all(gs[cap // 32:] == 0xA5)


def _sr_edge_blocks(rng, nblk):
    """MX blocks of 32 at the edges of the kernels' stochastic-rounding fast path (every value of a group of
    8 zero or at least 2^(e-6), e >= -120, done by the hardware SR convert) and of its general path."""
    out = np.empty((nblk, 32), f32)
    for b in range(nblk):
        e = int(rng.integers(-20, 21))
        top = f32(448.0) * f32(2.0) ** e
        kind = b % 8
        v = (rng.uniform(2.0 ** (e - 6), float(top), 32) * rng.choice([-1.0, 1.0], 32)).astype(f32)
        if kind == 0:    # exactly at the fast-path threshold 2^(e-6), block maximum exactly 448 2^e
            v[:] = f32(2.0) ** (e - 6) * rng.choice([-1.0, 1.0], 32).astype(f32)
        elif kind == 1:  # one value just below the threshold: that group of 8 takes the general path
            v[int(rng.integers(32))] = np.nextafter(f32(2.0) ** (e - 6), f32(0.0))
        elif kind == 2:  # all-ones mantissas: rounding up carries into the exponent
            v = (f32(2.0) ** rng.integers(e - 6, e + 8, 32) * f32(1.99999)).astype(f32) * \
                rng.choice([-1.0, 1.0], 32).astype(f32)
        elif kind == 3:  # zeros of both signs among normal values
            v[::3] = f32(0.0)
            v[1::5] = f32(-0.0)
        elif kind == 4:  # a tiny block: E8M0 exponent below -120, general path throughout
            v = (rng.standard_normal(32) * 1e-39).astype(f32)
        elif kind == 5:  # values already on the E4M3 grid (nothing dropped)
            v = (F.e4m3_decode(rng.integers(0x08, 0x7F, 32).astype(np.uint8)) * f32(2.0) ** e).astype(f32)
        elif kind == 6:  # block maximum just above 448 2^e: the next exponent
            v[0] = np.nextafter(top, f32(np.inf))
        if kind not in (2, 4, 5, 6):
            v[int(rng.integers(32))] = top * f32(rng.choice([-1.0, 1.0]))
        out[b] = v
    return out


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_mxfp8_sr_fast_path_edges(dtype):
    """SR to MXFP8 at the edges of the hardware-SR fast path, row-wise and transposed, bit-exact."""
    log(f"quantize_mxfp8 SR fast-path edges {dtype}")
    rng = np.random.default_rng(21)
    blocks = _sr_edge_blocks(rng, 64 * 8)
    if dtype == "bf16":  # round to bf16 first; both sides then see the same values
        bits = synth.bf16_bits(blocks)
        blocks = synth.bf16_to_f32(bits).reshape(blocks.shape)
    dev_in = (lambda a: bf16_t(synth.bf16_bits(a))) if dtype == "bf16" else t
    x = np.ascontiguousarray(blocks.reshape(64, 256))          # row-wise: each block along a row
    gc, gs = bsq.quantize_mxfp8(dev_in(x), "sr", seed=9, stream_id=4)
    oc, os_ = Q.quantize_mxfp8(x, Q.SR, 9, 4)
    assert np.array_equal(h(gs), os_)
    assert np.array_equal(h(gc), oc)
    xt = np.ascontiguousarray(blocks.reshape(128, 4, 32).transpose(1, 2, 0).reshape(128, 128))  # blocks along tokens
    _, n = bsq.padded_segment_layout([0, 128], 128)
    gc, gs = bsq.quantize_mxfp8(dev_in(xt), "sr", seed=9, stream_id=5, transpose=True, out_elems=n)
    oc, os_ = Q.quantize_mxfp8_transposed(xt, [0, 128], Q.SR, 9, 5)
    assert np.array_equal(h(gs), os_)
    assert np.array_equal(h(gc), oc)


# (3, 48, 64) and (2, 80, 64): 192 and 320 blocks of 16 per item, so workgroups of
# 256 blocks span two items in the NVFP4-target maximum pass
_REQ_SHAPES = [(2, 64, 128), (1, 160, 64), (3, 256, 192), (1, 48, 128), (3, 48, 64), (2, 80, 64)]


@pytest.mark.parametrize("rnd", ["rn", "sr"])
@pytest.mark.parametrize("in_mode", ["tensor", "row"])
@pytest.mark.parametrize("fmt,B,R,C", [(f, *shp) for f in ("mxfp8", "nvfp4") for shp in _REQ_SHAPES
                                       if f == "nvfp4" or shp[1] % 32 == 0])  # MXFP8 output: rows % 32 == 0
def test_requant_batch_small(fmt, rnd, in_mode, B, R, C):
    log(f"requant batch {fmt} {rnd} {in_mode} {(B, R, C)}")
    rng = np.random.default_rng(B * 1000 + R + C)
    x = _data(rng, (B, R, C), "t3")
    im = Q.OUTER_TENSOR if in_mode == "tensor" else Q.OUTER_ROW
    p, s, o = Q.quantize_nvfp4(x, im)
    of = Q.MXFP8 if fmt == "mxfp8" else Q.NVFP4
    r = Q.RN if rnd == "rn" else Q.SR
    got = bsq.requant_transpose_sr(t(p), t(s), t(np.asarray(o).reshape(-1)), in_mode, fmt, seed=99, stream_id=3, rnd=rnd)
    want = Q.requant_transpose_sr(p, s, o, im, of, 99, 3, rnd=r)
    for g, w in zip(got, want):
        assert np.array_equal(h(g), np.asarray(w).reshape(h(g).shape))


def test_requant_workload1_nvfp4_seed0():
    """Workload 1: 256x256 fp32 with outliers, NVFP4 quantize, dequantize,
    transpose, SR requantize to NVFP4 with seed 0."""
    log("requant workload1")
    X, _ = synth.workload1()
    p, s, o = Q.quantize_nvfp4(X[None], Q.OUTER_TENSOR)
    gc, gs, go = bsq.quantize_nvfp4(t(X), "tensor")
    assert np.array_equal(h(gc), p[0]) and np.array_equal(h(gs), s[0])
    rc, rs, ro = bsq.requant_transpose_sr(t(p[0]), t(s[0]), t(o), "tensor", "nvfp4", seed=0, stream_id=0)
    wc, ws, wo = Q.requant_transpose_sr(p, s, o, Q.OUTER_TENSOR, Q.NVFP4, 0, 0)
    assert np.array_equal(h(rc), wc[0]) and np.array_equal(h(rs), ws[0]) and np.array_equal(h(ro), wo)


@pytest.mark.parametrize("rnd", ["rn", "sr"])
def test_requant_gather_small(rnd):
    log(f"requant gather {rnd}")
    rng = np.random.default_rng(21)
    T, C, E, k = 300, 192, 6, 3
    x = _data(rng, (1, T, C), "normal")
    p, s, o = Q.quantize_nvfp4(x, Q.OUTER_ROW)
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :k]
    ids[ids == 4] = 5                                  # expert 4 receives nothing
    ids = np.sort(ids, axis=1)
    ok = np.all(np.diff(ids, axis=1) > 0, axis=1)
    ids = ids[ok]
    Tk = ids.shape[0]
    row_index, seg, _ = oroute(ids, E)
    r = Q.RN if rnd == "rn" else Q.SR
    _, n = bsq.padded_segment_layout(seg, C)
    gc, gs = bsq.requant_transpose_sr(t(p[0]), t(s[0]), t(o.reshape(-1)), "row", "mxfp8", seed=3, stream_id=3,
                                      rnd=rnd, row_gather=t(row_index), seg_offsets=t(seg), out_elems=n)
    wc, ws = Q.requant_transpose_sr_segmented(p[0], s[0], o.reshape(-1), Q.OUTER_ROW, row_index, seg, 3, 3, rnd=r)
    assert Tk > 0
    assert np.array_equal(h(gs), ws)
    assert np.array_equal(h(gc), wc)


def test_route_small_and_full():
    for T, E, k, wl in [(5, 4, 2, None), (1000, 16, 4, None), (16384, 64, 8, 2), (65536, 128, 8, 5)]:
        log(f"route T={T} E={E} k={k}")
        if wl is None:
            rng = np.random.default_rng(T)
            ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
        else:
            ids = synth.moe_routing(wl)
        ri, seg, pr = bsq.route(t(ids), E)
        ori, oseg, opr = oroute(ids, E)
        assert np.array_equal(h(seg), oseg)
        assert np.array_equal(h(ri), ori)
        assert np.array_equal(h(pr), opr)


def _square_oracle(x, mode, outer):
    m = {"tensor": Q.OUTER_TENSOR, "given": Q.OUTER_GIVEN}[mode]
    oc, os_, oo = Q.quantize_nvfp4_square(x, m, outer)
    oct_, ost, _ = Q.quantize_nvfp4_square(np.ascontiguousarray(x.transpose(0, 2, 1)), m, outer)
    return oc, os_, oo, oct_, ost


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["tensor", "given"])
@pytest.mark.parametrize("shape,kind", [((1, 16, 16), "normal"), ((2, 48, 80), "wide"), ((3, 144, 272), "zeros_mix"),
                                        ((1, 256, 384), "t3"), ((2, 400, 16), "normal"), ((1, 16, 400), "wide")])
def test_quantize_nvfp4_square_small(dtype, mode, shape, kind):
    """Square-tile NVFP4, both layouts, against the oracle (the transposed
    layout against the oracle run on x transposed), bit for bit; shapes span
    several 128 x 128 workgroup tiles with ragged 16-multiples."""
    log(f"quantize_nvfp4_square {dtype} {mode} {shape} {kind}")
    rng = np.random.default_rng(hash(("sq", dtype, mode, shape, kind)) % 2**32)
    x = _data(rng, shape, kind)
    if dtype == "bf16":
        bits = synth.bf16_bits(x)
        x = synth.bf16_to_f32(bits).reshape(shape)
        xd = bf16_t(bits.reshape(shape))
    else:
        xd = t(x)
    outer = (np.abs(rng.standard_normal(shape[0])) * 0.01 + 1e-3).astype(f32) if mode == "given" else None
    gc, gs, go, gct, gst = bsq.quantize_nvfp4_square(xd, mode, t(outer) if outer is not None else None)
    oc, os_, oo, oct_, ost = _square_oracle(x, mode, outer)
    assert np.array_equal(h(go), oo)
    assert np.array_equal(h(gs), os_) and np.array_equal(h(gc), oc)
    assert np.array_equal(h(gst), ost) and np.array_equal(h(gct), oct_)
    gc2, gs2, go2, n1, n2 = bsq.quantize_nvfp4_square(xd, mode, t(outer) if outer is not None else None,
                                                      transpose=False)
    assert n1 is None and n2 is None
    assert np.array_equal(h(gc2), oc) and np.array_equal(h(gs2), os_)


@pytest.mark.parametrize("dtype,shape", [("bf16", (3, 512, 1024)), ("bf16", (2, 1280, 2048)),
                                         ("bf16", (3, 1536, 3072)), ("bf16", (1, 4096, 2560)),
                                         ("f32", (2, 512, 1040)), ("f32", (1, 1024, 2560)),
                                         ("f32", (1, 4096, 2560)), ("bf16", (2, 1040, 528)),
                                         ("bf16", (10, 1024, 1024)), ("bf16", (5, 1536, 4096))])
def test_quantize_nvfp4_square_one_pass(dtype, shape):
    """Items of at least 1 MiB take the one-pass square kernel (1, 2 or 3
    units per workgroup, one or two interleaved groups, odd item counts and
    enough items per group for the steady-state pipeline, workgroups without
    a unit, ragged units); items needing more units per workgroup take the
    two-pass path. Both layouts must equal the oracle's bytes."""
    log(f"quantize_nvfp4_square tensor one-pass {dtype} {shape}")
    rng = np.random.default_rng(17 + shape[1])
    x = rng.standard_normal(shape).astype(f32)
    x[-1, 3, 7] = -250.0  # an outlier sets the last item's outer scale
    if dtype == "bf16":
        bits = synth.bf16_bits(x)
        x = synth.bf16_to_f32(bits).reshape(shape)
        xd = bf16_t(bits.reshape(shape))
    else:
        xd = t(x)
    gc, gs, go, gct, gst = bsq.quantize_nvfp4_square(xd, "tensor")
    oc, os_, oo, oct_, ost = _square_oracle(x, "tensor", None)
    assert np.array_equal(h(go), oo)
    assert np.array_equal(h(gs), os_) and np.array_equal(h(gc), oc)
    assert np.array_equal(h(gst), ost) and np.array_equal(h(gct), oct_)


def test_quantize_nvfp4_square_one_pass_wait_fallback():
    """A poll limit of 0 sends every workgroup of the one-pass square kernel that
    finds a slot unmarked through its fallback (it reduces the item itself);
    the bytes are unchanged."""
    log("quantize_nvfp4_square tensor one-pass, fallback")
    rng = np.random.default_rng(23)
    shape = (2, 512, 2048)
    bits = synth.bf16_bits(rng.standard_normal(shape).astype(f32))
    x = synth.bf16_to_f32(bits).reshape(shape)
    os.environ["BSQ_WAIT_POLLS"] = "0"
    try:
        gc, gs, go, gct, gst = bsq.quantize_nvfp4_square(bf16_t(bits.reshape(shape)), "tensor")
        torch.cuda.synchronize()
    finally:
        del os.environ["BSQ_WAIT_POLLS"]
    oc, os_, oo, oct_, ost = _square_oracle(x, "tensor", None)
    assert np.array_equal(h(go), oo)
    assert np.array_equal(h(gs), os_) and np.array_equal(h(gc), oc)
    assert np.array_equal(h(gst), ost) and np.array_equal(h(gct), oct_)


def test_quantize_nvfp4_square_outlier_figure():
    """The outlier figure's tile (one large value among values in [1, 2], outer
    scale 1): with one 16x16 scale only the outlier survives, on the GPU too."""
    log("quantize_nvfp4_square outlier figure")
    rng = np.random.default_rng(11)
    x = rng.uniform(1.0, 2.0, (16, 16)).astype(f32)
    x[15, 7] = 100.0
    gc, gs, _, gct, _ = bsq.quantize_nvfp4_square(t(x), "given", t(np.array([1.0], f32)))
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))
    assert int(np.count_nonzero(F.unpack_fp4(h(gc)) & 7)) == gold["figure3_outlier_tile"]["survive_16x16"]
    assert int(np.count_nonzero(F.unpack_fp4(h(gct)) & 7)) == gold["figure3_outlier_tile"]["survive_16x16"]


# ---------------------------------------------------------------- full sizes, sampled outputs
@pytest.fixture(scope="module")
def wl2():
    log("generate workload 2 inputs")
    return dict(x=synth.moe_activations(2), w=synth.moe_weights(2), ids=synth.moe_routing(2))


def test_quantize_nvfp4_workload2_full(wl2):
    """Activations per token, weights per expert, at full size; sampled rows
    (with the oracle's per-expert outer scale from the whole expert)."""
    log("quantize workload2 activations")
    x = wl2["x"]
    gc, gs, go = bsq.quantize_nvfp4(bf16_t(x), "row")
    rng = np.random.default_rng(20)
    rows = np.unique(np.r_[0, 1, 16383, rng.choice(16384, 256, replace=False)])
    xf = synth.bf16_to_f32(x[rows])
    oc, os_, oo = Q.quantize_nvfp4(xf[None], Q.OUTER_ROW)
    assert np.array_equal(h(gc[rows]), oc[0]) and np.array_equal(h(gs[rows]), os_[0])
    assert np.array_equal(h(go)[rows], oo[0])
    del gc, gs, go
    log("quantize workload2 weights")
    w = wl2["w"]
    gc, gs, go = bsq.quantize_nvfp4(bf16_t(w), "tensor")
    go = h(go)
    for e in range(64):  # every expert's outer scale (the whole expert's maximum)
        we = synth.bf16_to_f32(w[e])
        st = Q.outer_scale_from_amax(np.abs(we).max())
        assert go[e] == st, e
        if e in (0, 7, 18, 31, 40, 49, 58, 63):
            rows = np.unique(np.r_[0, 1535, rng.choice(1536, 14, replace=False)])
            oc, os_, _ = Q.quantize_nvfp4(we[rows][None], Q.OUTER_GIVEN, np.array([st], f32))
            assert np.array_equal(h(gc[e][rows]), oc[0]) and np.array_equal(h(gs[e][rows]), os_[0]), e


def test_quantize_nvfp4_four_over_six_workload2_full(wl2):
    """The activation quantizer of the quantized linear layer figure: per
    token, Four Over Six, at full size; sampled rows against the oracle."""
    log("quantize workload2 activations, four over six")
    x = wl2["x"]
    gc, gs, go = bsq.quantize_nvfp4(bf16_t(x), "row", four_over_six=True)
    rng = np.random.default_rng(21)
    rows = np.unique(np.r_[0, 16383, rng.choice(16384, 256, replace=False)])
    xf = synth.bf16_to_f32(x[rows])
    oc, os_, oo = Q.quantize_nvfp4(xf[None], Q.OUTER_ROW, four_over_six=True)
    assert np.array_equal(h(gs[rows]), os_[0])
    assert np.array_equal(h(gc[rows]), oc[0])
    assert np.array_equal(h(go)[rows], oo[0])


def test_requant_workload3_full(wl2):
    """64 experts of NVFP4 [1536, 4096] -> MXFP8 [4096, 1536] with seed 42; the
    input bytes come from the oracle for the checked experts."""
    log("requant workload3")
    E, N, K = 64, 1536, 4096
    rng = np.random.default_rng(3)
    from _gpu_util import filler_nvfp4
    codes, scales = filler_nvfp4(rng, (E, N), K)
    outer = np.full(E, 1e-4, f32)
    check = (0, 9, 17, 26, 38, 45, 57, 63)
    for e in check:
        we = synth.bf16_to_f32(wl2["w"][e])[None]
        p, s, o = Q.quantize_nvfp4(we, Q.OUTER_TENSOR)
        codes[e], scales[e], outer[e] = p[0], s[0], o[0]
    gc, gs = bsq.requant_transpose_sr(t(codes), t(scales), t(outer), "tensor", "mxfp8", seed=42, stream_id=0)
    for e in check:
        wc, ws = Q.requant_transpose_sr(codes[e:e + 1], scales[e:e + 1], outer[e:e + 1], Q.OUTER_TENSOR, Q.MXFP8,
                                        42, 0, item0=e)
        assert np.array_equal(h(gs[e]), ws[0]) and np.array_equal(h(gc[e]), wc[0])


def test_workload4_full_gradient_and_activation_requant(wl2):
    """Workload 4 at full size: g [131072, 1536] SR-quantized row-wise (stream 1)
    and transposed per expert (stream 2); x_q^T requantized per expert with a
    gather (stream 3); sampled rows / experts against the oracle."""
    ids = wl2["ids"]
    row_index, seg, _ = oroute(ids, 64)
    M, Cg = 131072, 1536
    log("generate workload 4 gradient")
    g = synth.output_grad(M, Cg)
    gd = bf16_t(g)
    log("quantize_mxfp8 rows workload4")
    gc, gs = bsq.quantize_mxfp8(gd, "sr", seed=42, stream_id=1)
    mp, n = bsq.padded_segment_layout(seg, Cg)
    (dc, ds), (dtc, dts) = bsq.quantize_mxfp8_dual(gd, "sr", seed=42, stream_rows=1, stream_t=2, seg_offsets=t(seg),
                                                   out_elems=n)
    rows = np.unique(np.r_[0, 3, 65535, 131071, np.random.default_rng(22).choice(M, 60, replace=False)])
    gf = synth.bf16_to_f32(g[rows])
    idx = (rows[:, None].astype(np.uint64) * np.uint64(Cg) + np.arange(Cg, dtype=np.uint64)[None, :])
    oc, os_ = Q.mxfp8_quantize(gf, idx, Q.SR, 42, 1)
    assert np.array_equal(h(gc[rows]), oc) and np.array_equal(h(gs[rows]), os_)
    assert np.array_equal(h(dc[rows]), oc) and np.array_equal(h(ds[rows]), os_)   # the one-read variant
    del gc, gs, dc, ds
    log("quantize_mxfp8 transposed workload4")
    tc, ts = bsq.quantize_mxfp8(gd, "sr", seed=42, stream_id=2, transpose=True, seg_offsets=t(seg), out_elems=n)
    tc, ts, dtc, dts = h(tc), h(ts), h(dtc), h(dts)
    _, base = Q.segmented_layout(seg, Cg)
    sel = [0, 11, 25, 40, 52, 63]
    gf = synth.bf16_to_f32(g).reshape(M, Cg)
    for e in sel:
        oc, os_ = Q.quantize_mxfp8_transposed(gf, seg, Q.SR, 42, 2, segments=[e])
        for c_, s_ in ((tc, ts), (dtc, dts)):
            assert np.array_equal(c_[base[e]:base[e] + Cg * mp[e]], oc)
            assert np.array_equal(s_[base[e] // 32:(base[e] + Cg * mp[e]) // 32], os_)
    del tc, ts, dtc, dts, gd, gf
    log("requant x_q^T gather workload4")
    T, Kx = 16384, 4096
    rng = np.random.default_rng(4)
    from _gpu_util import filler_nvfp4
    xc, xs = filler_nvfp4(rng, (T,), Kx)
    xo = np.full(T, 1e-3, f32)
    toks = np.unique(np.concatenate([row_index[seg[e]:seg[e + 1]] for e in sel]))
    p, s, o = Q.quantize_nvfp4(synth.bf16_to_f32(wl2["x"][toks])[None], Q.OUTER_ROW)
    xc[toks], xs[toks], xo[toks] = p[0], s[0], o[0]
    mpx, nx = bsq.padded_segment_layout(seg, Kx)
    rc, rs = bsq.requant_transpose_sr(t(xc), t(xs), t(xo), "row", "mxfp8", seed=42, stream_id=3, rnd="sr",
                                      row_gather=t(row_index), seg_offsets=t(seg), out_elems=nx)
    rc, rs = h(rc), h(rs)
    _, basex = Q.segmented_layout(seg, Kx)
    for e in sel:
        wc, ws = Q.requant_transpose_sr_segmented(xc, xs, xo, Q.OUTER_ROW, row_index, seg, 42, 3, segments=[e])
        assert np.array_equal(rc[basex[e]:basex[e] + Kx * mpx[e]], wc)
        assert np.array_equal(rs[basex[e] // 32:(basex[e] + Kx * mpx[e]) // 32], ws)


# ---------------------------------------------------------------- statistics and determinism
def _sr_mean_test(vals_mean, z, step, n):
    frac = np.clip((np.abs(z) - np.floor(np.abs(z) / step) * step) / step, 0, 1)
    sigma = step * np.sqrt(frac * (1 - frac))
    dev = np.abs(vals_mean - z)
    bad = dev > 4 * sigma / np.sqrt(n) + step / n + step * 2.0 ** -17
    pooled = np.sum(vals_mean - z) / np.sqrt(np.sum(sigma ** 2) / n)
    return int(bad.sum()), float(pooled)


def test_sr_unbiased_gpu_workload1():
    """Workload 1 on the GPU: the mean of the SR requantization (NVFP4 target)
    over 10^4 seeds lies within 4 sigma of the dequantized input."""
    log("SR statistics workload1 (10^4 seeds)")
    X, _ = synth.workload1()
    p, s, o = Q.quantize_nvfp4(X[None], Q.OUTER_TENSOR)
    z = Q.dequantize_nvfp4(p, s, o, Q.OUTER_TENSOR)[0].T.astype(np.float64)
    pc, ps, po = t(p[0]), t(s[0]), t(o)
    lut = torch.tensor(F.e2m1_decode(np.arange(16)), dtype=torch.float64, device=DEV)
    slut = torch.tensor(np.nan_to_num(F.e4m3_decode(np.arange(256))), dtype=torch.float64, device=DEV)
    acc = torch.zeros((256, 256), dtype=torch.float64, device=DEV)
    n = 10_000
    for seed in range(n):
        rc, rs, ro = bsq.requant_transpose_sr(pc, ps, po, "tensor", "nvfp4", seed=seed, stream_id=0)
        q = torch.stack([rc & 15, rc >> 4], dim=-1).reshape(256, 256).long()
        acc += lut[q] * slut[rs.long()].repeat_interleave(16, dim=1) * ro.double()
        if seed == 0:
            s0, st0 = h(rs), float(h(ro)[0])
    mean = h(acc) / n
    step = np.repeat(F.e4m3_decode(s0), 16, axis=1) * st0
    y = z / step
    step = step * np.where(np.abs(y) < 2, 0.5, np.where(np.abs(y) < 4, 1.0, 2.0))
    sat = np.abs(y) >= 6
    bad, pooled = _sr_mean_test(mean[~sat], z[~sat], step[~sat], n)
    assert bad <= 16, bad
    assert abs(pooled) <= 4, pooled


def test_determinism():
    log("determinism")
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 96, 4096)).astype(f32)
    a = [h(v) for v in bsq.quantize_nvfp4(t(x), "row")]
    b = [h(v) for v in bsq.quantize_nvfp4(t(x), "row")]
    assert all(np.array_equal(u, v) for u, v in zip(a, b))
    p, s, o = (t(v) for v in a)
    r1 = [h(v) for v in bsq.requant_transpose_sr(p, s, o, "row", "mxfp8", seed=9, stream_id=1)]
    r2 = [h(v) for v in bsq.requant_transpose_sr(p, s, o, "row", "mxfp8", seed=9, stream_id=1)]
    assert all(np.array_equal(u, v) for u, v in zip(r1, r2))


def test_quantize_nvfp4_square_workload2_weights_full(wl2):
    """The square-tile variant on the full expert weights [64, 1536, 4096]
    (bf16, per-expert outer scale): sampled experts against the oracle in
    both layouts, and on every expert the transposed codes and scales are the
    transpose of the row-major ones (the property the square tile exists for)."""
    log("quantize_nvfp4_square workload2 weights")
    w = wl2["w"]
    gc, gs, go, gct, gst = bsq.quantize_nvfp4_square(bf16_t(w), "tensor")
    for e in (0, 29, 63):
        we = synth.bf16_to_f32(w[e])[None]
        oc, os_, oo, oct_, ost = _square_oracle(we, "tensor", None)
        assert np.array_equal(h(go)[e:e + 1], oo)
        assert np.array_equal(h(gs[e]), os_[0]) and np.array_equal(h(gc[e]), oc[0])
        assert np.array_equal(h(gst[e]), ost[0]) and np.array_equal(h(gct[e]), oct_[0])
    for e0 in range(0, 64, 16):
        c = gc[e0:e0 + 16]
        ct = gct[e0:e0 + 16]
        lo = torch.stack([c & 15, c >> 4], dim=-1).flatten(-2)       # [16, 1536, 4096] nibbles
        lot = torch.stack([ct & 15, ct >> 4], dim=-1).flatten(-2)    # [16, 4096, 1536]
        assert torch.equal(lot, lo.transpose(1, 2))
        del lo, lot
    gs_tiles = gs[:, ::16, :]                                          # [64, 96, 256]
    assert torch.equal(gs, gs_tiles.repeat_interleave(16, dim=1))
    assert torch.equal(gst, gs_tiles.transpose(1, 2).repeat_interleave(16, dim=1))   # [64, 4096, 96]
