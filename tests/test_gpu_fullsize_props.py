"""Every output byte of the step's stochastically rounded MXFP8 quantizers at
full size (the expert weights' requantization and the gradient's and the
activations' transposed quantizations), checked by properties that any
correct result has ("Re-quantization with stochastic rounding"):

* each block's E8M0 scale is the oracle's exponent rule applied to the
  block's largest magnitude;
* each code decodes to one of the two E4M3 grid neighbours of its scaled
  input (to the input itself when that lies on the grid), with the input's
  sign; the padding of every expert segment is therefore +0;
* over a whole tensor the rounding errors sum to zero within the bound of
  unbiased rounding (6 sigma, plus the 16-bit draw's resolution).

The exact draws are compared with the oracle on sampled outputs in
test_gpu_quant.py; these checks reach every other byte. Inputs are the
seeded synthetic workloads and random valid NVFP4 bytes; the expected
properties come from the oracle's dequantization and exponent rule and from
float64 torch arithmetic, never from the kernels."""
import numpy as np
import pytest
import torch

import block_scaled_bit_quantize_amd as bsq
import synth
from oracle import formats as F
from oracle import quant as Q
from oracle.route import route as oroute

from _gpu_util import DEV, bf16_t, filler_nvfp4, h, log, t

pytestmark = pytest.mark.gpu


class _Sums:
    """Rounding-error sums over one tensor (the unbiasedness bound)."""

    def __init__(self, name):
        self.name, self.err, self.var, self.slack, self.n = name, 0.0, 0.0, 0.0, 0

    def check(self):
        bound = 6.0 * self.var ** 0.5 + self.slack
        log(f"{self.name}: {self.n} values, error sum {self.err:.4g} (bound {bound:.4g})")
        assert abs(self.err) <= bound, (self.name, self.err, bound)


def _check_mx(codes, scales, z, sums):
    """codes uint8 [N, L] and scales uint8 [N, L/32] (device), z float32
    [N, L] (device): the values the quantizer rounds, in the output layout."""
    grid = torch.tensor(F.E4M3_VAL, dtype=torch.float64, device=DEV)  # codes 0x00..0x7E, ascending
    N, L = z.shape
    amax = z.abs().reshape(N, L // 32, 32).amax(-1)
    e = torch.from_numpy(Q.e8m0_exponent(amax.cpu().numpy()).astype(np.int64)).to(DEV)
    assert torch.equal(scales.reshape(N, L // 32).long(), e + 127), sums.name
    y = z.double() * torch.pow(2.0, -e.double()).repeat_interleave(32, dim=1)  # exact
    m = y.abs()
    lo = torch.searchsorted(grid, m.contiguous(), right=True) - 1
    hi = torch.clamp(lo + 1, max=grid.numel() - 1)
    exact = grid[lo] == m
    c = codes.reshape(N, L)
    cm = (c & 0x7F).long()
    ok = (cm == lo) | ((cm == hi) & ~exact)
    assert bool(ok.all()), (sums.name, int((~ok).sum()))
    assert torch.equal((c >> 7).bool(), torch.signbit(y)), sums.name
    step = torch.where(exact, torch.ones_like(m), grid[hi] - grid[lo])
    d = torch.where(exact, torch.zeros_like(m), (m - grid[lo]) / step)
    sums.err += float((grid[cm] - m).sum())
    sums.var += float((step * step * d * (1.0 - d)).sum())
    sums.slack += float(torch.where(exact, torch.zeros_like(m), step).sum()) * 2.0 ** -16
    sums.n += N * L


def test_requant_weights_fullsize_properties():
    """64 experts of NVFP4 [1536, 4096] -> MXFP8 [4096, 1536] (seed 42), every
    expert from random valid NVFP4 bytes."""
    log("fullsize requant weights")
    E, N, K = 64, 1536, 4096
    rng = np.random.default_rng(33)
    codes, scales = filler_nvfp4(rng, (E, N), K)
    outer = rng.uniform(1e-5, 1e-3, E).astype(np.float32)
    gc, gs = bsq.requant_transpose_sr(t(codes), t(scales), t(outer), "tensor", "mxfp8", seed=42, stream_id=0)
    sums = _Sums("requant weights")
    for e in range(E):
        z = Q.dequantize_nvfp4(codes[e:e + 1], scales[e:e + 1], outer[e:e + 1], Q.OUTER_TENSOR)[0]
        _check_mx(gc[e], gs[e], t(np.ascontiguousarray(z.T)), sums)
    sums.check()


def test_gradient_and_activation_fullsize_properties():
    """The backward's operands at full size: g [131072, 1536] row-wise (stream
    1) and transposed per expert segment (stream 2), and the gathered token
    rows of x_q (random valid NVFP4 bytes, per-token outer scales) transposed
    per expert segment (stream 3), with the step's routing."""
    ids = synth.moe_routing(2)
    row_index, seg, _ = oroute(ids, 64)
    M, Cg = 131072, 1536
    log("fullsize gradient: generate")
    g = synth.output_grad(M, Cg)
    gd = bf16_t(g)
    gz = gd.float()
    log("fullsize gradient rows")
    gc, gs = bsq.quantize_mxfp8(gd, "sr", seed=42, stream_id=1)
    sums = _Sums("gradient rows")
    for r0 in range(0, M, 16384):
        _check_mx(gc[r0:r0 + 16384], gs[r0:r0 + 16384], gz[r0:r0 + 16384], sums)
    sums.check()
    del gc, gs

    def per_segment(codes, scales, rows_of, C, name):
        mp, base = Q.segmented_layout(seg, C)
        sums = _Sums(name)
        for e in range(64):
            Me = int(seg[e + 1] - seg[e])
            Z = torch.zeros((C, mp[e]), dtype=torch.float32, device=DEV)
            Z[:, :Me] = rows_of(int(seg[e]), int(seg[e + 1])).T
            b = int(base[e])
            _check_mx(codes[b:b + C * mp[e]], scales[b // 32:(b + C * mp[e]) // 32], Z, sums)
        assert int(base[-1]) == codes.numel()
        sums.check()

    log("fullsize gradient transposed")
    _, n = bsq.padded_segment_layout(seg, Cg)
    tc, ts = bsq.quantize_mxfp8(gd, "sr", seed=42, stream_id=2, transpose=True, seg_offsets=t(seg), out_elems=n)
    per_segment(tc, ts, lambda a, b: gz[a:b], Cg, "gradient transposed")
    del tc, ts, gd, gz

    log("fullsize activations transposed with gather")
    T, Kx = 16384, 4096
    rng = np.random.default_rng(44)
    xc, xs = filler_nvfp4(rng, (T,), Kx)
    xo = rng.uniform(1e-4, 1e-2, T).astype(np.float32)
    zx = t(Q.dequantize_nvfp4(xc[None], xs[None], xo.reshape(1, -1), Q.OUTER_ROW)[0])
    _, nx = bsq.padded_segment_layout(seg, Kx)
    rc, rs = bsq.requant_transpose_sr(t(xc), t(xs), t(xo), "row", "mxfp8", seed=42, stream_id=3, rnd="sr",
                                      row_gather=t(row_index), seg_offsets=t(seg), out_elems=nx)
    ri = t(row_index.astype(np.int64))
    per_segment(rc, rs, lambda a, b: zx[ri[a:b]], Kx, "activations transposed")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_transposed_mxfp8_max_cols(dtype):
    """The transposed quantizer and the one-read dual at their largest column
    count (2^22: a float32 tile's row offsets reach 127 * 2^24 bytes), 160
    rows in two ragged segments: every output by the properties above, 64
    sampled channels bit-exact against the oracle's draws, and the dual equal
    to the two separate calls."""
    C = 1 << 22
    seg = np.array([0, 37, 160], dtype=np.int64)
    log(f"max cols transposed mxfp8 {dtype}")
    g = torch.Generator(device=DEV)
    g.manual_seed(2024)
    x = (torch.randn((160, C), generator=g, device=DEV) * 3e-3).to(dtype)
    mp, n = bsq.padded_segment_layout(seg, C)
    _, base = Q.segmented_layout(seg, C)
    sd = t(seg)
    tc, ts = bsq.quantize_mxfp8(x, "sr", seed=7, stream_id=2, transpose=True, seg_offsets=sd, out_elems=n)
    xf = x.float()
    sums = _Sums(f"max cols {dtype}")
    for e in range(2):
        a, b = int(seg[e]), int(seg[e + 1])
        for c0 in range(0, C, 1 << 20):
            Z = torch.zeros((1 << 20, mp[e]), dtype=torch.float32, device=DEV)
            Z[:, :b - a] = xf[a:b, c0:c0 + (1 << 20)].T
            lo = int(base[e]) + c0 * mp[e]
            hi = lo + (1 << 20) * mp[e]
            _check_mx(tc[lo:hi], ts[lo // 32:hi // 32], Z, sums)
    sums.check()
    rng = np.random.default_rng(5)
    chans = np.unique(np.r_[0, C - 1, rng.integers(0, C, 62)])
    tch, tsh = h(tc), h(ts)
    for e in range(2):
        a, b = int(seg[e]), int(seg[e + 1])
        zc = np.zeros((len(chans), mp[e]), dtype=np.float32)
        zc[:, :b - a] = h(xf[a:b][:, t(chans)]).T
        idx = (np.uint64(base[e]) + chans.astype(np.uint64)[:, None] * np.uint64(mp[e])
               + np.arange(mp[e], dtype=np.uint64)[None, :])
        oc, os_ = Q.mxfp8_quantize(zc, idx, Q.SR, 7, 2)
        for i, c in enumerate(chans):
            lo = int(base[e]) + int(c) * mp[e]
            assert np.array_equal(tch[lo:lo + mp[e]], oc[i]), (e, c)
            assert np.array_equal(tsh[lo // 32:(lo + mp[e]) // 32], os_[i]), (e, c)
    del tch, tsh
    rc, rs = bsq.quantize_mxfp8(x, "sr", seed=7, stream_id=1)
    (dc, ds), (dtc, dts) = bsq.quantize_mxfp8_dual(x, "sr", seed=7, stream_rows=1, stream_t=2, seg_offsets=sd,
                                                   out_elems=n)
    assert torch.equal(dc, rc) and torch.equal(ds, rs)
    assert torch.equal(dtc, tc) and torch.equal(dts, ts)
