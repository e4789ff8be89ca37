"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, and rejects invalid arguments on the host before any HIP
call (the documented status codes)."""
import ctypes
import os
import re

import pytest

from block_scaled_bit_quantize_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsq.h")

OK, E_NULL, E_SHAPE, E_ALIGN, E_DTYPE, E_ENUM, E_WORKSPACE, E_LAUNCH = range(8)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.library_path()):
        from block_scaled_bit_quantize_amd.build import build
        build()
    return _lib.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsq_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, f"binding lacks {n}"
    assert set(_lib.SIGNATURES) == set(names)


def test_status_strings_and_version(lib):
    for s in range(8):
        assert lib.bsq_status_string(s)
    assert lib.bsq_status_string(99) == b"unknown status"
    assert lib.bsq_version() == 100


FAKE = 0x10000  # a 16-byte aligned non-null value; never dereferenced on these paths


def test_quantize_nvfp4_validation(lib):
    q = lib.bsq_quantize_nvfp4
    assert q(FAKE, 7, 1, 1, 16, 0, None, FAKE, FAKE, FAKE, FAKE, 256, None) == E_DTYPE
    assert q(FAKE, 1, 1, 1, 16, 9, None, FAKE, FAKE, FAKE, FAKE, 256, None) == E_ENUM
    assert q(FAKE, 1, 1, 1, 24, 1, None, FAKE, FAKE, FAKE, None, 0, None) == E_SHAPE
    assert q(FAKE, 1, 1, 1, 32784, 1, None, FAKE, FAKE, FAKE, None, 0, None) == E_SHAPE
    assert q(FAKE, 1, -1, 1, 16, 1, None, FAKE, FAKE, FAKE, None, 0, None) == E_SHAPE
    assert q(None, 1, 1, 1, 16, 1, None, FAKE, FAKE, FAKE, None, 0, None) == E_NULL
    assert q(FAKE, 1, 1, 1, 16, 2, None, FAKE, FAKE, FAKE, None, 0, None) == E_NULL      # GIVEN needs outer_in
    assert q(FAKE + 8, 1, 1, 1, 16, 1, None, FAKE, FAKE, FAKE, None, 0, None) == E_ALIGN
    assert q(FAKE, 1, 1, 1, 16, 0, None, FAKE, FAKE, FAKE, None, 0, None) == E_NULL      # TENSOR needs ws
    assert q(FAKE, 1, 1, 1, 16, 0, None, FAKE, FAKE, FAKE, FAKE, 4, None) == E_WORKSPACE
    assert q(None, 1, 0, 1, 16, 1, None, None, None, None, None, 0, None) == OK          # empty batch: no work
    assert lib.bsq_quantize_nvfp4_workspace(3, 4, 16, 0) >= 12
    assert lib.bsq_quantize_nvfp4_workspace(3, 4, 16, 1) == 0


def test_quantize_nvfp4_square_validation(lib):
    q = lib.bsq_quantize_nvfp4_square
    # x, dtype, B, R, C, mode, outer_in, codes, scales, codes_t, scales_t, outer_out, ws, ws_bytes, stream
    assert q(FAKE, 7, 1, 16, 16, 2, FAKE, FAKE, FAKE, None, None, FAKE, None, 0, None) == E_DTYPE
    assert q(FAKE, 1, 1, 16, 16, 1, None, FAKE, FAKE, None, None, FAKE, None, 0, None) == E_ENUM   # per-row
    assert q(FAKE, 1, 1, 16, 16, 16, FAKE, FAKE, FAKE, None, None, FAKE, None, 0, None) == E_ENUM  # a flag
    assert q(FAKE, 1, 1, 24, 16, 2, FAKE, FAKE, FAKE, None, None, FAKE, None, 0, None) == E_SHAPE
    assert q(FAKE, 1, 1, 16, 8, 2, FAKE, FAKE, FAKE, None, None, FAKE, None, 0, None) == E_SHAPE
    assert q(FAKE, 1, 1, 2 ** 32, 16, 2, FAKE, FAKE, FAKE, None, None, FAKE, None, 0, None) == E_SHAPE
    assert q(FAKE, 1, 1, 16, 16, 2, None, FAKE, FAKE, None, None, FAKE, None, 0, None) == E_NULL   # GIVEN needs outer_in
    assert q(FAKE, 1, 1, 16, 16, 2, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, 0, None) == E_NULL   # codes_t alone
    assert q(FAKE, 1, 1, 16, 16, 2, FAKE, FAKE, FAKE, FAKE + 8, FAKE, FAKE, None, 0, None) == E_ALIGN
    assert q(FAKE, 1, 1, 16, 16, 0, None, FAKE, FAKE, None, None, FAKE, None, 0, None) == E_NULL   # TENSOR needs ws
    assert q(FAKE, 1, 1, 16, 16, 0, None, FAKE, FAKE, None, None, FAKE, FAKE, 4, None) == E_WORKSPACE
    assert q(None, 1, 0, 16, 16, 0, None, None, None, None, None, None, None, 0, None) == OK      # empty batch
    assert lib.bsq_quantize_nvfp4_square_workspace(3, 16, 16, 0) >= 12
    assert lib.bsq_quantize_nvfp4_square_workspace(3, 1024, 1024, 0) >= 3 * 4 * 256
    assert lib.bsq_quantize_nvfp4_square_workspace(3, 1024, 1024, 2) == 0


def test_codec_validation(lib):
    e = lib.bsq_rht_s2f6_encode
    assert e(FAKE, 7, 1, 32, 0, FAKE, FAKE, None) == E_DTYPE
    assert e(FAKE, 1, 1, 48, 0, FAKE, FAKE, None) == E_SHAPE
    assert e(FAKE, 1, -1, 32, 0, FAKE, FAKE, None) == E_SHAPE
    assert e(FAKE, 1, 2 ** 40, 2 ** 20, 0, FAKE, FAKE, None) == E_SHAPE
    assert e(None, 1, 1, 32, 0, FAKE, FAKE, None) == E_NULL
    assert e(FAKE + 8, 1, 1, 32, 0, FAKE, FAKE, None) == E_ALIGN
    assert e(None, 1, 0, 32, 0, None, None, None) == OK                       # empty: no work
    c = lib.bsq_rht_s2f6_combine
    # codes, scales, rows, cols, pair_row, tokens, k, signs, out, out_dtype, stream
    assert c(FAKE, FAKE, 4, 32, FAKE, 2, 2, 0, FAKE, 9, None) == E_DTYPE
    assert c(FAKE, FAKE, 4, 40, FAKE, 2, 2, 0, FAKE, 1, None) == E_SHAPE
    assert c(FAKE, FAKE, 4, 32, FAKE, 2, 0, 0, FAKE, 1, None) == E_SHAPE       # k >= 1
    assert c(FAKE, FAKE, 4, 32, FAKE, 2, 65, 0, FAKE, 1, None) == E_SHAPE      # k <= 64
    assert c(FAKE, FAKE, 0, 32, FAKE, 2, 2, 0, FAKE, 1, None) == E_SHAPE       # tokens need rows
    assert c(FAKE, FAKE, 4, 32, None, 2, 2, 0, FAKE, 1, None) == E_NULL
    assert c(FAKE, FAKE, 4, 32, FAKE + 2, 2, 2, 0, FAKE, 1, None) == E_ALIGN
    assert c(None, None, 4, 32, None, 0, 2, 0, None, 1, None) == OK            # no tokens: no work


def test_chain_entries_validation(lib):
    q = lib.bsq_swiglu_quantize_nvfp4
    # h13, dtype, rows, ffn, flags, codes, scales, outer_out, stream
    assert q(FAKE, 7, 4, 16, 0, FAKE, FAKE, FAKE, None) == E_DTYPE
    assert q(FAKE, 1, 4, 16, 1, FAKE, FAKE, FAKE, None) == E_ENUM               # only the Four Over Six flag
    assert q(FAKE, 1, 4, 24, 0, FAKE, FAKE, FAKE, None) == E_SHAPE
    assert q(FAKE, 1, 4, 32784, 0, FAKE, FAKE, FAKE, None) == E_SHAPE
    assert q(None, 1, 4, 16, 16, FAKE, FAKE, FAKE, None) == E_NULL
    assert q(FAKE + 8, 1, 4, 16, 0, FAKE, FAKE, FAKE, None) == E_ALIGN
    assert q(None, 1, 0, 16, 0, None, None, None, None) == OK                  # no rows: no work
    g = lib.bsq_grouped_gemm_nvfp4_s2f6
    # a_codes, a_scales, a_outer, per_row, a_rows, row_index, b_codes, b_scales, b_outer, seg, E, M, N, K,
    # signs, out_codes, out_scales, stream
    base = [FAKE, FAKE, FAKE, 1, 8, None, FAKE, FAKE, FAKE, FAKE, 2, 8, 256, 64, 0, FAKE, FAKE, None]
    def call(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return g(*a)
    assert call(a12=100) == E_SHAPE                                              # N % 256
    assert call(a13=48) == E_SHAPE                                               # K % 64
    assert call(a10=0) == E_SHAPE                                                # E >= 1
    assert call(a16=None) == E_NULL
    assert call(a15=FAKE + 8) == E_ALIGN
    assert call(a11=0) == OK                                                     # no rows: no work


def test_quantize_mxfp8_validation(lib):
    q = lib.bsq_quantize_mxfp8
    assert q(FAKE, 1, 4, 48, 0, None, 0, 1, 0, 0, FAKE, FAKE, None, 0, None) == E_SHAPE
    assert q(FAKE, 1, 4, 64, 0, None, 0, 5, 0, 0, FAKE, FAKE, None, 0, None) == E_ENUM
    assert q(FAKE, 3, 4, 64, 0, None, 0, 1, 0, 0, FAKE, FAKE, None, 0, None) == E_DTYPE
    assert q(FAKE, 1, 4, 64, 2, None, 0, 1, 0, 0, FAKE, FAKE, None, 0, None) == E_ENUM
    assert q(FAKE, 1, 4, 96, 1, None, 0, 1, 0, 0, FAKE, FAKE, FAKE, 1 << 20, None) == E_SHAPE   # cols % 64
    assert q(FAKE, 1, 4, (1 << 22) + 64, 1, None, 0, 1, 0, 0, FAKE, FAKE, FAKE, 1 << 20, None) == E_SHAPE  # cols <= 2^22
    assert q(FAKE, 1, 4, 64, 1, FAKE, 0, 1, 0, 0, FAKE, FAKE, FAKE, 1 << 20, None) == E_SHAPE   # 0 segments
    assert q(FAKE, 1, 4, 64, 1, None, 0, 1, 0, 0, FAKE, FAKE, None, 0, None) == E_NULL
    assert q(FAKE, 1, 4, 64, 1, None, 0, 1, 0, 0, FAKE, FAKE, FAKE, 8, None) == E_WORKSPACE
    assert q(FAKE, 1, 4, 64, 0, None, 0, 1, 0, 0, FAKE + 4, FAKE, None, 0, None) == E_ALIGN
    d = lib.bsq_quantize_mxfp8_dual  # x, dtype, rows, cols, seg, nseg, rnd, seed, s_rows, s_t, c, s, c_t, s_t, ws, wsb
    ok = [FAKE, 1, 4, 64, None, 0, 1, 0, 1, 2, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None]
    def dcall(i, v):
        a = list(ok); a[i] = v; return d(*a)
    assert dcall(3, 96) == E_SHAPE            # cols % 64
    assert dcall(3, (1 << 22) + 64) == E_SHAPE  # cols <= 2^22
    assert dcall(4, FAKE) == E_SHAPE          # seg_offsets with 0 segments
    assert dcall(6, 5) == E_ENUM
    assert dcall(1, 3) == E_DTYPE
    assert dcall(12, None) == E_NULL          # codes_t
    assert dcall(10, None) == E_NULL          # row codes
    assert dcall(10, FAKE + 4) == E_ALIGN
    assert dcall(15, 8) == E_WORKSPACE
    assert dcall(2, 0) == OK                  # empty


def test_requant_validation(lib):
    r = lib.bsq_requant_transpose_sr
    args = lambda **kw: [kw.get(k, v) for k, v in [
        ("codes", FAKE), ("scales", FAKE), ("outer", FAKE), ("in_mode", 0), ("batch", 1), ("rows", 64),
        ("cols", 64), ("in_rows", 64), ("gather", None), ("seg", None), ("nseg", 0), ("fmt", 1), ("rnd", 1),
        ("seed", 0), ("sid", 0), ("oc", FAKE), ("os", FAKE), ("oo", FAKE), ("ws", FAKE), ("wsb", 1 << 20),
        ("stream", None)]]
    assert r(*args(in_mode=2)) == E_ENUM
    assert r(*args(fmt=3)) == E_ENUM
    assert r(*args(rnd=4)) == E_ENUM
    assert r(*args(cols=96)) == E_SHAPE
    assert r(*args(rows=48)) == E_SHAPE                        # MXFP8 needs rows % 32
    assert r(*args(in_rows=65)) == E_SHAPE
    assert r(*args(codes=None)) == E_NULL
    assert r(*args(oc=FAKE + 1)) == E_ALIGN
    assert r(*args(fmt=0, oo=None)) == E_NULL
    assert r(*args(fmt=0, wsb=0)) == E_WORKSPACE
    assert r(*args(gather=FAKE)) == E_NULL                     # gather needs seg_offsets
    assert r(*args(gather=FAKE, seg=FAKE, nseg=2, fmt=0)) == E_SHAPE
    assert r(*args(gather=FAKE, seg=FAKE, nseg=2, wsb=16)) == E_WORKSPACE


def test_gemm_and_route_validation(lib):
    g = lib.bsq_grouped_gemm_nvfp4
    base = [FAKE, FAKE, FAKE, 1, 8, None, FAKE, FAKE, FAKE, FAKE, 2, 16, 256, 256, FAKE, 1, None]
    def call(i, v):
        a = list(base); a[i] = v; return g(*a)
    assert call(12, 200) == E_SHAPE          # N % 256
    assert call(13, 96) == E_SHAPE           # K % 64
    assert call(10, 0) == E_SHAPE            # E >= 1
    assert call(0, None) == E_NULL
    assert call(14, FAKE + 2) == E_ALIGN
    assert call(15, 7) == E_DTYPE
    m = lib.bsq_grouped_gemm_mxfp8
    assert m(2, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 256, 256, 128, FAKE, 1, None) == E_ENUM
    assert m(0, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 256, 256, 100, FAKE, 1, None) == E_SHAPE
    assert m(1, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 200, 256, 0, FAKE, 0, None) == E_SHAPE
    assert m(0, FAKE, None, FAKE, FAKE, FAKE, 2, 256, 256, 128, FAKE, 1, None) == E_NULL
    assert m(0, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 256, 256, 128, FAKE, 5, None) == E_DTYPE
    ir = lib.bsq_gemm_nvfp4_inreg_scale
    assert ir(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 100, 128, 64, FAKE, None) == E_SHAPE     # M % 128
    assert ir(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 128, 128, 32, FAKE, None) == E_SHAPE     # K % 64
    assert ir(FAKE, FAKE, FAKE, None, FAKE, FAKE, 128, 128, 64, FAKE, None) == E_NULL
    assert ir(FAKE, FAKE + 1, FAKE, FAKE, FAKE, FAKE, 128, 128, 64, FAKE, None) == E_ALIGN
    assert ir(None, None, None, None, None, None, 0, 128, 64, None, None) == 0              # empty
    rt = lib.bsq_route
    assert rt(FAKE, 10, 0, 4, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == E_SHAPE
    assert rt(FAKE, 10, 2, 2000, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == E_SHAPE
    assert rt(FAKE, 10, 2, 4, FAKE, None, FAKE, FAKE, 1 << 20, None) == E_NULL
    assert rt(FAKE, 10, 2, 4, FAKE, FAKE, FAKE, FAKE, 4, None) == E_WORKSPACE
    rn = lib.bsq_route_noalloc  # checked before any device call
    assert rn(FAKE, 10, 0, 4, FAKE, FAKE, FAKE, None) == E_SHAPE
    assert rn(FAKE, 10, 2, 4, FAKE, None, FAKE, None) == E_NULL
    assert rn(None, 10, 2, 4, FAKE, FAKE, FAKE, None) == E_NULL
    # counts need ceil(T / 256) * E int32 slots: 1 MiB holds 4096 chunks at E = 64
    assert rn(FAKE, 4096 * 256 + 1, 1, 64, FAKE, FAKE, FAKE, None) == E_WORKSPACE
    assert rn(FAKE, 256 * 256 + 1, 1, 1024, FAKE, FAKE, FAKE, None) == E_WORKSPACE
    assert lib.bsq_route_workspace(4096 * 256, 64) == _lib.ROUTE_NOALLOC_MAX_BYTES


def test_mfma_rate_probe_validation(lib):
    p = lib.bsq_mfma_rate_probe  # checked before any device call
    assert p(5, 0, 10, 8, FAKE, None) == E_ENUM
    assert p(0, 3, 10, 8, FAKE, None) == E_ENUM
    assert p(0, 0, 0, 8, FAKE, None) == E_SHAPE
    assert p(0, 0, 10, 0, FAKE, None) == E_SHAPE
    assert p(0, 0, 10, 70000, FAKE, None) == E_SHAPE
    assert p(0, 0, 10, 8, None, None) == E_NULL
    assert p(0, 0, 10, 8, FAKE + 2, None) == E_ALIGN
