"""Pins of the oracle's generator: published known-answer vectors and the
uniformity of the 16-bit draws."""
import json
import os

import numpy as np

from oracle.rng import philox4x32_10, sr_bits16, sr_uniform

KAT = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.json")))


def test_philox_known_answers():
    for v in KAT["vectors"]:
        c = [int(x, 16) for x in v["ctr"]]
        k = [int(x, 16) for x in v["key"]]
        out = philox4x32_10(*c, *k)
        assert [int(o) for o in out] == [int(x, 16) for x in v["out"]]


def test_word_mapping():
    # eight consecutive indices share one generator call; index i takes half i&1 of word (i>>1)&3
    seed, stream = 0x123456789ABCDEF0, 77
    idx = np.arange(16, dtype=np.uint64) + np.uint64(8 * 1000)
    r = sr_bits16(seed, stream, idx)
    w = philox4x32_10(1000, 0, stream, 0, seed & 0xFFFFFFFF, seed >> 32)
    w2 = philox4x32_10(1001, 0, stream, 0, seed & 0xFFFFFFFF, seed >> 32)
    for i in range(8):
        word = int(w[i >> 1])
        assert r[i] == (word >> (16 * (i & 1))) & 0xFFFF
        assert r[8 + i] == (int(w2[i >> 1]) >> (16 * (i & 1))) & 0xFFFF
    # high index bits and the stream id change the draw
    big = np.array([8 * (1 << 33)], dtype=np.uint64)
    w3 = philox4x32_10(0, 2, stream, 0, seed & 0xFFFFFFFF, seed >> 32)
    assert sr_bits16(seed, stream, big)[0] == int(w3[0]) & 0xFFFF


def test_uniformity_chi2():
    r = sr_bits16(42, 1, np.arange(1 << 20, dtype=np.uint64))
    hist = np.bincount(r >> 8, minlength=256)              # 256 bins, 4096 expected each
    chi2 = float(np.sum((hist - 4096.0) ** 2 / 4096.0))
    # 255 degrees of freedom: mean 255, sd 22.6; 6 sd bounds
    assert 255 - 6 * 22.6 < chi2 < 255 + 6 * 22.6
    u = sr_uniform(42, 1, np.arange(1 << 16, dtype=np.uint64))
    assert u.min() > 0 and u.max() < 1
