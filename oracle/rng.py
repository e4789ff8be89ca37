"""Counter-based random numbers for stochastic rounding.

The pages define stochastic rounding only as rounding up or down with
probabilities inversely proportional to the distances to the two neighbours
(section "Re-quantization with stochastic rounding"). They do not name a
generator. This oracle fixes one published counter-based generator so that
the GPU output is reproducible bit-for-bit:

  Philox4x32-10 (J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw,
  "Parallel random numbers: as easy as 1, 2, 3", SC'11).  One round maps a
  4x32-bit counter (c0, c1, c2, c3) under a 2x32-bit key (k0, k1) to
      (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0))
  with M0 = 0xD2511F53, M1 = 0xCD9E8D57; between rounds the key is bumped by
  (0x9E3779B9, 0xBB67AE85).  Ten rounds.

Mapping used by every stochastic rounding in this project (a reading; the
pages leave it open): for a 64-bit linear element index ``idx`` in the OUTPUT
tensor, a 64-bit ``seed`` and a 64-bit ``stream`` id,
  key     = (seed mod 2^32, seed >> 32)
  counter = ((idx >> 3) mod 2^32, (idx >> 3) >> 32, stream mod 2^32, stream >> 32)
  word    = output[(idx >> 1) & 3]
  r       = (word >> (16 * (idx & 1))) & 0xFFFF          (16 random bits)
  u       = (r + 1/2) / 2^16                              (uniform in (0, 1))
so one generator call serves eight consecutive output elements.
"""
import numpy as np

M0 = np.uint64(0xD2511F53)
M1 = np.uint64(0xCD9E8D57)
W0 = 0x9E3779B9
W1 = 0xBB67AE85
MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x32-10. Counter words are arrays (or scalars) of
    values < 2^32; key words are Python ints. Returns four uint32 arrays."""
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) & MASK32 for c in (c0, c1, c2, c3))
    k0 = int(k0) & 0xFFFFFFFF
    k1 = int(k1) & 0xFFFFFFFF
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + W0) & 0xFFFFFFFF
            k1 = (k1 + W1) & 0xFFFFFFFF
        p0 = M0 * c0                         # exact: both factors < 2^32
        p1 = M1 * c2
        n0 = (p1 >> np.uint64(32)) ^ c1 ^ np.uint64(k0)
        n1 = p1 & MASK32
        n2 = (p0 >> np.uint64(32)) ^ c3 ^ np.uint64(k1)
        n3 = p0 & MASK32
        c0, c1, c2, c3 = n0, n1, n2, n3
    return tuple(c.astype(np.uint32) for c in (c0, c1, c2, c3))


def sr_bits16(seed, stream, idx):
    """16 random bits for each 64-bit output index in ``idx`` (array)."""
    idx = np.asarray(idx, dtype=np.uint64)
    grp = idx >> np.uint64(3)
    seed = int(seed)
    stream = int(stream)
    w = philox4x32_10(grp & MASK32, grp >> np.uint64(32),
                      np.full(idx.shape, stream & 0xFFFFFFFF, dtype=np.uint64),
                      np.full(idx.shape, (stream >> 32) & 0xFFFFFFFF, dtype=np.uint64),
                      seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    words = np.stack(w, axis=-1)                               # [..., 4]
    sel = ((idx >> np.uint64(1)) & np.uint64(3)).astype(np.int64)
    word = np.take_along_axis(words, sel[..., None], axis=-1)[..., 0].astype(np.uint64)
    shift = (np.uint64(16) * (idx & np.uint64(1)))
    return ((word >> shift) & np.uint64(0xFFFF)).astype(np.int64)


def sr_uniform(seed, stream, idx):
    """u = (r + 1/2) / 2^16 in float64 (exact)."""
    return (sr_bits16(seed, stream, idx).astype(np.float64) + 0.5) / 65536.0
