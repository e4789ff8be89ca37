"""bsq_route_noalloc (routing into a library-owned device array, for callers
that cannot allocate) against bsq_route on the same inputs: two calls in a
row, the second smaller, every output bit-exact."""
import numpy as np
import pytest
import torch

import block_scaled_bit_quantize_amd as bsq
import synth
from _gpu_util import DEV, h, log, t

pytestmark = pytest.mark.gpu


def _noalloc(ids, E):
    T, k = ids.shape
    ri = torch.full((T * k,), -7, dtype=torch.int32, device=DEV)
    pr = torch.full((T * k,), -7, dtype=torch.int32, device=DEV)
    seg = torch.full((E + 1,), -7, dtype=torch.int64, device=DEV)
    return bsq.route_noalloc(ids, E, ri, seg, pr)


def test_route_noalloc_matches_route_twice():
    # 16384 tokens top-8 of 64 experts (the MoE step's routing), then a
    # smaller ragged case with more experts, then an empty one
    cases = [(synth.moe_routing(2), 64)]
    rng = np.random.default_rng(11)
    T2, k2, E2 = 3001, 4, 96
    ids2 = np.argsort(rng.random((T2, E2)), axis=1)[:, :k2].astype(np.int32)
    cases.append((ids2, E2))
    cases.append((np.zeros((0, 2), dtype=np.int32), 8))
    for ids, E in cases:
        log(f"route_noalloc T={ids.shape[0]} k={ids.shape[1]} E={E}")
        d = t(ids)
        want = bsq.route(d, E)
        got = _noalloc(d, E)
        torch.cuda.synchronize()
        for w, g in zip(want, got):
            np.testing.assert_array_equal(h(g), h(w))
