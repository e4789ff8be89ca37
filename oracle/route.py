"""Routing of tokens to expert segments.

Page: "End-to-End 4-Bit Training", section "Quantized communications": a
router decides where each token goes and tokens are dispatched to the
experts they were routed to.  On one GPU dispatch becomes a permutation:
each (token, slot) pair of the top-k routing becomes one row of the expert
GEMM, rows grouped by expert.

Reading: within an expert's segment, rows are ordered by (token, slot)
ascending, i.e. a stable sort of the flattened top-k ids by expert.
"""
import numpy as np


def route(topk_ids, num_experts):
    """topk_ids [T, k] int -> (row_index [T*k] int32: token of each dispatched
    row, seg_offsets [E+1] int64, pair_row [T*k] int32: dispatched row of pair
    t*k + j)."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    order = np.argsort(flat, kind="stable")
    row_index = (order // k).astype(np.int32)
    counts = np.bincount(flat, minlength=num_experts)
    seg = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    pair_row = np.empty(T * k, dtype=np.int32)
    pair_row[order] = np.arange(T * k, dtype=np.int32)
    return row_index, seg, pair_row
