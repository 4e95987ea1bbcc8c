"""Algorithmic HBM byte counts for one decode step.

Only what the method itself has to move is counted: cached K and V rows,
local K and V rows, signatures, queries, outputs and indices.  Workspace
partials, a second (cache-resident) signature pass and launch overheads are
not counted; they are costs the kernels must hide.

The document KV state of a model is 2 * n * L * H * d entries ("Nectar: Neural
Estimation of Cached-Token Attention via Regression", slide "A fixed document
is expensive to read repeatedly"); one decode step of one layer reads the
2 * n * H * d entries of that layer.
"""
from __future__ import annotations

import numpy as np


def doc_kv_state_bytes(n: int, layers: int, kv_heads: int, d: int, elem_bytes: int = 2) -> int:
    """Bytes of the cached K and V of a document: 2 n L H d entries."""
    return 2 * n * layers * kv_heads * d * elem_bytes


def dense_step_bytes(B: int, Hq: int, Hkv: int, d: int, n: int, elem_bytes: int,
                     shared_doc: bool = False, n_loc_total: int = 0, fused: bool = False) -> int:
    """cached_attn_lse (+ lse_merge_local) for one layer.

    n_loc_total: sum over batch items of the local tokens merged (0: no merge).
    fused: the two as one call (dense_decode_step), which reads q once and
    writes only the merged out and alpha; the two-call form also writes A and
    alpha and reads them and q again."""
    Bkv = 1 if shared_doc else B
    kv = 2 * Bkv * Hkv * n * d * elem_bytes
    loc = 2 * Hkv * n_loc_total * d * elem_bytes
    q = B * Hq * d * elem_bytes
    out = B * Hq * (d + 1) * 4                      # A and alpha (or out and alpha), fp32
    if fused or not n_loc_total:
        return kv + loc + q + out
    merged = B * Hq * (d + 1) * 4
    merge_in = B * Hq * (d + 1) * 4 + B * Hq * d * elem_bytes
    return kv + loc + q + out + merged + merge_in


def unique_rows(idx: np.ndarray, count: np.ndarray, G: int) -> int:
    """Distinct (b, KV head, position) triples over the selected sets.

    idx [B, Hq, cap], count [B, Hq]; query heads g*G..g*G+G-1 share KV head g."""
    B, Hq, cap = idx.shape
    total = 0
    for b in range(B):
        for h in range(Hq // G):
            sets = [idx[b, h * G + g, :count[b, h * G + g]] for g in range(G)]
            total += int(np.unique(np.concatenate(sets)).size) if sets else 0
    return total


def sparse_step_bytes(B: int, Hq: int, Hkv: int, d: int, n: int, elem_bytes: int, cap: int,
                      unique_kv_rows: int) -> int:
    """sig_score_topk + gather_attn: signatures, unique selected K+V rows, indices, q, outputs."""
    sigs = B * Hkv * n * 4 + B * Hq * 4
    rows = unique_kv_rows * 2 * d * elem_bytes
    idx = 2 * B * Hq * (cap + 1) * 4                # written by TOPK, read by GATHER-ATT
    q = B * Hq * d * elem_bytes
    out = B * Hq * (d + 1) * 4
    return sigs + rows + idx + q + out
