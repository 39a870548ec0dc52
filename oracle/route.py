"""Routing sort and top-k combine around the grouped GEMM (oracle; test only).

Sources: "grouped-nf4-gemm releases", v0.2.6 section "The patch point": the
grouped GEMM replaces a per-expert loop, its rows grouped by expert with
`sizes[e]` rows for expert e. "grouped-nf4-gemm capability index" (index.json),
`entrypoints`: `router_epilogue` and `combine_rows` are the steps on either side
of the GEMM.

Readings: the (token, slot) entries are ordered by expert and, within an expert,
by flat index t * k + slot (the order a per-expert loop meets them; a stable
sort); an id outside [0, E) is dropped (no row, row_of = -1). The combine is the
router-weighted sum over a token's slots.
"""
from __future__ import annotations

import numpy as np


def route_sort_ref(topk_ids: np.ndarray, E: int):
    """(sizes [E], row_of [T*k], src_of [T*k]) of a stable sort by expert."""
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    valid = (ids >= 0) & (ids < E)
    order = np.argsort(np.where(valid, ids, E), kind="stable")
    n_valid = int(valid.sum())
    src_of = np.full(ids.size, -1, np.int32)
    src_of[:n_valid] = order[:n_valid]
    row_of = np.full(ids.size, -1, np.int32)
    row_of[order[:n_valid]] = np.arange(n_valid, dtype=np.int32)
    sizes = np.bincount(ids[valid], minlength=E).astype(np.int32)
    return sizes, row_of, src_of


def gather_ref(x_bits: np.ndarray, src_of: np.ndarray, k: int) -> np.ndarray:
    """x_sorted[r] = x[src_of[r] // k] for rows with a source (others all-zero bits)."""
    x_bits = np.asarray(x_bits)
    out = np.zeros((len(src_of), x_bits.shape[1]), dtype=x_bits.dtype)
    have = np.asarray(src_of) >= 0
    out[have] = x_bits[np.asarray(src_of)[have] // k]
    return out


def combine_ref(y: np.ndarray, row_of: np.ndarray, weights, T: int, k: int) -> np.ndarray:
    """out[t] = sum over slots s (with a row) of w[t, s] * y[row_of[t*k + s]], fp64."""
    y = np.asarray(y, dtype=np.float64)
    w = np.ones((T, k)) if weights is None else np.asarray(weights, dtype=np.float64).reshape(T, k)
    out = np.zeros((T, y.shape[1]), dtype=np.float64)
    r = np.asarray(row_of).reshape(T, k)
    for s in range(k):
        have = r[:, s] >= 0
        out[have] += w[have, s][:, None] * y[r[have, s]]
    return out


def brute_force_route(topk_ids, E: int):
    """Pure-Python version of route_sort_ref (tiny inputs)."""
    ids = [int(v) for v in np.asarray(topk_ids).reshape(-1)]
    src = [f for e in range(E) for f in range(len(ids)) if ids[f] == e]
    row_of = [-1] * len(ids)
    for r, f in enumerate(src):
        row_of[f] = r
    sizes = [sum(1 for v in ids if v == e) for e in range(E)]
    return sizes, row_of, src + [-1] * (len(ids) - len(src))
