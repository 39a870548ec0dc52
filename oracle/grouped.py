"""Grouped expert GEMM, its input gradient and brute-force checks (oracle; test only).

Definition ("grouped-nf4-gemm releases", v0.2.6 section "The patch point"): the
caller sorts routed rows by expert, so rows off[e] .. off[e+1]-1 of `a` belong
to expert e, with off the exclusive prefix sum of the per-expert row counts
`sizes`. The grouped GEMM returns, for every expert, a_e times W_e transposed —
exactly what a loop of one matmul per expert returns. Here every expert's
weight is decoded to fp64 (exact) and the matmul runs in fp64.

The input gradient ("grouped-nf4-gemm capability index", system_manifest.owns:
the dgrad of the grouped packed GEMM) is dX_e = dY_e W_e on the same weights.

Weights are passed as a callable `weights(e) -> fp64 [N, K]` so that callers
decode with the format's own decoder (see oracle.pack) and so that large
workloads never hold every expert at once.
"""
from __future__ import annotations

import math
from typing import Callable, Sequence

import numpy as np

WeightFn = Callable[[int], np.ndarray]


def _bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def offsets(sizes: Sequence[int]) -> np.ndarray:
    """Exclusive prefix sum of the per-expert row counts, int64 [E+1]."""
    s = np.asarray(sizes, dtype=np.int64)
    if (s < 0).any():
        raise ValueError("negative expert size")
    off = np.zeros(len(s) + 1, dtype=np.int64)
    np.cumsum(s, out=off[1:])
    return off


def grouped_ref(a_bits: np.ndarray, sizes, weights: WeightFn, N: int) -> np.ndarray:
    """out[off[e]:off[e+1]] = a_e @ W_e^T in fp64; rows past sum(sizes) are 0."""
    a_bits = np.asarray(a_bits)
    M = a_bits.shape[0]
    off = offsets(sizes)
    if off[-1] > M:
        raise ValueError(f"sum(sizes)={off[-1]} exceeds M={M}")
    out = np.zeros((M, N), dtype=np.float64)
    for e in range(len(off) - 1):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        out[lo:hi] = _bf16_to_f64(a_bits[lo:hi]) @ weights(e).T
    return out


def loop_ref(x_bits: np.ndarray, topk_ids: np.ndarray, weights: WeightFn, N: int) -> np.ndarray:
    """The per-expert loop as the model runs it, from unsorted tokens.

    Flatten the top-k expert ids, stable-argsort them, gather tokens (index //
    top_k), count rows per expert, then one matmul per expert over its slice.
    Returns the outputs in that sorted row order, plus sizes.
    """
    topk_ids = np.asarray(topk_ids)
    T, k = topk_ids.shape
    flat = topk_ids.reshape(-1)
    idxs = np.argsort(flat, kind="stable")
    sorted_x = _bf16_to_f64(np.asarray(x_bits)[idxs // k])
    E = int(flat.max()) + 1 if flat.size else 0
    counts = np.bincount(flat, minlength=E)
    out = np.zeros((T * k, N), dtype=np.float64)
    start = 0
    for e, num in enumerate(counts):
        if num == 0:
            continue
        out[start:start + num] = sorted_x[start:start + num] @ weights(e).T
        start += num
    return out, counts.astype(np.int32)


def dgrad_ref(dy_bits: np.ndarray, sizes, weights: WeightFn, K: int) -> np.ndarray:
    """dX[off[e]:off[e+1]] = dY_e @ W_e in fp64 (contracts over N)."""
    dy_bits = np.asarray(dy_bits)
    M = dy_bits.shape[0]
    off = offsets(sizes)
    out = np.zeros((M, K), dtype=np.float64)
    for e in range(len(off) - 1):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        out[lo:hi] = _bf16_to_f64(dy_bits[lo:hi]) @ weights(e)
    return out


def _expert_of_rows(sizes, rows) -> np.ndarray:
    off = offsets(sizes)
    return np.searchsorted(off, np.asarray(rows, dtype=np.int64), side="right") - 1


def sampled_fwd_ref(a_bits, sizes, weight_rows: Callable[[int, np.ndarray], np.ndarray],
                    rows: np.ndarray, cols: np.ndarray) -> np.ndarray:
    """out[rows[i], cols[i]] for sampled positions, one dot product each.

    weight_rows(e, n_idx) -> fp64 [len(n_idx), K] decodes only the needed rows.
    """
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    ex = _expert_of_rows(sizes, rows)
    res = np.empty(len(rows), dtype=np.float64)
    for e in np.unique(ex):
        sel = np.nonzero(ex == e)[0]
        ucols, inv = np.unique(cols[sel], return_inverse=True)
        w = weight_rows(int(e), ucols)
        a = _bf16_to_f64(np.asarray(a_bits)[rows[sel]])
        res[sel] = np.einsum("ik,ik->i", a, w[inv])
    return res


def sampled_dgrad_ref(dy_bits, sizes, weight_cols: Callable[[int, np.ndarray], np.ndarray],
                      rows: np.ndarray, cols: np.ndarray) -> np.ndarray:
    """dX[rows[i], cols[i]] for sampled positions: sum over n of dY[r, n] W[e, n, k].

    weight_cols(e, k_idx) -> fp64 [N, len(k_idx)] decodes only the needed columns.
    """
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    ex = _expert_of_rows(sizes, rows)
    res = np.empty(len(rows), dtype=np.float64)
    for e in np.unique(ex):
        sel = np.nonzero(ex == e)[0]
        ucols, inv = np.unique(cols[sel], return_inverse=True)
        w = weight_cols(int(e), ucols)                 # [N, u]
        dy = _bf16_to_f64(np.asarray(dy_bits)[rows[sel]])  # [s, N]
        res[sel] = np.einsum("in,ni->i", dy, w[:, inv])
    return res


def brute_force_ref(a_bits, sizes, weights: WeightFn) -> list:
    """Pure-Python triple loop with exactly rounded sums (math.fsum); tiny inputs only."""
    a = _bf16_to_f64(a_bits)
    off = offsets(sizes)
    out = []
    for e in range(len(off) - 1):
        w = weights(e)
        for r in range(int(off[e]), int(off[e + 1])):
            out.append([math.fsum(float(a[r, k]) * float(w[n, k]) for k in range(w.shape[1]))
                        for n in range(w.shape[0])])
    return out


def brute_force_dgrad(dy_bits, sizes, weights: WeightFn) -> list:
    dy = _bf16_to_f64(dy_bits)
    off = offsets(sizes)
    out = []
    for e in range(len(off) - 1):
        w = weights(e)
        for r in range(int(off[e]), int(off[e + 1])):
            out.append([math.fsum(float(dy[r, n]) * float(w[n, k]) for n in range(w.shape[0]))
                        for k in range(w.shape[1])])
    return out
