"""Low-rank adapter delta on the grouped expert projection (oracle; test only).

Source: "grouped-nf4-gemm releases", v0.2.4 section (the differentiable grouped
NF4 GEMM): the frozen 4-bit projection is composed with a trainable low-rank
delta B(Ax), added at the pre-activation point, and the whole is trainable (a
backward pass for the input and for the adapter).

The page gives no formula beyond B(Ax). Readings taken here (the LoRA
parameterisation, Hu et al. 2021, eq. 3, per expert):

* per expert e, A_e is [r, K], B_e is [N, r], and for each row x of expert e
  y = x W_e^T + s * (x A_e^T) B_e^T, with one scalar s for the layer (LoRA's
  alpha / r), added to the projection before any activation;
* backward, with g = dL/dy and u = x A_e^T:
  dL/dx = g W_e + s (g B_e) A_e,  dL/dB_e = s g^T u,  dL/dA_e = s (g B_e)^T x,
  summed over the rows of expert e. The 4-bit weights W_e are frozen.

Everything is fp64 on bf16-exact inputs; the frozen part is oracle.grouped.
"""
from __future__ import annotations

import numpy as np

from .grouped import grouped_ref, dgrad_ref, offsets, _bf16_to_f64


def _f64(x):
    x = np.asarray(x)
    return _bf16_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)


def lora_delta_ref(a_bits, sizes, lora_a, lora_b, s: float):
    """(delta [M, N], u [M, r]): u = x A_e^T and delta = s u B_e^T per expert.
    lora_a [E, r, K], lora_b [E, N, r] as bf16 bits or floats."""
    x = _f64(a_bits)
    A, B = _f64(lora_a), _f64(lora_b)
    off = offsets(sizes)
    M = x.shape[0]
    u = np.zeros((M, A.shape[1]))
    delta = np.zeros((M, B.shape[1]))
    for e in range(len(off) - 1):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            u[lo:hi] = x[lo:hi] @ A[e].T
            delta[lo:hi] = s * (u[lo:hi] @ B[e].T)
    return delta, u


def lora_forward_ref(a_bits, sizes, weights, lora_a, lora_b, s: float, N: int):
    """y = grouped_ref(x, W) + s (x A_e^T) B_e^T, fp64 [M, N]."""
    delta, _ = lora_delta_ref(a_bits, sizes, lora_a, lora_b, s)
    return grouped_ref(a_bits, sizes, weights, N) + delta


def lora_backward_ref(a_bits, dy_bits, sizes, weights, lora_a, lora_b, s: float, K: int):
    """(dx [M, K], dA [E, r, K], dB [E, N, r]) in fp64 for upstream gradient dy."""
    x, g = _f64(a_bits), _f64(dy_bits)
    A, B = _f64(lora_a), _f64(lora_b)
    off = offsets(sizes)
    dx = dgrad_ref(dy_bits, sizes, weights, K)
    dA = np.zeros_like(A)
    dB = np.zeros_like(B)
    for e in range(len(off) - 1):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        u = x[lo:hi] @ A[e].T                      # [rows, r]
        gb = g[lo:hi] @ B[e]                       # [rows, r]
        dx[lo:hi] += s * (gb @ A[e])
        dB[e] = s * (g[lo:hi].T @ u)
        dA[e] = s * (gb.T @ x[lo:hi])
    return dx, dA, dB


def brute_force_lora(a_bits, dy_bits, sizes, lora_a, lora_b, s: float):
    """Pure-Python loops (math.fsum) for the adapter part only: (delta, dx_delta,
    dA, dB) as nested lists. Tiny inputs only."""
    import math
    x, g = _f64(a_bits), _f64(dy_bits)
    A, B = _f64(lora_a), _f64(lora_b)
    E, r, K = A.shape
    N = B.shape[1]
    off = [0]
    for v in sizes:
        off.append(off[-1] + int(v))
    delta = [[0.0] * N for _ in range(x.shape[0])]
    dxd = [[0.0] * K for _ in range(x.shape[0])]
    dA = [[[0.0] * K for _ in range(r)] for _ in range(E)]
    dB = [[[0.0] * r for _ in range(N)] for _ in range(E)]
    for e in range(E):
        rows = range(off[e], off[e + 1])
        for m in rows:
            u = [math.fsum(x[m, k] * A[e, j, k] for k in range(K)) for j in range(r)]
            gb = [math.fsum(g[m, n] * B[e, n, j] for n in range(N)) for j in range(r)]
            for n in range(N):
                delta[m][n] = s * math.fsum(u[j] * B[e, n, j] for j in range(r))
            for k in range(K):
                dxd[m][k] = s * math.fsum(gb[j] * A[e, j, k] for j in range(r))
        for j in range(r):
            for k in range(K):
                dA[e][j][k] = s * math.fsum(
                    math.fsum(g[m, n] * B[e, n, j] for n in range(N)) * x[m, k] for m in rows)
            for n in range(N):
                dB[e][n][j] = s * math.fsum(
                    g[m, n] * math.fsum(x[m, k] * A[e, j, k] for k in range(K)) for m in rows)
    return delta, dxd, dA, dB
