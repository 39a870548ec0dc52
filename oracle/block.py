"""Fused expert block: gate_up grouped GEMM -> SwiGLU -> down grouped GEMM
(oracle; test only).

Sources:

* "grouped-nf4-gemm releases", v0.2.5 section ("arena_experts — arena →
  kernel"): a MoE layer's forward runs the gate projection, the gated linear
  unit and the down projection straight off the grouped GEMM's packed weights.
* "grouped-nf4-gemm capability index" (index.json): `system_manifest.owns`
  lists the decode glue kernels (swiglu among them) next to the grouped GEMM,
  and `entrypoints` names `swiglu_rows`.

The pages print neither the gated unit's formula nor the order of the gate and
up rows inside the fused gate_up weight. Readings taken here:

* SwiGLU (Shazeer 2020, "GLU Variants Improve Transformer", eq. 5 family):
  act = silu(gate) * up, with silu(x) = x * sigmoid(x) = x / (1 + e^-x).
* gate and up rows are interleaved: row 2i of the fused weight [2I, H] is the
  gate of unit i and row 2i + 1 its up projection.
* The intermediate act is rounded once to bf16 (round to nearest, ties to even)
  before the down projection, as a separately stored activation would be.

Everything else is the grouped GEMM of oracle.grouped, twice, on the same routing.
"""
from __future__ import annotations

import math
from typing import Callable

import numpy as np

from .grouped import grouped_ref, offsets, _bf16_to_f64

WeightFn = Callable[[int], np.ndarray]


def silu(x: np.ndarray) -> np.ndarray:
    """x / (1 + e^-x) in fp64 (e^-x overflowing to inf gives -0 for very negative x)."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def swiglu_ref(h: np.ndarray) -> np.ndarray:
    """act[:, i] = silu(h[:, 2i]) * h[:, 2i + 1] (gate/up interleaved), fp64."""
    h = np.asarray(h, dtype=np.float64)
    if h.shape[-1] % 2:
        raise ValueError("the fused gate_up width must be even")
    return silu(h[..., 0::2]) * h[..., 1::2]


def bf16_rne_from_f64(x: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bits with one rounding to nearest, ties to even (no detour
    through fp32, which could round twice). Finite inputs only."""
    x = np.asarray(x, dtype=np.float64)
    if not np.isfinite(x).all():
        raise ValueError("finite values only")
    mag = np.abs(x)
    # bf16 keeps 8 significant bits; below 2^-126 its spacing is fixed at 2^-133
    _, e = np.frexp(mag)                      # mag = m * 2^e, m in [0.5, 1)
    q = np.where(mag >= 2.0 ** -126, e - 8, -133).astype(np.int64)
    r = np.round(np.ldexp(mag, -q))           # numpy rounds halves to even
    val = np.copysign(np.ldexp(r, q), x)
    with np.errstate(over="ignore"):
        f32 = val.astype(np.float32)          # exact: every bf16 value is an fp32 value
    return (f32.view(np.uint32) >> 16).astype(np.uint16)


def expert_block_ref(a_bits: np.ndarray, sizes, w13: WeightFn, w2: WeightFn, H: int, I: int):
    """(act_bits [M, I] bf16 bits, out [M, H] fp64) of the fused expert block.

    h = a_e W13_e^T (fp64, [rows, 2I]); act = bf16(silu(h_gate) * h_up);
    out = act_e W2_e^T (fp64). Rows past sum(sizes) are 0 in both.
    """
    h = grouped_ref(a_bits, sizes, w13, 2 * I)
    act_bits = bf16_rne_from_f64(swiglu_ref(h))
    out = grouped_ref(act_bits, sizes, w2, H)
    return act_bits, out


def sampled_block_ref(a_bits, sizes, rows: np.ndarray, w13_fn: WeightFn, w2_fn: WeightFn) -> np.ndarray:
    """out[rows, :] of the fused block for a few rows (each row needs its whole
    intermediate, so whole output rows are returned), fp64 [len(rows), H]."""
    off = offsets(sizes)
    rows = np.asarray(rows, dtype=np.int64)
    ex = np.searchsorted(off, rows, side="right") - 1
    res = []
    cache = {}
    for r, e in zip(rows, ex):
        e = int(e)
        if e not in cache:
            cache = {e: (w13_fn(e), w2_fn(e))}
        w13, w2 = cache[e]
        h = _bf16_to_f64(np.asarray(a_bits)[r:r + 1]) @ w13.T
        act = _bf16_to_f64(bf16_rne_from_f64(swiglu_ref(h)))
        res.append((act @ w2.T)[0])
    return np.stack(res) if res else np.zeros((0, 0))


def brute_force_block(a_bits, sizes, w13: WeightFn, w2: WeightFn) -> list:
    """Pure-Python loops with exactly rounded sums (math.fsum) and math.exp;
    the bf16 rounding goes through math.frexp. Tiny inputs only."""
    def round_bf16(v: float) -> float:
        if v == 0.0:
            return v
        m, e = math.frexp(abs(v))
        q = e - 8 if abs(v) >= 2.0 ** -126 else -133
        t = abs(v) / 2.0 ** q
        lo = math.floor(t)
        d = t - lo
        r = lo + 1 if (d > 0.5 or (d == 0.5 and lo % 2 == 1)) else lo
        return math.copysign(r * 2.0 ** q, v)

    a = _bf16_to_f64(a_bits)
    off = offsets(sizes)
    out = []
    for e in range(len(off) - 1):
        g13, g2 = w13(e), w2(e)
        for r in range(int(off[e]), int(off[e + 1])):
            h = [math.fsum(float(a[r, k]) * float(g13[n, k]) for k in range(g13.shape[1]))
                 for n in range(g13.shape[0])]
            act = []
            for i in range(len(h) // 2):
                g, u = h[2 * i], h[2 * i + 1]
                den = 1.0 + math.exp(-g) if g > -700.0 else math.inf
                act.append(round_bf16(g / den * u))
            out.append([math.fsum(act[i] * float(g2[j, i]) for i in range(len(act)))
                        for j in range(g2.shape[0])])
    return out
