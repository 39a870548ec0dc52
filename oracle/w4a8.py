"""W4A8 variant of the MXFP4 grouped GEMM: e2m1 weights x MXFP8 (e4m3) activations
(oracle; test only).

Source: "bw24 releases, v0.9.0", section "Changes since v0.8.0" (Features and
Documentation lists): a W4A8-FP8 prefill tile that quantises the activations to
e4m3 and multiplies them with the native e2m1 weight bytes in one block-scaled
matrix instruction (e4m3 x e2m1), the weights' own scales kept.

The page does not say how the activations are scaled. Readings taken here, from
the OCP Microscaling Formats (MX) v1.0 specification, section 6.3 (conversion
to an MX format) and the E4M3 element format it defines:

* Blocks of 32 consecutive k along each activation row (the weights' block), one
  e8m0 scale byte X per block: X = floor(log2(amax)) - 8 + 127 (8 = exponent of
  e4m3's largest power of two, 256), clamped to [0, 254]; an all-zero block gets
  X = 0.
* Elements: v = x / 2^(X - 127) (exact), rounded to the nearest e4m3 value, ties
  to even; magnitudes above 448 (the largest finite e4m3) saturate to 448. The
  block's largest element lands in [256, 512) before saturation.
* E4M3 (OCP, "FN"): sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent
  field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no infinities.
* Activations must be finite (bf16 inf or NaN is refused here).

The product is then the grouped GEMM of oracle.grouped on the decoded values:
out_e = dequant(a_e) . dequant(W_e)^T in fp64, every product exact.
"""
from __future__ import annotations

import math

import numpy as np

from .grouped import offsets, _bf16_to_f64

MX_BLOCK = 32
E4M3_MAX = 448.0
E4M3_EMAX = 8          # exponent of the largest power of two in e4m3


def e4m3_value(code: int) -> float:
    """Value of one e4m3 byte (OCP FN encoding); NaN for 0x7F / 0xFF."""
    s, e, m = (code >> 7) & 1, (code >> 3) & 0xF, code & 7
    if e == 0xF and m == 7:
        return math.nan
    mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_round(v: np.ndarray) -> np.ndarray:
    """fp64 -> e4m3 code bytes: nearest value, ties to even mantissa, |v| > 448
    saturating to 448, sign kept (negative values that round to 0 give -0).
    Finite inputs only."""
    v = np.asarray(v, dtype=np.float64)
    if not np.isfinite(v).all():
        raise ValueError("finite values only")
    mag = np.abs(v)
    # spacing of the e4m3 grid at |v|: 2^-9 below the smallest normal 2^-6, else
    # 2^(floor(log2 |v|) - 3)
    _, ex = np.frexp(mag)                          # mag = f * 2^ex, f in [0.5, 1)
    q = np.where(mag >= 2.0 ** -6, ex - 1 - 3, -9).astype(np.int64)
    r = np.round(np.ldexp(mag, -q))                # halves to even
    val = np.minimum(np.ldexp(r, q), E4M3_MAX)
    # encode val (now on the grid, <= 448)
    code = np.zeros(v.shape, dtype=np.int64)
    sub = val < 2.0 ** -6
    code[sub] = np.round(np.ldexp(val[sub], 9)).astype(np.int64)     # m with e = 0
    nv = val[~sub]
    f, e2 = np.frexp(nv)                            # nv = f * 2^e2, f in [0.5, 1)
    e_field = e2 - 1 + 7
    m = np.round((2.0 * f - 1.0) * 8.0).astype(np.int64)
    code[~sub] = (e_field << 3) | m
    # the sign is kept, also where the magnitude rounds to 0 (-0 is 0x80)
    return (code | (np.signbit(v).astype(np.int64) << 7)).astype(np.uint8)


def mxfp8_scale_bytes(a: np.ndarray) -> np.ndarray:
    """e8m0 scale byte of every 32-block of the rows of a (fp64 [.., K])."""
    a = np.asarray(a, dtype=np.float64)
    K = a.shape[-1]
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    amax = np.abs(a.reshape(a.shape[:-1] + (K // MX_BLOCK, MX_BLOCK))).max(axis=-1)
    _, ex = np.frexp(amax)                          # floor(log2 amax) = ex - 1 for amax > 0
    x = np.where(amax > 0, ex - 1 - E4M3_EMAX + 127, 0)
    return np.clip(x, 0, 254).astype(np.uint8)


def quantize_mxfp8(a_bits: np.ndarray):
    """bf16 bits [M, K] -> (e4m3 codes u8 [M, K], e8m0 scales u8 [M, K/32])."""
    a = _bf16_to_f64(a_bits)
    if not np.isfinite(a).all():
        raise ValueError("activations must be finite")
    X = mxfp8_scale_bytes(a)
    step = np.ldexp(1.0, X.astype(np.int64) - 127)               # 2^(X - 127)
    v = a / np.repeat(step, MX_BLOCK, axis=-1)                    # exact (power of two)
    return e4m3_round(v), X


def dequant_mxfp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """fp64 values of e4m3 codes [.., K] with e8m0 scales [.., K/32]."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    step = np.ldexp(1.0, scales.astype(np.int64) - 127)
    return E4M3_TABLE[codes] * np.repeat(step, MX_BLOCK, axis=-1)


def w4a8_grouped_ref(a_bits, sizes, weights, N: int) -> np.ndarray:
    """fp64 [M, N]: per expert e, the MXFP8-quantised activation rows of e times
    the decoded MXFP4 weights (weights(e) -> fp64 [N, K]) transposed; rows past
    sum(sizes) are 0."""
    codes, X = quantize_mxfp8(a_bits)
    a = dequant_mxfp8(codes, X)
    off = offsets(sizes)
    out = np.zeros((a.shape[0], N), dtype=np.float64)
    for e in range(len(off) - 1):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            out[lo:hi] = a[lo:hi] @ weights(e).T
    return out


def sampled_w4a8_ref(a_bits, sizes, weight_rows, rows, cols) -> np.ndarray:
    """out[rows[i], cols[i]] of the W4A8 product for sampled positions, one dot
    product each (weight_rows(e, n_idx) -> fp64 [len(n_idx), K])."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    off = offsets(sizes)
    ex = np.searchsorted(off, rows, side="right") - 1
    res = np.empty(len(rows), dtype=np.float64)
    for e in np.unique(ex):
        sel = np.nonzero(ex == e)[0]
        codes, X = quantize_mxfp8(np.asarray(a_bits)[rows[sel]])
        w = weight_rows(int(e), cols[sel])
        res[sel] = np.einsum("ik,ik->i", dequant_mxfp8(codes, X), w)
    return res


def brute_force_w4a8(a_bits, sizes, weights) -> list:
    """Pure-Python loops: per-element scale and rounding by exhaustive nearest
    search over the e4m3 table (ties to the even code), exactly rounded sums
    (math.fsum). Tiny inputs only."""
    a = _bf16_to_f64(a_bits)
    finite = [(E4M3_TABLE[c], c) for c in range(0x7F)]             # +0 .. 448
    out = []
    off = [0]
    for s in sizes:
        off.append(off[-1] + int(s))
    for e in range(len(sizes)):
        w = weights(e)
        for r in range(off[e], off[e + 1]):
            q = []
            for b in range(0, a.shape[1], MX_BLOCK):
                blk = [float(x) for x in a[r, b:b + MX_BLOCK]]
                amax = max(abs(x) for x in blk)
                X = 0 if amax == 0 else min(254, max(0, math.frexp(amax)[1] - 1 - 8 + 127))
                sc = 2.0 ** (X - 127)
                for x in blk:
                    t = min(abs(x) / sc, E4M3_MAX)
                    best = min(finite, key=lambda vc: (abs(vc[0] - t), vc[1] & 1))
                    q.append(math.copysign(best[0], x) * sc)
            out.append([math.fsum(q[k] * float(w[n, k]) for k in range(len(q))) for n in range(w.shape[0])])
    return out
