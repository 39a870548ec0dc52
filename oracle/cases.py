"""Oracle-side assembly of a workload's packed inputs (test infrastructure only).

Raw draws come from `synthetic`; NF4 bytes are made here by this package's own
quantiser, so nothing the oracle checks against ever comes from the GPU path.
"""
from __future__ import annotations

import numpy as np

import synthetic
from .pack import quantize_pack_nf4, dequant_nf4, dequant_mxfp4, NF4_BLOCK


def nf4_expert(c: synthetic.Case, seed: int, e: int):
    """Packed NF4 (codes [N, K/2], absmax [N, K/64]) of expert e."""
    return quantize_pack_nf4(synthetic.nf4_weight_f32(c, seed, e))


def build(c: synthetic.Case, seed: int, experts=None):
    """Packed inputs of a workload small enough to hold whole.

    Returns dict with a_bits [M,K] u16, sizes [E] i32, and for NF4 codes
    [E,N,K/2] u8 + absmax [E,N,K/64] f32, for MXFP4 codes [E,N,K/2] u8 +
    scales [E,N,K/32] u8; for dgrad cases also dy_bits [M,N] u16.
    `experts` (optional) limits which experts are packed (others are zero).
    """
    a, sizes = synthetic.rows_bf16(c, seed)
    d = {"case": c, "seed": seed, "a_bits": a, "sizes": sizes}
    which = range(c.E) if experts is None else experts
    if c.fmt == "nf4":
        codes = np.zeros((c.E, c.N, c.K // 2), dtype=np.uint8)
        absmax = np.zeros((c.E, c.N, c.K // NF4_BLOCK), dtype=np.float32)
        for e in which:
            codes[e], absmax[e] = nf4_expert(c, seed, e)
        d.update(codes=codes, scales=absmax)
    else:
        codes = np.zeros((c.E, c.N, c.K // 2), dtype=np.uint8)
        scales = np.zeros((c.E, c.N, c.K // 32), dtype=np.uint8)
        for e in which:
            codes[e], scales[e] = synthetic.mxfp4_bytes(c, seed, e)
        d.update(codes=codes, scales=scales)
    if c.op == "dgrad":
        d["dy_bits"] = synthetic.dgrad_dy_bf16(c, seed)
    return d


def weight_fn(d):
    """fp64 decoder of expert e for a dict from `build`."""
    fmt = d["case"].fmt
    codes, scales = d["codes"], d["scales"]
    if fmt == "nf4":
        return lambda e: dequant_nf4(codes[e], scales[e])
    return lambda e: dequant_mxfp4(codes[e], scales[e])


def nf4_rows_fn(c: synthetic.Case, seed: int):
    """weight_rows(e, n_idx) for sampled checks: draws expert e, packs only the
    requested rows with the oracle quantiser and decodes them in fp64."""
    def f(e, n_idx):
        w = synthetic.nf4_weight_f32(c, seed, e, rows=np.asarray(n_idx))
        q, s = quantize_pack_nf4(w)
        return dequant_nf4(q, s)
    return f


def nf4_cols_fn(c: synthetic.Case, seed: int):
    """weight_cols(e, k_idx) -> fp64 [N, len(k_idx)]: packs only the 64-wide
    blocks that hold the requested columns (NF4 blocks are row-local, so this
    gives the same bytes as packing the whole expert)."""
    def f(e, k_idx):
        k_idx = np.asarray(k_idx)
        w = synthetic.nf4_weight_f32(c, seed, e)
        blocks = np.unique(k_idx // NF4_BLOCK)
        cols = np.concatenate([np.arange(b * NF4_BLOCK, (b + 1) * NF4_BLOCK) for b in blocks])
        q, s = quantize_pack_nf4(np.ascontiguousarray(w[:, cols]))
        dq = dequant_nf4(q, s)
        pos = {int(k): i for i, k in enumerate(cols)}
        return dq[:, [pos[int(k)] for k in k_idx]]
    return f


def mxfp4_cols_fn(c: synthetic.Case, seed: int):
    """weight_cols(e, k_idx) -> fp64 [N, len(k_idx)]: decodes only the 32-wide
    blocks (16 code bytes and one scale byte per row) that hold the columns."""
    def f(e, k_idx):
        k_idx = np.asarray(k_idx)
        codes, scales = synthetic.mxfp4_bytes(c, seed, e)
        blocks = np.unique(k_idx // 32)
        sub_c = np.concatenate([codes[:, 16 * b:16 * (b + 1)] for b in blocks], axis=1)
        dq = dequant_mxfp4(np.ascontiguousarray(sub_c), np.ascontiguousarray(scales[:, blocks]))
        pos = {int(b): i for i, b in enumerate(blocks)}
        return dq[:, [32 * pos[int(k) // 32] + int(k) % 32 for k in k_idx]]
    return f


def mxfp4_rows_fn(c: synthetic.Case, seed: int):
    def f(e, n_idx):
        codes, scales = synthetic.mxfp4_bytes(c, seed, e)
        n_idx = np.asarray(n_idx)
        return dequant_mxfp4(codes[n_idx], scales[n_idx])
    return f
