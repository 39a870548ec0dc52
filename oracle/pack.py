"""Packers and decoders of the two 4-bit weight formats (oracle; test only).

Storage follows the shapes on "grouped-nf4-gemm 0.33.1", section "Try it on
CPU right now": an NF4 weight [N, K] packs to codes [N, K/2] u8 and absmax
[N, K/64] fp32; an MXFP4 weight [.., K] packs to blocks [.., K/32, 16] u8 and
e8m0 scales [.., K/32] u8 (the same bytes as [.., K/2]).

Nibble order inside a byte is not printed on the pages. Reading taken:
* NF4 (bitsandbytes 4-bit layout): element 2j in the HIGH nibble of byte j.
* MXFP4 (released-checkpoint byte order): element 2j in the LOW nibble.

Decoding (opening description of the same page: table lookup, then blockwise
scaling): NF4 w = T[c] * absmax[k // 64]; MXFP4 w = e2m1(c) * 2^(s - 127) with
one scale byte per 32 elements. Both products are exact in fp64.
"""
from __future__ import annotations

import numpy as np

from .codebooks import NF4_TABLE_F32, E2M1_TABLE, e8m0_value

NF4_BLOCK = 64
MX_BLOCK = 32


# ----------------------------------------------------------------------------- nibbles
def unpack_nf4_codes(packed: np.ndarray) -> np.ndarray:
    """[.., K/2] u8 -> [.., K] codes; element 2j is the high nibble of byte j."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p >> 4
    out[..., 1::2] = p & 0x0F
    return out


def pack_nf4_codes(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8)
    return ((c[..., 0::2] << 4) | (c[..., 1::2] & 0x0F)).astype(np.uint8)


def unpack_mxfp4_codes(blocks: np.ndarray) -> np.ndarray:
    """[.., K/2] u8 -> [.., K] codes; element 2j is the low nibble of byte j."""
    p = np.asarray(blocks, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def pack_mxfp4_codes(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8)
    return ((c[..., 0::2] & 0x0F) | (c[..., 1::2] << 4)).astype(np.uint8)


# ----------------------------------------------------------------------------- NF4
def quantize_pack_nf4(w: np.ndarray):
    """NF4 quantiser (a fixture that makes the NF4 workloads' bytes).

    Per row and per 64 consecutive k: absmax = max |w| (fp32); x = w / absmax in
    fp64 (0 for an all-zero block); the code is the nearest table entry, a value
    exactly on a midpoint goes to the lower code. Refuses non-2-D input.
    Returns (codes u8 [N, K/2], absmax fp32 [N, K/64]).
    """
    w = np.asarray(w)
    if w.ndim != 2:
        raise ValueError(f"quantize_pack_nf4 expects a 2-D [N, K] weight, got shape {w.shape}")
    n, k = w.shape
    if k % NF4_BLOCK:
        raise ValueError(f"K={k} is not a multiple of {NF4_BLOCK}")
    w32 = w.astype(np.float32)
    blocks = w32.reshape(n, k // NF4_BLOCK, NF4_BLOCK)
    absmax = np.abs(blocks).max(axis=2).astype(np.float32)
    denom = absmax.astype(np.float64)[:, :, None]
    with np.errstate(invalid="ignore", divide="ignore"):
        x = np.where(denom > 0, blocks.astype(np.float64) / np.where(denom > 0, denom, 1.0), 0.0)
    t = NF4_TABLE_F32.astype(np.float64)
    mids = (t[:-1] + t[1:]) * 0.5               # exact in fp64
    codes = (x[..., None] > mids).sum(axis=-1).astype(np.uint8)
    return pack_nf4_codes(codes.reshape(n, k)), absmax


def dequant_nf4(packed: np.ndarray, absmax: np.ndarray) -> np.ndarray:
    """Exact fp64 decode: W[.., n, k] = T[code] * absmax[.., n, k // 64]."""
    codes = unpack_nf4_codes(packed)
    t = NF4_TABLE_F32.astype(np.float64)[codes]
    s = np.repeat(np.asarray(absmax, dtype=np.float32).astype(np.float64), NF4_BLOCK, axis=-1)
    return t * s


def nf4_w32(packed: np.ndarray, absmax: np.ndarray) -> np.ndarray:
    """The fp32 weight: IEEE fp32 product of the two fp32 factors (== fp32(W64))."""
    return dequant_nf4(packed, absmax).astype(np.float32)


# ----------------------------------------------------------------------------- MXFP4
_E2M1_MAG = E2M1_TABLE[:8]                      # 0, .5, 1, 1.5, 2, 3, 4, 6
_E2M1_MID = (_E2M1_MAG[:-1] + _E2M1_MAG[1:]) * 0.5


def quantize_pack_mxfp4(w: np.ndarray):
    """MXFP4 quantiser (round-trip fixture only; the MXFP4 workloads draw raw bytes).

    Per 32 consecutive k: X = floor(log2 amax) - 2 (2 = largest e2m1 exponent),
    scale byte = X + 127 clamped to [0, 254] (127 for an all-zero block); each
    element is the nearest e2m1 value of w / 2^X, saturating at 6, ties to the
    even code. Returns (blocks u8 [.., K/32, 16], scales u8 [.., K/32]).
    """
    w = np.asarray(w, dtype=np.float32)
    k = w.shape[-1]
    if k % MX_BLOCK:
        raise ValueError(f"K={k} is not a multiple of {MX_BLOCK}")
    lead = w.shape[:-1]
    b = w.astype(np.float64).reshape(lead + (k // MX_BLOCK, MX_BLOCK))
    amax = np.abs(b).max(axis=-1)
    with np.errstate(divide="ignore"):
        X = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, 0)
    sbyte = np.clip(X + 127, 0, 254).astype(np.int64)
    v = b / np.ldexp(1.0, (sbyte - 127).astype(np.int32))[..., None]
    a = np.abs(v)
    lo = (a[..., None] > _E2M1_MID).sum(axis=-1)       # ties -> lower
    hi = (a[..., None] >= _E2M1_MID).sum(axis=-1)      # ties -> upper
    idx = np.where(lo == hi, lo, np.where(lo % 2 == 0, lo, hi))
    codes = (idx | np.where(np.signbit(v), 8, 0)).astype(np.uint8)
    blocks = pack_mxfp4_codes(codes.reshape(lead + (k,))).reshape(lead + (k // MX_BLOCK, 16))
    return blocks, sbyte.astype(np.uint8)


def dequant_mxfp4(blocks: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Exact fp64 decode: W[.., k] = e2m1(code) * 2^(scale[.., k // 32] - 127).

    blocks is [.., K/2] or the page's [.., K/32, 16] view of the same bytes."""
    blocks = np.asarray(blocks, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    if blocks.ndim == scales.ndim + 1 and blocks.shape[:-1] == scales.shape:
        blocks = blocks.reshape(scales.shape[:-1] + (scales.shape[-1] * blocks.shape[-1],))
    codes = unpack_mxfp4_codes(blocks)
    v = E2M1_TABLE[codes]
    s = np.repeat(e8m0_value(scales), MX_BLOCK, axis=-1)
    with np.errstate(invalid="ignore", over="ignore"):
        return v * s


def mxfp4_w32(blocks: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """fp32 of the exact value: RNE, fp32 subnormals kept, overflow to +-inf, NaN scale -> NaN."""
    with np.errstate(over="ignore", invalid="ignore"):
        return dequant_mxfp4(blocks, scales).astype(np.float32)


# ----------------------------------------------------------------------------- roundings
def bf16_rne_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest even on the bit pattern; NaN stays a
    (quiet) NaN with its sign."""
    b = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    is_nan = (b & 0x7FFFFFFF) > 0x7F800000
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return np.where(is_nan, (b >> 16) | 0x40, rounded).astype(np.uint16)


def fp16_rne_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 -> IEEE binary16 bits, round to nearest even (numpy's conversion)."""
    with np.errstate(over="ignore"):
        return np.asarray(x32, dtype=np.float32).astype(np.float16).view(np.uint16)
