"""Seeded synthetic inputs for the grouped 4-bit expert GEMM.

This module is shared by the CPU oracle, the tests and the benchmark. It draws
random numbers and lays them out; it holds none of the GEMM's arithmetic: no
codebook, no e2m1/e8m0 decode, no quantiser, no matmul.

Workload shapes follow the five configurations the method is measured on: a tiny
NF4 case, OLMoE-1B-7B, Qwen3-30B-A3B and Mixtral-8x7B shaped NF4 experts and
gpt-oss shaped MXFP4 experts. The pages measure on real text and real
checkpoints; none is available here, so these seeded draws stand in for them.

Every array is drawn from its own numpy PCG64 stream keyed by (seed, purpose,
...), so any piece can be regenerated alone:

* routing      default_rng([seed, 0])     N(0,1) logits [T, E] (+ Zipf(1.1) bias)
* activations  default_rng([seed, 1])     N(0,1) fp32 [T, K], rounded to bf16
* NF4 weights  default_rng([seed, 2, e])  N(0, 0.02) fp32 [N, K] per expert
* MXFP4 bytes  default_rng([seed, 3, e])  code bytes [N, K/2], e8m0 [N, K/32]
* dgrad dY     default_rng([seed, 4])     N(0,1) fp32 [M, N], rounded to bf16

bf16 values are carried as uint16 bit patterns (numpy has no bf16 type).
"""
from __future__ import annotations

import dataclasses
import numpy as np

__all__ = [
    "Case", "CASES", "case", "topk_ids", "routing", "activations_bf16", "rows_bf16",
    "nf4_weight_f32", "mxfp4_bytes", "dgrad_dy_bf16", "f32_to_bf16_bits",
    "bf16_bits_to_f32",
]


@dataclasses.dataclass(frozen=True)
class Case:
    """One workload: a projection of one MoE layer at one token count."""
    name: str
    fmt: str          # "nf4" or "mxfp4"
    E: int            # experts
    K: int            # contraction (input features)
    N: int            # output features of the projection
    T: int            # tokens
    top_k: int
    zipf: float = 0.0  # >0: Zipf-skewed router logits
    op: str = "fwd"    # "fwd" or "dgrad"

    @property
    def M(self) -> int:
        return self.T * self.top_k


def _mk(name, fmt, E, K, N, T, k, zipf=0.0, op="fwd"):
    return Case(name, fmt, E, K, N, T, k, zipf, op)


# The five workload families. The benchmark's headline is Mixtral w1/w3 (the
# largest single-GPU configuration) with its dgrad, beside every T=1 and T=64
# decode case; every case is a parity case.
CASES = {c.name: c for c in [
    _mk("tiny", "nf4", 8, 256, 512, 64, 2),
    _mk("olmoe_gate_up_t1", "nf4", 64, 2048, 2048, 1, 8),
    _mk("olmoe_gate_up_t2048", "nf4", 64, 2048, 2048, 2048, 8),
    _mk("qwen3_gate_up_t1", "nf4", 128, 2048, 1536, 1, 8, 1.1),
    _mk("qwen3_down_t1", "nf4", 128, 768, 2048, 1, 8, 1.1),
    _mk("qwen3_gate_up_t64", "nf4", 128, 2048, 1536, 64, 8, 1.1),
    _mk("qwen3_down_t64", "nf4", 128, 768, 2048, 64, 8, 1.1),
    _mk("qwen3_gate_up_t4096", "nf4", 128, 2048, 1536, 4096, 8, 1.1),
    _mk("qwen3_down_t4096", "nf4", 128, 768, 2048, 4096, 8, 1.1),
    _mk("gptoss_gate_up_t1", "mxfp4", 32, 2880, 5760, 1, 4),
    _mk("gptoss_down_t1", "mxfp4", 32, 2880, 2880, 1, 4),
    _mk("gptoss_gate_up_t2048", "mxfp4", 32, 2880, 5760, 2048, 4),
    _mk("gptoss_down_t2048", "mxfp4", 32, 2880, 2880, 2048, 4),
    _mk("mixtral_w13_t4096", "nf4", 8, 4096, 28672, 4096, 2),
    _mk("mixtral_w2_t4096", "nf4", 8, 14336, 4096, 4096, 2),
    _mk("mixtral_dgrad_w13", "nf4", 8, 4096, 28672, 4096, 2, op="dgrad"),
    _mk("mixtral_dgrad_w2", "nf4", 8, 14336, 4096, 4096, 2, op="dgrad"),
    # input gradient of the gpt-oss gate_up projection on its released MXFP4 bytes
    _mk("gptoss_dgrad_gate_up", "mxfp4", 32, 2880, 5760, 2048, 4, op="dgrad"),
]}


def case(name: str) -> Case:
    return CASES[name]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 round-to-nearest-even, as uint16 bit patterns (NaN kept quiet)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = (b & 0x7FFFFFFF) > 0x7F800000
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    r = np.where(nan, (b >> 16) | 0x40, r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def topk_ids(c: Case, seed: int) -> np.ndarray:
    """Router draw: expert ids [T, top_k] from softmax of N(0,1) logits (plus a
    Zipf(s) bias -s*ln(rank) over a seeded expert permutation when zipf > 0);
    ties go to the lower expert id."""
    rr = np.random.default_rng([seed, 0])
    logits = rr.standard_normal((c.T, c.E))
    if c.zipf > 0.0:
        rank = rr.permutation(c.E) + 1
        logits = logits - c.zipf * np.log(rank)
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return np.argsort(-p, axis=1, kind="stable")[:, : c.top_k]


def routing(c: Case, seed: int):
    """The caller-side sort that the GEMM consumes.

    Returns (sizes int32 [E], token int64 [M]): rows are grouped by expert in
    (expert, token, slot) order; row r holds token token[r].
    """
    expert = topk_ids(c, seed).ravel()
    token = np.repeat(np.arange(c.T), c.top_k)
    order = np.lexsort((np.tile(np.arange(c.top_k), c.T), token, expert))
    sizes = np.bincount(expert, minlength=c.E).astype(np.int32)
    return sizes, token[order].astype(np.int64)


def activations_bf16(c: Case, seed: int) -> np.ndarray:
    """Token hidden states [T, K] as bf16 bits."""
    rx = np.random.default_rng([seed, 1])
    x = rx.standard_normal((c.T, c.K), dtype=np.float32)
    return f32_to_bf16_bits(x)


def rows_bf16(c: Case, seed: int):
    """Grouped activation rows a [M, K] (bf16 bits) and sizes [E]."""
    sizes, token = routing(c, seed)
    x = activations_bf16(c, seed)
    return np.ascontiguousarray(x[token]), sizes


def nf4_weight_f32(c: Case, seed: int, e: int, rows=None, first_rows=None) -> np.ndarray:
    """Unquantised weights of expert e, [N, K] fp32 drawn from N(0, 0.02).

    rows: optional index array to return only those output rows (the whole
    expert is still drawn, so the values do not depend on `rows`).
    first_rows: optional n to return rows 0..n-1 only; the stream is drawn in
    row-major order, so drawing its first n * K values gives the same rows.
    """
    g = np.random.default_rng([seed, 2, e])
    n = c.N if first_rows is None else min(int(first_rows), c.N)
    w = g.standard_normal((n, c.K), dtype=np.float32)
    w *= np.float32(0.02)
    return w if rows is None else np.ascontiguousarray(w[rows])


def mxfp4_bytes(c: Case, seed: int, e: int):
    """Raw MXFP4 storage of expert e: code bytes [N, K/2] u8 (uniform over all
    nibbles) and e8m0 scale bytes [N, K/32] u8 drawn from 119..129 (2^-8..2^2)."""
    g = np.random.default_rng([seed, 3, e])
    codes = g.integers(0, 256, (c.N, c.K // 2), dtype=np.uint8)
    scales = g.integers(119, 130, (c.N, c.K // 32), dtype=np.uint8)
    return codes, scales


def dgrad_dy_bf16(c: Case, seed: int) -> np.ndarray:
    """Upstream gradient dY [M, N] as bf16 bits, N(0,1)."""
    r = np.random.default_rng([seed, 4])
    return f32_to_bf16_bits(r.standard_normal((c.M, c.N), dtype=np.float32))
