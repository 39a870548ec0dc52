"""Helpers for the GPU parity tests: uploads, tolerance checks, case assembly.

Inputs come from `synthetic` (seeded draws) and, for NF4 bytes, from the oracle's
quantiser (small cases) or the library's GPU quantiser (full-size cases, whose
bytes are themselves checked against the oracle quantiser on sampled rows).
Expected values come only from `oracle`.
"""
from __future__ import annotations

import hashlib
import sys

import numpy as np

import oracle
import synthetic
from oracle import cases as C

TOL = 1e-2  # |gpu - ref| <= TOL * max(1, |ref|), elementwise, on bf16 outputs


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    return torch


def dev():
    return torch_mod().device("cuda", 0)


def up_u16_as_bf16(x: np.ndarray):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev())


def up(x: np.ndarray):
    return torch_mod().from_numpy(np.ascontiguousarray(x)).to(dev())


def bf16_to_f64(t) -> np.ndarray:
    torch = torch_mod()
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def bits16(t) -> np.ndarray:
    torch = torch_mod()
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.max(np.abs(got - ref) / np.maximum(1.0, np.abs(ref)))) if ref.size else 0.0


def assert_close(got: np.ndarray, ref: np.ndarray, what: str):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = rel_err(got, ref)
    log(f"  {what}: max |err|/max(1,|ref|) = {err:.5f}")
    assert err <= TOL, f"{what}: max rel err {err} > {TOL}"
    return err


def sha(t) -> str:
    return hashlib.sha256(t.detach().contiguous().view(-1).view(torch_mod().uint8).cpu().numpy().tobytes()).hexdigest()


def upload_case(d):
    """Upload a dict from oracle.cases.build to the GPU (weights as packed bytes)."""
    g = {"a": up_u16_as_bf16(d["a_bits"]), "sizes": up(d["sizes"].astype(np.int32)),
         "w": up(d["codes"]), "s": up(d["scales"])}
    if "dy_bits" in d:
        g["dy"] = up_u16_as_bf16(d["dy_bits"])
    return g


def gpu_weights_nf4(c: synthetic.Case, seed: int, experts=None):
    """Pack every expert's N(0,0.02) weights on the GPU with the library's NF4
    packer. Returns (codes [E,N,K/2], absmax [E,N,K/64]) on the device."""
    import grouped_expert_gemm_amd as geg
    torch = torch_mod()
    codes = torch.zeros((c.E, c.N, c.K // 2), dtype=torch.uint8, device=dev())
    absmax = torch.zeros((c.E, c.N, c.K // 64), dtype=torch.float32, device=dev())
    for e in (range(c.E) if experts is None else experts):
        w = up(synthetic.nf4_weight_f32(c, seed, e))
        q, s = geg.gnf4_quantize(w)
        codes[e].copy_(q)
        absmax[e].copy_(s)
        del w
    return codes, absmax


def gpu_weights_mxfp4(c: synthetic.Case, seed: int, experts=None):
    torch = torch_mod()
    codes = torch.zeros((c.E, c.N, c.K // 2), dtype=torch.uint8, device=dev())
    scales = torch.zeros((c.E, c.N, c.K // 32), dtype=torch.uint8, device=dev())
    for e in (range(c.E) if experts is None else experts):
        q, s = synthetic.mxfp4_bytes(c, seed, e)
        codes[e].copy_(up(q))
        scales[e].copy_(up(s))
    return codes, scales


def sample_positions(sizes: np.ndarray, ncols: int, n: int, seed: int):
    """Rows/cols to check: first and last row of every non-empty expert, the last
    column (tail), plus uniform random positions."""
    rng = np.random.default_rng(seed)
    off = oracle.offsets(sizes)
    rows, cols = [], []
    for e in range(len(sizes)):
        if sizes[e] > 0:
            for r in (off[e], off[e + 1] - 1):
                rows += [r, r]
                cols += [int(rng.integers(0, ncols)), ncols - 1]
    M = int(off[-1])
    rows += list(rng.integers(0, M, n))
    cols += list(rng.integers(0, ncols, n))
    return np.array(rows, np.int64), np.array(cols, np.int64)
