"""Offsets past 2^31 elements, one case per process (run by
tests/test_gpu_full.py::test_offsets_past_2_31_elements_in_own_process).

The pages record an int32 offset overflow in the grouped kernel ("Current
status", "What changed — retired, superseded, corrected") and its boundary test,
run one case per process. Here the activation tensor holds M * K > 2^31 elements
(M = 540674 routed rows, K = 4096), and the dgrad's dY as many; one expert's
rows straddle element 2^31 and the last expert's rows all lie past it. Rows repeat 4096 seeded token vectors
(row r holds token r % 4096), so the oracle computes any sampled output row from
the token block. Whole output rows are compared: the first and last row of every
expert, rows on both sides of the 2^31-element boundary and random rows.

Prints progress lines and, last, one JSON line {case: max |err| / max(1, |ref|)}.
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synthetic  # noqa: E402


def log(msg):
    print(msg, flush=True)


def main():
    import torch
    import grouped_expert_gemm_amd as geg

    dev = torch.device("cuda", 0)
    K, N, T0 = 4096, 256, 4096
    # expert 2 straddles element 2^31 (row 524288); expert 3 lies wholly past it
    sizes = np.array([170000, 180000, 174290, 16384], np.int32)
    E, M = len(sizes), int(sizes.sum())
    s2, s3 = int(sizes[2]), int(sizes[3])
    assert M * K > 2 ** 31 and (M - s3) * K > 2 ** 31 > (M - s3 - s2) * K
    rng = np.random.default_rng(2031)
    tok = synthetic.f32_to_bf16_bits(rng.standard_normal((T0, K)).astype(np.float32))
    off = oracle.offsets(sizes)
    first_past = -(-(2 ** 31) // K)   # first row whose elements all lie past 2^31
    rows = np.unique(np.concatenate([off[:-1], off[1:] - 1, [first_past - 1, first_past, M - 1],
                                     rng.integers(0, M, 24)])).astype(np.int64)
    ex = np.searchsorted(off, rows, side="right") - 1
    res = {}

    tok_t = torch.from_numpy(tok.view(np.int16)).to(dev)
    idx = torch.arange(M, device=dev, dtype=torch.int64) % T0
    sz = torch.from_numpy(sizes).to(dev)

    # ---- forward, NF4 and MXFP4: a [M, K] (more than 2^31 elements)
    a = tok_t[idx].view(torch.bfloat16)
    for fmt in ("nf4", "mxfp4"):
        log(f"case: boundary forward {fmt} M={M} K={K} N={N} E={E} (M*K={M * K})")
        if fmt == "nf4":
            packs = [oracle.quantize_pack_nf4((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
                     for _ in range(E)]
            dec = oracle.dequant_nf4
            fn = geg.gnf4_grouped_gemm
        else:
            packs = [(rng.integers(0, 256, (N, K // 2), dtype=np.uint8), rng.integers(119, 130, (N, K // 32),
                                                                                     dtype=np.uint8))
                     for _ in range(E)]
            dec = oracle.dequant_mxfp4
            fn = geg.gmxfp4_grouped_gemm
        w = torch.from_numpy(np.stack([p[0] for p in packs])).to(dev)
        s = torch.from_numpy(np.stack([p[1] for p in packs])).to(dev)
        ws = geg.Workspace(geg.geg_workspace_bytes(0 if fmt == "nf4" else 1, M, N, K, E))
        out = fn(a, sz, w, s, workspace=ws, check_errors=True)
        got = out[torch.from_numpy(rows).to(dev)].float().cpu().numpy().astype(np.float64)
        del out, ws
        torch.cuda.empty_cache()
        x = (tok[rows % T0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        ref = np.stack([x[i] @ dec(*packs[e]).T for i, e in enumerate(ex)])
        err = float(np.max(np.abs(got - ref) / np.maximum(1.0, np.abs(ref))))
        log(f"  forward {fmt}: {len(rows)} whole rows, max |err|/max(1,|ref|) = {err:.5f}")
        res[f"forward_{fmt}"] = err
    del a
    torch.cuda.empty_cache()

    # ---- NF4 dgrad: dY [M, 4096] (more than 2^31 elements) -> dX [M, 256]
    Nd, Kd = 4096, 256
    log(f"case: boundary dgrad nf4 M={M} N={Nd} K={Kd} E={E} (M*N={M * Nd})")
    dy = tok_t[idx].view(torch.bfloat16)
    packs = [oracle.quantize_pack_nf4((rng.standard_normal((Nd, Kd)) * 0.02).astype(np.float32)) for _ in range(E)]
    w = torch.from_numpy(np.stack([p[0] for p in packs])).to(dev)
    s = torch.from_numpy(np.stack([p[1] for p in packs])).to(dev)
    dx = geg.gnf4_grouped_dgrad(dy, sz, w, s, check_errors=True)
    got = dx[torch.from_numpy(rows).to(dev)].float().cpu().numpy().astype(np.float64)
    g = (tok[rows % T0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = np.stack([g[i] @ oracle.dequant_nf4(*packs[e]) for i, e in enumerate(ex)])
    err = float(np.max(np.abs(got - ref) / np.maximum(1.0, np.abs(ref))))
    log(f"  dgrad nf4: {len(rows)} whole rows, max |err|/max(1,|ref|) = {err:.5f}")
    res["dgrad_nf4"] = err
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
