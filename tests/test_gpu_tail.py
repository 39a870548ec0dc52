"""GPU parity of split remainder tiles, on every output element.

With a contraction of at least 1024, the tiled kernel splits the remainder
tiles (blocks of at most 128 rows) that are left over for a last, partial
persistent round into up to four pieces of consecutive contraction stages;
every piece writes fp32 partial sums and a second launch adds them in piece
order (with the gated epilogue applied there in the fused block). The number of
pieces follows from the plan and the grid, so `cu_limit` picks it: sizes
[1024, 5] give 4 full row blocks and one 5-row remainder per expert pair; with
2 output-column tiles that is 8 class-0 tiles and 2 remainder tiles, so a grid
of 8 splits each remainder tile 4 ways, a grid of 4 splits it 2 ways, and a grid
of 14 runs the remainder tiles beside the last class-0 round unsplit.

Definition of the result: "grouped-nf4-gemm releases", v0.2.6 "The patch point"
(the per-expert loop); tolerance |gpu - ref| <= 1e-2 max(1, |ref|).
"""
import ctypes

import numpy as np
import pytest

import oracle
import synthetic
from oracle import cases as C
from oracle import lora as L
from gpu_util import assert_close, bf16_to_f64, log, up, up_u16_as_bf16, upload_case

pytestmark = pytest.mark.gpu

SIZES = [1024, 5]
GRIDS = {4: "4 pieces", 2: "2 pieces", 1: "unsplit"}
CU_FOR_PIECES = {4: 8, 2: 4, 1: 16}


@pytest.fixture(scope="module")
def geg():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_expert_gemm_amd as g
    g.lib()
    return g


def _case(fmt, K, N, seed, sizes=SIZES):
    rng = np.random.default_rng(seed)
    E, M = len(sizes), int(np.sum(sizes))
    sizes = np.array(sizes, np.int32)
    a = synthetic.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    if fmt == "nf4":
        codes = np.zeros((E, N, K // 2), np.uint8)
        sc = np.zeros((E, N, K // 64), np.float32)
        for e in range(E):
            codes[e], sc[e] = oracle.quantize_pack_nf4((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    else:
        codes = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
        sc = rng.integers(119, 124, (E, N, K // 32), dtype=np.uint8)
    c = synthetic.Case("tail", fmt, E, K, N, 0, 1)
    return c, {"case": c, "a_bits": a, "sizes": sizes, "codes": codes, "scales": sc}


@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
@pytest.mark.parametrize("pieces", [4, 2, 1])
def test_forward_split_remainder_tiles(geg, fmt, pieces):
    cu = CU_FOR_PIECES[pieces]
    log(f"case: tiled forward {fmt}, K=8192 N=320 sizes={SIZES} cu_limit={cu} ({GRIDS[pieces]})")
    c, d = _case(fmt, 8192, 320, seed=51)
    g = upload_case(d)
    fn = geg.gnf4_grouped_gemm if fmt == "nf4" else geg.gmxfp4_grouped_gemm
    out = fn(g["a"], g["sizes"], g["w"], g["s"], opts=geg.Opts(2, 0, None, cu), check_errors=True)
    assert_close(bf16_to_f64(out), oracle.grouped_ref(d["a_bits"], d["sizes"], C.weight_fn(d), c.N),
                 f"forward {fmt} {GRIDS[pieces]}")


@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
@pytest.mark.parametrize("pieces", [4, 2, 1])
def test_dgrad_split_remainder_tiles(geg, fmt, pieces):
    # dX [M, 320] contracts over N = 8192
    cu = CU_FOR_PIECES[pieces]
    log(f"case: dgrad {fmt}, K=320 N=8192 sizes={SIZES} cu_limit={cu} ({GRIDS[pieces]})")
    c, d = _case(fmt, 320, 8192, seed=52)
    rng = np.random.default_rng(53)
    M = int(np.sum(SIZES))
    dyf = rng.standard_normal((M, 8192)).astype(np.float32)
    dyf[1026] *= 1e-6     # a remainder row far below fp16's range (row scaling)
    dy = synthetic.f32_to_bf16_bits(dyf)
    g = upload_case(d)
    fn = geg.gnf4_grouped_dgrad if fmt == "nf4" else geg.gmxfp4_grouped_dgrad
    dx = fn(up_u16_as_bf16(dy), g["sizes"], g["w"], g["s"], opts=geg.Opts(0, 0, None, cu), check_errors=True)
    ref = oracle.dgrad_ref(dy, d["sizes"], C.weight_fn(d), 320)
    got = bf16_to_f64(dx)
    assert_close(got, ref, f"dgrad {fmt} {GRIDS[pieces]}")
    row_rel = float(np.max(np.abs(got[1026] - ref[1026])) / np.max(np.abs(ref[1026])))
    log(f"  small remainder row: max|err|/max|ref| = {row_rel:.2e}")
    assert row_rel <= 1e-2


@pytest.mark.parametrize("direction", ["forward", "backward"])
def test_adapter_with_split_remainder_tiles(geg, direction):
    # the adapter delta joins exactly one piece of a split tile (the first)
    K, N = (8192, 320) if direction == "forward" else (320, 8192)
    r, s = 16, 0.5
    log(f"case: nf4 adapter {direction}, K={K} N={N} r={r} sizes={SIZES} cu_limit=8 (4 pieces)")
    c, d = _case("nf4", K, N, seed=54)
    rng = np.random.default_rng(55)
    M = int(np.sum(SIZES))
    A = (rng.standard_normal((2, r, K)) / np.sqrt(K)).astype(np.float32)
    B = (rng.standard_normal((2, N, r)) * 0.5).astype(np.float32)
    Wf = C.weight_fn(d)
    g = upload_case(d)
    o = geg.Opts(0, 0, None, 8)
    At, Bt = up(A), up(B)
    out, u = geg.gnf4_grouped_gemm_lora(g["a"], g["sizes"], g["w"], g["s"], At, Bt, s, opts=o, check_errors=True)
    if direction == "forward":
        assert_close(bf16_to_f64(out), L.lora_forward_ref(d["a_bits"], d["sizes"], Wf, A, B, s, N), "adapter forward")
        return
    dy = synthetic.f32_to_bf16_bits(rng.standard_normal((M, N)).astype(np.float32))
    dx, ga, gb = geg.gnf4_grouped_dgrad_lora(up_u16_as_bf16(dy), g["sizes"], g["w"], g["s"], g["a"], At, Bt, u, s,
                                             opts=o, check_errors=True)
    dx_ref, dA_ref, dB_ref = L.lora_backward_ref(d["a_bits"], dy, d["sizes"], Wf, A, B, s, K)
    assert_close(bf16_to_f64(dx), dx_ref, "adapter dx")
    assert_close(ga.cpu().numpy().astype(np.float64), dA_ref, "adapter dA")
    assert_close(gb.cpu().numpy().astype(np.float64), dB_ref, "adapter dB")


def test_block_gated_epilogue_on_split_tiles(geg):
    # gate_up contracts over H = 8192: the fixup launch applies silu(gate) * up.
    # Over so long a contraction many intermediate values sit within the fp32
    # error band of a bf16 rounding midpoint, where either rounding of the
    # block's bf16 intermediate is a correct result; the bound adds what such a
    # flip can move each output (the same allowance as the full-size blocks).
    from test_gpu_block import block_case
    from test_gpu_full import _act_rounding_allowance
    d = block_case("nf4", 2, 8192, 192, SIZES, seed=56)
    n = int(d["sizes"].sum())
    _, ref = oracle.expert_block_ref(d["a"], d["sizes"], d["w13"], d["w2"], d["H"], d["I"])
    ref = ref[:n]
    x = synthetic.bf16_bits_to_f32(d["a"][:n]).astype(np.float64)
    off = np.concatenate([[0], np.cumsum(d["sizes"])])
    allow = np.zeros_like(ref)
    for e in range(2):
        allow[off[e]:off[e + 1]], _ = _act_rounding_allowance(x[off[e]:off[e + 1]], d["w13"](e), d["w2"](e))
    plain = 1e-2 * np.maximum(1.0, np.abs(ref))
    for cu in (8, 16):
        log(f"case: fused block nf4 H=8192 I=192 sizes={SIZES} tiled, cu_limit={cu}")
        out = geg.gnf4_expert_block(up_u16_as_bf16(d["a"]), up(d["sizes"]), up(d["c13"]), up(d["s13"]), up(d["c2"]),
                                    up(d["s2"]), opts=geg.Opts(2, 0, None, cu), check_errors=True)
        err = np.abs(bf16_to_f64(out)[:n] - ref)
        log(f"  block cu_limit={cu}: max |err|/max(1,|ref|) = {np.max(err / np.maximum(1.0, np.abs(ref))):.5f}; "
            f"share within 1e-2 max(1,|ref|) = {float(np.mean(err <= plain)):.7f}; "
            f"max err / (plain bound + rounding allowance) = {np.max(err / (plain + allow)):.4f}")
        assert np.all(err <= plain + allow)
        # the split remainder rows (expert 1) carry no ambiguity at this size
        assert np.all(err[1024:] <= plain[1024:])


# Three experts of one full block each and two 5- and 7-row remainders, over 2
# output-column tiles: 6 class-0 tiles, then 4 remainder tiles. A grid of 4
# leaves 2 free slots in the second round, so the first 2 remainder tiles run
# whole there and the last 2 split in 2 pieces; a grid of 3 has no free slot and
# 1 tile left over, which splits in 3 pieces of uneven stage counts.
MIXED = [256, 256, 256, 5, 7]


@pytest.mark.parametrize("fmt,K", [("nf4", 2048), ("mxfp4", 2080)])
@pytest.mark.parametrize("cu", [4, 3])
def test_forward_whole_and_split_remainder_tiles(geg, fmt, K, cu):
    log(f"case: tiled forward {fmt}, K={K} N=512 sizes={MIXED} cu_limit={cu}")
    c, d = _case(fmt, K, 512, seed=57, sizes=MIXED)
    g = upload_case(d)
    fn = geg.gnf4_grouped_gemm if fmt == "nf4" else geg.gmxfp4_grouped_gemm
    out = fn(g["a"], g["sizes"], g["w"], g["s"], opts=geg.Opts(2, 0, None, cu), check_errors=True)
    assert_close(bf16_to_f64(out), oracle.grouped_ref(d["a_bits"], d["sizes"], C.weight_fn(d), c.N),
                 f"forward {fmt} K={K} cu={cu}")


@pytest.mark.parametrize("fmt,N", [("nf4", 2048), ("mxfp4", 2056)])
@pytest.mark.parametrize("cu", [4, 3])
def test_dgrad_whole_and_split_remainder_tiles(geg, fmt, N, cu):
    log(f"case: dgrad {fmt}, K=512 N={N} sizes={MIXED} cu_limit={cu}")
    c, d = _case(fmt, 512, N, seed=58, sizes=MIXED)
    rng = np.random.default_rng(59)
    M = int(np.sum(MIXED))
    dy = synthetic.f32_to_bf16_bits(rng.standard_normal((M, N)).astype(np.float32))
    g = upload_case(d)
    fn = geg.gnf4_grouped_dgrad if fmt == "nf4" else geg.gmxfp4_grouped_dgrad
    dx = fn(up_u16_as_bf16(dy), g["sizes"], g["w"], g["s"], opts=geg.Opts(0, 0, None, cu), check_errors=True)
    assert_close(bf16_to_f64(dx), oracle.dgrad_ref(dy, d["sizes"], C.weight_fn(d), 512), f"dgrad {fmt} N={N} cu={cu}")


@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
def test_workspace_without_split_region_runs_unsplit(geg, fmt):
    # a workspace that holds everything but the split partials: the call that
    # would split each remainder tile 4 ways (grid of 8) runs it whole instead
    import torch
    K, N = 8192, 320
    log(f"case: tiled forward {fmt}, K={K} N={N} sizes={SIZES} cu_limit=8, workspace without the split region")
    c, d = _case(fmt, K, N, seed=51)
    g = upload_case(d)
    M = int(np.sum(SIZES))
    op = geg.GEG_OP_NF4_FWD if fmt == "nf4" else geg.GEG_OP_MXFP4_FWD
    o = geg.Opts(2, 0, None, 8)
    need = geg.geg_workspace_bytes(op, M, N, K, 2, o)
    tail = 256 * 128 * 256 * 4
    ws = geg.Workspace(need)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=g["a"].device)
    fn = getattr(geg.lib(), "gnf4_grouped_gemm" if fmt == "nf4" else "gmxfp4_grouped_gemm")
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = fn(p(g["a"]), p(g["sizes"]), p(g["w"]), p(g["s"]), p(out), M, N, K, 2, p(ws.buf), need - tail,
            ctypes.byref(o), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, geg.lib().geg_last_error()
    assert ws.read_error() == 0
    ref = oracle.grouped_ref(d["a_bits"], d["sizes"], C.weight_fn(d), c.N)
    assert_close(bf16_to_f64(out), ref, f"forward {fmt} without the split region")
    # the same call with the whole workspace splits and agrees within fp32 order
    full = geg.gnf4_grouped_gemm if fmt == "nf4" else geg.gmxfp4_grouped_gemm
    split = full(g["a"], g["sizes"], g["w"], g["s"], workspace=ws, opts=o, check_errors=True)
    assert_close(bf16_to_f64(split), ref, f"forward {fmt} split")
