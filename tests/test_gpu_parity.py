"""GPU parity of the grouped GEMMs against the fp64 oracle, on small and medium
seeded cases where the oracle computes every output, through every path."""
import numpy as np
import pytest

import oracle
import synthetic
from oracle import cases as C
from oracle import pack as P
from gpu_util import (TOL, assert_close, bf16_to_f64, bits16, log, up, up_u16_as_bf16,
                      upload_case, sha)

pytestmark = pytest.mark.gpu

PATHS = {"auto": None, "skinny": (1, 0), "tiled": (2, 0), "vec": (3, 0), "narrow": (4, 0)}


@pytest.fixture(scope="module")
def geg():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_expert_gemm_amd as g
    g.lib()
    return g


def _opts(geg, path, split=0):
    if path is None:
        return geg.Opts(0, split) if split else None
    return geg.Opts(path[0], split or path[1])


def run_fwd(geg, c, g, path=None, split=0, ws=None):
    opts = _opts(geg, PATHS.get(path, path) if isinstance(path, str) else path, split)
    fn = geg.gnf4_grouped_gemm if c.fmt == "nf4" else geg.gmxfp4_grouped_gemm
    return fn(g["a"], g["sizes"], g["w"], g["s"], opts=opts, workspace=ws)


def custom_case(fmt, E, K, N, sizes, seed=0, extra_rows=0):
    """A case with hand-chosen sizes; weights packed by the oracle."""
    rng = np.random.default_rng(seed)
    sizes = np.array(sizes, np.int32)
    M = int(sizes.sum()) + extra_rows
    a = synthetic.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    if fmt == "nf4":
        codes = np.zeros((E, N, K // 2), np.uint8)
        sc = np.zeros((E, N, K // 64), np.float32)
        for e in range(E):
            codes[e], sc[e] = oracle.quantize_pack_nf4((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    else:
        codes = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
        sc = rng.integers(119, 130, (E, N, K // 32), dtype=np.uint8)
    c = synthetic.Case("custom", fmt, E, K, N, 0, 1)
    d = {"case": c, "a_bits": a, "sizes": sizes, "codes": codes, "scales": sc}
    return c, d


def ref_of(d):
    c = d["case"]
    return oracle.grouped_ref(d["a_bits"], d["sizes"], C.weight_fn(d), c.N)


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("path", ["auto", "skinny", "tiled", "vec", "narrow"])
def test_tiny_config(geg, seed, path):
    c = synthetic.case("tiny")
    log(f"case: tiny seed={seed} path={path}")
    d = C.build(c, seed)
    out = run_fwd(geg, c, upload_case(d), path)
    assert_close(bf16_to_f64(out), ref_of(d), f"tiny s{seed} {path}")


@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
@pytest.mark.parametrize("path", ["auto", "skinny", "tiled", "vec", "narrow"])
def test_medium_ragged(geg, fmt, path):
    # several 128x128 tiles, ragged row and column tails, zero-row experts at both
    # ends, skinny (<=32 rows) and tiled experts mixed, K with a 64 (NF4) or 96
    # (MXFP4) tail past the last 128-step
    K = 448 if fmt == "nf4" else 416
    sizes = [0, 3, 130, 0, 33, 1, 257, 32, 0]
    log(f"case: medium ragged {fmt} path={path} sizes={sizes} K={K} N=200")
    c, d = custom_case(fmt, len(sizes), K, 200, sizes, seed=5)
    out = run_fwd(geg, c, upload_case(d), path)
    assert_close(bf16_to_f64(out), ref_of(d), f"medium {fmt} {path}")


@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
def test_exact_integer_case_is_bitwise(geg, fmt):
    # sparse small codes, power-of-two scales and activations in {-1, 0, 1}: every
    # product and partial sum is exact in fp32 and every result exact in bf16
    log(f"case: exact integer {fmt}")
    E, N, K = 3, 48, 256
    sizes = np.array([0, 5, 40], np.int32)
    rng = np.random.default_rng(3)
    a = synthetic.f32_to_bf16_bits(rng.integers(-1, 2, (45, K)).astype(np.float32))
    nz = rng.random((E, N, K)) < 0.125
    if fmt == "nf4":
        c4 = np.where(nz, rng.choice(np.array([0, 15], np.uint8), size=(E, N, K)), 7).astype(np.uint8)
        codes = P.pack_nf4_codes(c4)
        sc = (2.0 ** rng.integers(-2, 3, (E, N, K // 64))).astype(np.float32)
    else:
        c4 = np.where(nz, rng.choice(np.array([1, 2, 3, 9, 10, 11], np.uint8), size=(E, N, K)),
                      rng.choice(np.array([0, 8], np.uint8), size=(E, N, K))).astype(np.uint8)
        codes = P.pack_mxfp4_codes(c4)
        sc = rng.integers(126, 129, (E, N, K // 32)).astype(np.uint8)
    c = synthetic.Case("exact", fmt, E, K, N, 0, 1)
    d = {"case": c, "a_bits": a, "sizes": sizes, "codes": codes, "scales": sc}
    ref = ref_of(d)
    refbits = P.bf16_rne_bits(ref.astype(np.float32))
    assert np.array_equal(synthetic.bf16_bits_to_f32(refbits), ref)       # exact in bf16
    for path in ["skinny", "tiled", "vec", "narrow"]:
        out = run_fwd(geg, c, upload_case(d), path)
        gb = bits16(out)
        bad = np.argwhere(gb != refbits)
        log(f"  {path}: {len(bad)} mismatches {bad[:5].tolist()}")
        assert len(bad) == 0, path


@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
def test_decode_equals_tiled_and_splits_agree(geg, fmt):
    name = "olmoe_gate_up_t1" if fmt == "nf4" else "gptoss_down_t1"
    c = synthetic.case(name)
    log(f"case: {name} paths and split-K")
    d = C.build(c, 0, experts=np.nonzero(synthetic.routing(c, 0)[0])[0])
    g = upload_case(d)
    ref = ref_of(d)
    outs = {}
    for path, split in [("skinny", 1), ("skinny", 2), ("skinny", 3), ("skinny", 8), ("tiled", 0), ("vec", 0),
                        ("narrow", 0), ("auto", 0)]:
        o = run_fwd(geg, c, g, path, split)
        assert_close(bf16_to_f64(o), ref, f"{name} {path} split={split}")
        outs[(path, split)] = bf16_to_f64(o)
    assert np.max(np.abs(outs[("skinny", 1)] - outs[("tiled", 0)])) <= 2 * TOL * max(1, np.abs(ref).max())


@pytest.mark.parametrize("fmt,K", [("nf4", 768), ("nf4", 2048), ("nf4", 4096), ("mxfp4", 1024),
                                   ("mxfp4", 2880)])
def test_vector_path_shapes(geg, fmt, K):
    # the vector path's lane layouts: rows of <= 32 chunks (two weight rows per
    # load, K = 768 / 1024), exactly one row per load (2048), several loads per
    # row with a partial last one (2880: 90 chunks) or full ones (4096); N = 200
    # leaves a ragged last unit; 5 and 9 rows take 2 and 3 row chunks
    sizes = [1, 0, 2, 3, 4, 5, 9, 0, 1]
    log(f"case: vector path {fmt} K={K} N=200 sizes={sizes}")
    c, d = custom_case(fmt, len(sizes), K, 200, sizes, seed=11)
    g = upload_case(d)
    ref = ref_of(d)
    for path in ["vec", "narrow", "auto"]:
        out = run_fwd(geg, c, g, path)
        assert_close(bf16_to_f64(out), ref, f"vector {fmt} K={K} {path}")


def test_determinism_nonmutation_and_canary(geg):
    import torch
    log("case: determinism / non-mutation / canary rows past sum(sizes)")
    c, d = custom_case("nf4", 6, 512, 320, [20, 0, 140, 7, 0, 33], seed=9, extra_rows=16)
    g = upload_case(d)
    before = {k: sha(v) for k, v in g.items()}
    for path in ["auto", "skinny", "tiled"]:
        out = torch.full((g["a"].shape[0], c.N), 7.0, dtype=torch.bfloat16, device=g["a"].device)
        opts = _opts(geg, PATHS[path])
        o1 = geg.gnf4_grouped_gemm(g["a"], g["sizes"], g["w"], g["s"], out=out, opts=opts).clone()
        o2 = geg.gnf4_grouped_gemm(g["a"], g["sizes"], g["w"], g["s"], opts=opts)
        m = int(d["sizes"].sum())
        assert torch.equal(o1[:m], o2[:m]), path                       # bitwise run to run
        assert torch.all(o1[m:] == 7.0), path                          # rows past sum(sizes) untouched
        assert_close(bf16_to_f64(o1[:m]), ref_of(d)[:m], f"canary case {path}")
    after = {k: sha(v) for k, v in g.items()}
    assert before == after                                             # inputs not modified


def test_skewed_single_expert_matches_dense_fp32_matmul(geg):
    import torch
    log("case: all rows on one expert vs torch fp32 matmul over the fp32 export")
    c, d = custom_case("nf4", 4, 1024, 384, [0, 0, 300, 0], seed=11)
    g = upload_case(d)
    out = run_fwd(geg, c, g)
    w32, _, _ = geg.gnf4_dequant(g["w"], g["s"], bf16=False, f16=False)
    dense = (g["a"].float() @ w32[2].T).double().cpu().numpy()
    assert_close(bf16_to_f64(out), dense, "dense cross-check")


def test_bad_sizes_are_flagged_and_clamped(geg):
    import torch
    log("case: negative sizes / sum(sizes) > M")
    c, d = custom_case("nf4", 3, 256, 128, [10, 20, 5], seed=2)
    g = upload_case(d)
    ws = geg.Workspace(1 << 16)
    bad = up(np.array([10, -4, 5], np.int32))
    geg.gnf4_grouped_gemm(g["a"], bad, g["w"], g["s"], workspace=ws)
    assert ws.read_error() & geg.DEVERR_NEGATIVE_SIZE
    ws.reset()
    over = up(np.array([10, 20, 50], np.int32))                        # sum 80 > M = 35
    out = geg.gnf4_grouped_gemm(g["a"], over, g["w"], g["s"], workspace=ws)
    assert ws.read_error() & geg.DEVERR_SIZES_EXCEED_M
    # rows of the clamped last expert are still correct (5 rows fit under M)
    d2 = dict(d, sizes=np.array([10, 20, 5], np.int32))
    assert_close(bf16_to_f64(out), ref_of(d2), "clamped sizes")
    ws.reset()
    assert ws.read_error() == 0


def test_fp16_range_flag(geg):
    # An activation beyond fp16 range: the decode paths convert bf16 -> fp16
    # directly and flag the overflow; the tiled path scales each row by a power
    # of two first, so the same row is computed exactly and nothing is flagged;
    # a non-finite activation is flagged on the tiled path too.
    log("case: activation beyond fp16 range on the NF4 path")
    c, d = custom_case("nf4", 2, 128, 64, [3, 40], seed=4)
    d["a_bits"][1, 5] = synthetic.f32_to_bf16_bits(np.array([1.0e5], np.float32))[0]
    g = upload_case(d)
    for path in ["skinny", "narrow", "vec"]:
        ws = geg.Workspace(1 << 16)
        run_fwd(geg, c, g, path, ws=ws)
        assert ws.read_error() & geg.DEVERR_FP16_RANGE, path
    ws = geg.Workspace(1 << 16)
    out = run_fwd(geg, c, g, "tiled", ws=ws)
    assert ws.read_error() == 0
    assert_close(bf16_to_f64(out), ref_of(d), "tiled, row holding 1e5")
    d["a_bits"][1, 5] = 0x7F80                                            # +inf
    ws = geg.Workspace(1 << 16)
    run_fwd(geg, c, upload_case(d), "tiled", ws=ws)
    assert ws.read_error() & geg.DEVERR_FP16_RANGE
    with pytest.raises(geg.GegDeviceError, match="fp16"):
        run_fwd_checked = geg.gnf4_grouped_gemm
        run_fwd_checked(*(upload_case(d)[k] for k in ("a", "sizes", "w", "s")), opts=geg.Opts(2, 0),
                        workspace=ws, check_errors=True)
    assert ws.read_error() == 0                                           # cleared when it raised
    ws = geg.Workspace(1 << 16)
    d["a_bits"][1, 5] = 0
    run_fwd(geg, c, upload_case(d), "auto", ws=ws)
    assert ws.read_error() == 0


@pytest.mark.parametrize("scale", [1e-6, 1e-7, 1e-8, 1e6])
def test_nf4_dgrad_row_scaling_keeps_small_and_large_gradients(geg, scale):
    # Activation gradients of a training step sit far below fp16's normal range
    # (2^-14); the tiled NF4 path multiplies each dY row by a power of two before
    # its fp16 conversion and the results back after, so dX keeps its relative
    # precision at any scale. Checked against max|err| / max|ref|, which does not
    # fall back on the absolute floor of max(1, |ref|) when |ref| << 1.
    log(f"case: nf4 dgrad with dY ~ N(0, {scale:g})")
    c, d = custom_case("nf4", 4, 320, 136, [0, 37, 150, 5], seed=6)
    rng = np.random.default_rng(8)
    dyf = (rng.standard_normal((192, 136)) * scale).astype(np.float32)
    dyf[3, :] *= 1e-3                        # one row three decades smaller than the rest
    dy = synthetic.f32_to_bf16_bits(dyf)
    g = upload_case(d)
    dx = geg.gnf4_grouped_dgrad(up_u16_as_bf16(dy), g["sizes"], g["w"], g["s"], check_errors=True)
    ref = oracle.dgrad_ref(dy, d["sizes"], C.weight_fn(d), c.K)
    got = bf16_to_f64(dx)
    rel = float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
    row_rel = float(np.max(np.abs(got[3] - ref[3])) / np.max(np.abs(ref[3])))
    log(f"  max|err|/max|ref| = {rel:.2e}, small row {row_rel:.2e}")
    assert rel <= 1e-2 and row_rel <= 1e-2


@pytest.mark.parametrize("N", [9000, 20000])
def test_nf4_dgrad_long_rows(geg, N):
    # dY rows of more than 8192 values take the one-workgroup-per-row conversion
    # (up to 8 or 16 chunks per thread); one row four decades smaller than the rest
    log(f"case: nf4 dgrad with dY rows of {N} values")
    c, d = custom_case("nf4", 3, 128, N, [21, 0, 50], seed=14)
    rng = np.random.default_rng(15)
    dyf = rng.standard_normal((71, N)).astype(np.float32)
    dyf[30, :] *= 1e-4
    dy = synthetic.f32_to_bf16_bits(dyf)
    g = upload_case(d)
    dx = geg.gnf4_grouped_dgrad(up_u16_as_bf16(dy), g["sizes"], g["w"], g["s"], check_errors=True)
    ref = oracle.dgrad_ref(dy, d["sizes"], C.weight_fn(d), c.K)
    got = bf16_to_f64(dx)
    assert_close(got, ref, f"dgrad N={N}")
    row_rel = float(np.max(np.abs(got[30] - ref[30])) / np.max(np.abs(ref[30])))
    log(f"  small row max|err|/max|ref| = {row_rel:.2e}")
    assert row_rel <= 1e-2


def test_nf4_forward_long_rows(geg):
    # activation rows of 9216 values: the one-workgroup-per-row conversion
    log("case: nf4 tiled forward with K = 9216")
    c, d = custom_case("nf4", 2, 9216, 96, [33, 60], seed=16)
    out = run_fwd(geg, c, upload_case(d), "tiled")
    assert_close(bf16_to_f64(out), ref_of(d), "forward K=9216")


@pytest.mark.parametrize("scale", [1e-7, 1e4])
def test_nf4_forward_row_scaling(geg, scale):
    # the same on the forward tiled path: activations far below or above fp16's
    # range are computed at full relative precision
    log(f"case: nf4 tiled forward with activations ~ N(0, {scale:g})")
    c, d = custom_case("nf4", 3, 256, 200, [40, 0, 260], seed=12)
    d["a_bits"] = synthetic.f32_to_bf16_bits(synthetic.bf16_bits_to_f32(d["a_bits"]) * np.float32(scale))
    out = run_fwd(geg, c, upload_case(d), "tiled")
    ref = ref_of(d)
    rel = float(np.max(np.abs(bf16_to_f64(out) - ref)) / np.max(np.abs(ref)))
    log(f"  max|err|/max|ref| = {rel:.2e}")
    assert rel <= 1e-2


def test_empty_and_single_expert(geg):
    import torch
    log("case: M=0, E=1")
    c, d = custom_case("mxfp4", 1, 64, 32, [0], seed=1)
    g = upload_case(d)
    out = geg.gmxfp4_grouped_gemm(g["a"], g["sizes"], g["w"], g["s"])
    assert out.shape == (0, 32)
    c, d = custom_case("mxfp4", 1, 64, 32, [77], seed=1)
    out = run_fwd(geg, c, upload_case(d))
    assert_close(bf16_to_f64(out), ref_of(d), "E=1")


def test_dgrad_small(geg):
    log("case: dgrad small ragged")
    c, d = custom_case("nf4", 4, 320, 136, [0, 37, 150, 5], seed=6)
    rng = np.random.default_rng(7)
    dy = synthetic.f32_to_bf16_bits(rng.standard_normal((192, 136)).astype(np.float32))
    g = upload_case(d)
    dx = geg.gnf4_grouped_dgrad(up_u16_as_bf16(dy), g["sizes"], g["w"], g["s"])
    ref = oracle.dgrad_ref(dy, d["sizes"], C.weight_fn(d), c.K)
    assert_close(bf16_to_f64(dx), ref, "dgrad small")


def test_dgrad_medium_ragged(geg):
    # two row blocks for one expert, a K that ends inside an output tile, and an
    # N (the contraction) that ends 8 into its last 64-wide stage
    log("case: dgrad medium ragged")
    c, d = custom_case("nf4", 5, 448, 200, [0, 300, 3, 0, 70], seed=9)
    rng = np.random.default_rng(10)
    dy = synthetic.f32_to_bf16_bits(rng.standard_normal((373, 200)).astype(np.float32))
    g = upload_case(d)
    dx = geg.gnf4_grouped_dgrad(up_u16_as_bf16(dy), g["sizes"], g["w"], g["s"])
    ref = oracle.dgrad_ref(dy, d["sizes"], C.weight_fn(d), c.K)
    assert_close(bf16_to_f64(dx), ref, "dgrad medium")


def test_graph_capture_replays(geg):
    import torch
    log("case: hip graph capture of decode + prefill calls, 3 replays")
    c, d = custom_case("nf4", 5, 256, 192, [2, 0, 150, 1, 40], seed=8)
    g = upload_case(d)
    ref = ref_of(d)
    ws = geg.Workspace(geg.geg_workspace_bytes(0, int(d["sizes"].sum()), c.N, c.K, c.E, geg.Opts(0, 4)))
    out = torch.empty((int(d["sizes"].sum()), c.N), dtype=torch.bfloat16, device=g["a"].device)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        geg.gnf4_grouped_gemm(g["a"], g["sizes"], g["w"], g["s"], out=out, workspace=ws, opts=geg.Opts(0, 4))
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        geg.gnf4_grouped_gemm(g["a"], g["sizes"], g["w"], g["s"], out=out, workspace=ws, opts=geg.Opts(0, 4))
    for i in range(3):
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), i
    assert_close(bf16_to_f64(out), ref, "graph replay")


def test_dgrad_mxfp4_ragged(geg):
    # MXFP4 dgrad on the released bytes: two row blocks for one expert, K that
    # ends inside an output tile, an N (the contraction) that ends 8 into its
    # last 64-wide stage, zero-row experts at both ends
    log("case: dgrad mxfp4 ragged")
    c, d = custom_case("mxfp4", 5, 416, 200, [0, 300, 3, 70, 0], seed=11)
    rng = np.random.default_rng(12)
    dy = synthetic.f32_to_bf16_bits(rng.standard_normal((373, 200)).astype(np.float32))
    g = upload_case(d)
    dx = geg.gmxfp4_grouped_dgrad(up_u16_as_bf16(dy), g["sizes"], g["w"], g["s"])
    ref = oracle.dgrad_ref(dy, d["sizes"], C.weight_fn(d), c.K)
    assert_close(bf16_to_f64(dx), ref, "dgrad mxfp4 ragged")


@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
def test_autograd_grouped_linear(geg, fmt):
    # forward through the grouped GEMM, backward through the dgrad kernel, driven
    # by torch autograd; dA checked against the oracle's dgrad of the same dOut
    import torch
    K = 320 if fmt == "nf4" else 288
    c, d = custom_case(fmt, 4, K, 136, [5, 0, 90, 30], seed=13)
    g = upload_case(d)
    a = g["a"].clone().requires_grad_(True)
    out = geg.grouped_linear(a, g["sizes"], g["w"], g["s"], fmt)
    rng = np.random.default_rng(14)
    dout = synthetic.f32_to_bf16_bits(rng.standard_normal((125, 136)).astype(np.float32))
    out.backward(up_u16_as_bf16(dout))
    assert_close(bf16_to_f64(out), ref_of(d), f"autograd forward {fmt}")
    assert_close(bf16_to_f64(a.grad), oracle.dgrad_ref(dout, d["sizes"], C.weight_fn(d), K), f"autograd dA {fmt}")
