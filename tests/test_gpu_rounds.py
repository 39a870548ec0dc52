"""GPU parity of the persistent kernels past their first round of work, on every
output element.

Every kernel here runs a persistent grid that walks a work list in rounds of
`grid` units. Two ways to make the walk take several rounds while the fp64
oracle still computes every output in seconds:

* `cu_limit` (geg_opts): the library sizes every grid as if the device had that
  many compute units, so small problems take many rounds on every kernel (tiled
  forward and dgrad, narrow, vector, skinny, W4A8, the adapter kernels, the
  fused block). Results must equal the oracle within the path's tolerance and,
  for the kernels whose per-element arithmetic does not depend on the grid,
  equal the uncapped launch bit for bit.
* natural sizes: problems whose tiles number at least three times the full grid
  (256 workgroups for the tiled and W4A8 kernels, the resident workgroups of the
  narrow kernel), with remainder blocks of both tile classes.

Definition of the result: "grouped-nf4-gemm releases", v0.2.6 "The patch point"
(the per-expert loop); tolerance |gpu - ref| <= 1e-2 max(1, |ref|).
"""
import numpy as np
import pytest

import oracle
import synthetic
from oracle import cases as C
from oracle import lora as L
from oracle import w4a8 as W8
from gpu_util import assert_close, bf16_to_f64, bits16, log, up, up_u16_as_bf16, upload_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def geg():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_expert_gemm_amd as g
    g.lib()
    return g


def _case(fmt, E, K, N, sizes, seed, extra_rows=0):
    rng = np.random.default_rng(seed)
    sizes = np.array(sizes, np.int32)
    M = int(sizes.sum()) + extra_rows
    a = synthetic.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    if fmt == "nf4":
        codes = np.zeros((E, N, K // 2), np.uint8)
        sc = np.zeros((E, N, K // 64), np.float32)
        for e in range(E):
            if sizes[e] > 0:
                codes[e], sc[e] = oracle.quantize_pack_nf4((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    else:
        codes = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
        sc = rng.integers(119, 130, (E, N, K // 32), dtype=np.uint8)
    c = synthetic.Case("rounds", fmt, E, K, N, 0, 1)
    return c, {"case": c, "a_bits": a, "sizes": sizes, "codes": codes, "scales": sc}


def _fwd(geg, d, g, force, cu_limit):
    fn = geg.gnf4_grouped_gemm if d["case"].fmt == "nf4" else geg.gmxfp4_grouped_gemm
    return fn(g["a"], g["sizes"], g["w"], g["s"], opts=geg.Opts(force, 0, None, cu_limit), check_errors=True)


# ---------------------------------------------------------------- capped grids

FWD_PATHS = {"tiled": 2, "narrow": 4, "vec": 3, "skinny": 1}


@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
@pytest.mark.parametrize("path", ["tiled", "narrow", "vec", "skinny"])
def test_forward_capped_grid(geg, fmt, path):
    # N = 700: three output-column tiles (the last partial), 11 narrow units of
    # 64 columns, 22 vector row groups of 32; with one or two compute units the
    # tiled kernel walks 23 tiles in 12 rounds, the others tens of rounds
    K = 448 if fmt == "nf4" else 416
    sizes = [0, 3, 130, 0, 33, 1, 257, 32, 0]
    cu = 2 if path == "tiled" else 1
    log(f"case: capped grid forward {fmt} path={path} cu_limit={cu} sizes={sizes} K={K} N=700")
    c, d = _case(fmt, len(sizes), K, 700, sizes, seed=31)
    g = upload_case(d)
    ref = oracle.grouped_ref(d["a_bits"], d["sizes"], C.weight_fn(d), c.N)
    capped = _fwd(geg, d, g, FWD_PATHS[path], cu)
    assert_close(bf16_to_f64(capped), ref, f"capped {fmt} {path}")
    full = _fwd(geg, d, g, FWD_PATHS[path], 0)
    same = bool((bits16(capped) == bits16(full)).all())
    log(f"  bitwise equal to the uncapped launch: {same}")
    if path in ("tiled", "narrow"):
        assert same, "the tile/unit arithmetic does not depend on the grid"


@pytest.mark.parametrize("split", [1, 3])
def test_skinny_split_k_capped_grid(geg, split):
    sizes = [5, 0, 17, 2, 33]
    log(f"case: capped grid skinny split={split} sizes={sizes} K=1024 N=300")
    c, d = _case("nf4", len(sizes), 1024, 300, sizes, seed=32)
    g = upload_case(d)
    out = geg.gnf4_grouped_gemm(g["a"], g["sizes"], g["w"], g["s"], opts=geg.Opts(1, split, None, 1),
                                check_errors=True)
    assert_close(bf16_to_f64(out), oracle.grouped_ref(d["a_bits"], d["sizes"], C.weight_fn(d), c.N),
                 f"capped skinny split={split}")


@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
def test_dgrad_capped_grid(geg, fmt):
    # dX [M, K=704]: three output tiles per row block, two row blocks for one
    # expert, the contraction N = 200 ends 8 into its last stage
    K = 704
    sizes = [0, 300, 3, 0, 70]
    log(f"case: capped grid dgrad {fmt} cu_limit=2 sizes={sizes} K={K} N=200")
    c, d = _case(fmt, len(sizes), K, 200, sizes, seed=33)
    rng = np.random.default_rng(34)
    M = int(np.sum(sizes))
    dy = synthetic.f32_to_bf16_bits(rng.standard_normal((M, 200)).astype(np.float32))
    g = upload_case(d)
    fn = geg.gnf4_grouped_dgrad if fmt == "nf4" else geg.gmxfp4_grouped_dgrad
    dyt = up_u16_as_bf16(dy)
    dx = fn(dyt, g["sizes"], g["w"], g["s"], opts=geg.Opts(0, 0, None, 2), check_errors=True)
    assert_close(bf16_to_f64(dx), oracle.dgrad_ref(dy, d["sizes"], C.weight_fn(d), K), f"capped dgrad {fmt}")
    full = fn(dyt, g["sizes"], g["w"], g["s"])
    assert (bits16(dx) == bits16(full)).all()


def test_w4a8_capped_grid(geg):
    sizes = [0, 3, 130, 0, 257, 1, 0]
    K, N = 2880, 300
    log(f"case: capped grid w4a8 cu_limit=1 sizes={sizes} K={K} N={N}")
    c, d = _case("mxfp4", len(sizes), K, N, sizes, seed=35)
    g = upload_case(d)
    out = geg.gmxfp4_w4a8_grouped_gemm(g["a"], g["sizes"], g["w"], g["s"], opts=geg.Opts(0, 0, None, 1),
                                       check_errors=True)
    ref = W8.w4a8_grouped_ref(d["a_bits"], d["sizes"], C.weight_fn(d), N)
    assert_close(bf16_to_f64(out), ref, "capped w4a8")
    full = geg.gmxfp4_w4a8_grouped_gemm(g["a"], g["sizes"], g["w"], g["s"])
    assert (bits16(out) == bits16(full)).all()


@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
def test_lora_capped_grid(geg, fmt):
    # the adapter kernels (x A^T pass over 16-row units, the gradient row
    # reductions, the transposes) with one compute unit's grid
    E, K, N, r = 5, 256, 200, 16
    sizes = [40, 0, 130, 1, 70]
    log(f"case: capped grid lora {fmt} r={r} sizes={sizes}")
    c, d = _case(fmt, E, K, N, sizes, seed=36)
    rng = np.random.default_rng(37)
    M = int(np.sum(sizes))
    dy = synthetic.f32_to_bf16_bits(rng.standard_normal((M, N)).astype(np.float32))
    A = (rng.standard_normal((E, r, K)) / np.sqrt(K)).astype(np.float32)
    B = (rng.standard_normal((E, N, r)) * 0.5).astype(np.float32)
    Wf = C.weight_fn(d)
    s = 0.5
    g = upload_case(d)
    o = geg.Opts(0, 0, None, 1)
    fwd = geg.gnf4_grouped_gemm_lora if fmt == "nf4" else geg.gmxfp4_grouped_gemm_lora
    bwd = geg.gnf4_grouped_dgrad_lora if fmt == "nf4" else geg.gmxfp4_grouped_dgrad_lora
    At, Bt = up(A), up(B)
    out, u = fwd(g["a"], g["sizes"], g["w"], g["s"], At, Bt, s, opts=o, check_errors=True)
    assert_close(bf16_to_f64(out), L.lora_forward_ref(d["a_bits"], d["sizes"], Wf, A, B, s, N), f"lora fwd {fmt}")
    dx, ga, gb = bwd(up_u16_as_bf16(dy), g["sizes"], g["w"], g["s"], g["a"], At, Bt, u, s, opts=o, check_errors=True)
    dx_ref, dA_ref, dB_ref = L.lora_backward_ref(d["a_bits"], dy, d["sizes"], Wf, A, B, s, K)
    assert_close(bf16_to_f64(dx), dx_ref, f"lora dx {fmt}")
    assert_close(ga.cpu().numpy().astype(np.float64), dA_ref, f"lora dA {fmt}")
    assert_close(gb.cpu().numpy().astype(np.float64), dB_ref, f"lora dB {fmt}")


def test_block_capped_grid(geg):
    from test_gpu_block import block_case, run_block
    d = block_case("nf4", 6, 448, 192, [0, 37, 1, 300, 5, 0], seed=38)
    n = int(d["sizes"].sum())
    _, ref = oracle.expert_block_ref(d["a"], d["sizes"], d["w13"], d["w2"], d["H"], d["I"])
    for path, force in (("tiled", 2), ("narrow", 4), ("vec", 3)):
        log(f"case: capped grid block path={path} cu_limit=1")
        fn = geg.gnf4_expert_block
        out = fn(up_u16_as_bf16(d["a"]), up(d["sizes"]), up(d["c13"]), up(d["s13"]), up(d["c2"]), up(d["s2"]),
                 opts=geg.Opts(force, 0, None, 1), check_errors=True)
        assert_close(bf16_to_f64(out)[:n], ref[:n], f"capped block {path}")


# ---------------------------------------------------------------- natural sizes

# 700 = 2 full blocks + 188 (class 0), 650 = 2 + 138 (class 0), 100 and 40 are
# class-1 remainders, 701 = 2 + 189: 11 row blocks; with 80 output tiles per
# row block that is 880 tiles, 3.4 rounds of the 256-workgroup grid
BIG_SIZES = [700, 650, 100, 701, 40]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
def test_tiled_forward_three_rounds(geg, fmt):
    K, N = (256, 20480) if fmt == "nf4" else (288, 20480)   # MXFP4: a 32-wide K tail
    log(f"case: tiled forward {fmt} sizes={BIG_SIZES} K={K} N={N} (880 tiles)")
    c, d = _case(fmt, len(BIG_SIZES), K, N, BIG_SIZES, seed=41)
    g = upload_case(d)
    out = _fwd(geg, d, g, 0, 0)
    assert_close(bf16_to_f64(out), oracle.grouped_ref(d["a_bits"], d["sizes"], C.weight_fn(d), N),
                 f"tiled forward {fmt} 3+ rounds")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
def test_tiled_dgrad_three_rounds(geg, fmt):
    K, N = 20480, 256   # dX [M, 20480]: 80 output tiles per row block
    log(f"case: tiled dgrad {fmt} sizes={BIG_SIZES} K={K} N={N} (880 tiles)")
    c, d = _case(fmt, len(BIG_SIZES), K, N, BIG_SIZES, seed=42)
    rng = np.random.default_rng(43)
    M = int(np.sum(BIG_SIZES))
    dy = synthetic.f32_to_bf16_bits(rng.standard_normal((M, N)).astype(np.float32))
    g = upload_case(d)
    fn = geg.gnf4_grouped_dgrad if fmt == "nf4" else geg.gmxfp4_grouped_dgrad
    dx = fn(up_u16_as_bf16(dy), g["sizes"], g["w"], g["s"], check_errors=True)
    assert_close(bf16_to_f64(dx), oracle.dgrad_ref(dy, d["sizes"], C.weight_fn(d), K), f"tiled dgrad {fmt} 3+ rounds")


@pytest.mark.timeout(600)
def test_w4a8_three_rounds(geg):
    K, N = 256, 10240   # 256 x 128 tiles: 80 per row block, 880 in all
    log(f"case: w4a8 sizes={BIG_SIZES} K={K} N={N} (880 tiles)")
    c, d = _case("mxfp4", len(BIG_SIZES), K, N, BIG_SIZES, seed=44)
    g = upload_case(d)
    out = geg.gmxfp4_w4a8_grouped_gemm(g["a"], g["sizes"], g["w"], g["s"], check_errors=True)
    ref = W8.w4a8_grouped_ref(d["a_bits"], d["sizes"], C.weight_fn(d), N)
    assert_close(bf16_to_f64(out), ref, "w4a8 3+ rounds")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
def test_narrow_three_rounds(geg, fmt):
    # 64 experts of 17..40 rows (a decode batch: M <= 32 E, every expert narrow,
    # 32-row units over 128 weight rows); N = 8192 gives 64 column blocks, so
    # about 5000 units against the 768 or so resident workgroups
    rng = np.random.default_rng(45)
    sizes = rng.integers(17, 41, 64).astype(np.int32)
    sizes[[3, 40]] = 0
    K, N = 256, 8192
    log(f"case: narrow {fmt} E=64 M={int(sizes.sum())} K={K} N={N}")
    c, d = _case(fmt, 64, K, N, sizes, seed=46)
    g = upload_case(d)
    out = _fwd(geg, d, g, 0, 0)
    assert_close(bf16_to_f64(out), oracle.grouped_ref(d["a_bits"], d["sizes"], C.weight_fn(d), N),
                 f"narrow {fmt} 3+ rounds")
