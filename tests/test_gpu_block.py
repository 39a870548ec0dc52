"""GPU parity of the fused expert block (gate_up grouped GEMM -> SwiGLU in its
epilogue -> down grouped GEMM) against the fp64 oracle, through every path that
carries the gated epilogue (tiled, narrow, vector) and the automatic choice."""
import numpy as np
import pytest

import oracle
import synthetic
from gpu_util import assert_close, bf16_to_f64, bits16, log, up, up_u16_as_bf16

pytestmark = pytest.mark.gpu

PATHS = {"auto": 0, "tiled": 2, "vec": 3, "narrow": 4}


@pytest.fixture(scope="module")
def geg():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_expert_gemm_amd as g
    g.lib()
    return g


def _pack(fmt, rng, E, N, K):
    if fmt == "nf4":
        codes = np.zeros((E, N, K // 2), np.uint8)
        sc = np.zeros((E, N, K // 64), np.float32)
        for e in range(E):
            codes[e], sc[e] = oracle.quantize_pack_nf4((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
        return codes, sc, (lambda e: oracle.dequant_nf4(codes[e], sc[e]))
    codes = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    sc = rng.integers(119, 124, (E, N, K // 32), dtype=np.uint8)
    return codes, sc, (lambda e: oracle.dequant_mxfp4(codes[e], sc[e]))


def block_case(fmt, E, H, I, sizes, seed=0, extra_rows=0):
    rng = np.random.default_rng(seed)
    sizes = np.array(sizes, np.int32)
    M = int(sizes.sum()) + extra_rows
    a = synthetic.f32_to_bf16_bits(rng.standard_normal((M, H)).astype(np.float32))
    c13, s13, w13 = _pack(fmt, rng, E, 2 * I, H)
    c2, s2, w2 = _pack(fmt, rng, E, H, I)
    return dict(fmt=fmt, a=a, sizes=sizes, c13=c13, s13=s13, c2=c2, s2=s2, w13=w13, w2=w2, H=H, I=I)


def run_block(geg, d, path="auto", out=None):
    fn = geg.gnf4_expert_block if d["fmt"] == "nf4" else geg.gmxfp4_expert_block
    opts = geg.Opts(PATHS[path], 0) if PATHS[path] else None
    return fn(up_u16_as_bf16(d["a"]), up(d["sizes"]), up(d["c13"]), up(d["s13"]), up(d["c2"]),
              up(d["s2"]), out=out, opts=opts)


def check(geg, d, path, what):
    out = run_block(geg, d, path)
    n = int(d["sizes"].sum())
    _, ref = oracle.expert_block_ref(d["a"], d["sizes"], d["w13"], d["w2"], d["H"], d["I"])
    assert_close(bf16_to_f64(out)[:n], ref[:n], what)


@pytest.mark.parametrize("path", ["auto", "tiled", "vec", "narrow"])
def test_block_small(geg, path):
    # E=8, H=256, I=256: the tiny configuration's shape as an expert MLP
    log(f"case: block small path={path}")
    d = block_case("nf4", 8, 256, 256, [16, 7, 30, 0, 1, 20, 9, 45], seed=0)
    check(geg, d, path, f"block small {path}")


@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
@pytest.mark.parametrize("path", ["auto", "tiled", "vec", "narrow"])
def test_block_ragged(geg, fmt, path):
    # zero-row experts at both ends, one-row and tiled experts, a fused width
    # (2I) and a hidden size that leave partial column tiles
    H, I = (448, 192) if fmt == "nf4" else (416, 96)
    log(f"case: block ragged fmt={fmt} path={path} H={H} I={I}")
    d = block_case(fmt, 6, H, I, [0, 37, 1, 300, 5, 0], seed=1)
    check(geg, d, path, f"block ragged {fmt} {path}")


@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
def test_block_decode_shapes(geg, fmt):
    # one token over its top-8 experts (vector path), then a decode batch of
    # 64 tokens spread over the experts (narrow kernel)
    H, I = (2048, 512) if fmt == "nf4" else (960, 480)   # 64 and 30 chunks per row
    rng = np.random.default_rng(7)
    s1 = np.zeros(64, np.int32)
    s1[rng.choice(64, 8, replace=False)] = 1
    log(f"case: block decode T=1 fmt={fmt}")
    check(geg, block_case(fmt, 64, H, I, s1, seed=2), "auto", f"block T=1 {fmt}")
    s64 = np.bincount(rng.integers(0, 64, 512), minlength=64).astype(np.int32)
    log(f"case: block decode T=64 fmt={fmt}")
    check(geg, block_case(fmt, 64, H, I, s64, seed=3), "auto", f"block T=64 {fmt}")


def test_block_rows_past_routed_untouched_and_empty(geg):
    import torch
    d = block_case("nf4", 4, 256, 128, [3, 0, 40, 2], seed=4, extra_rows=5)
    M, H = d["a"].shape
    out = torch.full((M, H), 7.0, dtype=torch.bfloat16, device="cuda")
    run_block(geg, d, "auto", out=out)
    tail = bf16_to_f64(out)[45:]
    assert (tail == 7.0).all()
    # M = 0 is a no-op
    e = block_case("nf4", 4, 256, 128, [0, 0, 0, 0], seed=5)
    z = run_block(geg, e, "auto")
    assert z.shape == (0, 256)


def test_block_refuses_skinny_and_bad_shapes(geg):
    d = block_case("nf4", 2, 128, 64, [3, 4], seed=6)
    with pytest.raises(geg.GegError):
        geg.gnf4_expert_block(up_u16_as_bf16(d["a"]), up(d["sizes"]), up(d["c13"]), up(d["s13"]),
                              up(d["c2"]), up(d["s2"]), opts=geg.Opts(1, 0))
    # I not a multiple of 64 (the down projection's K)
    import torch
    a = up_u16_as_bf16(d["a"])
    w13 = torch.zeros((2, 2 * 96, 64), dtype=torch.uint8, device="cuda")
    s13 = torch.ones((2, 2 * 96, 2), dtype=torch.float32, device="cuda")
    w2 = torch.zeros((2, 128, 48), dtype=torch.uint8, device="cuda")
    s2 = torch.ones((2, 128, 1), dtype=torch.float32, device="cuda")
    with pytest.raises(geg.GegError):
        geg.gnf4_expert_block(a, up(d["sizes"]), w13, s13, w2, s2)
