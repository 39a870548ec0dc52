"""GPU parity of the W4A8 variant (MXFP8 e4m3 activations x MXFP4 weights on the
block-scaled matrix instruction) against oracle.w4a8.

The activation quantisation is integer work decided on exactly scaled values:
codes and scales must match the oracle bit for bit.

The GEMM is asserted at the path's tolerance, |gpu - ref| <= 1e-2 max(1, |ref|)
per element, against the oracle of the quantised operands. The instruction's
128-wide dot products keep about 12 bits below the largest product (in-bounds
probes on gfx950 measured errors up to 3e-4 of max |a w| per instruction,
unbiased), so the error is also printed against S = sum_k |a_k w_k| as a
diagnostic of that arithmetic (err / (2^-10 S) stays below 1 on every case).
"""
import numpy as np
import pytest

import oracle
import synthetic
from oracle import cases as C
from oracle import w4a8 as W
from gpu_util import bf16_to_f64, log, up, up_u16_as_bf16, sample_positions

pytestmark = pytest.mark.gpu

TOL = 1e-2
ACC = 2.0 ** -10


@pytest.fixture(scope="module")
def geg():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_expert_gemm_amd as g
    g.lib()
    return g


def _codes_of(t):
    return t.cpu().numpy()


def _act_bits(rng, M, K):
    # rows of different magnitudes, a zero block, a block of tiny values, -0
    a = rng.standard_normal((M, K)).astype(np.float32) * (10.0 ** rng.uniform(-3, 3, (M, 1))).astype(np.float32)
    a[0, :32] = 0.0
    if M > 1:
        a[1, 32:64] *= 1e-30
    bits = synthetic.f32_to_bf16_bits(a)
    bits[0, 5] = 0x8000
    return bits


@pytest.mark.parametrize("M,K", [(1, 32), (37, 2880), (300, 128), (64, 2048)])
def test_quantize_bit_exact(geg, M, K):
    log(f"case: mxfp8 quantize M={M} K={K}")
    rng = np.random.default_rng(M + K)
    bits = _act_bits(rng, M, K)
    codes, scales = geg.gmxfp8_quantize(up_u16_as_bf16(bits))
    rc, rs = W.quantize_mxfp8(bits)
    assert np.array_equal(_codes_of(scales), rs)
    got = _codes_of(codes)
    bad = np.argwhere(got != rc)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:3].tolist()}: {got[tuple(bad[0])]:#x} vs {rc[tuple(bad[0])]:#x}"


def test_quantize_ties_and_saturation(geg):
    # one block per row; element 0 fixes the scale (amax 1 -> X = 119, step 2^-8),
    # the rest are bf16 values whose scaled value sits exactly between two e4m3
    # values, or just past 448 (saturation)
    vals = [(1 + m / 8 + 1 / 16) * 2.0 ** e for e in range(-6, 9) for m in range(8)]   # normal grid
    vals += [(k + 0.5) * 2.0 ** -9 for k in range(8)]                                  # 2^-9 grid
    vals = np.array(vals, dtype=np.float64)
    rows = []
    for i in range(0, len(vals), 31):
        chunk = vals[i:i + 31] / 256.0
        row = np.zeros(32, np.float32)
        row[0] = 1.0
        row[1:1 + len(chunk)] = chunk.astype(np.float32)
        rows.append(row)
    rows.append(np.array([1.9375, -1.90625, 1.75, 1.8125] + [0.0] * 28, np.float32))
    bits = synthetic.f32_to_bf16_bits(np.stack(rows))
    assert np.array_equal(synthetic.bf16_bits_to_f32(bits), np.stack(rows)), "fixture values must be exact in bf16"
    log(f"case: mxfp8 ties rows={len(rows)}")
    codes, scales = geg.gmxfp8_quantize(up_u16_as_bf16(bits))
    rc, rs = W.quantize_mxfp8(bits)
    assert np.array_equal(_codes_of(scales), rs)
    assert np.array_equal(_codes_of(codes), rc)


def _sum_abs(a_bits, sizes, wfn, N):
    codes, X = W.quantize_mxfp8(a_bits)
    a = np.abs(W.dequant_mxfp8(codes, X))
    off = oracle.offsets(sizes)
    S = np.zeros((a.shape[0], N))
    for e in range(len(sizes)):
        if sizes[e]:
            S[off[e]:off[e + 1]] = a[off[e]:off[e + 1]] @ np.abs(wfn(e)).T
    return S


def _check(got, ref, S, what):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = TOL * np.maximum(1.0, np.abs(ref))
    acc_bound = ACC * S   # diagnostic only: the instruction's dot-product arithmetic
    log(f"  {what}: max |err|/max(1,|ref|) = {np.max(err / np.maximum(1.0, np.abs(ref))):.5f}, "
        f"max err/(2^-10 S) = {np.max(err / np.maximum(acc_bound, 1e-30)):.4f}, "
        f"share within 1e-2 max(1,|ref|) = {float(np.mean(err <= bound)):.5f}")
    assert np.all(err <= bound), f"{what}: err exceeds 1e-2 max(1,|ref|) at {np.argwhere(err > bound)[:3].tolist()}"


@pytest.mark.parametrize("K,N,sizes", [
    (2880, 200, [0, 3, 130, 0, 257, 1, 0]),      # K tail of 64 in the last step, ragged tiles
    (416, 99, [5, 0, 140, 2]),                    # odd N (single-element stores), K tail of 32
    (32, 64, [3, 7]),                             # one 32-block: the first step is the tail
    (1024, 384, [128, 256, 0, 1]),                # whole tiles
])
def test_w4a8_matches_oracle(geg, K, N, sizes):
    log(f"case: w4a8 K={K} N={N} sizes={sizes}")
    rng = np.random.default_rng(K + N)
    E = len(sizes)
    M = int(sum(sizes)) + 3                        # rows past sum(sizes) stay untouched
    a = synthetic.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    codes = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    sc = rng.integers(119, 130, (E, N, K // 32), dtype=np.uint8)
    wfn = lambda e: oracle.dequant_mxfp4(codes[e], sc[e])
    import torch
    out = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    geg.gmxfp4_w4a8_grouped_gemm(up_u16_as_bf16(a), up(np.array(sizes, np.int32)), up(codes), up(sc), out=out)
    got = bf16_to_f64(out)
    m = int(sum(sizes))
    assert (got[m:] == 7.0).all(), "rows past sum(sizes) were written"
    ref = W.w4a8_grouped_ref(a, sizes, wfn, N)[:m]
    _check(got[:m], ref, _sum_abs(a, sizes, wfn, N)[:m], f"w4a8 K={K} N={N}")


def test_w4a8_exact_values(geg):
    # activations in {0, +-0.5, +-1} (exact in e4m3 at the block's scale), weights
    # in {0, +-0.5, +-1} at scale 2^0: every product and sum is a multiple of 2^-2,
    # the sums stay below 64 (so they are exact in bf16, 8 significant bits) and
    # in any accumulator the instruction may use: the result must equal the
    # oracle bit for bit
    rng = np.random.default_rng(7)
    E, K, N = 3, 128, 128
    sizes = [40, 0, 90]
    M = sum(sizes)
    a = rng.choice([0.0, 0.5, -0.5, 1.0, -1.0], (M, K)).astype(np.float32)
    a[:, ::32] = 1.0                               # every block's amax is 1
    a_bits = synthetic.f32_to_bf16_bits(a)
    nib = rng.choice([0, 1, 2, 8, 9, 10], (E, N, K))
    codes = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    sc = np.full((E, N, K // 32), 127, np.uint8)
    log("case: w4a8 exact values")
    out = geg.gmxfp4_w4a8_grouped_gemm(up_u16_as_bf16(a_bits), up(np.array(sizes, np.int32)), up(codes), up(sc))
    ref = W.w4a8_grouped_ref(a_bits, sizes, lambda e: oracle.dequant_mxfp4(codes[e], sc[e]), N)
    assert np.abs(ref).max() < 64 and np.all(ref * 4 == np.round(ref * 4))
    assert np.array_equal(bf16_to_f64(out), ref)


def test_w4a8_full_size_sampled(geg):
    c = synthetic.case("gptoss_gate_up_t2048")
    seed = 0
    log(f"case: w4a8 full size {c.name} (M={c.M} N={c.N} K={c.K} E={c.E})")
    from gpu_util import gpu_weights_mxfp4
    a_bits, sizes = synthetic.rows_bf16(c, seed)
    w, s = gpu_weights_mxfp4(c, seed, experts=np.nonzero(sizes)[0])
    out = geg.gmxfp4_w4a8_grouped_gemm(up_u16_as_bf16(a_bits), up(sizes), w, s)
    rows, cols = sample_positions(sizes, c.N, 1500, seed=1)
    got = bf16_to_f64(out)[rows, cols]
    rows_fn = C.mxfp4_rows_fn(c, seed)
    ref = W.sampled_w4a8_ref(a_bits, sizes, lambda e, n: rows_fn(e, n), rows, cols)
    # S for the sampled positions
    # S at the sampled positions: the same product with |a| (sign bit cleared, which
    # quantises to |codes| with the same scales) and |w|
    S = W.sampled_w4a8_ref(np.asarray(a_bits) & np.uint16(0x7FFF), sizes, lambda e, n: np.abs(rows_fn(e, n)), rows, cols)
    _check(got, ref, S, "w4a8 gpt-oss gate_up T=2048 (sampled)")


def test_w4a8_flags_non_finite(geg):
    import torch
    rng = np.random.default_rng(9)
    a = rng.standard_normal((8, 64)).astype(np.float32)
    a[3, 40] = np.inf
    codes = rng.integers(0, 256, (1, 16, 32), dtype=np.uint8)
    sc = np.full((1, 16, 2), 127, np.uint8)
    ws = geg.Workspace(geg.geg_workspace_bytes(geg.GEG_OP_MXFP4_W4A8, 8, 16, 64, 1))
    log("case: w4a8 non-finite flag")
    geg.gmxfp4_w4a8_grouped_gemm(up_u16_as_bf16(synthetic.f32_to_bf16_bits(a)), up(np.array([8], np.int32)),
                                 up(codes), up(sc), workspace=ws)
    assert ws.read_error() & geg.DEVERR_NON_FINITE


def test_w4a8_empty_and_zero_rows(geg):
    import torch
    z = geg.gmxfp4_w4a8_grouped_gemm(torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda"),
                                     up(np.zeros(2, np.int32)), up(np.zeros((2, 16, 32), np.uint8)),
                                     up(np.zeros((2, 16, 2), np.uint8)))
    assert z.shape == (0, 16)
    out = torch.full((4, 16), 3.0, dtype=torch.bfloat16, device="cuda")
    geg.gmxfp4_w4a8_grouped_gemm(torch.ones((4, 64), dtype=torch.bfloat16, device="cuda"),
                                 up(np.zeros(2, np.int32)), up(np.zeros((2, 16, 32), np.uint8)),
                                 up(np.full((2, 16, 2), 127, np.uint8)), out=out)
    assert (bf16_to_f64(out) == 3.0).all()
