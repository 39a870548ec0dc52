"""Pins of the W4A8 oracle (e4m3 activations with e8m0 block scales x MXFP4
weights): the e4m3 value table and rounding against torch's float8_e4m3fn (a
library routine that shares nothing with the oracle), the OCP scale rule on
worked examples, and the grouped product against an exhaustive-search brute force."""
import math

import numpy as np
import pytest

import oracle
import synthetic
from oracle import w4a8 as W


def test_e4m3_table_matches_torch_and_closed_form():
    torch = pytest.importorskip("torch")
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(t), np.isnan(W.E4M3_TABLE))
    assert np.array_equal(np.nan_to_num(t), np.nan_to_num(W.E4M3_TABLE))
    T = W.E4M3_TABLE
    assert T[0x7E] == 448.0 and T[0x38] == 1.0 and T[0x08] == 2.0 ** -6 and T[0x01] == 2.0 ** -9
    assert np.isnan(T[0x7F]) and np.isnan(T[0xFF])
    assert T[0x80] == 0.0 and math.copysign(1.0, T[0x80]) == -1.0
    assert np.all(np.diff(T[:0x7F]) > 0)                   # increasing over +0 .. 448
    assert np.array_equal(T[0x80:0xFF], -T[:0x7F])           # sign symmetry


def test_e4m3_round_matches_torch_including_ties():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    v = rng.standard_normal(50000) * 10.0 ** rng.uniform(-4.5, 2.6, 50000)
    v = np.concatenate([v, [0.0, -0.0, 448.0, -448.0, 2.0 ** -10, -2.0 ** -10, 3 * 2.0 ** -11]])
    got = W.e4m3_round(v)
    # torch turns magnitudes past 448 into NaN; the oracle saturates (tested below)
    ref = torch.from_numpy(np.clip(v, -448, 448)).float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)
    # every midpoint between neighbouring finite values goes to the even code
    vals = W.E4M3_TABLE[:0x7F]
    mids = (vals[:-1] + vals[1:]) / 2
    got = W.e4m3_round(mids)
    assert np.all(got % 2 == 0)
    assert np.array_equal(got, torch.from_numpy(mids).float().to(torch.float8_e4m3fn).view(torch.uint8).numpy())


def test_e4m3_round_saturates_above_448():
    got = W.e4m3_round(np.array([449.0, 463.9, 464.0, 480.0, 511.0, -500.0]))
    assert list(got) == [0x7E] * 5 + [0xFE]


def test_scale_rule_worked_examples():
    # amax 1: floor(log2 1) = 0, X = 0 - 8 + 127 = 119, step 2^-8, 1 -> 256 (0x78)
    # amax 3: X = 1 - 8 + 127 = 120, step 2^-7, 3 -> 384 = 1.5 * 2^8 (0x7C)
    # amax 1.9375: X = 119, 1.9375 * 256 = 496 -> saturates to 448 (0x7E)
    # all-zero block: X = 0, codes 0
    K = 32
    rows = np.zeros((4, K), dtype=np.float32)
    rows[0, 5] = 1.0
    rows[1, 7] = -3.0
    rows[2, 0] = 1.9375
    rows[2, 1] = 0.5
    a_bits = synthetic.f32_to_bf16_bits(rows)
    codes, X = W.quantize_mxfp8(a_bits)
    assert list(X[:, 0]) == [119, 120, 119, 0]
    assert codes[0, 5] == 0x78 and codes[1, 7] == 0xFC and codes[2, 0] == 0x7E
    assert codes[2, 1] == 0x70          # 0.5 * 256 = 128 = 2^7: e field 14, m 0
    assert not codes[3].any()


def test_scale_rule_puts_block_max_in_range():
    rng = np.random.default_rng(1)
    a = (rng.standard_normal((64, 256)) * 10.0 ** rng.uniform(-3, 3, (64, 1))).astype(np.float32)
    a_bits = synthetic.f32_to_bf16_bits(a)
    codes, X = W.quantize_mxfp8(a_bits)
    af = synthetic.bf16_bits_to_f32(a_bits).astype(np.float64)
    blk = np.abs(af.reshape(64, 8, 32)).max(-1) / np.ldexp(1.0, X.astype(np.int64) - 127)
    assert np.all((blk >= 256) & (blk < 512))
    # dequantised activations are within half an e4m3 step (or the 448 clamp) of the input
    d = W.dequant_mxfp8(codes, X)
    step = np.repeat(np.ldexp(1.0, X.astype(np.int64) - 127), 32, -1)
    v = af / step
    err = np.abs(d / step - np.clip(v, -448, 448))
    spacing = np.where(np.abs(v) >= 2.0 ** -6, np.ldexp(1.0, np.frexp(np.abs(v))[1] - 4), 2.0 ** -9)
    assert np.all(err <= spacing / 2)


def test_w4a8_grouped_matches_brute_force():
    rng = np.random.default_rng(2)
    E, K, N = 3, 64, 8
    sizes = [2, 0, 3]
    M = sum(sizes)
    a_bits = synthetic.f32_to_bf16_bits((rng.standard_normal((M, K)) * np.array([1.0, 0.01, 30.0, 1e-3, 5.0])[:, None]).astype(np.float32))
    packs = [(rng.integers(0, 256, (N, K // 2), dtype=np.uint8), rng.integers(118, 130, (N, K // 32), dtype=np.uint8))
             for _ in range(E)]
    wf = lambda e: oracle.dequant_mxfp4(*packs[e])
    got = W.w4a8_grouped_ref(a_bits, sizes, wf, N)
    ref = np.array(W.brute_force_w4a8(a_bits, sizes, wf))
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-300)
    rows = np.array([0, 1, 2, 4, 3])
    cols = np.array([0, 7, 3, 5, 1])
    samp = W.sampled_w4a8_ref(a_bits, sizes, lambda e, n: wf(e)[n], rows, cols)
    np.testing.assert_allclose(samp, ref[rows, cols], rtol=1e-13)


def test_w4a8_is_close_to_the_bf16_product():
    # the quantisation error only: relative Frobenius error of a few percent
    rng = np.random.default_rng(3)
    E, K, N = 2, 256, 32
    sizes = [20, 12]
    a_bits = synthetic.f32_to_bf16_bits(rng.standard_normal((32, K)).astype(np.float32))
    packs = [(rng.integers(0, 256, (N, K // 2), dtype=np.uint8), rng.integers(119, 130, (N, K // 32), dtype=np.uint8))
             for _ in range(E)]
    wf = lambda e: oracle.dequant_mxfp4(*packs[e])
    q = W.w4a8_grouped_ref(a_bits, sizes, wf, N)
    r = oracle.grouped_ref(a_bits, sizes, wf, N)
    rel = np.linalg.norm(q - r) / np.linalg.norm(r)
    assert 1e-3 < rel < 0.05


def test_quantize_refuses_non_finite():
    bits = synthetic.f32_to_bf16_bits(np.array([[np.inf] + [0.0] * 31], dtype=np.float32))
    with pytest.raises(ValueError):
        W.quantize_mxfp8(bits)
