"""Pins of the oracle's fused expert block (CPU only).

silu and the SwiGLU pairing are pinned by closed forms; the one-step bf16
rounding by the bit-pattern rounding on fp32 inputs and by cases where a detour
through fp32 would round twice; the whole block by a pure-Python brute force and
by cases with a known result (zero up rows, an exact integer case).
"""
import math

import numpy as np
import pytest

import oracle
import synthetic
from oracle import pack as P


def test_silu_closed_forms():
    x = np.array([0.0, math.log(3.0), -math.log(3.0), 40.0, -800.0])
    s = oracle.silu(x)
    assert s[0] == 0.0
    # sigmoid(ln 3) = 3/4, sigmoid(-ln 3) = 1/4
    assert abs(s[1] - 0.75 * math.log(3.0)) < 1e-15
    assert abs(s[2] + 0.25 * math.log(3.0)) < 1e-15
    assert abs(s[3] - 40.0) < 1e-15          # sigmoid(40) = 1 - 4e-18
    assert s[4] == 0.0 and math.copysign(1.0, s[4]) < 0


def test_silu_odd_part_identity():
    # x sigmoid(x) - (-x) sigmoid(-x) = x (sigmoid(x) + sigmoid(-x)) = x
    x = np.random.default_rng(0).standard_normal(1000) * 5
    np.testing.assert_allclose(oracle.silu(x) - oracle.silu(-x), x, rtol=1e-14, atol=1e-14)


def test_swiglu_pairs_are_interleaved():
    h = np.array([[1.0, 2.0, -3.0, 0.5, 0.0, 7.0]])
    act = oracle.swiglu_ref(h)
    sil = lambda v: v / (1 + math.exp(-v))
    np.testing.assert_allclose(act[0], [sil(1.0) * 2.0, sil(-3.0) * 0.5, 0.0], rtol=1e-15)
    with pytest.raises(ValueError):
        oracle.swiglu_ref(np.zeros((1, 3)))


def test_bf16_rounding_matches_bit_pattern_rounding_on_fp32_inputs():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 3.3e38)]
    want = P.bf16_rne_bits(f)
    got = oracle.bf16_rne_from_f64(f.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_bf16_rounding_is_one_step():
    # 1 + 2^-8 + 2^-40 lies just above the tie between 1 and 1 + 2^-7: one
    # rounding goes up; rounding to fp32 first lands on the tie and then goes
    # down to even (1.0)
    x = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert oracle.bf16_rne_from_f64(np.array([x]))[0] == 0x3F81
    assert P.bf16_rne_bits(np.array([x], np.float32))[0] == 0x3F80
    # exact ties go to even
    assert oracle.bf16_rne_from_f64(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80
    assert oracle.bf16_rne_from_f64(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 0x3F82
    # subnormal spacing 2^-133, and signs
    assert oracle.bf16_rne_from_f64(np.array([2.0 ** -133]))[0] == 0x0001
    assert oracle.bf16_rne_from_f64(np.array([-3 * 2.0 ** -134]))[0] == 0x8002
    assert oracle.bf16_rne_from_f64(np.array([-0.0]))[0] == 0x8000


def _block_case(E=3, H=64, I=64, sizes=(2, 0, 3), seed=0):
    rng = np.random.default_rng(seed)
    M = int(sum(sizes))
    a = synthetic.f32_to_bf16_bits(rng.standard_normal((M, H)).astype(np.float32))
    p13 = [oracle.quantize_pack_nf4((rng.standard_normal((2 * I, H)) * 0.05).astype(np.float32)) for _ in range(E)]
    p2 = [oracle.quantize_pack_nf4((rng.standard_normal((H, I)) * 0.05).astype(np.float32)) for _ in range(E)]
    return (a, np.array(sizes, np.int32), (lambda e: oracle.dequant_nf4(*p13[e])),
            (lambda e: oracle.dequant_nf4(*p2[e])))


def test_block_matches_brute_force():
    a, sizes, w13, w2 = _block_case()
    act, out = oracle.expert_block_ref(a, sizes, w13, w2, 64, 64)
    bf = np.array(oracle.brute_force_block(a, sizes, w13, w2))
    assert out.shape == (5, 64) and act.shape == (5, 64)
    np.testing.assert_allclose(out, bf, rtol=1e-12, atol=1e-14)


def test_block_sampled_rows_match_whole_block():
    a, sizes, w13, w2 = _block_case(sizes=(3, 1, 4), seed=2)
    _, out = oracle.expert_block_ref(a, sizes, w13, w2, 64, 64)
    rows = np.array([0, 3, 7, 4])
    np.testing.assert_allclose(oracle.sampled_block_ref(a, sizes, rows, w13, w2), out[rows], rtol=1e-13, atol=1e-15)


def test_block_zero_up_rows_give_zero():
    # NF4 code 7 is exactly 0.0: with every up row zero, act and out are zero
    E, H, I = 2, 64, 64
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 16, (E, 2 * I, H)).astype(np.uint8)
    codes[:, 1::2, :] = 7
    absmax = np.full((E, 2 * I, 1), 0.5, np.float32)
    q = P.pack_nf4_codes(codes)
    c2 = rng.integers(0, 16, (E, H, I)).astype(np.uint8)
    q2 = P.pack_nf4_codes(c2)
    a2 = np.full((E, H, 1), 0.25, np.float32)
    a = synthetic.f32_to_bf16_bits(rng.standard_normal((5, H)).astype(np.float32))
    act, out = oracle.expert_block_ref(a, [2, 3], lambda e: oracle.dequant_nf4(q[e], absmax[e]),
                                       lambda e: oracle.dequant_nf4(q2[e], a2[e]), H, I)
    assert not act.any() or not (act & 0x7FFF).any()
    assert not out.any()


def test_block_exact_integer_case():
    # gate = up = +-1 weights on integer activations: h is an integer, silu(h) h
    # is known per row; down weights of +-1 and 0 keep the second sum exact in
    # fp64 after the bf16 rounding of act
    E, H, I = 1, 64, 64
    rng = np.random.default_rng(5)
    codes = rng.choice(np.array([0, 7, 15], np.uint8), size=(E, 2 * I, H))
    absmax = np.ones((E, 2 * I, 1), np.float32)
    c2 = rng.choice(np.array([0, 7, 15], np.uint8), size=(E, H, I))
    a2 = np.ones((E, H, 1), np.float32)
    q, q2 = P.pack_nf4_codes(codes), P.pack_nf4_codes(c2)
    ai = rng.integers(-2, 3, (4, H))
    a = synthetic.f32_to_bf16_bits(ai.astype(np.float32))
    act, out = oracle.expert_block_ref(a, [4], lambda e: oracle.dequant_nf4(q[e], absmax[e]),
                                       lambda e: oracle.dequant_nf4(q2[e], a2[e]), H, I)
    sign = {0: -1.0, 7: 0.0, 15: 1.0}
    for r in range(4):
        h = [sum(sign[int(codes[0, n, k])] * ai[r, k] for k in range(H)) for n in range(2 * I)]
        act_r = []
        for i in range(I):
            g, u = h[2 * i], h[2 * i + 1]
            v = g / (1 + math.exp(-g)) * u
            bits = oracle.bf16_rne_from_f64(np.array([v])).astype(np.uint32) << 16
            act_r.append(float(bits.view(np.float32)[0]))
        for j in range(H):
            want = math.fsum(act_r[i] * sign[int(c2[0, j, i])] for i in range(I))
            assert out[r, j] == want
