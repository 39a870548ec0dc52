"""Pins of the oracle's grouped GEMM and input gradient (CPU only).

The grouped result is pinned by a pure-Python brute force (exactly rounded
sums), by exact integer cases whose result is known in closed form, by the
per-expert loop as the model runs it from unsorted tokens, and by the block
locality of the scales; the input gradient by brute force and by the adjoint
identity <dY, A W^T> = <dY W, A>.
"""
import numpy as np
import pytest

import oracle
import synthetic
from oracle import cases as C
from oracle import pack as P


def _small_nf4(E=3, N=16, K=128, sizes=(0, 5, 3), seed=0):
    rng = np.random.default_rng(seed)
    M = int(sum(sizes))
    a = synthetic.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    packs = [oracle.quantize_pack_nf4((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
             for _ in range(E)]
    return a, np.array(sizes, np.int32), (lambda e: oracle.dequant_nf4(*packs[e])), packs


def test_grouped_matches_brute_force():
    a, sizes, W, _ = _small_nf4()
    ref = oracle.grouped_ref(a, sizes, W, 16)
    bf = np.array(oracle.brute_force_ref(a, sizes, W))
    assert ref.shape == (8, 16)
    np.testing.assert_allclose(ref, bf, rtol=1e-13, atol=1e-15)


def test_grouped_is_a_times_w_transposed_nonsquare():
    # out[m, n] = sum_k a[m, k] W[n, k]; with N != K a transposed operand cannot fit
    a, sizes, W, _ = _small_nf4(E=2, N=24, K=64, sizes=(3, 4))
    ref = oracle.grouped_ref(a, sizes, W, 24)
    af = synthetic.bf16_bits_to_f32(a).astype(np.float64)
    m, n = 5, 17
    want = sum(af[m, k] * W(1)[n, k] for k in range(64))
    assert abs(ref[m, n] - want) < 1e-12


def test_grouped_exact_integer_case():
    # NF4 codes in {0, 7, 15} are exactly -1, 0, +1; absmax powers of two and
    # integer activations make every product and partial sum exact.
    E, N, K = 3, 16, 64
    sizes = np.array([0, 5, 3], np.int32)
    rng = np.random.default_rng(3)
    codes = rng.choice(np.array([0, 7, 15], np.uint8), size=(E, N, K))
    absmax = (2.0 ** rng.integers(-2, 3, (E, N, 1))).astype(np.float32)
    ai = rng.integers(-2, 3, (8, K))
    a = synthetic.f32_to_bf16_bits(ai.astype(np.float32))
    q = P.pack_nf4_codes(codes)
    ref = oracle.grouped_ref(a, sizes, lambda e: oracle.dequant_nf4(q[e], absmax[e]), N)
    sign = {0: -1, 7: 0, 15: 1}
    off = [0, 0, 5, 8]
    for e in range(E):
        for r in range(off[e], off[e + 1]):
            for n in range(N):
                want = sum(int(ai[r, k]) * sign[int(codes[e, n, k])] for k in range(K)) * float(absmax[e, n, 0])
                assert ref[r, n] == want
    # and the result is exactly representable in bf16
    assert np.array_equal(synthetic.bf16_bits_to_f32(P.bf16_rne_bits(ref.astype(np.float32))), ref.astype(np.float32))


def test_grouped_exact_mxfp4_case():
    # any e2m1 code at scale byte 127 (x1) times integer activations is exact
    E, N, K = 2, 16, 64
    rng = np.random.default_rng(4)
    blocks = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    scales = np.full((E, N, K // 32), 127, np.uint8)
    sizes = np.array([2, 3], np.int32)
    ai = rng.integers(-2, 3, (5, K))
    a = synthetic.f32_to_bf16_bits(ai.astype(np.float32))
    ref = oracle.grouped_ref(a, sizes, lambda e: oracle.dequant_mxfp4(blocks[e], scales[e]), N)
    codes = P.unpack_mxfp4_codes(blocks)
    mags = {0: 0, 1: 0.5, 2: 1, 3: 1.5, 4: 2, 5: 3, 6: 4, 7: 6}
    val = lambda c: (-1 if c & 8 else 1) * mags[c & 7]
    for r, e in [(0, 0), (1, 0), (2, 1), (4, 1)]:
        for n in range(N):
            assert ref[r, n] == sum(int(ai[r, k]) * val(int(codes[e, n, k])) for k in range(K))


def test_scale_blocks_are_64_wide_and_row_local():
    a, sizes, _, packs = _small_nf4(E=1, N=4, K=256, sizes=(3,))
    q, s = packs[0]
    base = oracle.grouped_ref(a, sizes, lambda e: oracle.dequant_nf4(q, s), 4)
    s2 = s.copy()
    s2[2, 1] *= 2.0                                # row n=2, k in [64, 128)
    moved = oracle.grouped_ref(a, sizes, lambda e: oracle.dequant_nf4(q, s2), 4)
    assert np.array_equal(moved[:, [0, 1, 3]], base[:, [0, 1, 3]])
    W = oracle.dequant_nf4(q, s)
    af = synthetic.bf16_bits_to_f32(a).astype(np.float64)
    want = base[:, 2] + af[:, 64:128] @ W[2, 64:128]
    np.testing.assert_allclose(moved[:, 2], want, rtol=1e-12)


def test_mxfp4_scale_blocks_are_32_wide():
    blocks = np.zeros((1, 32), np.uint8) + 0x22      # every code = 2 (1.0)
    scales = np.array([[127, 128]], np.uint8)
    w = oracle.dequant_mxfp4(blocks, scales)
    assert np.all(w[0, :32] == 1.0) and np.all(w[0, 32:] == 2.0)


def test_grouped_equals_per_expert_loop_from_unsorted_tokens():
    c = synthetic.case("tiny")
    d = C.build(c, 0)
    W = C.weight_fn(d)
    ref = oracle.grouped_ref(d["a_bits"], d["sizes"], W, c.N)
    x = synthetic.activations_bf16(c, 0)
    loop, counts = oracle.loop_ref(x, synthetic.topk_ids(c, 0), W, c.N)
    assert np.array_equal(counts, d["sizes"])
    assert np.array_equal(loop, ref)               # bitwise: the same fp64 operations


def test_zero_row_experts_and_tail_rows():
    a, sizes, W, _ = _small_nf4(E=4, sizes=(0, 3, 0, 2))
    a_pad = np.concatenate([a, np.zeros((3, a.shape[1]), np.uint16)])
    ref = oracle.grouped_ref(a_pad, sizes, W, 16)
    assert np.all(ref[5:] == 0)
    with pytest.raises(ValueError):
        oracle.offsets([1, -1])


def test_dgrad_brute_force_and_adjoint_identity():
    a, sizes, W, _ = _small_nf4(E=3, N=32, K=64, sizes=(4, 0, 6))
    rng = np.random.default_rng(5)
    dy = synthetic.f32_to_bf16_bits(rng.standard_normal((10, 32)).astype(np.float32))
    dx = oracle.dgrad_ref(dy, sizes, W, 64)
    bf = np.array(oracle.brute_force_dgrad(dy, sizes, W))
    np.testing.assert_allclose(dx, bf, rtol=1e-13, atol=1e-15)
    y = oracle.grouped_ref(a, sizes, W, 32)
    dyf = synthetic.bf16_bits_to_f32(dy).astype(np.float64)
    af = synthetic.bf16_bits_to_f32(a).astype(np.float64)
    lhs = float(np.sum(dyf * y))
    rhs = float(np.sum(dx * af))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


def test_sampled_refs_match_full_refs():
    c = synthetic.Case("t", "nf4", 4, 128, 64, 16, 2)
    d = C.build(c, 1)
    W = C.weight_fn(d)
    full = oracle.grouped_ref(d["a_bits"], d["sizes"], W, c.N)
    rng = np.random.default_rng(0)
    rows = rng.integers(0, c.M, 50)
    cols = rng.integers(0, c.N, 50)
    got = oracle.sampled_fwd_ref(d["a_bits"], d["sizes"], C.nf4_rows_fn(c, 1), rows, cols)
    np.testing.assert_allclose(got, full[rows, cols], rtol=1e-12, atol=1e-14)
    dy = synthetic.dgrad_dy_bf16(c, 1)
    fulld = oracle.dgrad_ref(dy, d["sizes"], W, c.K)
    kcols = rng.integers(0, c.K, 50)
    gotd = oracle.sampled_dgrad_ref(dy, d["sizes"], C.nf4_cols_fn(c, 1), rows, kcols)
    np.testing.assert_allclose(gotd, fulld[rows, kcols], rtol=1e-12, atol=1e-14)


def test_sampled_mxfp4_refs_match_full_refs():
    # the MXFP4 row and column decoders used at full size against the whole-expert
    # decode (K of 288: nine 32-blocks, an odd count of them)
    c = synthetic.Case("t", "mxfp4", 3, 288, 96, 16, 2)
    d = C.build(c, 2)
    W = C.weight_fn(d)
    rng = np.random.default_rng(1)
    rows = rng.integers(0, c.M, 40)
    cols = rng.integers(0, c.N, 40)
    full = oracle.grouped_ref(d["a_bits"], d["sizes"], W, c.N)
    got = oracle.sampled_fwd_ref(d["a_bits"], d["sizes"], C.mxfp4_rows_fn(c, 2), rows, cols)
    np.testing.assert_allclose(got, full[rows, cols], rtol=1e-12, atol=1e-14)
    dy = synthetic.dgrad_dy_bf16(c, 2)
    fulld = oracle.dgrad_ref(dy, d["sizes"], W, c.K)
    kcols = np.append(rng.integers(0, c.K, 40), [0, 31, 32, c.K - 1])
    rows2 = np.append(rows, rows[:4])
    gotd = oracle.sampled_dgrad_ref(dy, d["sizes"], C.mxfp4_cols_fn(c, 2), rows2, kcols)
    np.testing.assert_allclose(gotd, fulld[rows2, kcols], rtol=1e-12, atol=1e-14)
