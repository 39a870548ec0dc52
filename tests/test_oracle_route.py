"""Pins of the oracle's routing sort and top-k combine (CPU only)."""
import numpy as np

import oracle
import synthetic


def test_route_sort_matches_brute_force_and_invariants():
    rng = np.random.default_rng(0)
    for T, k, E in [(1, 8, 64), (7, 2, 5), (64, 4, 16), (33, 1, 3)]:
        ids = rng.integers(0, E, (T, k))
        sizes, row_of, src_of = oracle.route_sort_ref(ids, E)
        bs, br, bsrc = oracle.brute_force_route(ids, E)
        assert list(sizes) == bs and list(row_of) == br and list(src_of) == bsrc
        assert sizes.sum() == T * k
        assert (src_of[row_of] == np.arange(T * k)).all()            # inverse permutations
        flat = ids.reshape(-1)
        key = flat[src_of] * (T * k) + src_of                         # (expert, flat index)
        assert (np.diff(key) > 0).all()                                # sorted and stable


def test_route_sort_drops_invalid_ids():
    ids = np.array([[0, 5], [-1, 2], [2, 0]])
    sizes, row_of, src_of = oracle.route_sort_ref(ids, 3)
    assert list(sizes) == [2, 0, 2]
    assert list(row_of) == [0, -1, -1, 2, 3, 1]
    assert list(src_of) == [0, 5, 3, 4, -1, -1]


def test_route_order_is_the_loop_order():
    # loop_ref gathers each expert's rows in stable order of flat index: the
    # grouped GEMM on the sorted rows reproduces it row for row
    rng = np.random.default_rng(1)
    T, k, E, K, N = 9, 3, 4, 64, 16
    ids = rng.integers(0, E, (T, k))
    x = synthetic.f32_to_bf16_bits(rng.standard_normal((T, K)).astype(np.float32))
    packs = [oracle.quantize_pack_nf4((rng.standard_normal((N, K)) * 0.05).astype(np.float32)) for _ in range(E)]
    W = lambda e: oracle.dequant_nf4(*packs[e])
    sizes, row_of, src_of = oracle.route_sort_ref(ids, E)
    xs = oracle.gather_ref(x, src_of, k)
    y = oracle.grouped_ref(xs, sizes, W, N)
    lr, cnt = oracle.loop_ref(x, ids, W, N)      # the loop's outputs in its own row order
    np.testing.assert_array_equal(lr, y)
    assert list(cnt) == list(sizes[:len(cnt)])


def test_combine_closed_forms():
    rng = np.random.default_rng(2)
    T, k, N = 5, 3, 8
    y = rng.standard_normal((T * k, N))
    row_of = rng.permutation(T * k).astype(np.int32)
    # one-hot weights give the routed row exactly
    w = np.zeros((T, k)); w[:, 1] = 1.0
    np.testing.assert_array_equal(oracle.combine_ref(y, row_of, w, T, k), y[row_of.reshape(T, k)[:, 1]])
    # linear in the weights
    w1, w2 = rng.random((T, k)), rng.random((T, k))
    lhs = oracle.combine_ref(y, row_of, w1 + 2 * w2, T, k)
    rhs = oracle.combine_ref(y, row_of, w1, T, k) + 2 * oracle.combine_ref(y, row_of, w2, T, k)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-13, atol=1e-13)
    # a dropped slot contributes nothing
    r2 = row_of.copy(); r2[4] = -1
    got = oracle.combine_ref(y, r2, None, T, k)
    want = oracle.combine_ref(y, row_of, None, T, k)
    want[1] -= y[row_of[4]]
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)
