"""Pins of the low-rank adapter oracle: the backward formulas against torch's
autograd in fp64 on the CPU (derivatives computed independently of the
hand-derived formulas), pure-Python brute force, and the reductions that must
hold (s = 0 gives the frozen projection; the adapter part is linear in s)."""
import numpy as np
import pytest

import oracle
import synthetic
from oracle import lora as L


def _case(seed, E=3, K=64, N=48, r=8, sizes=(5, 0, 7)):
    rng = np.random.default_rng(seed)
    M = sum(sizes)
    x = synthetic.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    dy = synthetic.f32_to_bf16_bits(rng.standard_normal((M, N)).astype(np.float32))
    A = synthetic.f32_to_bf16_bits((rng.standard_normal((E, r, K)) * 0.1).astype(np.float32))
    B = synthetic.f32_to_bf16_bits((rng.standard_normal((E, N, r)) * 0.1).astype(np.float32))
    packs = [oracle.quantize_pack_nf4((rng.standard_normal((N, K)) * 0.05).astype(np.float32)) for _ in range(E)]
    W = lambda e: oracle.dequant_nf4(*packs[e])
    return x, dy, A, B, list(sizes), W


def test_backward_matches_torch_autograd():
    torch = pytest.importorskip("torch")
    x, dy, A, B, sizes, W = _case(0)
    s = 0.75
    K, N = x.shape[1], dy.shape[1]
    dx, dA, dB = L.lora_backward_ref(x, dy, sizes, W, A, B, s, K)
    off = oracle.offsets(sizes)
    xt = torch.tensor(L._f64(x), requires_grad=True)
    At = torch.tensor(L._f64(A), requires_grad=True)
    Bt = torch.tensor(L._f64(B), requires_grad=True)
    outs = []
    for e in range(len(sizes)):
        lo, hi = int(off[e]), int(off[e + 1])
        We = torch.tensor(W(e))
        xe = xt[lo:hi]
        outs.append(xe @ We.T + s * (xe @ At[e].T) @ Bt[e].T)
    y = torch.cat(outs)
    y.backward(torch.tensor(L._f64(dy)))
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dA, At.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dB, Bt.grad.numpy(), rtol=1e-12, atol=1e-12)
    y_ref = L.lora_forward_ref(x, sizes, W, A, B, s, N)
    np.testing.assert_allclose(y_ref, y.detach().numpy(), rtol=1e-12, atol=1e-12)


def test_matches_brute_force():
    x, dy, A, B, sizes, W = _case(1, E=2, K=64, N=6, r=3, sizes=(2, 3))
    s = 1.5
    delta, u = L.lora_delta_ref(x, sizes, A, B, s)
    dx, dA, dB = L.lora_backward_ref(x, dy, sizes, W, A, B, s, 64)
    dxf = dx - oracle.dgrad_ref(dy, sizes, W, 64)
    bd, bdx, bdA, bdB = L.brute_force_lora(x, dy, sizes, A, B, s)
    np.testing.assert_allclose(delta, np.array(bd), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dxf, np.array(bdx), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dA, np.array(bdA), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dB, np.array(bdB), rtol=1e-12, atol=1e-14)


def test_scale_zero_and_linearity():
    x, dy, A, B, sizes, W = _case(2)
    N, K = dy.shape[1], x.shape[1]
    y0 = L.lora_forward_ref(x, sizes, W, A, B, 0.0, N)
    np.testing.assert_array_equal(y0, oracle.grouped_ref(x, sizes, W, N))
    d1, _ = L.lora_delta_ref(x, sizes, A, B, 1.0)
    d3, _ = L.lora_delta_ref(x, sizes, A, B, 3.0)
    np.testing.assert_allclose(d3, 3.0 * d1, rtol=1e-13, atol=1e-15)
    # an expert with no rows gets zero adapter gradients
    _, dA, dB = L.lora_backward_ref(x, dy, sizes, W, A, B, 2.0, K)
    assert not dA[1].any() and not dB[1].any()
