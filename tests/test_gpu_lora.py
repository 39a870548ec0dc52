"""GPU parity of the low-rank adapter delta (forward at the pre-activation point
and backward for the input and both adapter matrices) against oracle.lora, on
top of the grouped 4-bit projection and its dgrad. Tolerance: the path's
|gpu - ref| <= 1e-2 max(1, |ref|) on every output (bf16 activations, fp32
adapter gradients)."""
import numpy as np
import pytest

import oracle
import synthetic
from oracle import lora as L
from gpu_util import assert_close, bf16_to_f64, log, up, up_u16_as_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def geg():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_expert_gemm_amd as g
    g.lib()
    return g


def _case(fmt, E, K, N, r, sizes, seed):
    rng = np.random.default_rng(seed)
    M = int(sum(sizes))
    x = synthetic.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    dy = synthetic.f32_to_bf16_bits(rng.standard_normal((M, N)).astype(np.float32))
    A = (rng.standard_normal((E, r, K)) / np.sqrt(K)).astype(np.float32)
    B = (rng.standard_normal((E, N, r)) * 0.5).astype(np.float32)
    if fmt == "nf4":
        packs = [oracle.quantize_pack_nf4((rng.standard_normal((N, K)) * 0.02).astype(np.float32)) for _ in range(E)]
        W = lambda e: oracle.dequant_nf4(*packs[e])
    else:
        packs = [(rng.integers(0, 256, (N, K // 2), dtype=np.uint8), rng.integers(119, 124, (N, K // 32), dtype=np.uint8))
                 for _ in range(E)]
        W = lambda e: oracle.dequant_mxfp4(*packs[e])
    codes = np.stack([p[0] for p in packs])
    scales = np.stack([p[1] for p in packs])
    return x, dy, A, B, np.array(sizes, np.int32), W, codes, scales


@pytest.mark.parametrize("fmt,r,K,N,sizes", [
    ("nf4", 16, 256, 200, [0, 5, 40, 0, 130, 1]),     # ragged rows and columns, empty experts
    ("nf4", 8, 512, 96, [17, 3]),
    ("mxfp4", 64, 288, 136, [9, 0, 70]),               # rank 64: two 32-wide contraction steps
    ("mxfp4", 32, 128, 57, [4, 33]),                   # odd N (forward only)
])
def test_lora_forward_and_backward(geg, fmt, r, K, N, sizes):
    import torch
    log(f"case: lora {fmt} r={r} K={K} N={N} sizes={sizes}")
    x, dy, A, B, sz, W, codes, scales = _case(fmt, len(sizes), K, N, r, sizes, seed=K + N + r)
    s = 0.5
    fwd = geg.gnf4_grouped_gemm_lora if fmt == "nf4" else geg.gmxfp4_grouped_gemm_lora
    xt, szt, At, Bt = up_u16_as_bf16(x), up(sz), up(A), up(B)
    wt, st = up(codes), up(scales)
    out, u = fwd(xt, szt, wt, st, At, Bt, s)
    assert_close(bf16_to_f64(out), L.lora_forward_ref(x, sz, W, A, B, s, N), f"lora forward {fmt} r={r}")
    _, u_ref = L.lora_delta_ref(x, sz, A, B, s)
    assert_close(u.cpu().numpy().astype(np.float64), u_ref, f"lora u {fmt} r={r}")
    if N % 8:
        return
    bwd = geg.gnf4_grouped_dgrad_lora if fmt == "nf4" else geg.gmxfp4_grouped_dgrad_lora
    dx, ga, gb = bwd(up_u16_as_bf16(dy), szt, wt, st, xt, At, Bt, u, s)
    dx_ref, dA_ref, dB_ref = L.lora_backward_ref(x, dy, sz, W, A, B, s, K)
    assert_close(bf16_to_f64(dx), dx_ref, f"lora dx {fmt} r={r}")
    assert_close(ga.cpu().numpy().astype(np.float64), dA_ref, f"lora dA {fmt} r={r}")
    assert_close(gb.cpu().numpy().astype(np.float64), dB_ref, f"lora dB {fmt} r={r}")


@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
def test_lora_backward_small_gradients(geg, fmt):
    # dY ~ N(0, 1e-7), the scale of activation gradients in training: dx, dA and
    # dB keep their relative precision (checked against max|err| / max|ref|, not
    # the absolute floor of max(1, |ref|)); the NF4 dgrad scales each dY row by a
    # power of two before its fp16 conversion
    log(f"case: lora backward {fmt} with dY ~ N(0, 1e-7)")
    x, dy, A, B, sz, W, codes, scales = _case(fmt, 4, 320 if fmt == "nf4" else 288, 136, 16, [5, 0, 90, 30],
                                               seed=23)
    K = x.shape[1]
    dy = synthetic.f32_to_bf16_bits(synthetic.bf16_bits_to_f32(dy) * np.float32(1e-7))
    s = 0.5
    fwd = geg.gnf4_grouped_gemm_lora if fmt == "nf4" else geg.gmxfp4_grouped_gemm_lora
    bwd = geg.gnf4_grouped_dgrad_lora if fmt == "nf4" else geg.gmxfp4_grouped_dgrad_lora
    xt, szt, At, Bt, wt, st = up_u16_as_bf16(x), up(sz), up(A), up(B), up(codes), up(scales)
    _, u = fwd(xt, szt, wt, st, At, Bt, s)
    dx, ga, gb = bwd(up_u16_as_bf16(dy), szt, wt, st, xt, At, Bt, u, s, check_errors=True)
    dx_ref, dA_ref, dB_ref = L.lora_backward_ref(x, dy, sz, W, A, B, s, K)
    for got, ref, what in ((bf16_to_f64(dx), dx_ref, "dx"), (ga.cpu().numpy().astype(np.float64), dA_ref, "dA"),
                           (gb.cpu().numpy().astype(np.float64), dB_ref, "dB")):
        rel = float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
        log(f"  {what}: max|err|/max|ref| = {rel:.2e}")
        assert rel <= 1e-2, what


def test_lora_autograd_op(geg):
    import torch
    log("case: lora autograd op")
    x, dy, A, B, sz, W, codes, scales = _case("nf4", 4, 320, 136, 16, [5, 0, 90, 30], seed=21)
    s = 2.0
    a = up_u16_as_bf16(x).requires_grad_(True)
    At = up(A).requires_grad_(True)
    Bt = up(B).requires_grad_(True)
    out = geg.grouped_linear_lora(a, up(sz), up(codes), up(scales), At, Bt, s, "nf4")
    out.backward(up_u16_as_bf16(dy))
    assert_close(bf16_to_f64(out), L.lora_forward_ref(x, sz, W, A, B, s, 136), "autograd lora forward")
    dx_ref, dA_ref, dB_ref = L.lora_backward_ref(x, dy, sz, W, A, B, s, 320)
    assert_close(bf16_to_f64(a.grad), dx_ref, "autograd lora dx")
    assert_close(At.grad.cpu().numpy().astype(np.float64), dA_ref, "autograd lora dA")
    assert_close(Bt.grad.cpu().numpy().astype(np.float64), dB_ref, "autograd lora dB")


def test_lora_empty_batch_gives_zero_gradients(geg):
    import torch
    log("case: lora M=0")
    E, K, N, r = 3, 64, 32, 8
    x = torch.zeros((0, K), dtype=torch.bfloat16, device="cuda")
    dy = torch.zeros((0, N), dtype=torch.bfloat16, device="cuda")
    u = torch.zeros((0, r), dtype=torch.float32, device="cuda")
    A = torch.ones((E, r, K), dtype=torch.float32, device="cuda")
    B = torch.ones((E, N, r), dtype=torch.float32, device="cuda")
    w = torch.zeros((E, N, K // 2), dtype=torch.uint8, device="cuda")
    am = torch.ones((E, N, K // 64), dtype=torch.float32, device="cuda")
    ga = torch.full((E, r, K), 5.0, device="cuda")
    gb = torch.full((E, N, r), 5.0, device="cuda")
    geg.gnf4_grouped_dgrad_lora(dy, up(np.zeros(E, np.int32)), w, am, x, A, B, u, 1.0, grad_a=ga, grad_b=gb)
    assert not ga.any() and not gb.any()


@pytest.mark.timeout(900)
def test_lora_full_size_sampled(geg):
    """OLMoE gate_up NF4 at T=2048 (16384 routed rows, E=64, K=N=2048) with a
    rank-16 adapter, through the same entry points the adapter bench times: the
    projection on sampled outputs (the oracle computes them one by one), the
    adapter parts (u, dA, dB and the adapter's share of dx) on every element."""
    from oracle import cases as C
    from gpu_util import gpu_weights_nf4, sample_positions
    c = synthetic.case("olmoe_gate_up_t2048")
    seed, r, s = 0, 16, 2.0
    log(f"case: lora full size {c.name} (M={c.M} N={c.N} K={c.K} E={c.E}) r={r}")
    a_bits, sizes = synthetic.rows_bf16(c, seed)
    w, sc = gpu_weights_nf4(c, seed, experts=np.nonzero(sizes)[0])
    rng = np.random.default_rng([seed, 9])
    A = (rng.standard_normal((c.E, r, c.K)) / np.sqrt(c.K)).astype(np.float32)
    B = (rng.standard_normal((c.E, c.N, r)) * 0.5).astype(np.float32)
    dy = synthetic.f32_to_bf16_bits(rng.standard_normal((c.M, c.N)).astype(np.float32))
    xt, szt, At, Bt = up_u16_as_bf16(a_bits), up(sizes), up(A), up(B)
    out, u = geg.gnf4_grouped_gemm_lora(xt, szt, w, sc, At, Bt, s)
    dx, ga, gb = geg.gnf4_grouped_dgrad_lora(up_u16_as_bf16(dy), szt, w, sc, xt, At, Bt, u, s)
    # forward: frozen projection on samples + the adapter delta
    delta, u_ref = L.lora_delta_ref(a_bits, sizes, A, B, s)
    rows, cols = sample_positions(sizes, c.N, 1500, seed=1)
    ref = oracle.sampled_fwd_ref(a_bits, sizes, C.nf4_rows_fn(c, seed), rows, cols) + delta[rows, cols]
    assert_close(bf16_to_f64(out)[rows, cols], ref, "lora full forward (sampled)")
    assert_close(u.cpu().numpy().astype(np.float64), u_ref, "lora full u")
    # backward: the adapter parts in full (frozen weight set to zero), the frozen
    # dgrad on samples inside a few 64-wide column blocks (plus the last one)
    zero_w = lambda e: np.zeros((c.N, c.K))
    dx_ad, dA_ref, dB_ref = L.lora_backward_ref(a_bits, dy, sizes, zero_w, A, B, s, c.K)
    assert_close(ga.cpu().numpy().astype(np.float64), dA_ref, "lora full dA")
    assert_close(gb.cpu().numpy().astype(np.float64), dB_ref, "lora full dB")
    rows, cols = sample_positions(sizes, c.K, 600, seed=2)
    blocks = np.append(np.random.default_rng(3).choice(c.K // 64 - 1, 3, replace=False), c.K // 64 - 1)
    cols = blocks[cols % 4] * 64 + cols % 64
    ref = oracle.sampled_dgrad_ref(dy, sizes, C.nf4_cols_fn(c, seed), rows, cols) + dx_ad[rows, cols]
    assert_close(bf16_to_f64(dx)[rows, cols], ref, "lora full dx (sampled)")
