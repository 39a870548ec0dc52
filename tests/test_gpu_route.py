"""GPU parity of the routing sort, the row gather and the top-k combine against
the oracle (index work bit-exact, the combine within the bf16 tolerance), and of
a whole MoE layer (sort -> fused expert block -> combine)."""
import numpy as np
import pytest

import oracle
import synthetic
from gpu_util import assert_close, bf16_to_f64, bits16, log, up, up_u16_as_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def geg():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_expert_gemm_amd as g
    g.lib()
    return g


def _ids(rng, T, k, E, zipf=False):
    # distinct experts per token, as a router's top-k gives
    logits = rng.standard_normal((T, E))
    if zipf:
        logits -= 1.1 * np.log(rng.permutation(E) + 1)
    return np.argsort(-logits, axis=1, kind="stable")[:, :k].astype(np.int32)


@pytest.mark.parametrize("T,k,E,H", [(1, 8, 64, 256), (64, 8, 128, 512), (4096, 8, 128, 2048),
                                     (300, 2, 8, 128), (257, 1, 1024, 64), (1000, 4, 32, 2880)])
def test_route_sort_bit_exact(geg, T, k, E, H):
    import torch
    rng = np.random.default_rng(T + k + E)
    ids = _ids(rng, T, k, E, zipf=(E == 128))
    x = synthetic.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    log(f"case: route sort T={T} k={k} E={E} H={H}")
    sizes, row_of, src_of, xs = geg.route_sort(up(ids), E, x=up_u16_as_bf16(x))
    rs, rr, rsrc = oracle.route_sort_ref(ids, E)
    np.testing.assert_array_equal(sizes.cpu().numpy(), rs)
    np.testing.assert_array_equal(row_of.cpu().numpy(), rr)
    np.testing.assert_array_equal(src_of.cpu().numpy(), rsrc)
    np.testing.assert_array_equal(bits16(xs), oracle.gather_ref(x, rsrc, k))


def test_route_sort_flags_and_drops_invalid_ids(geg):
    import torch
    ids = np.array([[0, 5], [-1, 2], [2, 0]], np.int32)
    ws = geg.Workspace(1 << 20)
    sizes, row_of, src_of, _ = geg.route_sort(up(ids), 3, workspace=ws)
    assert list(sizes.cpu().numpy()) == [2, 0, 2]
    assert list(row_of.cpu().numpy()) == [0, -1, -1, 2, 3, 1]
    assert list(src_of.cpu().numpy()) == [0, 5, 3, 4, -1, -1]
    assert ws.read_error() & geg.DEVERR_BAD_EXPERT_ID


def test_route_sort_empty(geg):
    import torch
    ids = torch.zeros((0, 4), dtype=torch.int32, device="cuda")
    sizes, row_of, src_of, _ = geg.route_sort(ids, 16)
    assert sizes.shape == (16,) and not sizes.cpu().numpy().any()


@pytest.mark.parametrize("T,k,N,weighted", [(1, 8, 2048, True), (64, 8, 1536, True), (4096, 8, 2048, True),
                                            (300, 2, 128, False), (17, 4, 2880, True)])
def test_route_combine(geg, T, k, N, weighted):
    rng = np.random.default_rng(T * 7 + k)
    row_of = rng.permutation(T * k).astype(np.int32)
    row_of[rng.random(T * k) < 0.05] = -1
    y = synthetic.f32_to_bf16_bits(rng.standard_normal((T * k, N)).astype(np.float32))
    w = rng.random((T, k)).astype(np.float32) if weighted else None
    log(f"case: combine T={T} k={k} N={N} weighted={weighted}")
    out = geg.route_combine(up_u16_as_bf16(y), up(row_of), up(w) if w is not None else None, k)
    ref = oracle.combine_ref(synthetic.bf16_bits_to_f32(y), row_of, w, T, k)
    assert_close(bf16_to_f64(out), ref, f"combine T={T} k={k}")


@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
@pytest.mark.parametrize("T", [1, 64, 512])
def test_moe_layer(geg, fmt, T):
    # router top-k ids and weights -> sort + gather -> fused expert block ->
    # weighted combine, all on the device, against the oracle's composition
    E, k, H, I = 32, 4, 512, 256
    rng = np.random.default_rng(T)
    ids = _ids(rng, T, k, E)
    wts = rng.random((T, k)).astype(np.float32)
    x = synthetic.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    if fmt == "nf4":
        p13 = [oracle.quantize_pack_nf4((rng.standard_normal((2 * I, H)) * 0.02).astype(np.float32)) for _ in range(E)]
        p2 = [oracle.quantize_pack_nf4((rng.standard_normal((H, I)) * 0.02).astype(np.float32)) for _ in range(E)]
        dq = oracle.dequant_nf4
    else:
        # scales 2^-8..2^-6 keep the block's outputs of order one, like the NF4 case
        p13 = [(rng.integers(0, 256, (2 * I, H // 2), dtype=np.uint8), rng.integers(119, 122, (2 * I, H // 32), dtype=np.uint8)) for _ in range(E)]
        p2 = [(rng.integers(0, 256, (H, I // 2), dtype=np.uint8), rng.integers(119, 122, (H, I // 32), dtype=np.uint8)) for _ in range(E)]
        dq = oracle.dequant_mxfp4
    c13 = np.stack([p[0] for p in p13]); s13 = np.stack([p[1] for p in p13])
    c2 = np.stack([p[0] for p in p2]); s2 = np.stack([p[1] for p in p2])
    log(f"case: moe layer fmt={fmt} T={T}")
    sizes, row_of, src_of, xs = geg.route_sort(up(ids), E, x=up_u16_as_bf16(x))
    blk = geg.gnf4_expert_block if fmt == "nf4" else geg.gmxfp4_expert_block
    y = blk(xs, sizes, up(c13), up(s13), up(c2), up(s2))
    out = geg.route_combine(y, row_of, up(wts), k)
    rs, rr, rsrc = oracle.route_sort_ref(ids, E)
    xs_ref = oracle.gather_ref(x, rsrc, k)
    _, yref = oracle.expert_block_ref(xs_ref, rs, lambda e: dq(*p13[e]), lambda e: dq(*p2[e]), H, I)
    # the block hands its output over in bf16 (its API type); the combine sums those
    ybf = synthetic.bf16_bits_to_f32(oracle.bf16_rne_from_f64(yref)).astype(np.float64)
    ref = oracle.combine_ref(ybf, rr, wts, T, k)
    assert_close(bf16_to_f64(out), ref, f"moe layer {fmt} T={T}")
