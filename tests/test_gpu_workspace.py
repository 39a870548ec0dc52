"""One workspace shared by every entry point that writes scratch (W4A8 codes,
routing chunk counts, the fused block's intermediate, the adapter backward's
transposed weights), then a split-K decode GEMM on the same workspace: whatever
the earlier calls left there, its output matches the oracle (every call writes
its scratch before reading it)."""
import numpy as np
import pytest

import oracle
import synthetic
from gpu_util import assert_close, bf16_to_f64, log, up, up_u16_as_bf16

pytestmark = pytest.mark.gpu


def test_shared_workspace_then_split_k(geg_mod):
    geg = geg_mod
    import torch
    rng = np.random.default_rng(31)
    ws = geg.Workspace(64 << 20)
    # W4A8 (codes right after the header), routing sort, adapter backward
    E, K, N, M = 4, 256, 128, 64
    sizes = np.array([20, 0, 30, 14], np.int32)
    a = up_u16_as_bf16(synthetic.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32)))
    blocks = up(rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8))
    sc = up(rng.integers(119, 124, (E, N, K // 32), dtype=np.uint8))
    geg.gmxfp4_w4a8_grouped_gemm(a, up(sizes), blocks, sc, workspace=ws)
    ids = up(rng.integers(0, E, (M // 4, 4)).astype(np.int32))
    geg.route_sort(ids, E, workspace=ws)
    r = 8
    A = up((rng.standard_normal((E, r, K)) * 0.1).astype(np.float32))
    B = up((rng.standard_normal((E, N, r)) * 0.1).astype(np.float32))
    out, u = geg.gmxfp4_grouped_gemm_lora(a, up(sizes), blocks, sc, A, B, 1.0, workspace=ws)
    dy = up_u16_as_bf16(synthetic.f32_to_bf16_bits(rng.standard_normal((M, N)).astype(np.float32)))
    geg.gmxfp4_grouped_dgrad_lora(dy, up(sizes), blocks, sc, a, A, B, u, 1.0, workspace=ws)
    torch.cuda.synchronize()
    # then a split-K decode GEMM on the same workspace
    c = synthetic.case("olmoe_gate_up_t1")
    log("case: shared workspace, then skinny split-K on olmoe_gate_up_t1")
    d = oracle.cases.build(c, 0)
    o = geg.gnf4_grouped_gemm(up_u16_as_bf16(d["a_bits"]), up(d["sizes"].astype(np.int32)), up(d["codes"]),
                              up(d["scales"]), workspace=ws, opts=geg.Opts(1, 2))
    ref = oracle.grouped_ref(d["a_bits"], d["sizes"], oracle.cases.weight_fn(d), c.N)
    assert_close(bf16_to_f64(o), ref, "split-K after shared use")
    assert ws.read_error() == 0


@pytest.fixture(scope="module")
def geg_mod():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_expert_gemm_amd as g
    g.lib()
    return g
