"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (automatic path choice). The oracle computes sampled outputs one
dot product at a time: first and last row of every expert, the last column, and
uniform random positions. NF4 bytes are made on the GPU by the library's packer;
the sampled rows' bytes are checked bit for bit against the oracle's packer."""
import numpy as np
import pytest

import oracle
import synthetic
from oracle import cases as C
from gpu_util import (assert_close, bf16_to_f64, gpu_weights_mxfp4, gpu_weights_nf4, log, up,
                      up_u16_as_bf16, sample_positions)

pytestmark = pytest.mark.gpu

FWD = [n for n, c in synthetic.CASES.items() if c.op == "fwd" and n != "tiny"]
DGRAD = [n for n, c in synthetic.CASES.items() if c.op == "dgrad"]


@pytest.fixture(scope="module")
def geg():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_expert_gemm_amd as g
    g.lib()
    return g


def _inputs(c, seed):
    a_bits, sizes = synthetic.rows_bf16(c, seed)
    touched = np.nonzero(sizes)[0]
    if c.fmt == "nf4":
        w, s = gpu_weights_nf4(c, seed, experts=touched)
    else:
        w, s = gpu_weights_mxfp4(c, seed, experts=touched)
    return a_bits, sizes, w, s


def _check_packed_rows(c, seed, w, s, rows_by_expert):
    for e, n_idx in rows_by_expert.items():
        wf = synthetic.nf4_weight_f32(c, seed, e, rows=n_idx)
        q, sc = oracle.quantize_pack_nf4(wf)
        assert np.array_equal(w[e][n_idx].cpu().numpy(), q), e
        assert np.array_equal(s[e][n_idx].cpu().numpy().view(np.uint32), sc.view(np.uint32)), e


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", FWD)
def test_forward_full_size(geg, name):
    c = synthetic.case(name)
    seed = 0
    log(f"case: {name} (M={c.M} N={c.N} K={c.K} E={c.E} {c.fmt}) seed={seed}")
    a_bits, sizes, w, s = _inputs(c, seed)
    fn = geg.gnf4_grouped_gemm if c.fmt == "nf4" else geg.gmxfp4_grouped_gemm
    out = fn(up_u16_as_bf16(a_bits), up(sizes), w, s)
    rows, cols = sample_positions(sizes, c.N, 1500, seed=1)
    got = bf16_to_f64(out)[rows, cols]
    rows_fn = C.nf4_rows_fn(c, seed) if c.fmt == "nf4" else C.mxfp4_rows_fn(c, seed)
    ref = oracle.sampled_fwd_ref(a_bits, sizes, rows_fn, rows, cols)
    assert_close(got, ref, name)
    if c.fmt == "nf4":
        e0 = int(np.nonzero(sizes)[0][0])
        _check_packed_rows(c, seed, w, s, {e0: np.unique(cols)[:64]})


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", DGRAD)
def test_dgrad_full_size(geg, name):
    c = synthetic.case(name)
    seed = 0
    log(f"case: {name} dgrad (M={c.M} N={c.N} K={c.K} E={c.E}) seed={seed}")
    a_bits, sizes, w, s = _inputs(c, seed)
    dy = synthetic.dgrad_dy_bf16(c, seed)
    fn = geg.gnf4_grouped_dgrad if c.fmt == "nf4" else geg.gmxfp4_grouped_dgrad
    dx = fn(up_u16_as_bf16(dy), up(sizes), w, s)
    rows, cols = sample_positions(sizes, c.K, 600, seed=2)
    # keep the sampled columns inside a few 64-wide blocks (plus the last one) so
    # the oracle packs only those blocks of each expert
    rng = np.random.default_rng(3)
    blocks = np.append(rng.choice(c.K // 64 - 1, 3, replace=False), c.K // 64 - 1)
    cols = blocks[cols % 4] * 64 + cols % 64
    got = bf16_to_f64(dx)[rows, cols]
    cols_fn = C.nf4_cols_fn(c, seed) if c.fmt == "nf4" else C.mxfp4_cols_fn(c, seed)
    ref = oracle.sampled_dgrad_ref(dy, sizes, cols_fn, rows, cols)
    assert_close(got, ref, name + " dgrad")
