"""The entry point that allocates nothing (gnf4_grouped_gemm_noalloc), for callers
that cannot allocate device memory: called through the C ABI, its output must
equal gnf4_grouped_gemm's (the same kernels; with a workspace) bit for bit and the
oracle within 1e-2 max(1, |ref|), on two calls in a row, the second smaller, on
the tiled, narrow and vector paths; device errors reach the caller's word; a call
whose scratch exceeds the library-held array is refused before any launch."""
import ctypes

import numpy as np
import pytest

import oracle
from oracle import cases as C
from gpu_util import assert_close, bf16_to_f64, bits16, log, upload_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def geg():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_expert_gemm_amd as g
    g.lib()
    return g


def _case(E, K, N, sizes, seed):
    from test_gpu_parity import custom_case
    return custom_case("nf4", E, K, N, sizes, seed=seed)


def _noalloc(geg, g, c, out, err=None):
    import torch
    M = g["a"].shape[0]
    st = geg.lib().gnf4_grouped_gemm_noalloc(
        ctypes.c_void_p(g["a"].data_ptr()), ctypes.c_void_p(g["sizes"].data_ptr()),
        ctypes.c_void_p(g["w"].data_ptr()), ctypes.c_void_p(g["s"].data_ptr()), ctypes.c_void_p(out.data_ptr()),
        M, c.N, c.K, c.E, None if err is None else ctypes.c_void_p(err.data_ptr()), None,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


def test_noalloc_matches_workspace_entry_point(geg):
    import torch
    # first call: a prefill batch (tiled path with the row-scaled fp16 copy in the
    # library-held scratch, small experts on the narrow kernel); second call: a
    # smaller decode batch (vector path), so the second call leaves most of what
    # the first wrote in the scratch untouched
    for i, (E, K, N, sizes) in enumerate([(6, 512, 704, [300, 7, 0, 1800, 20, 257]),
                                          (8, 256, 320, [1, 0, 1, 1, 0, 1, 1, 1])]):
        c, d = _case(E, K, N, sizes, seed=50 + i)
        g = upload_case(d)
        log(f"case: noalloc call {i + 1}: M={g['a'].shape[0]} N={N} K={K} E={E} sizes={sizes}")
        out = torch.full((g["a"].shape[0], N), 7.0, dtype=torch.bfloat16, device="cuda")
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        assert _noalloc(geg, g, c, out, err) == 0, geg.lib().geg_last_error()
        ref_ws = geg.gnf4_grouped_gemm(g["a"], g["sizes"], g["w"], g["s"])
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        same = bool((bits16(out) == bits16(ref_ws)).all())
        log(f"  bitwise equal to gnf4_grouped_gemm: {same}")
        assert same
        assert_close(bf16_to_f64(out), oracle.grouped_ref(d["a_bits"], d["sizes"], C.weight_fn(d), N),
                     f"noalloc call {i + 1}")


def test_noalloc_reports_device_errors_to_the_callers_word(geg):
    import torch
    c, d = _case(3, 256, 128, [10, 20, 5], seed=53)
    g = upload_case(d)
    g["sizes"] = torch.tensor([10, -4, 5], dtype=torch.int32, device="cuda")
    out = torch.empty((35, 128), dtype=torch.bfloat16, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    assert _noalloc(geg, g, c, out, err) == 0
    torch.cuda.synchronize()
    assert int(err.item()) & geg.DEVERR_NEGATIVE_SIZE
    # no error word: the bits are dropped, the call still succeeds
    assert _noalloc(geg, g, c, out, None) == 0
    torch.cuda.synchronize()


def test_noalloc_refuses_scratch_past_its_array(geg):
    # M * K * 2 bytes of row-scaled fp16 activations past 144 MiB: refused on the
    # host before any device work (no pointer is touched)
    P = 0x10000
    st = geg.lib().gnf4_grouped_gemm_noalloc(P, P, P, P, P, 40000, 256, 2048, 4, None, None, None)
    assert st == 5
    assert b"144 MiB" in geg.lib().geg_last_error()
    # within the array (117 MiB of fp16 rows; the optional 32 MiB of split
    # remainder tiles left out) the same sizes go on to the pointer checks
    st = geg.lib().gnf4_grouped_gemm_noalloc(P, P, P, P, P, 30000, 256, 2048, 4, None, None, None)
    assert st not in (0, 5)
