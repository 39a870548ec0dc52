"""The C ABI without a GPU: the library loads, exports every declared function,
and refuses bad arguments before any launch (no device call is made)."""
import ctypes

import pytest

import grouped_expert_gemm_amd as geg

P = 0x10000          # a fake 64 KiB-aligned address; never dereferenced by these checks


def L():
    return geg.lib()


def test_library_exports_every_header_function():
    names = geg.header_functions()
    assert len(names) >= 13
    for n in ["gnf4_grouped_gemm", "gmxfp4_grouped_gemm", "gnf4_grouped_dgrad",
              "geg_workspace_bytes", "gnf4_dequant", "gmxfp4_dequant", "gnf4_quantize"]:
        assert n in names
    lib = L()
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_version_and_status_strings():
    assert L().geg_version() == 113
    assert L().geg_status_string(0) == b"GEG_OK"
    assert L().geg_status_string(5) == b"GEG_ERR_WORKSPACE"


def _gemm(name="gnf4_grouped_gemm", a=P, sizes=P, w=P, s=P, out=P, M=16, N=64, K=128, E=4,
          ws=P, ws_bytes=1 << 20, opts=None):
    f = getattr(L(), name)
    return f(a, sizes, w, s, out, M, N, K, E, ws, ws_bytes, ctypes.byref(opts) if opts else None, None)


def test_bad_shapes_are_refused():
    assert _gemm(K=100) == 2                        # K % 64
    assert b"multiple of 64" in L().geg_last_error()
    assert _gemm("gmxfp4_grouped_gemm", K=48) == 2  # K % 32
    assert b"multiple of 32" in L().geg_last_error()
    assert _gemm(M=-1) == 2
    assert _gemm(N=0) == 2
    assert _gemm(E=0) == 2
    assert _gemm(E=2000) == 2
    assert b"1024 experts" in L().geg_last_error()
    assert L().gnf4_grouped_dgrad(P, P, P, P, P, 16, 60, 128, 4, P, 1 << 20, None, None) == 2  # N % 8
    assert b"N % 8" in L().geg_last_error()


def test_buffer_windows_past_2gib_are_refused_not_clamped():
    # one expert's packed weights must fit one 32-bit buffer window: N * K / 2 bytes
    # just past 0x7FFFFFF0 is refused on the host (before any device check) by
    # every entry point, instead of the kernels reading zeros past the window
    N, K = 65536, 65536                              # N * K / 2 = 2^31
    for name in ("gnf4_grouped_gemm", "gmxfp4_grouped_gemm", "gnf4_grouped_dgrad", "gmxfp4_grouped_dgrad",
                 "gmxfp4_w4a8_grouped_gemm"):
        assert _gemm(name, N=N, K=K) == 2, name
        assert b"0x7FFFFFF0" in L().geg_last_error(), name
    assert _gemm(N=32768, K=131072) == 2               # 2^31 bytes again
    # within the window the shape passes and the call stops at a later check
    # (no GPU here, or P is not device memory)
    assert _gemm(N=32767, K=131072) not in (0, 2)      # 2^31 - 2^16 bytes
    assert _gemm(N=65536 - 64, K=65536) not in (0, 2)  # 2^31 - 2^21 bytes
    # 256 rows of the contraction or output width must fit one window (512 * max(N, K) bytes)
    assert _gemm(N=64, K=4194304) == 2
    assert b"4194303" in L().geg_last_error()
    assert L().gnf4_grouped_dgrad(P, P, P, P, P, 16, 4194304, 64, 4, P, 1 << 20, None, None) == 2
    # the W4A8 activation scales are read through one window: ceil(K/128) * M * 4 bytes
    assert _gemm("gmxfp4_w4a8_grouped_gemm", M=(1 << 28), N=64, K=512) == 2
    assert b"activation scales" in L().geg_last_error()
    # the block checks both projections
    assert L().gnf4_expert_block(P, P, P, P, P, P, P, 16, 65536, 32768, 4, P, 1 << 20, None, None) == 2


def test_bad_options_are_refused():
    assert _gemm(opts=geg.Opts(5, 0)) == 8
    assert _gemm(opts=geg.Opts(0, 17)) == 8
    assert _gemm(opts=geg.Opts(0, -1)) == 8
    assert _gemm(opts=geg.Opts(0, 0, None, -1)) == 8
    assert b"cu_limit" in L().geg_last_error()
    assert _gemm(opts=geg.Opts(0, 0, None, 3)) not in (0, 2, 8)   # accepted: stops at the device check


def test_empty_problem_is_a_noop_even_with_null_pointers():
    assert _gemm(a=None, sizes=None, w=None, s=None, out=None, M=0, ws=None) == 0


def test_null_pointers_are_refused():
    assert _gemm(a=None) == 1
    assert _gemm(sizes=None) == 1
    assert _gemm(out=None) == 1
    assert _gemm(ws=None) == 5


def test_misaligned_pointers_are_refused():
    assert _gemm(a=P + 2) == 3
    assert _gemm(out=P + 8) == 3
    assert _gemm(w=P + 4) == 3
    assert _gemm(ws=P + 16) == 5


def test_small_workspace_is_refused():
    o = geg.Opts(1, 4)                              # skinny path, 4 K splits
    need = geg.geg_workspace_bytes(geg.GEG_OP_NF4_FWD, 8, 2048, 2048, 64, o)
    assert need > 256                               # split-K needs its partials
    assert _gemm(M=8, N=2048, K=2048, E=64, ws_bytes=need - 256, opts=o) == 5
    assert b"workspace" in L().geg_last_error()


def test_split_region_of_the_workspace_is_optional():
    # a workspace that holds everything but the 32 MiB of split remainder tiles
    # passes the workspace check (the call then runs unsplit; here it stops at
    # the device check), one byte less than that is refused
    tail = 256 * 128 * 256 * 4
    for name, op, M, N, K in (("gnf4_grouped_gemm", geg.GEG_OP_NF4_FWD, 4096, 2048, 2048),
                              ("gmxfp4_grouped_gemm", geg.GEG_OP_MXFP4_FWD, 4096, 2048, 2048),
                              ("gnf4_grouped_dgrad", geg.GEG_OP_NF4_DGRAD, 4096, 2048, 1024),
                              ("gmxfp4_grouped_dgrad", geg.GEG_OP_MXFP4_DGRAD, 4096, 2048, 1024)):
        need = geg.geg_workspace_bytes(op, M, N, K, 8)
        base = need - tail
        assert base >= 256 and base % 256 == 0, name
        assert _gemm(name, M=M, N=N, K=K, E=8, ws_bytes=base) not in (0, 5), name
        assert _gemm(name, M=M, N=N, K=K, E=8, ws_bytes=base - 256) == 5, name
        assert b"workspace" in L().geg_last_error(), name


def test_workspace_sizes():
    # NF4 prefill: the 256-byte header (error word), then the fp16 copy of the
    # activations that the tiled path reads and the rows' int32 exponents;
    # MXFP4 reads bf16 activations as given
    # contraction >= 1024: plus the fp32 partials of up to 256 split remainder
    # tiles (128 x 256 values each)
    tail = 256 * 128 * 256 * 4
    assert geg.geg_workspace_bytes(geg.GEG_OP_NF4_FWD, 16384, 2048, 2048, 64) == \
        256 + 16384 * 2048 * 2 + 16384 * 4 + tail
    assert geg.geg_workspace_bytes(geg.GEG_OP_MXFP4_FWD, 8192, 5760, 2880, 32) == 256 + tail
    assert geg.geg_workspace_bytes(geg.GEG_OP_MXFP4_FWD, 8192, 5760, 992, 32) == 256
    assert geg.geg_workspace_bytes(geg.GEG_OP_NF4_FWD, 8192, 2048, 768, 128) == 256 + 8192 * 768 * 2 + 8192 * 4
    assert geg.geg_workspace_bytes(geg.GEG_OP_NF4_DGRAD, 8192, 28672, 4096, 8) == \
        256 + 8192 * 28672 * 2 + 8192 * 4 + tail
    assert geg.geg_workspace_bytes(geg.GEG_OP_NF4_DGRAD, 8192, 4096, 14336, 8) == \
        256 + 8192 * 4096 * 2 + 8192 * 4 + tail
    assert geg.geg_workspace_bytes(geg.GEG_OP_NF4_DGRAD, 8192, 512, 14336, 8) == \
        256 + 8192 * 512 * 2 + 8192 * 4
    assert geg.geg_workspace_bytes(geg.GEG_OP_MXFP4_DGRAD, 64, 8192, 256, 4) == 256 + tail
    assert geg.geg_workspace_bytes(geg.GEG_OP_NF4_FWD, 8192, 4096, 14336, 8) == \
        256 + 8192 * 14336 * 2 + 8192 * 4 + tail
    assert geg.geg_workspace_bytes(geg.GEG_OP_NF4_FWD, 3000, 2048, 64, 4) == \
        256 + 3000 * 64 * 2 + ((3000 * 4 + 255) & ~255)
    # skinny split-K partials; a small batch on the automatic path goes to the
    # vector path, which needs nothing beyond the header
    one = geg.geg_workspace_bytes(geg.GEG_OP_NF4_FWD, 8, 2048, 2048, 64, geg.Opts(1, 1))
    four = geg.geg_workspace_bytes(geg.GEG_OP_NF4_FWD, 8, 2048, 2048, 64, geg.Opts(1, 4))
    assert one == 256 and four >= 256 + 4 * 8 * 2048 * 4
    assert geg.geg_workspace_bytes(geg.GEG_OP_NF4_FWD, 8, 2048, 2048, 64) == 256
    assert geg.geg_workspace_bytes(7, 8, 8, 64, 1) == 0


def test_dequant_and_quantize_validation():
    assert L().gnf4_dequant(P, P, P, None, None, 16, 100, 2, None) == 2
    assert L().gnf4_dequant(None, P, P, None, None, 16, 128, 2, None) == 1
    assert L().gmxfp4_dequant(P, P, P + 4, None, None, 16, 128, 2, None) == 3
    assert L().gnf4_quantize(P, P, P, 4, 96, None) == 2
    assert L().gnf4_quantize(None, None, None, 0, 64, None) == 0


def test_python_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    a = torch.zeros((4, 64), dtype=torch.bfloat16)
    with pytest.raises(geg.GegError, match="GPU"):
        geg.gnf4_grouped_gemm(a, torch.zeros(1, dtype=torch.int32),
                              torch.zeros((1, 8, 32), dtype=torch.uint8),
                              torch.zeros((1, 8, 1), dtype=torch.float32))


def test_python_binding_checks_operand_types_and_shapes():
    # the C entry points take bare pointers, so the binding checks every operand's
    # dtype and shape before anything reaches the device: MXFP4 scale bytes handed
    # to the NF4 entry point (or the reverse) are refused, not read as fp32
    torch = pytest.importorskip("torch")
    E, N, K, M = 2, 8, 128, 4
    a = torch.zeros((M, K), dtype=torch.bfloat16)
    sizes = torch.zeros(E, dtype=torch.int32)
    w = torch.zeros((E, N, K // 2), dtype=torch.uint8)
    nf4_s = torch.zeros((E, N, K // 64), dtype=torch.float32)
    mx_s = torch.zeros((E, N, K // 32), dtype=torch.uint8)
    dy = torch.zeros((M, N), dtype=torch.bfloat16)
    for call in (lambda: geg.gnf4_grouped_gemm(a, sizes, w, mx_s),
                 lambda: geg.gmxfp4_grouped_gemm(a, sizes, w, nf4_s),
                 lambda: geg.gnf4_grouped_dgrad(dy, sizes, w, mx_s),
                 lambda: geg.gmxfp4_grouped_dgrad(dy, sizes, w, nf4_s),
                 lambda: geg.gnf4_grouped_gemm(a.float(), sizes, w, nf4_s),
                 lambda: geg.gnf4_grouped_gemm(a, sizes.long(), w, nf4_s),
                 lambda: geg.gnf4_grouped_gemm(a[:, :64], sizes, w, nf4_s),
                 lambda: geg.gnf4_grouped_gemm(a, sizes, w.transpose(1, 2).contiguous().transpose(1, 2), nf4_s),
                 lambda: geg.gnf4_dequant(w, mx_s),
                 lambda: geg.route_combine(torch.zeros((6, 16), dtype=torch.bfloat16),
                                           torch.zeros(8, dtype=torch.int32), None, 2)):
        with pytest.raises(geg.GegError, match="GEG_ERR_BAD_SHAPE"):
            call()
    # well-formed operands get as far as the device check
    with pytest.raises(geg.GegError, match="GPU"):
        geg.gmxfp4_grouped_dgrad(dy, sizes, w, mx_s)


def test_scratch_lies_past_the_header():
    # routing counts, the adapter backward's scratch and the W4A8 codes start
    # after the 256-byte header that holds the error word
    assert geg.lib().geg_route_workspace_bytes(64, 8, 64) == 256 + 2 * 64 * 4   # 512 entries: 2 chunks
    assert geg.lib().geg_lora_workspace_bytes(geg.GEG_OP_MXFP4_DGRAD, 64, 128, 256, 4, 8) == \
        256 + 4 * 8 * 128 * 4 + 4 * 256 * 8 * 4 + 64 * 8 * 4
    assert geg.geg_workspace_bytes(geg.GEG_OP_MXFP4_W4A8, 64, 128, 256, 4) >= 256 + 64 * 256
