"""grouped_expert_gemm_amd — Python binding of libgeg (grouped 4-bit expert GEMM, gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/geg.h. torch supplies device
memory and the current stream. There is no CPU fallback: host tensors are
refused, and a missing library raises.

    out = gnf4_grouped_gemm(a, sizes, w, absmax)          # NF4 forward
    out = gmxfp4_grouped_gemm(a, sizes, blocks, scales)   # MXFP4 forward
    dx  = gnf4_grouped_dgrad(dy, sizes, w, absmax)        # NF4 input gradient
"""
from __future__ import annotations

import ctypes
import os
import re
import threading

__all__ = [
    "GegError", "GegDeviceError", "Opts", "Workspace", "lib", "header_functions",
    "gnf4_grouped_gemm", "gnf4_grouped_gemm_noalloc", "gmxfp4_grouped_gemm", "gnf4_grouped_dgrad", "gmxfp4_grouped_dgrad",
    "grouped_linear", "gnf4_expert_block", "gmxfp4_expert_block", "route_sort", "route_combine",
    "gnf4_dequant", "gmxfp4_dequant", "gnf4_quantize", "geg_workspace_bytes",
    "gmxfp4_w4a8_grouped_gemm", "gmxfp8_quantize", "GEG_OP_MXFP4_W4A8", "DEVERR_NON_FINITE",
    "gnf4_grouped_gemm_lora", "gmxfp4_grouped_gemm_lora", "gnf4_grouped_dgrad_lora",
    "gmxfp4_grouped_dgrad_lora", "grouped_linear_lora",
    "geg_version", "geg_launch_count", "GEG_OP_NF4_FWD", "GEG_OP_MXFP4_FWD", "GEG_OP_NF4_DGRAD",
    "GEG_OP_NF4_BLOCK", "GEG_OP_MXFP4_BLOCK", "GEG_OP_MXFP4_DGRAD", "DEVERR_NEGATIVE_SIZE", "DEVERR_SIZES_EXCEED_M", "DEVERR_FP16_RANGE",
    "DEVERR_BAD_EXPERT_ID",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgeg.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "geg.h")

GEG_OP_NF4_FWD, GEG_OP_MXFP4_FWD, GEG_OP_NF4_DGRAD = 0, 1, 2
GEG_OP_NF4_BLOCK, GEG_OP_MXFP4_BLOCK, GEG_OP_MXFP4_DGRAD = 3, 4, 5
GEG_OP_MXFP4_W4A8 = 6
DEVERR_NEGATIVE_SIZE, DEVERR_SIZES_EXCEED_M, DEVERR_FP16_RANGE = 0x1, 0x2, 0x4
DEVERR_BAD_EXPERT_ID, DEVERR_NON_FINITE = 0x8, 0x10

_STATUS = {0: "GEG_OK", 1: "GEG_ERR_NULL_POINTER", 2: "GEG_ERR_BAD_SHAPE", 3: "GEG_ERR_MISALIGNED",
           4: "GEG_ERR_NOT_DEVICE_MEMORY", 5: "GEG_ERR_WORKSPACE", 6: "GEG_ERR_UNSUPPORTED_DEVICE",
           7: "GEG_ERR_HIP", 8: "GEG_ERR_BAD_OPTION", 9: "device error word"}


class GegError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{_STATUS.get(status, status)}: {detail}")


class Opts(ctypes.Structure):
    """geg_opts: force_path 0 auto / 1 skinny / 2 tiled / 3 vector / 4 narrow; split_k 0
    or 1 none / 2..16 (skinny); kernel_events: NULL or a pointer to 4 hipEvent_t (tile start/end,
    decode start/end) recorded around the call's kernels; cu_limit 0, or n > 0 to size every
    grid for at most n compute units (persistent loops then run more rounds; for tests)."""
    _fields_ = [("force_path", ctypes.c_int32), ("split_k", ctypes.c_int32),
                ("kernel_events", ctypes.c_void_p), ("cu_limit", ctypes.c_int32)]


class GegDeviceError(GegError):
    """A call's kernels flagged a condition in the workspace's device error word
    (GEG_DEVERR_* bits): raised by the wrappers when called with check_errors=True."""

    NAMES = {0x1: "negative sizes[e] (treated as 0)", 0x2: "sum(sizes) > M (rows past M not computed)",
             0x4: "an fp16 operand overflowed or is not finite", 0x8: "a top-k id outside [0, E) (dropped)",
             0x10: "a non-finite W4A8 activation"}

    def __init__(self, bits: int):
        self.bits = bits
        what = "; ".join(v for k, v in self.NAMES.items() if bits & k) or "unknown bits"
        super().__init__(9, f"device error word 0x{bits:x}: {what}")


_lib = None
_lib_lock = threading.Lock()
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t


def lib() -> ctypes.CDLL:
    """Load libgeg.so (built in-tree by grouped_expert_gemm_amd.build)."""
    global _lib
    with _lib_lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(
                    f"{LIB_PATH} is missing: build it with `python -m grouped_expert_gemm_amd.build` "
                    "(hipcc, gfx950). There is no fallback implementation.")
            L = ctypes.CDLL(LIB_PATH)
            gemm_args = [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, _SZ, _P, _P]
            for name in ("gnf4_grouped_gemm", "gmxfp4_grouped_gemm", "gnf4_grouped_dgrad",
                         "gmxfp4_grouped_dgrad", "gmxfp4_w4a8_grouped_gemm"):
                f = getattr(L, name)
                f.argtypes, f.restype = gemm_args, ctypes.c_int
            L.gmxfp8_quantize.argtypes, L.gmxfp8_quantize.restype = [_P, _P, _P, _I64, _I64, _P], ctypes.c_int
            L.gnf4_grouped_gemm_noalloc.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, _P, _P]
            L.gnf4_grouped_gemm_noalloc.restype = ctypes.c_int
            L.geg_lora_workspace_bytes.argtypes = [_I32, _I64, _I64, _I64, _I32, _I32]
            L.geg_lora_workspace_bytes.restype = _SZ
            for name in ("gnf4_grouped_gemm_lora", "gmxfp4_grouped_gemm_lora"):
                f = getattr(L, name)
                f.argtypes = [_P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _I64, _I64, _I64, _I32, _I32,
                              _P, _SZ, _P, _P]
                f.restype = ctypes.c_int
            for name in ("gnf4_grouped_dgrad_lora", "gmxfp4_grouped_dgrad_lora"):
                f = getattr(L, name)
                f.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P, _I64, _I64, _I64, _I32,
                              _I32, _P, _SZ, _P, _P]
                f.restype = ctypes.c_int
            L.geg_route_sort.argtypes = [_P, _I64, _I32, _I32, _P, _I64, _P, _P, _P, _P, _P, _SZ, _P]
            L.geg_route_sort.restype = ctypes.c_int
            L.geg_route_workspace_bytes.argtypes = [_I64, _I32, _I32]
            L.geg_route_workspace_bytes.restype = _SZ
            L.geg_route_combine.argtypes = [_P, _P, _P, _I64, _I32, _I64, _P, _P]
            L.geg_route_combine.restype = ctypes.c_int
            block_args = [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, _SZ, _P, _P]
            for name in ("gnf4_expert_block", "gmxfp4_expert_block"):
                f = getattr(L, name)
                f.argtypes, f.restype = block_args, ctypes.c_int
            L.geg_workspace_bytes.argtypes = [_I32, _I64, _I64, _I64, _I32, _P]
            L.geg_workspace_bytes.restype = _SZ
            L.geg_workspace_init.argtypes, L.geg_workspace_init.restype = [_P, _SZ, _P], ctypes.c_int
            L.geg_read_device_error.argtypes = [_P, ctypes.POINTER(ctypes.c_int32), _P]
            L.geg_read_device_error.restype = ctypes.c_int
            for name in ("gnf4_dequant", "gmxfp4_dequant"):
                f = getattr(L, name)
                f.argtypes, f.restype = [_P, _P, _P, _P, _P, _I64, _I64, _I32, _P], ctypes.c_int
            L.gnf4_quantize.argtypes, L.gnf4_quantize.restype = [_P, _P, _P, _I64, _I64, _P], ctypes.c_int
            L.geg_status_string.argtypes, L.geg_status_string.restype = [ctypes.c_int], ctypes.c_char_p
            L.geg_last_error.argtypes, L.geg_last_error.restype = [], ctypes.c_char_p
            L.geg_version.argtypes, L.geg_version.restype = [], ctypes.c_int32
            L.geg_launch_count.argtypes, L.geg_launch_count.restype = [], ctypes.c_uint64
            _lib = L
    return _lib


class KernelTimer:
    """Four HIP events (tiled-kernel start/end, decode-kernels start/end) that a
    call records around its kernels when passed through `opts()`; `elapsed_ms()`
    returns (tile_ms, decode_ms), None for kernels the call did not launch."""

    def __init__(self, force_path: int = 0, split_k: int = 0):
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._ev = (ctypes.c_void_p * 4)()
        for i in range(4):
            if self._hip.hipEventCreate(ctypes.byref(self._ev, i * ctypes.sizeof(ctypes.c_void_p))) != 0:
                raise GegError("hipEventCreate failed")
        self._opts = Opts(force_path, split_k, ctypes.cast(self._ev, ctypes.c_void_p))

    def opts(self) -> "Opts":
        return self._opts

    def _ms(self, a, b):
        ms = ctypes.c_float(0.0)
        ok = (self._hip.hipEventSynchronize(ctypes.c_void_p(self._ev[b])) == 0 and
              self._hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self._ev[a]),
                                            ctypes.c_void_p(self._ev[b])) == 0)
        # events the call did not record fail here; leave no error behind for
        # the next launch on this thread
        self._hip.hipGetLastError()
        return ms.value if ok else None

    def elapsed_ms(self):
        return self._ms(0, 1), self._ms(2, 3)

    def __del__(self):
        try:
            for i in range(4):
                self._hip.hipEventDestroy(ctypes.c_void_p(self._ev[i]))
        except Exception:
            pass


def header_functions() -> list:
    """Names of every function declared in include/geg.h."""
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b((?:geg|gnf4|gmxfp4)_\w+)\s*\(", txt)))


def _check(status: int) -> None:
    if status != 0:
        raise GegError(status, lib().geg_last_error().decode(errors="replace"))


def _check_device_errors(ws, check_errors: bool, stream) -> None:
    """With check_errors, wait for the call, read the workspace's device error word
    and raise GegDeviceError if any bit is set (the word is cleared first, so the
    next call starts clean). Without it, flagged conditions are visible only
    through Workspace.read_error()."""
    if not check_errors:
        return
    bits = ws.read_error(stream)
    if bits:
        ws.reset(stream)
        raise GegDeviceError(bits)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _require_gpu(*ts):
    for t in ts:
        if t is not None and t.device.type != "cuda":
            raise GegError(4, "tensors must be on the GPU: this library has no CPU path "
                              "(the CPU oracle under oracle/ is the reference for host data)")


def _check_tensor(t, name, dtype, shape):
    """dtype, shape and dense row-major layout of one operand: the C entry points
    take bare pointers and sizes, so this is the only place they can be checked."""
    if t is None:
        return
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise GegError(2, f"{name}: expected a contiguous {dtype} tensor of shape {list(shape)}, got "
                          f"{t.dtype} {list(t.shape)}{'' if t.is_contiguous() else ' (not contiguous)'}")


def _check_packed(nf4: bool, w, scales, E, N, K, wname, sname):
    """Packed 4-bit weights [E, N, K/2] with fp32 absmax [E, N, K/64] (NF4) or
    e8m0 bytes [E, N, K/32] (MXFP4)."""
    import torch
    _check_tensor(w, wname, torch.uint8, (E, N, K // 2))
    if nf4:
        _check_tensor(scales, sname, torch.float32, (E, N, K // 64))
    else:
        _check_tensor(scales, sname, torch.uint8, (E, N, K // 32))


def geg_version() -> int:
    return lib().geg_version()


def geg_launch_count() -> int:
    return lib().geg_launch_count()


def geg_workspace_bytes(op, M, N, K, E, opts: Opts | None = None) -> int:
    return lib().geg_workspace_bytes(op, M, N, K, E, ctypes.byref(opts) if opts else None)


class Workspace:
    """A device workspace (torch-allocated uint8 buffer), zeroed once on creation
    and grown on demand. One workspace must not be shared by concurrent calls."""

    def __init__(self, nbytes: int = 1 << 20, device=None):
        import torch
        self.device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        self.buf = None
        self.ensure(nbytes)

    def ensure(self, nbytes: int, stream=None):
        import torch
        nbytes = max(256, (int(nbytes) + 255) & ~255)
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
            _check(lib().geg_workspace_init(_ptr(self.buf), nbytes, _stream(stream)))
        return self

    @property
    def nbytes(self) -> int:
        return self.buf.numel()

    def read_error(self, stream=None) -> int:
        code = ctypes.c_int32(0)
        _check(lib().geg_read_device_error(_ptr(self.buf), ctypes.byref(code), _stream(stream)))
        return code.value

    def reset(self, stream=None):
        _check(lib().geg_workspace_init(_ptr(self.buf), self.nbytes, _stream(stream)))


_default_ws = {}


def _workspace(ws, need, device, stream):
    if ws is None:
        key = device.index
        ws = _default_ws.get(key)
        if ws is None:
            ws = _default_ws[key] = Workspace(max(need, 1 << 20), device)
    ws.ensure(need, stream)
    return ws


def _gemm(fn_name, op, a, sizes, wq, scales, out, workspace, opts, stream, check_errors=False):
    import torch
    M, K = a.shape
    E, N = wq.shape[0], wq.shape[1]
    _check_tensor(a, "a", torch.bfloat16, (M, K))
    _check_tensor(sizes, "sizes", torch.int32, (E,))
    _check_packed(op == GEG_OP_NF4_FWD, wq, scales, E, N, K, "weights", "scales")
    _check_tensor(out, "out", torch.bfloat16, (M, N))
    _require_gpu(a, sizes, wq, scales, out)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    need = geg_workspace_bytes(op, M, N, K, E, opts)
    ws = _workspace(workspace, need, a.device, stream)
    f = getattr(lib(), fn_name)
    _check(f(_ptr(a), _ptr(sizes), _ptr(wq), _ptr(scales), _ptr(out), M, N, K, E,
             _ptr(ws.buf), ws.nbytes, ctypes.byref(opts) if opts else None, _stream(stream)))
    _check_device_errors(ws, check_errors, stream)
    return out


def gnf4_grouped_gemm(a, sizes, w, absmax, out=None, workspace: Workspace | None = None,
                      opts: Opts | None = None, stream=None, check_errors: bool = False):
    """a bf16 [M,K] (rows grouped by expert), sizes int32 [E], w uint8 [E,N,K/2],
    absmax fp32 [E,N,K/64] -> out bf16 [M,N].

    Conditions the kernels flag on the device (negative sizes, sum(sizes) > M,
    fp16 overflow on a decode path) are clamped there and recorded in the
    workspace's error word; check_errors=True waits for the call and raises
    GegDeviceError when the word is set (the same holds for every wrapper below)."""
    return _gemm("gnf4_grouped_gemm", GEG_OP_NF4_FWD, a, sizes, w, absmax, out, workspace, opts, stream,
                 check_errors)


def gnf4_grouped_gemm_noalloc(a, sizes, w, absmax, out, error_word=None, opts: Opts | None = None, stream=None):
    """gnf4_grouped_gemm without a workspace, for callers that cannot allocate device
    memory: the library's kernels take their scratch from a library-held static
    array (144 MiB per GPU; larger calls raise GEG_ERR_WORKSPACE), so `out` must be
    given. error_word: None or a device int32 tensor of one element that receives
    the call's device error bits (OR-ed in). Calls that overlap on one GPU race on
    the shared array; calls ordered on one stream do not."""
    import torch
    M, K = a.shape
    E, N = w.shape[0], w.shape[1]
    _check_tensor(a, "a", torch.bfloat16, (M, K))
    _check_tensor(sizes, "sizes", torch.int32, (E,))
    _check_packed(True, w, absmax, E, N, K, "weights", "absmax")
    _check_tensor(out, "out", torch.bfloat16, (M, N))
    _check_tensor(error_word, "error_word", torch.int32, (1,))
    _require_gpu(a, sizes, w, absmax, out, error_word)
    _check(lib().gnf4_grouped_gemm_noalloc(_ptr(a), _ptr(sizes), _ptr(w), _ptr(absmax), _ptr(out), M, N, K, E,
                                           _ptr(error_word), ctypes.byref(opts) if opts else None, _stream(stream)))
    return out


def gmxfp4_grouped_gemm(a, sizes, blocks, scales, out=None, workspace: Workspace | None = None,
                        opts: Opts | None = None, stream=None, check_errors: bool = False):
    """a bf16 [M,K], sizes int32 [E], blocks uint8 [E,N,K/2] (or [E,N,K/32,16]),
    scales uint8 [E,N,K/32] -> out bf16 [M,N]."""
    if blocks.dim() == 4:
        blocks = blocks.reshape(blocks.shape[0], blocks.shape[1], -1)
    return _gemm("gmxfp4_grouped_gemm", GEG_OP_MXFP4_FWD, a, sizes, blocks, scales, out, workspace,
                 opts, stream, check_errors)


def _dgrad(fn_name, op, dy, sizes, w, scales, dx, workspace, opts, stream, check_errors=False):
    import torch
    M, N = dy.shape
    E, K = w.shape[0], w.shape[2] * 2
    _check_tensor(dy, "dy", torch.bfloat16, (M, N))
    _check_tensor(sizes, "sizes", torch.int32, (E,))
    _check_packed(op == GEG_OP_NF4_DGRAD, w, scales, E, N, K, "weights", "scales")
    _check_tensor(dx, "dx", torch.bfloat16, (M, K))
    _require_gpu(dy, sizes, w, scales, dx)
    if dx is None:
        dx = torch.empty((M, K), dtype=torch.bfloat16, device=dy.device)
    need = geg_workspace_bytes(op, M, N, K, E, opts)
    ws = _workspace(workspace, need, dy.device, stream)
    _check(getattr(lib(), fn_name)(_ptr(dy), _ptr(sizes), _ptr(w), _ptr(scales), _ptr(dx), M, N, K, E,
                                   _ptr(ws.buf), ws.nbytes, ctypes.byref(opts) if opts else None,
                                   _stream(stream)))
    _check_device_errors(ws, check_errors, stream)
    return dx


def gnf4_grouped_dgrad(dy, sizes, w, absmax, dx=None, workspace: Workspace | None = None,
                       opts: Opts | None = None, stream=None, check_errors: bool = False):
    """dy bf16 [M,N], w uint8 [E,N,K/2], absmax fp32 [E,N,K/64] -> dx bf16 [M,K]."""
    return _dgrad("gnf4_grouped_dgrad", GEG_OP_NF4_DGRAD, dy, sizes, w, absmax, dx, workspace, opts, stream,
                  check_errors)


def gmxfp4_grouped_dgrad(dy, sizes, blocks, scales, dx=None, workspace: Workspace | None = None,
                         opts: Opts | None = None, stream=None, check_errors: bool = False):
    """dy bf16 [M,N], blocks uint8 [E,N,K/2], scales uint8 [E,N,K/32] -> dx bf16 [M,K]."""
    if blocks.dim() == 4:
        blocks = blocks.reshape(blocks.shape[0], blocks.shape[1], -1)
    return _dgrad("gmxfp4_grouped_dgrad", GEG_OP_MXFP4_DGRAD, dy, sizes, blocks, scales, dx, workspace, opts,
                  stream, check_errors)


def gmxfp4_w4a8_grouped_gemm(a, sizes, blocks, scales, out=None, workspace: Workspace | None = None,
                             opts: Opts | None = None, stream=None, check_errors: bool = False):
    """W4A8: a bf16 [M,K] quantised on the device to MXFP8 (e4m3, one e8m0 scale per
    32 k) times MXFP4 blocks uint8 [E,N,K/2] (or [E,N,K/32,16]) with scales uint8
    [E,N,K/32] on the block-scaled matrix instruction -> out bf16 [M,N]."""
    if blocks.dim() == 4:
        blocks = blocks.reshape(blocks.shape[0], blocks.shape[1], -1)
    return _gemm("gmxfp4_w4a8_grouped_gemm", GEG_OP_MXFP4_W4A8, a, sizes, blocks, scales, out, workspace,
                 opts, stream, check_errors)


def gmxfp8_quantize(a, stream=None):
    """a bf16 [M,K] (K % 32 == 0) -> (e4m3 codes uint8 [M,K], e8m0 scales uint8 [M,K/32])."""
    import torch
    M, K = a.shape
    _check_tensor(a, "a", torch.bfloat16, (M, K))
    _require_gpu(a)
    codes = torch.empty((M, K), dtype=torch.uint8, device=a.device)
    scales = torch.empty((M, K // 32), dtype=torch.uint8, device=a.device)
    _check(lib().gmxfp8_quantize(_ptr(a), _ptr(codes), _ptr(scales), M, K, _stream(stream)))
    return codes, scales


def _check_lora(x, sizes, lora_a, lora_b):
    import torch
    M, K = x.shape
    E, r = lora_a.shape[0], lora_a.shape[1]
    N = lora_b.shape[1]
    _check_tensor(x, "x", torch.bfloat16, (M, K))
    _check_tensor(sizes, "sizes", torch.int32, (E,))
    _check_tensor(lora_a, "lora_a", torch.float32, (E, r, K))
    _check_tensor(lora_b, "lora_b", torch.float32, (E, N, r))
    return M, N, K, E, r


def _gemm_lora(fmt, a, sizes, w, scales, lora_a, lora_b, scale, out, u, workspace, opts, stream,
               check_errors=False):
    import torch
    M, N, K, E, r = _check_lora(a, sizes, lora_a, lora_b)
    _check_packed(fmt == "nf4", w, scales, E, N, K, "weights", "scales")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    if u is None:
        u = torch.empty((M, r), dtype=torch.float32, device=a.device)
    _check_tensor(out, "out", torch.bfloat16, (M, N))
    _check_tensor(u, "u", torch.float32, (M, r))
    _require_gpu(a, sizes, w, scales, lora_a, lora_b, out, u)
    op = GEG_OP_NF4_FWD if fmt == "nf4" else GEG_OP_MXFP4_FWD
    ws = _workspace(workspace, lib().geg_lora_workspace_bytes(op, M, N, K, E, r), a.device, stream)
    fn = getattr(lib(), "gnf4_grouped_gemm_lora" if fmt == "nf4" else "gmxfp4_grouped_gemm_lora")
    _check(fn(_ptr(a), _ptr(sizes), _ptr(w), _ptr(scales), _ptr(lora_a), _ptr(lora_b), float(scale), _ptr(out),
              _ptr(u), M, N, K, E, r, _ptr(ws.buf), ws.nbytes, ctypes.byref(opts) if opts else None, _stream(stream)))
    _check_device_errors(ws, check_errors, stream)
    return out, u


def gnf4_grouped_gemm_lora(a, sizes, w, absmax, lora_a, lora_b, scale: float, out=None, u=None,
                           workspace: Workspace | None = None, opts: Opts | None = None, stream=None,
                           check_errors: bool = False):
    """out = a_e W_e^T + scale (a_e A_e^T) B_e^T per expert, the adapter delta added
    to the fp32 accumulators before the bf16 rounding; lora_a fp32 [E, r, K],
    lora_b fp32 [E, N, r]. Returns (out bf16 [M, N], u = a A_e^T fp32 [M, r])."""
    return _gemm_lora("nf4", a, sizes, w, absmax, lora_a, lora_b, scale, out, u, workspace, opts, stream,
                      check_errors)


def gmxfp4_grouped_gemm_lora(a, sizes, blocks, scales, lora_a, lora_b, scale: float, out=None, u=None,
                             workspace: Workspace | None = None, opts: Opts | None = None, stream=None,
                             check_errors: bool = False):
    """The same on MXFP4 weights (blocks uint8 [E, N, K/2], scales uint8 [E, N, K/32])."""
    if blocks.dim() == 4:
        blocks = blocks.reshape(blocks.shape[0], blocks.shape[1], -1)
    return _gemm_lora("mxfp4", a, sizes, blocks, scales, lora_a, lora_b, scale, out, u, workspace, opts, stream,
                      check_errors)


def _dgrad_lora(fmt, dy, sizes, w, scales, x, lora_a, lora_b, u, scale, dx, grad_a, grad_b, workspace, opts,
                stream, check_errors=False):
    import torch
    M, N, K, E, r = _check_lora(x, sizes, lora_a, lora_b)
    _check_packed(fmt == "nf4", w, scales, E, N, K, "weights", "scales")
    _check_tensor(dy, "dy", torch.bfloat16, (M, N))
    _check_tensor(u, "u", torch.float32, (M, r))
    if dx is None:
        dx = torch.empty((M, K), dtype=torch.bfloat16, device=dy.device)
    if grad_a is None:
        grad_a = torch.empty((E, r, K), dtype=torch.float32, device=dy.device)
    if grad_b is None:
        grad_b = torch.empty((E, N, r), dtype=torch.float32, device=dy.device)
    _check_tensor(dx, "dx", torch.bfloat16, (M, K))
    _check_tensor(grad_a, "grad_a", torch.float32, (E, r, K))
    _check_tensor(grad_b, "grad_b", torch.float32, (E, N, r))
    _require_gpu(dy, sizes, w, scales, x, lora_a, lora_b, u, dx, grad_a, grad_b)
    op = GEG_OP_NF4_DGRAD if fmt == "nf4" else GEG_OP_MXFP4_DGRAD
    ws = _workspace(workspace, lib().geg_lora_workspace_bytes(op, M, N, K, E, r), dy.device, stream)
    fn = getattr(lib(), "gnf4_grouped_dgrad_lora" if fmt == "nf4" else "gmxfp4_grouped_dgrad_lora")
    _check(fn(_ptr(dy), _ptr(sizes), _ptr(w), _ptr(scales), _ptr(x), _ptr(lora_a), _ptr(lora_b), _ptr(u),
              float(scale), _ptr(dx), _ptr(grad_a), _ptr(grad_b), M, N, K, E, r, _ptr(ws.buf), ws.nbytes,
              ctypes.byref(opts) if opts else None, _stream(stream)))
    _check_device_errors(ws, check_errors, stream)
    return dx, grad_a, grad_b


def gnf4_grouped_dgrad_lora(dy, sizes, w, absmax, x, lora_a, lora_b, u, scale: float, dx=None, grad_a=None,
                            grad_b=None, workspace: Workspace | None = None, opts: Opts | None = None, stream=None,
                            check_errors: bool = False):
    """Backward of gnf4_grouped_gemm_lora: (dx = dy W_e + scale (dy B_e) A_e bf16
    [M, K], grad_a fp32 [E, r, K], grad_b fp32 [E, N, r])."""
    return _dgrad_lora("nf4", dy, sizes, w, absmax, x, lora_a, lora_b, u, scale, dx, grad_a, grad_b, workspace,
                       opts, stream, check_errors)


def gmxfp4_grouped_dgrad_lora(dy, sizes, blocks, scales, x, lora_a, lora_b, u, scale: float, dx=None, grad_a=None,
                              grad_b=None, workspace: Workspace | None = None, opts: Opts | None = None, stream=None,
                              check_errors: bool = False):
    """The same on MXFP4 weights."""
    if blocks.dim() == 4:
        blocks = blocks.reshape(blocks.shape[0], blocks.shape[1], -1)
    return _dgrad_lora("mxfp4", dy, sizes, blocks, scales, x, lora_a, lora_b, u, scale, dx, grad_a, grad_b,
                       workspace, opts, stream, check_errors)


def grouped_linear_lora(a, sizes, w, scales, lora_a, lora_b, scale: float, fmt: str = "nf4",
                        check_errors: bool = False):
    """The grouped 4-bit projection with a trainable low-rank delta at the
    pre-activation point, as a torch autograd op: out = a_e W_e^T + scale *
    (a_e A_e^T) B_e^T per expert. Backward: dA (through the dgrad kernel and the
    adapter kernels), d lora_a, d lora_b (fp32); the 4-bit weights are frozen.
    check_errors=True makes both directions raise GegDeviceError on a flagged
    device condition (see gnf4_grouped_gemm)."""
    return _GroupedLinearLora.apply(a, sizes, w, scales, lora_a, lora_b, float(scale), fmt, bool(check_errors))


def grouped_linear(a, sizes, w, scales, fmt: str = "nf4", check_errors: bool = False):
    """The grouped 4-bit GEMM as a differentiable op (torch autograd): out = per
    expert a_e W_e^T; the backward returns dA = per expert dOut_e W_e through the
    library's dgrad kernel on the same packed bytes. The 4-bit weights are frozen
    (no gradient), as in 4-bit adapter training. check_errors=True makes both
    directions raise GegDeviceError on a flagged device condition."""
    return _GroupedLinear.apply(a, sizes, w, scales, fmt, bool(check_errors))


def _make_grouped_linear():
    import torch

    class GroupedLinear(torch.autograd.Function):
        @staticmethod
        def forward(ctx, a, sizes, w, scales, fmt, check_errors):
            ctx.save_for_backward(sizes, w, scales)
            ctx.fmt, ctx.check_errors = fmt, check_errors
            fn = gnf4_grouped_gemm if fmt == "nf4" else gmxfp4_grouped_gemm
            return fn(a, sizes, w, scales, check_errors=check_errors)

        @staticmethod
        def backward(ctx, grad_out):
            sizes, w, scales = ctx.saved_tensors
            fn = gnf4_grouped_dgrad if ctx.fmt == "nf4" else gmxfp4_grouped_dgrad
            da = (fn(grad_out.contiguous().to(torch.bfloat16), sizes, w, scales, check_errors=ctx.check_errors)
                  if ctx.needs_input_grad[0] else None)
            return da, None, None, None, None, None

    return GroupedLinear


def _make_grouped_linear_lora():
    import torch

    class GroupedLinearLora(torch.autograd.Function):
        @staticmethod
        def forward(ctx, a, sizes, w, scales, lora_a, lora_b, scale, fmt, check_errors):
            fn = gnf4_grouped_gemm_lora if fmt == "nf4" else gmxfp4_grouped_gemm_lora
            out, u = fn(a, sizes, w, scales, lora_a, lora_b, scale, check_errors=check_errors)
            ctx.save_for_backward(a, sizes, w, scales, lora_a, lora_b, u)
            ctx.fmt, ctx.scale, ctx.check_errors = fmt, scale, check_errors
            return out

        @staticmethod
        def backward(ctx, grad_out):
            a, sizes, w, scales, lora_a, lora_b, u = ctx.saved_tensors
            fn = gnf4_grouped_dgrad_lora if ctx.fmt == "nf4" else gmxfp4_grouped_dgrad_lora
            da, ga, gb = fn(grad_out.contiguous(), sizes, w, scales, a, lora_a, lora_b, u, ctx.scale,
                            check_errors=ctx.check_errors)
            return (da if ctx.needs_input_grad[0] else None), None, None, None, ga, gb, None, None, None

    return GroupedLinearLora


class _LazyFn:
    def __init__(self, make):
        self._make = make
        self._f = None

    def apply(self, *args):
        if self._f is None:
            self._f = self._make()
        return self._f.apply(*args)


_GroupedLinear = _LazyFn(_make_grouped_linear)
_GroupedLinearLora = _LazyFn(_make_grouped_linear_lora)


def _block(fn_name, op, a, sizes, w13, s13, w2, s2, out, workspace, opts, stream, check_errors=False):
    import torch
    M, H = a.shape
    E, I = w13.shape[0], w13.shape[1] // 2
    nf4 = op == GEG_OP_NF4_BLOCK
    _check_tensor(a, "a", torch.bfloat16, (M, H))
    _check_tensor(sizes, "sizes", torch.int32, (E,))
    _check_packed(nf4, w13, s13, E, 2 * I, H, "w13", "scales13")
    _check_packed(nf4, w2, s2, E, H, I, "w2", "scales2")
    _check_tensor(out, "out", torch.bfloat16, (M, H))
    _require_gpu(a, sizes, w13, s13, w2, s2, out)
    if out is None:
        out = torch.empty((M, H), dtype=torch.bfloat16, device=a.device)
    need = geg_workspace_bytes(op, M, H, I, E, opts)
    ws = _workspace(workspace, need, a.device, stream)
    _check(getattr(lib(), fn_name)(_ptr(a), _ptr(sizes), _ptr(w13), _ptr(s13), _ptr(w2), _ptr(s2),
                                   _ptr(out), M, H, I, E, _ptr(ws.buf), ws.nbytes,
                                   ctypes.byref(opts) if opts else None, _stream(stream)))
    _check_device_errors(ws, check_errors, stream)
    return out


def gnf4_expert_block(a, sizes, w13, absmax13, w2, absmax2, out=None,
                      workspace: Workspace | None = None, opts: Opts | None = None, stream=None,
                      check_errors: bool = False):
    """Fused SwiGLU expert MLP: a bf16 [M,H], w13 uint8 [E,2I,H/2] (rows 2i gate,
    2i+1 up), absmax13 fp32 [E,2I,H/64], w2 uint8 [E,H,I/2], absmax2 fp32
    [E,H,I/64] -> out bf16 [M,H]."""
    return _block("gnf4_expert_block", GEG_OP_NF4_BLOCK, a, sizes, w13, absmax13, w2, absmax2, out,
                  workspace, opts, stream, check_errors)


def gmxfp4_expert_block(a, sizes, blocks13, scales13, blocks2, scales2, out=None,
                        workspace: Workspace | None = None, opts: Opts | None = None, stream=None,
                        check_errors: bool = False):
    """The same block on MXFP4: blocks13 uint8 [E,2I,H/2], scales13 uint8
    [E,2I,H/32], blocks2 uint8 [E,H,I/2], scales2 uint8 [E,H,I/32]."""
    if blocks13.dim() == 4:
        blocks13 = blocks13.reshape(blocks13.shape[0], blocks13.shape[1], -1)
    if blocks2.dim() == 4:
        blocks2 = blocks2.reshape(blocks2.shape[0], blocks2.shape[1], -1)
    return _block("gmxfp4_expert_block", GEG_OP_MXFP4_BLOCK, a, sizes, blocks13, scales13, blocks2,
                  scales2, out, workspace, opts, stream, check_errors)


def route_sort(topk_ids, E: int, x=None, workspace: Workspace | None = None, stream=None,
               check_errors: bool = False):
    """Device-side routing sort of topk_ids int32 [T, k] over E experts.

    Returns (sizes int32 [E], row_of int32 [T*k], src_of int32 [T*k], x_sorted):
    entries ordered by expert, then by t*k + slot; x_sorted bf16 [T*k, H] holds
    x[src_of[r] // k] in sorted row r when x (bf16 [T, H]) is given, else None."""
    import torch
    T, k = topk_ids.shape
    _check_tensor(topk_ids, "topk_ids", torch.int32, (T, k))
    if x is not None:
        _check_tensor(x, "x", torch.bfloat16, (T, x.shape[1]))
    _require_gpu(topk_ids, x)
    dev = topk_ids.device
    sizes = torch.empty((E,), dtype=torch.int32, device=dev)
    row_of = torch.empty((T * k,), dtype=torch.int32, device=dev)
    src_of = torch.empty((T * k,), dtype=torch.int32, device=dev)
    xs = None
    H = 0
    if x is not None:
        H = x.shape[1]
        xs = torch.empty((T * k, H), dtype=torch.bfloat16, device=dev)
    need = lib().geg_route_workspace_bytes(T, k, E)
    ws = _workspace(workspace, need, dev, stream)
    _check(lib().geg_route_sort(_ptr(topk_ids), T, k, E, _ptr(x), H, _ptr(sizes), _ptr(row_of),
                                _ptr(src_of), _ptr(xs), _ptr(ws.buf), ws.nbytes, _stream(stream)))
    _check_device_errors(ws, check_errors, stream)
    return sizes, row_of, src_of, xs


def route_combine(y, row_of, weights, k: int, out=None, stream=None):
    """out bf16 [T, N] = sum over slots of weights[t, s] * y[row_of[t*k + s]] (fp32 in
    slot order); y bf16 [T*k, N] in routing-sort order, weights fp32 [T, k] or None."""
    import torch
    T = row_of.numel() // k
    N = y.shape[1]
    _check_tensor(row_of, "row_of", torch.int32, (T * k,))
    _check_tensor(y, "y", torch.bfloat16, (T * k, N))
    _check_tensor(weights, "weights", torch.float32, (T, k))
    _check_tensor(out, "out", torch.bfloat16, (T, N))
    _require_gpu(y, row_of, weights, out)
    if out is None:
        out = torch.empty((T, N), dtype=torch.bfloat16, device=y.device)
    _check(lib().geg_route_combine(_ptr(y), _ptr(row_of), _ptr(weights), T, k, N, _ptr(out), _stream(stream)))
    return out


def _dequant(fn_name, wq, scales, bf16, f16, stream):
    import torch
    E, N, K = wq.shape[0], wq.shape[1], wq.shape[2] * 2
    _check_packed(fn_name == "gnf4_dequant", wq, scales, E, N, K, "weights", "scales")
    _require_gpu(wq, scales)
    f32 = torch.empty((E, N, K), dtype=torch.float32, device=wq.device)
    ob = torch.empty((E, N, K), dtype=torch.bfloat16, device=wq.device) if bf16 else None
    oh = torch.empty((E, N, K), dtype=torch.float16, device=wq.device) if f16 else None
    _check(getattr(lib(), fn_name)(_ptr(wq), _ptr(scales), _ptr(f32), _ptr(ob), _ptr(oh), N, K, E,
                                   _stream(stream)))
    return f32, ob, oh


def gnf4_dequant(w, absmax, bf16=True, f16=True, stream=None):
    """Decode NF4 [E,N,K/2] + [E,N,K/64] to (fp32, bf16|None, fp16|None) [E,N,K]."""
    return _dequant("gnf4_dequant", w, absmax, bf16, f16, stream)


def gmxfp4_dequant(blocks, scales, bf16=True, f16=True, stream=None):
    """Decode MXFP4 [E,N,K/2] + [E,N,K/32] to (fp32, bf16|None, fp16|None) [E,N,K]."""
    if blocks.dim() == 4:
        blocks = blocks.reshape(blocks.shape[0], blocks.shape[1], -1)
    return _dequant("gmxfp4_dequant", blocks, scales, bf16, f16, stream)


def gnf4_quantize(w, stream=None):
    """NF4-pack fp32 weights [..., K] on the GPU -> (codes uint8 [..., K/2], absmax fp32 [..., K/64])."""
    import torch
    _require_gpu(w)
    if w.dtype != torch.float32 or not w.is_contiguous():
        raise GegError(2, "gnf4_quantize expects a contiguous fp32 tensor")
    K = w.shape[-1]
    rows = w.numel() // K
    codes = torch.empty(w.shape[:-1] + (K // 2,), dtype=torch.uint8, device=w.device)
    absmax = torch.empty(w.shape[:-1] + (K // 64,), dtype=torch.float32, device=w.device)
    _check(lib().gnf4_quantize(_ptr(w), _ptr(codes), _ptr(absmax), rows, K, _stream(stream)))
    return codes, absmax
