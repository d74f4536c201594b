"""NVFP4 W4A4 linear layer for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI in ``include/nvfp4.h`` (library
``libnvfp4.so`` built from ``csrc/``).  The binding only marshals arguments:
PyTorch provides device memory and the current stream, and every step of the
computation runs in the HIP kernels.  If the library is missing the import
fails; there is no fallback.

Entry points (same names as the C ABI):

* ``nvfp4_quantize(x)`` -> ``(codes, scales, gs)``: on-the-fly NVFP4
  quantization (paper "Why Gated DeltaNet Survives 4-Bit Quantization",
  section 2 "NVFP4").
* ``nvfp4_dequantize(codes, scales, gs, out_dtype)``: two-level dequant.
* ``nvfp4_fuse_rescale(scales_list, gs_list)`` -> ``gs_shared``: the
  fused-module repair (same paper, section 6), in place.
* ``nvfp4_gemm(x, w_codes, w_scales, w_gs, out_dtype)``: the W4A4 linear
  ``Y = X W^T`` with X quantized on the fly.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads the HIP runtime the library must share with PyTorch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnvfp4.so")

NVFP4_F32 = 0
NVFP4_BF16 = 1
MAX_FUSED = 16

_STATUS = {
    0: "NVFP4_OK", 1: "NVFP4_ERR_NULL", 2: "NVFP4_ERR_SHAPE", 3: "NVFP4_ERR_DTYPE",
    4: "NVFP4_ERR_ALIGN", 5: "NVFP4_ERR_WORKSPACE", 6: "NVFP4_ERR_INVALID", 7: "NVFP4_ERR_DEVICE",
}

# Every symbol include/nvfp4.h declares.
EXPORTS = (
    "nvfp4_status_string", "nvfp4_version", "nvfp4_quantize_workspace_size", "nvfp4_quantize",
    "nvfp4_dequantize", "nvfp4_fuse_rescale", "nvfp4_gemm_workspace_size", "nvfp4_gemm",
    "nvfp4_gemm_prepare", "nvfp4_gemm_run", "nvfp4_quantize_static", "nvfp4_gemm_prepare_static",
    "nvfp4_gemm_static", "nvfp4_gemm_w4a16_workspace_size", "nvfp4_gemm_w4a16",
    "nvfp4_fp8_quantize_workspace_size", "nvfp4_fp8_quantize", "nvfp4_fp8_quantize_static", "nvfp4_fp8_dequantize",
    "nvfp4_gemm_w8a16_workspace_size", "nvfp4_gemm_w8a8_workspace_size", "nvfp4_gemm_w8a16", "nvfp4_gemm_w8a8",
    "nvfp4_gemm_noalloc",
)

# Size of the library's fixed scratch array behind nvfp4_gemm_noalloc.
NOALLOC_SCRATCH_BYTES = 128 << 20


class Nvfp4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (%s)" % (where, _STATUS.get(status, "?"), status_string(status)))


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError("libnvfp4.so is not built; run `python nvfp4_w4a4_quantized_02_amd/build.py` "
                          "(or __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    I = ctypes.c_int
    L.nvfp4_status_string.argtypes = [I]
    L.nvfp4_status_string.restype = ctypes.c_char_p
    L.nvfp4_version.restype = I
    L.nvfp4_quantize_workspace_size.argtypes = [I64, I64]
    L.nvfp4_quantize_workspace_size.restype = SZ
    L.nvfp4_quantize.argtypes = [P, I, I64, I64, I64, P, P, P, P, SZ, P]
    L.nvfp4_quantize.restype = I
    L.nvfp4_dequantize.argtypes = [P, P, P, I64, I64, P, I, I64, P]
    L.nvfp4_dequantize.restype = I
    L.nvfp4_fuse_rescale.argtypes = [I, ctypes.POINTER(P), ctypes.POINTER(I64), I64, ctypes.POINTER(P), P, P]
    L.nvfp4_fuse_rescale.restype = I
    L.nvfp4_gemm_workspace_size.argtypes = [I64, I64, I64]
    L.nvfp4_gemm_workspace_size.restype = SZ
    L.nvfp4_gemm.argtypes = [P, I, I64, I64, I64, P, P, P, I64, P, I, I64, P, SZ, P]
    L.nvfp4_gemm.restype = I
    L.nvfp4_gemm_prepare.argtypes = [P, I, I64, I64, I64, P, SZ, P]
    L.nvfp4_gemm_prepare.restype = I
    L.nvfp4_gemm_run.argtypes = [I64, I64, P, P, P, I64, P, I, I64, P, SZ, P]
    L.nvfp4_gemm_run.restype = I
    L.nvfp4_quantize_static.argtypes = [P, I, I64, I64, I64, P, P, P, P]
    L.nvfp4_quantize_static.restype = I
    L.nvfp4_gemm_prepare_static.argtypes = [P, I, I64, I64, I64, P, P, SZ, P]
    L.nvfp4_gemm_prepare_static.restype = I
    L.nvfp4_gemm_static.argtypes = [P, I, I64, I64, I64, P, P, P, P, I64, P, I, I64, P, SZ, P]
    L.nvfp4_gemm_static.restype = I
    L.nvfp4_gemm_w4a16_workspace_size.argtypes = [I64, I64, I64]
    L.nvfp4_gemm_w4a16_workspace_size.restype = SZ
    L.nvfp4_gemm_w4a16.argtypes = [P, I, I64, I64, I64, P, P, P, I64, P, I, I64, P, SZ, P]
    L.nvfp4_gemm_w4a16.restype = I
    L.nvfp4_fp8_quantize_workspace_size.argtypes = [I64, I64]
    L.nvfp4_fp8_quantize_workspace_size.restype = SZ
    L.nvfp4_fp8_quantize.argtypes = [P, I, I64, I64, I64, P, P, P, SZ, P]
    L.nvfp4_fp8_quantize.restype = I
    L.nvfp4_fp8_quantize_static.argtypes = [P, I, I64, I64, I64, P, P, P]
    L.nvfp4_fp8_quantize_static.restype = I
    L.nvfp4_fp8_dequantize.argtypes = [P, P, I64, I64, P, I, I64, P]
    L.nvfp4_fp8_dequantize.restype = I
    for n in ("nvfp4_gemm_w8a16_workspace_size", "nvfp4_gemm_w8a8_workspace_size"):
        getattr(L, n).argtypes = [I64, I64, I64]
        getattr(L, n).restype = SZ
    L.nvfp4_gemm_w8a16.argtypes = [P, I, I64, I64, I64, P, P, I64, P, I, I64, P, SZ, P]
    L.nvfp4_gemm_w8a16.restype = I
    L.nvfp4_gemm_w8a8.argtypes = [P, I, I64, I64, I64, P, P, P, I64, P, I, I64, P, SZ, P]
    L.nvfp4_gemm_w8a8.restype = I
    L.nvfp4_gemm_noalloc.argtypes = [P, I, I64, I64, I64, P, P, P, I64, P, I, I64, P]
    L.nvfp4_gemm_noalloc.restype = I
    _check_single_hip_runtime()
    return L


def _check_single_hip_runtime():
    """The library must use the HIP runtime PyTorch loaded; two copies in one
    process would not share streams or device pointers."""
    try:
        with open("/proc/self/maps") as f:
            paths = {line.split()[-1] for line in f if "libamdhip64" in line}
    except OSError:
        return
    real = {os.path.realpath(p) for p in paths}
    if len(real) > 1:
        raise ImportError("two HIP runtimes are loaded (%s); import torch before libnvfp4" % sorted(real))


lib = _load()


def status_string(status: int) -> str:
    return lib.nvfp4_status_string(status).decode()


def _check(status: int, where: str):
    if status != 0:
        raise Nvfp4Error(status, where)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return NVFP4_F32
    if dt == torch.bfloat16:
        return NVFP4_BF16
    raise TypeError("supported dtypes are float32 and bfloat16, got %s" % dt)


def _stream_ptr(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


_workspaces: dict = {}


def workspace(nbytes: int, device) -> torch.Tensor:
    """A scratch buffer of at least nbytes (256-byte aligned), one per
    (device, current stream): calls that use it are ordered on that stream,
    so calls on different streams never share one, and a buffer replaced by a
    larger one was only ever used on the stream it was allocated on (torch's
    allocator then reuses its memory in that stream's order).  Code under
    graph capture should pass its own workspace where an entry point takes
    one, or run once eagerly on the capture stream first."""
    dev = torch.device(device)
    if dev.type != "cuda":
        raise ValueError("workspaces live on a GPU, got device %s" % dev)
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    key = (idx, torch.cuda.current_stream(idx).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 1 << 16), dtype=torch.uint8, device=torch.device("cuda", idx))
        assert ws.data_ptr() % 256 == 0
        _workspaces[key] = ws
    return ws


def _rows_view(x: torch.Tensor) -> tuple:
    """(rows, K, ld) of a 2-D float32/bfloat16 tensor on a GPU whose last
    dimension is contiguous."""
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda":
        raise ValueError("expected a tensor on a GPU")
    if x.dim() != 2:
        raise ValueError("expected a 2-D tensor, got shape %s" % (tuple(x.shape),))
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("supported dtypes are float32 and bfloat16, got %s" % x.dtype)
    if x.stride(1) != 1 and x.shape[1] > 1:
        raise ValueError("the last dimension must be contiguous")
    return x.shape[0], x.shape[1], x.stride(0) if x.shape[0] > 1 else max(x.shape[1], x.stride(0))


def _check_u8(t: torch.Tensor, shape: tuple, device, what: str):
    if not isinstance(t, torch.Tensor) or t.dtype != torch.uint8 or tuple(t.shape) != tuple(shape) \
            or t.device != device or not t.is_contiguous():
        raise ValueError("%s must be a contiguous uint8 tensor of shape %s on %s, got %s" % (
            what, tuple(shape), device, "%s %s on %s" % (t.dtype, tuple(t.shape), t.device)
            if isinstance(t, torch.Tensor) else type(t).__name__))


def _check_scalar(t: torch.Tensor, device, what: str):
    """A float32 device scalar (the first element is used)."""
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.numel() < 1 or t.device != device \
            or not t.is_contiguous():
        raise ValueError("%s must be a contiguous float32 tensor with at least one element on %s" % (what, device))


def nvfp4_quantize(x: torch.Tensor):
    """Quantize a [rows, K] float32/bfloat16 CUDA tensor.

    Returns (codes uint8 [rows, K/2], scales uint8 [rows, K/16], gs float32 [1])."""
    rows, K, ld = _rows_view(x)
    codes = torch.empty((rows, K // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, K // 16), dtype=torch.uint8, device=x.device)
    gs = torch.empty(1, dtype=torch.float32, device=x.device)
    nws = lib.nvfp4_quantize_workspace_size(rows, K)
    ws = workspace(nws, x.device)
    _check(lib.nvfp4_quantize(x.data_ptr(), _dtype_code(x.dtype), rows, K, ld, codes.data_ptr(),
                              scales.data_ptr(), gs.data_ptr(), ws.data_ptr(), ws.numel(),
                              _stream_ptr(x.device)), "nvfp4_quantize")
    return codes, scales, gs


def nvfp4_quantize_static(x: torch.Tensor, gs: torch.Tensor):
    """Quantize with a given (calibrated) tensor scale gs (float32 [1] on the
    device).  Returns (codes uint8 [rows, K/2], scales uint8 [rows, K/16])."""
    rows, K, ld = _rows_view(x)
    _check_scalar(gs, x.device, "gs")
    codes = torch.empty((rows, K // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, K // 16), dtype=torch.uint8, device=x.device)
    _check(lib.nvfp4_quantize_static(x.data_ptr(), _dtype_code(x.dtype), rows, K, ld, gs.data_ptr(),
                                     codes.data_ptr(), scales.data_ptr(), _stream_ptr(x.device)),
           "nvfp4_quantize_static")
    return codes, scales


def nvfp4_dequantize(codes: torch.Tensor, scales: torch.Tensor, gs: torch.Tensor,
                     out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    if not isinstance(codes, torch.Tensor) or codes.dim() != 2 or codes.device.type != "cuda":
        raise ValueError("codes must be a 2-D uint8 tensor [rows, K/2] on a GPU")
    rows, half = codes.shape
    K = 2 * half
    _check_u8(codes, (rows, half), codes.device, "codes")
    _check_u8(scales, (rows, K // 16), codes.device, "scales")
    _check_scalar(gs, codes.device, "gs")
    out = torch.empty((rows, K), dtype=out_dtype, device=codes.device)
    _check(lib.nvfp4_dequantize(codes.data_ptr(), scales.data_ptr(), gs.data_ptr(), rows, K, out.data_ptr(),
                                _dtype_code(out_dtype), K, _stream_ptr(codes.device)), "nvfp4_dequantize")
    return out


def nvfp4_fuse_rescale(scales_list, gs_list) -> torch.Tensor:
    """Repair a fused group in place; returns the shared tensor scale [1]."""
    n = len(scales_list)
    if not 1 <= n <= MAX_FUSED or len(gs_list) != n:
        raise ValueError("need 1..%d members with one tensor scale each" % MAX_FUSED)
    kb = scales_list[0].shape[1]
    dev = scales_list[0].device
    if dev.type != "cuda":
        raise ValueError("member scales must be on a GPU")
    for s in scales_list:
        if s.dim() != 2 or s.shape[1] != kb:
            raise ValueError("member scales must be uint8 [rows, K/16] with one K")
        _check_u8(s, tuple(s.shape), dev, "member scales")
    for g in gs_list:
        _check_scalar(g, dev, "member tensor scale")
    shared = torch.empty(1, dtype=torch.float32, device=dev)
    ptrs = (ctypes.c_void_p * n)(*[s.data_ptr() for s in scales_list])
    rows = (ctypes.c_int64 * n)(*[s.shape[0] for s in scales_list])
    gptrs = (ctypes.c_void_p * n)(*[g.data_ptr() for g in gs_list])
    _check(lib.nvfp4_fuse_rescale(n, ptrs, rows, kb, gptrs, shared.data_ptr(), _stream_ptr(dev)),
           "nvfp4_fuse_rescale")
    return shared


def _out_tensor(M, N, out_dtype, device):
    # rows padded to a 16-byte multiple, as the kernels store 16-byte aligned
    _dtype_code(out_dtype)
    per16 = 16 // torch.empty((), dtype=out_dtype).element_size()
    ld_pad = (N + per16 - 1) // per16 * per16
    return torch.empty((M, ld_pad), dtype=out_dtype, device=device)[:, :N]


def _check_out(out: torch.Tensor, M: int, N: int, device) -> torch.Tensor:
    """A caller-supplied output: [M, N] float32/bfloat16 on the device, unit
    inner stride and rows at least N apart (the library checks alignment)."""
    if not isinstance(out, torch.Tensor) or tuple(out.shape) != (M, N) or out.device != device:
        raise ValueError("out must be a tensor of shape %s on %s" % ((M, N), device))
    if out.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out must be float32 or bfloat16, got %s" % out.dtype)
    if N > 1 and out.stride(1) != 1:
        raise ValueError("out rows must be contiguous")
    if M > 1 and out.stride(0) < N:
        raise ValueError("out rows overlap (row stride %d < N = %d)" % (out.stride(0), N))
    return out


def _ld_out(out, M, N):
    return out.stride(0) if M > 1 else max(N, out.stride(0))


def _output(out, M, N, out_dtype, device):
    return _out_tensor(M, N, out_dtype, device) if out is None else _check_out(out, M, N, device)


def _check_weight(w_codes, w_scales, w_gs, K, device):
    if not isinstance(w_codes, torch.Tensor) or w_codes.dim() != 2:
        raise ValueError("w_codes must be a 2-D uint8 tensor [N, K/2]")
    N = w_codes.shape[0]
    _check_u8(w_codes, (N, K // 2), device, "w_codes")
    _check_u8(w_scales, (N, K // 16), device, "w_scales")
    _check_scalar(w_gs, device, "w_gs")
    return N


def nvfp4_gemm(x: torch.Tensor, w_codes: torch.Tensor, w_scales: torch.Tensor, w_gs: torch.Tensor,
               out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
               x_gs: torch.Tensor | None = None, ws: torch.Tensor | None = None) -> torch.Tensor:
    """Y = X W^T with X [M, K] quantized on the fly and W given as NVFP4
    (codes [N, K/2], scales [N, K/16], w_gs [1]).  x_gs: a calibrated
    activation tensor scale (float32 [1] on the device) instead of the
    absmax one.  ws: a uint8 workspace of the caller's (256-byte aligned, at
    least nvfp4_gemm_workspace_size bytes), e.g. for graph capture; by
    default the per-stream one."""
    M, K, ld = _rows_view(x)
    N = _check_weight(w_codes, w_scales, w_gs, K, x.device)
    out = _output(out, M, N, out_dtype, x.device)
    if x_gs is not None:
        _check_scalar(x_gs, x.device, "x_gs")
    nws = lib.nvfp4_gemm_workspace_size(M, N, K)
    if ws is None:
        ws = workspace(nws, x.device)
    else:
        _check_u8(ws, (ws.numel(),), x.device, "ws")
        if ws.data_ptr() % 256 or ws.numel() < nws:
            raise ValueError("the workspace must be 256-byte aligned and hold %d bytes" % nws)
    if x_gs is None:
        _check(lib.nvfp4_gemm(x.data_ptr(), _dtype_code(x.dtype), M, K, ld, w_codes.data_ptr(),
                              w_scales.data_ptr(), w_gs.data_ptr(), N, out.data_ptr(), _dtype_code(out.dtype),
                              _ld_out(out, M, N), ws.data_ptr(), ws.numel(), _stream_ptr(x.device)), "nvfp4_gemm")
    else:
        _check(lib.nvfp4_gemm_static(x.data_ptr(), _dtype_code(x.dtype), M, K, ld, x_gs.data_ptr(),
                                     w_codes.data_ptr(), w_scales.data_ptr(), w_gs.data_ptr(), N, out.data_ptr(),
                                     _dtype_code(out.dtype), _ld_out(out, M, N), ws.data_ptr(), ws.numel(),
                                     _stream_ptr(x.device)), "nvfp4_gemm_static")
    return out


def nvfp4_gemm_noalloc(x: torch.Tensor, w_codes: torch.Tensor, w_scales: torch.Tensor, w_gs: torch.Tensor,
                       out: torch.Tensor) -> torch.Tensor:
    """nvfp4_gemm into a caller-given output with no workspace and no
    allocation: the library's fixed scratch array (NOALLOC_SCRATCH_BYTES per
    device) holds the intermediate data.  Calls that overlap on one device
    race on that array."""
    M, K, ld = _rows_view(x)
    N = _check_weight(w_codes, w_scales, w_gs, K, x.device)
    _check_out(out, M, N, x.device)
    _check(lib.nvfp4_gemm_noalloc(x.data_ptr(), _dtype_code(x.dtype), M, K, ld, w_codes.data_ptr(),
                                  w_scales.data_ptr(), w_gs.data_ptr(), N, out.data_ptr(), _dtype_code(out.dtype),
                                  _ld_out(out, M, N), _stream_ptr(x.device)), "nvfp4_gemm_noalloc")
    return out


class PreparedActivations:
    """Result of nvfp4_gemm_prepare: X quantized into its own workspace,
    reusable by several nvfp4_gemm_run calls (same M and K)."""

    def __init__(self, M, K, ws):
        self.M, self.K, self.ws = M, K, ws


def nvfp4_gemm_prepare(x: torch.Tensor, ws: torch.Tensor | None = None, max_n: int = 0,
                       x_gs: torch.Tensor | None = None) -> PreparedActivations:
    """Quantize X into a workspace of its own (or the given uint8 tensor),
    sized for later runs against weights with up to max_n rows.  x_gs: a
    calibrated activation tensor scale instead of the absmax one."""
    M, K, ld = _rows_view(x)
    nws = lib.nvfp4_gemm_workspace_size(M, max_n, K)
    if ws is None or ws.numel() < nws:
        ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=x.device)
    _check_u8(ws, (ws.numel(),), x.device, "ws")
    if ws.data_ptr() % 256:
        raise ValueError("the workspace must be 256-byte aligned")
    if x_gs is not None:
        _check_scalar(x_gs, x.device, "x_gs")
    if x_gs is None:
        _check(lib.nvfp4_gemm_prepare(x.data_ptr(), _dtype_code(x.dtype), M, K, ld, ws.data_ptr(), ws.numel(),
                                      _stream_ptr(x.device)), "nvfp4_gemm_prepare")
    else:
        _check(lib.nvfp4_gemm_prepare_static(x.data_ptr(), _dtype_code(x.dtype), M, K, ld, x_gs.data_ptr(),
                                             ws.data_ptr(), ws.numel(), _stream_ptr(x.device)),
               "nvfp4_gemm_prepare_static")
    return PreparedActivations(M, K, ws)


def nvfp4_gemm_run(prep: PreparedActivations, w_codes: torch.Tensor, w_scales: torch.Tensor,
                   w_gs: torch.Tensor, out_dtype: torch.dtype = torch.bfloat16,
                   out: torch.Tensor | None = None) -> torch.Tensor:
    M, K = prep.M, prep.K
    N = _check_weight(w_codes, w_scales, w_gs, K, prep.ws.device)
    out = _output(out, M, N, out_dtype, prep.ws.device)
    _check(lib.nvfp4_gemm_run(M, K, w_codes.data_ptr(), w_scales.data_ptr(), w_gs.data_ptr(), N, out.data_ptr(),
                              _dtype_code(out.dtype), _ld_out(out, M, N), prep.ws.data_ptr(), prep.ws.numel(),
                              _stream_ptr(prep.ws.device)), "nvfp4_gemm_run")
    return out


def nvfp4_gemm_w4a16(x: torch.Tensor, w_codes: torch.Tensor, w_scales: torch.Tensor, w_gs: torch.Tensor,
                     out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None) -> torch.Tensor:
    """W4A16: Y = X W^T with X [M, K] bf16 used as given (no activation
    quantization) and W given as NVFP4 (codes [N, K/2], scales [N, K/16],
    w_gs [1])."""
    M, K, ld = _rows_view(x)
    N = _check_weight(w_codes, w_scales, w_gs, K, x.device)
    out = _output(out, M, N, out_dtype, x.device)
    nws = lib.nvfp4_gemm_w4a16_workspace_size(M, N, K)
    ws = workspace(nws, x.device) if nws else None
    _check(lib.nvfp4_gemm_w4a16(x.data_ptr(), _dtype_code(x.dtype), M, K, ld, w_codes.data_ptr(),
                                w_scales.data_ptr(), w_gs.data_ptr(), N, out.data_ptr(), _dtype_code(out.dtype),
                                _ld_out(out, M, N), ws.data_ptr() if ws is not None else None,
                                ws.numel() if ws is not None else 0, _stream_ptr(x.device)), "nvfp4_gemm_w4a16")
    return out


def nvfp4_fp8_quantize(x: torch.Tensor, scale: torch.Tensor | None = None):
    """FP8 E4M3 with one per-tensor scale.  Returns (bytes uint8 [rows, K],
    scale float32 [1]): the scale is RN(amax / 448) unless a device scale
    (float32 [1], e.g. a calibrated KV-cache scale) is given."""
    rows, K, ld = _rows_view(x)
    q = torch.empty((rows, K), dtype=torch.uint8, device=x.device)
    if scale is None:
        s = torch.empty(1, dtype=torch.float32, device=x.device)
        ws = workspace(lib.nvfp4_fp8_quantize_workspace_size(rows, K), x.device)
        _check(lib.nvfp4_fp8_quantize(x.data_ptr(), _dtype_code(x.dtype), rows, K, ld, q.data_ptr(), s.data_ptr(),
                                      ws.data_ptr(), ws.numel(), _stream_ptr(x.device)), "nvfp4_fp8_quantize")
        return q, s
    _check_scalar(scale, x.device, "scale")
    _check(lib.nvfp4_fp8_quantize_static(x.data_ptr(), _dtype_code(x.dtype), rows, K, ld, scale.data_ptr(),
                                         q.data_ptr(), _stream_ptr(x.device)), "nvfp4_fp8_quantize_static")
    return q, scale


def nvfp4_fp8_dequantize(q: torch.Tensor, scale: torch.Tensor, out_dtype: torch.dtype = torch.float32):
    if not isinstance(q, torch.Tensor) or q.dim() != 2 or q.device.type != "cuda":
        raise ValueError("q must be a 2-D uint8 tensor on a GPU")
    rows, K = q.shape
    _check_u8(q, (rows, K), q.device, "q")
    _check_scalar(scale, q.device, "scale")
    out = torch.empty((rows, K), dtype=out_dtype, device=q.device)
    _check(lib.nvfp4_fp8_dequantize(q.data_ptr(), scale.data_ptr(), rows, K, out.data_ptr(), _dtype_code(out_dtype),
                                    K, _stream_ptr(q.device)), "nvfp4_fp8_dequantize")
    return out


def _check_fp8_weight(w_q: torch.Tensor, w_scale: torch.Tensor, K: int, device) -> int:
    if not isinstance(w_q, torch.Tensor) or w_q.dim() != 2:
        raise ValueError("FP8 weights must be a 2-D uint8 tensor [N, K=%d]" % K)
    _check_u8(w_q, (w_q.shape[0], K), device, "FP8 weights")
    _check_scalar(w_scale, device, "w_scale")
    return w_q.shape[0]


def nvfp4_gemm_w8a16(x: torch.Tensor, w_q: torch.Tensor, w_scale: torch.Tensor,
                     out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None) -> torch.Tensor:
    """W8A16: Y = X (E4M3(W) * s_w)^T, X [M, K] bf16 as given, W [N, K] E4M3
    bytes with one per-tensor scale (float32 [1])."""
    M, K, ld = _rows_view(x)
    N = _check_fp8_weight(w_q, w_scale, K, x.device)
    out = _output(out, M, N, out_dtype, x.device)
    nws = lib.nvfp4_gemm_w8a16_workspace_size(M, N, K)
    ws = workspace(nws, x.device) if nws else None
    _check(lib.nvfp4_gemm_w8a16(x.data_ptr(), _dtype_code(x.dtype), M, K, ld, w_q.data_ptr(), w_scale.data_ptr(), N,
                                out.data_ptr(), _dtype_code(out.dtype), _ld_out(out, M, N),
                                ws.data_ptr() if ws is not None else None, ws.numel() if ws is not None else 0,
                                _stream_ptr(x.device)), "nvfp4_gemm_w8a16")
    return out


def nvfp4_gemm_w8a8(x: torch.Tensor, w_q: torch.Tensor, w_scale: torch.Tensor, x_scale: torch.Tensor | None = None,
                    out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None) -> torch.Tensor:
    """W8A8: X quantized to E4M3 with one per-tensor scale (RN(amax/448), or
    the calibrated x_scale), then Y = RN(s_x s_w) * E4M3(X) E4M3(W)^T."""
    M, K, ld = _rows_view(x)
    N = _check_fp8_weight(w_q, w_scale, K, x.device)
    out = _output(out, M, N, out_dtype, x.device)
    if x_scale is not None:
        _check_scalar(x_scale, x.device, "x_scale")
    ws = workspace(lib.nvfp4_gemm_w8a8_workspace_size(M, N, K), x.device)
    _check(lib.nvfp4_gemm_w8a8(x.data_ptr(), _dtype_code(x.dtype), M, K, ld,
                               x_scale.data_ptr() if x_scale is not None else None, w_q.data_ptr(),
                               w_scale.data_ptr(), N, out.data_ptr(), _dtype_code(out.dtype), _ld_out(out, M, N),
                               ws.data_ptr(), ws.numel(), _stream_ptr(x.device)), "nvfp4_gemm_w8a8")
    return out


__all__ = ["nvfp4_quantize", "nvfp4_quantize_static", "nvfp4_dequantize", "nvfp4_fuse_rescale", "nvfp4_gemm",
           "nvfp4_gemm_w4a16", "nvfp4_fp8_quantize", "nvfp4_fp8_dequantize", "nvfp4_gemm_w8a16", "nvfp4_gemm_w8a8",
           "nvfp4_gemm_prepare", "nvfp4_gemm_run", "nvfp4_gemm_noalloc", "PreparedActivations", "Nvfp4Error",
           "status_string", "lib", "EXPORTS", "LIB_PATH", "workspace"]
