"""Python binding of libq4gemv.so (4-bit weight-only dequant-GEMV for gfx950).

Argument marshalling only: every step runs in the HIP library.  Tensors must
be CUDA (ROCm) tensors, contiguous, with the dtypes the C header documents;
calls are enqueued on torch's current stream of the tensors' device.  There is
no CPU fallback: importing fails loudly if the library has not been built
(``python bit_weight_only_q4g128_amd/_build.py``).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "q4g128_gemv", "q4g128_gemv_grouped", "q4g128_gemv_grouped_noalloc", "NOALLOC_SCRATCH_BYTES", "nvfp4g16_gemv", "bf16_gemv", "q4g128_dequant_f32", "nvfp4g16_dequant_f32",
    "nvfp4g16_gemv_grouped", "nvfp4g16_workspace_bytes", "bf16_gemv_grouped", "bf16_workspace_bytes",
    "q4g128_gemv_fused", "q4g128_fused_workspace_bytes", "sample_topk", "bf16_head_sample", "bf16_head_sample_workspace_bytes", "q4g128_gemm", "gemv_grouped_mixed", "mixed_workspace_bytes",
    "variant_name", "strerror", "Q4GemvError", "LIB_PATH", "lib", "stream_read", "stream_read_sink_words",
    "VARIANT_AUTO", "VARIANT_DOT2", "VARIANT_MFMA", "VARIANT_STREAM", "VARIANT_TILED", "VARIANT_GEMM", "FMT_Q4G128", "FMT_NVFP4G16", "FMT_BF16",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libq4gemv.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing; build it with: python bit_weight_only_q4g128_amd/_build.py")
lib = ctypes.CDLL(LIB_PATH)

VARIANT_AUTO, VARIANT_DOT2, VARIANT_MFMA, VARIANT_STREAM, VARIANT_TILED, VARIANT_GEMM = 0, 1, 2, 3, 4, 5
FMT_Q4G128, FMT_NVFP4G16, FMT_BF16 = 0, 1, 2

_p, _i, _f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
lib.q4g128_gemv_variant.argtypes = [_p, _i, _i, _p, _p, _p, _i, _p, _i, _p]
lib.q4g128_gemm_variant.argtypes = [_p, _i, _i, _p, _p, _p, _i, _p, _i, _p]
lib.nvfp4g16_gemv_variant.argtypes = [_p, _i, _i, _p, _p, _f, _i, _p, _i, _p]
lib.bf16_gemv_variant.argtypes = [_p, _i, _i, _p, _i, _p, _i, _p]
lib.q4g128_gemv.argtypes = [_p, _i, _i, _p, _p, _p, _i, _p, _p]
lib.nvfp4g16_gemv.argtypes = [_p, _i, _i, _p, _p, _f, _i, _p, _p]
lib.bf16_gemv.argtypes = [_p, _i, _i, _p, _i, _p, _p]
lib.q4g128_dequant_f32.argtypes = [_p, _p, _p, _i, _i, _p, _p]
lib.nvfp4g16_dequant_f32.argtypes = [_p, _p, _f, _i, _i, _p, _p]
for _fn in ("q4g128_gemv_variant", "nvfp4g16_gemv_variant", "bf16_gemv_variant", "q4g128_gemv", "nvfp4g16_gemv",
            "bf16_gemv", "q4g128_dequant_f32", "nvfp4g16_dequant_f32"):
    getattr(lib, _fn).restype = ctypes.c_int
lib.q4gemv_variant_name.argtypes = [_i, _i, _i, _i, _i]
lib.q4gemv_variant_name.restype = ctypes.c_char_p
lib.q4gemv_strerror.argtypes = [_i]
lib.q4gemv_strerror.restype = ctypes.c_char_p
lib.q4gemv_time_next_launch.argtypes = [_p, _p]
lib.q4gemv_time_next_launch.restype = ctypes.c_int
lib.q4gemv_version.argtypes = []
lib.q4gemv_version.restype = ctypes.c_int
lib.q4gemv_stream_read.argtypes = [ctypes.POINTER(_p), ctypes.POINTER(ctypes.c_size_t), _i, _p, ctypes.c_size_t, _p]
lib.q4gemv_stream_read.restype = ctypes.c_int
lib.q4gemv_stream_read_sink_words.argtypes = [ctypes.POINTER(ctypes.c_size_t), _i]
lib.q4gemv_stream_read_sink_words.restype = ctypes.c_size_t


class Q4Task(ctypes.Structure):
    """Mirror of the C struct q4g128_task."""
    _fields_ = [("x", _p), ("qweight", _p), ("scale", _p), ("minv", _p), ("y", _p), ("N", _i), ("K", _i)]


lib.q4g128_gemv_grouped.argtypes = [ctypes.POINTER(Q4Task), _i, _i, _i, _p]
lib.q4g128_gemv_grouped.restype = ctypes.c_int
lib.q4g128_gemv_grouped_ws.argtypes = [ctypes.POINTER(Q4Task), _i, _i, _i, _p, ctypes.c_size_t, _p]
lib.q4g128_gemv_grouped_ws.restype = ctypes.c_int
lib.q4g128_workspace_bytes.argtypes = [ctypes.POINTER(Q4Task), _i, _i, ctypes.POINTER(ctypes.c_size_t)]
lib.q4g128_gemv_grouped_noalloc.argtypes = [ctypes.POINTER(Q4Task), _i, _i, _i, _p]
lib.q4g128_gemv_grouped_noalloc.restype = ctypes.c_int
NOALLOC_SCRATCH_BYTES = 8 << 20
lib.q4g128_workspace_bytes.restype = ctypes.c_int


class NvTask(ctypes.Structure):
    """Mirror of the C struct nvfp4g16_task."""
    _fields_ = [("x", _p), ("qweight", _p), ("scale_e4m3", _p), ("global_scale", _f), ("y", _p), ("N", _i), ("K", _i)]


class BfTask(ctypes.Structure):
    """Mirror of the C struct bf16_task."""
    _fields_ = [("x", _p), ("w", _p), ("y", _p), ("N", _i), ("K", _i)]


for _name, _T in (("nvfp4g16", NvTask), ("bf16", BfTask)):
    getattr(lib, f"{_name}_gemv_grouped_ws").argtypes = [ctypes.POINTER(_T), _i, _i, _i, _p, ctypes.c_size_t, _p]
    getattr(lib, f"{_name}_gemv_grouped_ws").restype = ctypes.c_int
    getattr(lib, f"{_name}_workspace_bytes").argtypes = [ctypes.POINTER(_T), _i, _i, ctypes.POINTER(ctypes.c_size_t)]
    getattr(lib, f"{_name}_workspace_bytes").restype = ctypes.c_int


class FusedTask(ctypes.Structure):
    _fields_ = [("x", _p), ("up", _p), ("qweight", _p), ("scale", _p), ("minv", _p), ("residual", _p), ("y", _p),
                ("N", _i), ("K", _i)]


lib.q4g128_gemv_fused.argtypes = [ctypes.POINTER(FusedTask), _i, _i, _p, ctypes.c_size_t, _p]
lib.q4g128_gemv_fused.restype = ctypes.c_int
lib.q4g128_fused_workspace_bytes.argtypes = [ctypes.POINTER(FusedTask), _i, _i, ctypes.POINTER(ctypes.c_size_t)]
lib.q4g128_fused_workspace_bytes.restype = ctypes.c_int


class MixedTask(ctypes.Structure):
    _fields_ = [("format", _i), ("x", _p), ("weight", _p), ("scale", _p), ("minv", _p), ("global_scale", _f), ("y", _p),
                ("N", _i), ("K", _i)]


lib.q4gemv_grouped_mixed.argtypes = [ctypes.POINTER(MixedTask), _i, _i, _p, ctypes.c_size_t, _p]
lib.q4gemv_grouped_mixed.restype = ctypes.c_int
lib.q4gemv_mixed_workspace_bytes.argtypes = [ctypes.POINTER(MixedTask), _i, _i, ctypes.POINTER(ctypes.c_size_t)]
lib.q4gemv_mixed_workspace_bytes.restype = ctypes.c_int
lib.q4g128_gemm.argtypes = [_p, _i, _i, _p, _p, _p, _i, _p, _p]
lib.q4g128_gemm.restype = ctypes.c_int
lib.q4_sample_topk.argtypes = [_p, _i, _i, _f, _i, _p, _p, _p, _p, _p]
lib.q4_sample_topk.restype = ctypes.c_int
lib.bf16_head_sample.argtypes = [_p, _i, _i, _p, _i, _p, _f, _i, _p, _p, _p, _p, _p]
lib.bf16_head_sample.restype = ctypes.c_int
lib.bf16_head_sample_ws.argtypes = [_p, _i, _i, _p, _i, _p, _f, _i, _p, _p, _p, _p, _p, ctypes.c_size_t, _p]
lib.bf16_head_sample_ws.restype = ctypes.c_int
lib.bf16_head_sample_workspace_bytes.argtypes = [_i, _i, _i, _i]
lib.bf16_head_sample_workspace_bytes.restype = ctypes.c_size_t


class Q4GemvError(ValueError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"q4gemv status {status}: {strerror(status)}")


def strerror(status: int) -> str:
    return lib.q4gemv_strerror(int(status)).decode()


def variant_name(fmt: int, variant: int, M: int, N: int, K: int) -> str:
    return lib.q4gemv_variant_name(fmt, variant, M, N, K).decode()


def _check(t: torch.Tensor, name: str, dtypes, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _out(out, shape, dtype, like):
    if out is None:
        return torch.empty(shape, dtype=dtype, device=like.device)
    _check(out, "out", (dtype,), len(shape))
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {tuple(shape)}")
    return out


def _raise(rc: int):
    if rc != 0:
        raise Q4GemvError(rc)


_U16 = (torch.bfloat16, torch.int16)
_F16 = (torch.float16, torch.int16)
_U8 = (torch.uint8,)
_E4M3 = (torch.uint8, torch.float8_e4m3fn)


def q4g128_gemv(x, qweight, scale, minv, out=None, variant: int = VARIANT_AUTO):
    """y[M, N] = x[M, K] . W^T, W int4 g128 min/max (qweight uint8 [N, K/2],
    scale/min fp16 [N, K/128])."""
    _check(x, "x", _U16, 2); _check(qweight, "qweight", _U8, 2)
    _check(scale, "scale", _F16, 2); _check(minv, "min", _F16, 2)
    M, K = x.shape
    N = qweight.shape[0]
    if qweight.shape[1] * 2 != K or tuple(scale.shape) != (N, K // 128) or tuple(minv.shape) != (N, K // 128):
        raise ValueError("inconsistent shapes")
    y = _out(out, (M, N), torch.bfloat16, x)
    _raise(lib.q4g128_gemv_variant(x.data_ptr(), M, K, qweight.data_ptr(), scale.data_ptr(), minv.data_ptr(), N,
                                   y.data_ptr(), int(variant), _stream(x)))
    return y


def _task_array(items):
    items = list(items)
    if not 1 <= len(items) <= 8:
        raise ValueError("1..8 tasks per call")
    arr = (Q4Task * len(items))()
    outs = []
    M = None
    for i, (x, qweight, scale, minv, out) in enumerate(items):
        _check(x, "x", _U16, 2); _check(qweight, "qweight", _U8, 2)
        _check(scale, "scale", _F16, 2); _check(minv, "min", _F16, 2)
        m, K = x.shape
        N = qweight.shape[0]
        if M is None:
            M = m
        if m != M:
            raise ValueError("all tasks must share the batch size M")
        if qweight.shape[1] * 2 != K or tuple(scale.shape) != (N, K // 128) or tuple(minv.shape) != (N, K // 128):
            raise ValueError(f"task {i}: inconsistent shapes")
        y = _out(out, (M, N), torch.bfloat16, x)
        outs.append(y)
        arr[i] = Q4Task(x.data_ptr(), qweight.data_ptr(), scale.data_ptr(), minv.data_ptr(), y.data_ptr(), N, K)
    return items, arr, outs, M


def q4g128_gemv_grouped(items, variant: int = VARIANT_AUTO, workspace=None):
    """Several independent int4 g128 GEMVs with one batch size, launched
    together.  items: sequence of (x, qweight, scale, min, out-or-None).
    workspace: optional uint8 device tensor of at least
    q4g128_workspace_bytes(items) bytes, zero-filled before its first use and
    reusable afterwards without clearing (lets large batches split K).
    Returns the list of outputs."""
    items, arr, outs, M = _task_array(items)
    st = _stream(items[0][0])
    if workspace is None:
        _raise(lib.q4g128_gemv_grouped(arr, len(items), M, int(variant), st))
    else:
        if workspace.device != items[0][0].device or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 tensor on the activations' device")
        _raise(lib.q4g128_gemv_grouped_ws(arr, len(items), M, int(variant), workspace.data_ptr(), workspace.numel(), st))
    return outs


def q4g128_gemv_grouped_noalloc(items, variant: int = VARIANT_AUTO):
    """q4g128_gemv_grouped with the library's built-in split-K scratch instead
    of a workspace (q4g128_gemv_grouped_noalloc in the C header: nothing is
    allocated; calls on one GPU must not overlap in time).  items as for
    q4g128_gemv_grouped.  Returns the list of outputs."""
    items, arr, outs, M = _task_array(items)
    _raise(lib.q4g128_gemv_grouped_noalloc(arr, len(items), M, int(variant), _stream(items[0][0])))
    return outs


def q4g128_workspace_bytes(items) -> int:
    """Bytes of zero-filled workspace q4g128_gemv_grouped may use for these
    tasks (0: it never splits them)."""
    items, arr, _, M = _task_array(items)
    n = ctypes.c_size_t(0)
    _raise(lib.q4g128_workspace_bytes(arr, len(items), M, ctypes.byref(n)))
    return int(n.value)


def nvfp4g16_gemv(x, qweight, scale_e4m3, global_scale: float, out=None, variant: int = VARIANT_AUTO):
    """y[M, N] = x . W^T, W NVFP4 (qweight uint8 [N, K/2] E2M1, scale_e4m3
    [N, K/16], global_scale fp32 multiplier)."""
    _check(x, "x", _U16, 2); _check(qweight, "qweight", _U8, 2); _check(scale_e4m3, "scale_e4m3", _E4M3, 2)
    M, K = x.shape
    N = qweight.shape[0]
    if qweight.shape[1] * 2 != K or tuple(scale_e4m3.shape) != (N, K // 16):
        raise ValueError("inconsistent shapes")
    y = _out(out, (M, N), torch.bfloat16, x)
    _raise(lib.nvfp4g16_gemv_variant(x.data_ptr(), M, K, qweight.data_ptr(), scale_e4m3.data_ptr(), float(global_scale), N,
                                     y.data_ptr(), int(variant), _stream(x)))
    return y


def _nv_task_array(items):
    items = list(items)
    if not 1 <= len(items) <= 8:
        raise ValueError("1..8 tasks per call")
    arr = (NvTask * len(items))()
    outs, M = [], None
    for i, (x, qweight, scale_e4m3, global_scale, out) in enumerate(items):
        _check(x, "x", _U16, 2); _check(qweight, "qweight", _U8, 2); _check(scale_e4m3, "scale_e4m3", _E4M3, 2)
        m, K = x.shape
        N = qweight.shape[0]
        M = m if M is None else M
        if m != M:
            raise ValueError("all tasks must share the batch size M")
        if qweight.shape[1] * 2 != K or tuple(scale_e4m3.shape) != (N, K // 16):
            raise ValueError(f"task {i}: inconsistent shapes")
        y = _out(out, (M, N), torch.bfloat16, x)
        outs.append(y)
        arr[i] = NvTask(x.data_ptr(), qweight.data_ptr(), scale_e4m3.data_ptr(), float(global_scale), y.data_ptr(), N, K)
    return items, arr, outs, M


def _bf_task_array(items):
    items = list(items)
    if not 1 <= len(items) <= 8:
        raise ValueError("1..8 tasks per call")
    arr = (BfTask * len(items))()
    outs, M = [], None
    for i, (x, w, out) in enumerate(items):
        _check(x, "x", _U16, 2); _check(w, "w", _U16, 2)
        m, K = x.shape
        N = w.shape[0]
        M = m if M is None else M
        if m != M:
            raise ValueError("all tasks must share the batch size M")
        if w.shape[1] != K:
            raise ValueError(f"task {i}: inconsistent shapes")
        y = _out(out, (M, N), torch.bfloat16, x)
        outs.append(y)
        arr[i] = BfTask(x.data_ptr(), w.data_ptr(), y.data_ptr(), N, K)
    return items, arr, outs, M


def _grouped(fn, items, arr, M, variant, workspace):
    st = _stream(items[0][0])
    if workspace is None:
        _raise(fn(arr, len(items), M, int(variant), None, 0, st))
    else:
        if workspace.device != items[0][0].device or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 tensor on the activations' device")
        _raise(fn(arr, len(items), M, int(variant), workspace.data_ptr(), workspace.numel(), st))


def nvfp4g16_gemv_grouped(items, variant: int = VARIANT_AUTO, workspace=None):
    """Several independent NVFP4 GEMVs with one batch size, launched together.
    items: sequence of (x, qweight, scale_e4m3, global_scale, out-or-None);
    workspace as for q4g128_gemv_grouped.  Returns the list of outputs."""
    items, arr, outs, M = _nv_task_array(items)
    _grouped(lib.nvfp4g16_gemv_grouped_ws, items, arr, M, variant, workspace)
    return outs


def nvfp4g16_workspace_bytes(items) -> int:
    items, arr, _, M = _nv_task_array(items)
    n = ctypes.c_size_t(0)
    _raise(lib.nvfp4g16_workspace_bytes(arr, len(items), M, ctypes.byref(n)))
    return int(n.value)


def bf16_gemv_grouped(items, variant: int = VARIANT_AUTO, workspace=None):
    """Several independent BF16 GEMVs with one batch size, launched together.
    items: sequence of (x, w, out-or-None); workspace as for
    q4g128_gemv_grouped.  Returns the list of outputs."""
    items, arr, outs, M = _bf_task_array(items)
    _grouped(lib.bf16_gemv_grouped_ws, items, arr, M, variant, workspace)
    return outs


def bf16_workspace_bytes(items) -> int:
    items, arr, _, M = _bf_task_array(items)
    n = ctypes.c_size_t(0)
    _raise(lib.bf16_workspace_bytes(arr, len(items), M, ctypes.byref(n)))
    return int(n.value)


def bf16_gemv(x, w, out=None, variant: int = VARIANT_AUTO):
    """y[M, N] = x . W^T with W bf16 [N, K]."""
    _check(x, "x", _U16, 2); _check(w, "w", _U16, 2)
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("inconsistent shapes")
    y = _out(out, (M, N), torch.bfloat16, x)
    _raise(lib.bf16_gemv_variant(x.data_ptr(), M, K, w.data_ptr(), N, y.data_ptr(), int(variant), _stream(x)))
    return y


def q4g128_dequant_f32(qweight, scale, minv, out=None):
    _check(qweight, "qweight", _U8, 2); _check(scale, "scale", _F16, 2); _check(minv, "min", _F16, 2)
    N, half = qweight.shape
    K = 2 * half
    w = _out(out, (N, K), torch.float32, qweight)
    _raise(lib.q4g128_dequant_f32(qweight.data_ptr(), scale.data_ptr(), minv.data_ptr(), N, K, w.data_ptr(), _stream(qweight)))
    return w


def nvfp4g16_dequant_f32(qweight, scale_e4m3, global_scale: float, out=None):
    _check(qweight, "qweight", _U8, 2); _check(scale_e4m3, "scale_e4m3", _E4M3, 2)
    N, half = qweight.shape
    K = 2 * half
    w = _out(out, (N, K), torch.float32, qweight)
    _raise(lib.nvfp4g16_dequant_f32(qweight.data_ptr(), scale_e4m3.data_ptr(), float(global_scale), N, K, w.data_ptr(),
                                    _stream(qweight)))
    return w


def _read_args(tensors):
    n = len(tensors)
    ptrs = (_p * n)(*[t.data_ptr() for t in tensors])
    sizes = (ctypes.c_size_t * n)(*[t.numel() * t.element_size() for t in tensors])
    return ptrs, sizes, n


def stream_read_sink_words(tensors) -> int:
    """Sink words stream_read needs for these device tensors (0: invalid)."""
    _, sizes, n = _read_args(tensors)
    return int(lib.q4gemv_stream_read_sink_words(sizes, n))


def stream_read(tensors, sink):
    """Diagnostic plain read of the bytes of up to 32 contiguous device tensors
    in one launch (the reference a GEMV launch of the same bytes is compared
    with); one XOR word per wave lands in the int32 device tensor `sink`."""
    for t in tensors:
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("stream_read takes contiguous device tensors")
    ptrs, sizes, n = _read_args(tensors)
    _raise(lib.q4gemv_stream_read(ptrs, sizes, n, sink.data_ptr(), sink.numel(), _stream(sink)))
    return sink


def _fused_task_array(items):
    items = [dict(it) for it in items]
    if not 1 <= len(items) <= 8:
        raise ValueError("1..8 tasks per call")
    arr = (FusedTask * len(items))()
    outs, M = [], None
    for i, it in enumerate(items):
        x, qweight, scale, minv = it["x"], it["qweight"], it["scale"], it["min"]
        up, res, out = it.get("up"), it.get("residual"), it.get("out")
        _check(x, "x", _U16, 2); _check(qweight, "qweight", _U8, 2)
        _check(scale, "scale", _F16, 2); _check(minv, "min", _F16, 2)
        m, K = x.shape
        N = qweight.shape[0]
        M = m if M is None else M
        if m != M:
            raise ValueError("all tasks must share the batch size M")
        if qweight.shape[1] * 2 != K or tuple(scale.shape) != (N, K // 128) or tuple(minv.shape) != (N, K // 128):
            raise ValueError(f"task {i}: inconsistent shapes")
        if up is not None:
            _check(up, "up", _U16, 2)
            if tuple(up.shape) != (M, K):
                raise ValueError(f"task {i}: up must be [M, K]")
        if res is not None:
            _check(res, "residual", _U16, 2)
            if tuple(res.shape) != (M, N):
                raise ValueError(f"task {i}: residual must be [M, N]")
        y = _out(out, (M, N), torch.bfloat16, x)
        outs.append(y)
        arr[i] = FusedTask(x.data_ptr(), up.data_ptr() if up is not None else None, qweight.data_ptr(), scale.data_ptr(),
                           minv.data_ptr(), res.data_ptr() if res is not None else None, y.data_ptr(), N, K)
    return items, arr, outs, M


def q4g128_gemv_fused(items, workspace=None):
    """int4 g128 GEMVs with the decode step's elementwise neighbours fused
    (q4g128_gemv_fused in the C header).  items: sequence of dicts with keys
    x, qweight, scale, min and optionally up (activations become
    RN_bf16(silu(x) * up)), residual (added to the output before its
    rounding; may be the out tensor itself) and out.  workspace as for
    q4g128_gemv_grouped.  Returns the list of outputs."""
    items, arr, outs, M = _fused_task_array(items)
    st = _stream(items[0]["x"])
    if workspace is None:
        _raise(lib.q4g128_gemv_fused(arr, len(items), M, None, 0, st))
    else:
        if workspace.device != items[0]["x"].device or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 tensor on the activations' device")
        _raise(lib.q4g128_gemv_fused(arr, len(items), M, workspace.data_ptr(), workspace.numel(), st))
    return outs


def q4g128_fused_workspace_bytes(items) -> int:
    items, arr, _, M = _fused_task_array(items)
    n = ctypes.c_size_t(0)
    _raise(lib.q4g128_fused_workspace_bytes(arr, len(items), M, ctypes.byref(n)))
    return int(n.value)


def _sample_outputs(M, top_k, like, want_topk):
    tok = torch.empty(M, dtype=torch.int32, device=like.device)
    if not want_topk:
        return tok, None, None
    return (tok, torch.empty((M, top_k), dtype=torch.int32, device=like.device),
            torch.empty((M, top_k), dtype=torch.float32, device=like.device))


def sample_topk(logits, u, temperature: float = 0.8, top_k: int = 30, return_topk: bool = False):
    """Top-k sampling from BF16 logits [M, V] with the caller's uniforms u
    (fp32 [M], in [0, 1)): returns token int32 [M], and with return_topk also
    the top-k indices int32 [M, k] and probabilities fp32 [M, k]."""
    _check(logits, "logits", _U16, 2); _check(u, "u", (torch.float32,), 1)
    M, V = logits.shape
    if u.shape[0] != M:
        raise ValueError("u must hold one draw per batch row")
    tok, ti, tp = _sample_outputs(M, top_k, logits, return_topk)
    _raise(lib.q4_sample_topk(logits.data_ptr(), M, V, float(temperature), int(top_k), u.data_ptr(), tok.data_ptr(),
                              ti.data_ptr() if ti is not None else None, tp.data_ptr() if tp is not None else None,
                              _stream(logits)))
    return (tok, ti, tp) if return_topk else tok


def bf16_head_sample_workspace_bytes(M: int, N: int, K: int, top_k: int = 30) -> int:
    """Bytes of zero-filled workspace for the workspace head sampling (one
    launch at M = 1, the split sampler for a batch; 0 if it does not apply to
    this shape)."""
    return int(lib.bf16_head_sample_workspace_bytes(M, N, K, top_k))


def bf16_head_sample(x, w, u, temperature: float = 0.8, top_k: int = 30, logits=None, return_topk: bool = False,
                     workspace=None):
    """The BF16 head GEMV logits = x W^T followed by top-k sampling: two
    launches; with a zero-filled uint8 workspace of at least
    bf16_head_sample_workspace_bytes() (when that is nonzero),
    bf16_head_sample_ws in the C header -- one launch for one row, the split
    sampler for a batch.  Returns (token, logits) or (token, topk_index,
    topk_prob, logits) with return_topk."""
    _check(x, "x", _U16, 2); _check(w, "w", _U16, 2); _check(u, "u", (torch.float32,), 1)
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K or u.shape[0] != M:
        raise ValueError("inconsistent shapes")
    lg = _out(logits, (M, N), torch.bfloat16, x)
    tok, ti, tp = _sample_outputs(M, top_k, x, return_topk)
    ti_p = ti.data_ptr() if ti is not None else None
    tp_p = tp.data_ptr() if tp is not None else None
    if workspace is None:
        _raise(lib.bf16_head_sample(x.data_ptr(), M, K, w.data_ptr(), N, lg.data_ptr(), float(temperature), int(top_k), u.data_ptr(),
                                    tok.data_ptr(), ti_p, tp_p, _stream(x)))
    else:
        if workspace.device != x.device or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 tensor on the activations' device")
        _raise(lib.bf16_head_sample_ws(x.data_ptr(), M, K, w.data_ptr(), N, lg.data_ptr(), float(temperature), int(top_k),
                                       u.data_ptr(), tok.data_ptr(), ti_p, tp_p, workspace.data_ptr(), workspace.numel(), _stream(x)))
    return (tok, ti, tp, lg) if return_topk else (tok, lg)


def q4g128_gemm(x, qweight, scale, minv, out=None, variant: int = VARIANT_AUTO):
    """Prefill GEMM y[M, N] = x[M, K] . W^T for int4 g128 weights, any M
    (q4g128_gemm_variant in the C header: VARIANT_AUTO, VARIANT_TILED for the
    tiled decode kernel over batch chunks, VARIANT_GEMM for the large-tile
    prefill kernel)."""
    _check(x, "x", _U16, 2); _check(qweight, "qweight", _U8, 2)
    _check(scale, "scale", _F16, 2); _check(minv, "min", _F16, 2)
    M, K = x.shape
    N = qweight.shape[0]
    if qweight.shape[1] * 2 != K or tuple(scale.shape) != (N, K // 128) or tuple(minv.shape) != (N, K // 128):
        raise ValueError("inconsistent shapes")
    y = _out(out, (M, N), torch.bfloat16, x)
    _raise(lib.q4g128_gemm_variant(x.data_ptr(), M, K, qweight.data_ptr(), scale.data_ptr(), minv.data_ptr(), N, y.data_ptr(),
                                   variant, _stream(x)))
    return y


def _mixed_task_array(items):
    """Tagged task tuples -> (MixedTask array, outputs, M):
      ("q4g128", x, qweight, scale, min, out), ("nvfp4g16", x, qweight,
      scale_e4m3, global_scale, out), ("bf16", x, w, out); out may be None."""
    items = list(items)
    if not 1 <= len(items) <= 8:
        raise ValueError("1..8 tasks per call")
    arr = (MixedTask * len(items))()
    outs, M = [], None
    for i, it in enumerate(items):
        kind = it[0]
        if kind == "q4g128":
            _, x, qw, sc, mn, out = it
            _check(qw, "qweight", _U8, 2); _check(sc, "scale", _F16, 2); _check(mn, "min", _F16, 2)
            fmt, w, G, N, K = FMT_Q4G128, qw, 0.0, qw.shape[0], qw.shape[1] * 2
            if tuple(sc.shape) != (N, K // 128) or tuple(mn.shape) != (N, K // 128):
                raise ValueError(f"task {i}: inconsistent shapes")
        elif kind == "nvfp4g16":
            _, x, qw, sc, G, out = it
            _check(qw, "qweight", _U8, 2); _check(sc, "scale_e4m3", _E4M3, 2)
            fmt, w, mn, N, K = FMT_NVFP4G16, qw, None, qw.shape[0], qw.shape[1] * 2
            if tuple(sc.shape) != (N, K // 16):
                raise ValueError(f"task {i}: inconsistent shapes")
        elif kind == "bf16":
            _, x, w, out = it
            _check(w, "w", _U16, 2)
            fmt, sc, mn, G, (N, K) = FMT_BF16, None, None, 0.0, w.shape
        else:
            raise ValueError(f"unknown task kind {kind!r} (q4g128, nvfp4g16, bf16)")
        _check(x, "x", _U16, 2)
        if x.shape[1] != K:
            raise ValueError(f"task {i}: x has K = {x.shape[1]}, the weights {K}")
        M = x.shape[0] if M is None else M
        if x.shape[0] != M:
            raise ValueError("all tasks must share the batch size M")
        y = _out(out, (M, N), torch.bfloat16, x)
        outs.append(y)
        arr[i] = MixedTask(fmt, x.data_ptr(), w.data_ptr(), sc.data_ptr() if sc is not None else None,
                           mn.data_ptr() if mn is not None else None, float(G), y.data_ptr(), N, K)
    return items, arr, outs, M


def gemv_grouped_mixed(items, workspace=None):
    """Independent GEMVs of mixed weight formats with one batch size, in one
    launch where the streaming kernel takes them all (M <= 4), else one
    grouped launch per format (q4gemv_grouped_mixed in the C header).
    Returns the list of outputs."""
    items, arr, outs, M = _mixed_task_array(items)
    st = _stream(items[0][1])
    if workspace is None:
        _raise(lib.q4gemv_grouped_mixed(arr, len(items), M, None, 0, st))
    else:
        if workspace.device != items[0][1].device or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 tensor on the activations' device")
        _raise(lib.q4gemv_grouped_mixed(arr, len(items), M, workspace.data_ptr(), workspace.numel(), st))
    return outs


def mixed_workspace_bytes(items) -> int:
    items, arr, _, M = _mixed_task_array(items)
    n = ctypes.c_size_t(0)
    _raise(lib.q4gemv_mixed_workspace_bytes(arr, len(items), M, ctypes.byref(n)))
    return int(n.value)
