"""Python binding of the qgemm C ABI (include/qgemm.h): argument marshalling only.

Every step of the GEMM runs in the HIP library ``libqgemm.so`` built next to this file;
torch serves only for device memory and the current stream.  Importing this package
fails loudly when the library has not been built.

Quick use::

    import weight_only_quantized_qgemm_amd as q
    p = q.problem(M, N, K, "int4", group_size=128)
    codes, scales, alpha = q.quantize(p, w_nk)          # host, numpy
    wpk, spk = q.pack(p, codes, scales)                  # host, numpy
    ... upload with torch, then q.run(p, A, wpk_dev, spk_dev, alpha_dev, out, ws)
"""
import ctypes
import os

import numpy as np
# torch first: it loads its HIP runtime (soname libamdhip64.so.7), and the library below then
# binds to that same runtime instance, so torch's pointers and streams are valid in it.  Loading
# the library first would bring in a second runtime that cannot share the device with torch's.
import torch  # noqa: F401

_PKG = os.path.dirname(os.path.abspath(__file__))
# QGEMM_LIB_PATH selects another build of the same library (the CPU tests load the
# host-sanitizer build this way); by default the in-tree libqgemm.so.
LIB_PATH = os.environ.get("QGEMM_LIB_PATH") or os.path.join(_PKG, "libqgemm.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python -m weight_only_quantized_qgemm_amd._build` (hipcc, gfx950)")
_lib = ctypes.CDLL(LIB_PATH)

# ----------------------------------------------------------------------------- enums
OK, ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED, ERR_MISALIGNED, ERR_WORKSPACE_TOO_SMALL, ERR_HIP = range(6)
DT_F16, DT_BF16, DT_F32, DT_INT4, DT_FP8_E4M3, DT_FP4_E2M1, DT_INT2, DT_NF4 = range(8)
SCALE_GROUP_F16, SCALE_TENSOR_F32, SCALE_BLOCK16_E4M3, SCALE_GROUP_F16_LUT16 = range(4)
KERNEL_AUTO, KERNEL_DECODE, KERNEL_PREFILL, KERNEL_PREFILL_STREAMK, KERNEL_PREFILL_TRANSFORM = range(5)


class Problem(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("a_dtype", ctypes.c_int32), ("w_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("scale_layout", ctypes.c_int32),
                ("kernel_hint", ctypes.c_int32), ("split_k_hint", ctypes.c_int32),
                ("tile_hint", ctypes.c_int32)]


assert ctypes.sizeof(Problem) == 56

_P = ctypes.POINTER(Problem)
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_lib.qgemm_quantize.argtypes = [_P, _vp, _vp, _vp, ctypes.POINTER(ctypes.c_float)]
_lib.qgemm_pack.argtypes = [_P, _vp, _vp, _vp, ctypes.POINTER(_sz), _vp, ctypes.POINTER(_sz)]
_lib.qgemm_workspace_bytes.argtypes = [_P, ctypes.POINTER(_sz)]
_lib.qgemm_run.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.qgemm_run_bias.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.qgemm_run_no_alloc.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.qgemm_plan_describe.argtypes = [_P, ctypes.c_char_p, _sz]
_lib.qgemm_status_string.argtypes = [ctypes.c_int]
_lib.qgemm_status_string.restype = ctypes.c_char_p
_lib.qgemm_last_error.argtypes = []
_lib.qgemm_last_error.restype = ctypes.c_char_p
_lib.qgemm_version.restype = ctypes.c_int32
NO_ALLOC_SCRATCH_BYTES = (32 << 20) + (64 << 10)    # QGEMM_NO_ALLOC_SCRATCH_BYTES of include/qgemm.h
for _f in ("qgemm_quantize", "qgemm_pack", "qgemm_workspace_bytes", "qgemm_run", "qgemm_run_bias",
           "qgemm_run_no_alloc", "qgemm_plan_describe"):
    getattr(_lib, _f).restype = ctypes.c_int

lib = _lib


class QgemmError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        self.detail = detail
        super().__init__(f"{_lib.qgemm_status_string(status).decode()}: {detail}")


def _check(status):
    if status != OK:
        raise QgemmError(status, _lib.qgemm_last_error().decode())


# ----------------------------------------------------------------------------- problems
_FORMATS = {
    "int4": (DT_F16, DT_INT4, SCALE_GROUP_F16, DT_F16),
    "fp8": (DT_BF16, DT_FP8_E4M3, SCALE_TENSOR_F32, DT_BF16),
    "fp8h": (DT_F16, DT_FP8_E4M3, SCALE_TENSOR_F32, DT_F16),      # FP8 weights, fp16 activations
    "fp4": (DT_BF16, DT_FP4_E2M1, SCALE_BLOCK16_E4M3, DT_BF16),
    "int2": (DT_F16, DT_INT2, SCALE_GROUP_F16, DT_F16),             # W2A16
    "nf4": (DT_F16, DT_NF4, SCALE_GROUP_F16_LUT16, DT_F16),         # 4-bit code-book index
}
GROUP_SCALED = ("int4", "int2", "nf4")


def problem(M, N, K, fmt, group_size=None, out_dtype=None, kernel_hint=KERNEL_AUTO, split_k_hint=0,
            tile_hint=0):
    """Problem descriptor for one of the formats 'int4', 'int2', 'nf4', 'fp8' (bf16
    activations), 'fp8h' (fp16 activations), 'fp4'."""
    a, w, sl, o = _FORMATS[fmt]
    if group_size is None:
        group_size = {"int4": 128, "int2": 128, "nf4": 128, "fp8": 0, "fp8h": 0, "fp4": 16}[fmt]
    if out_dtype is not None:
        o = out_dtype
    return Problem(M, N, K, a, w, o, group_size, sl, kernel_hint, split_k_hint, tile_hint)


def fmt_of(p):
    if p.w_dtype == DT_FP8_E4M3:
        return "fp8h" if p.a_dtype == DT_F16 else "fp8"
    return {DT_INT4: "int4", DT_INT2: "int2", DT_NF4: "nf4", DT_FP4_E2M1: "fp4"}[p.w_dtype]


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    return x.data_ptr()          # torch tensor


# ----------------------------------------------------------------------------- host calls
def quantize(p, w_nk):
    """fp32 [N, K] weights -> (canonical codes uint8, canonical scales or None, alpha).

    NF4 scales are one flat fp16 (uint16) array: the 16 code-book entries, then [K/G][N]."""
    w = np.ascontiguousarray(w_nk, dtype=np.float32)
    N, K = int(p.N), int(p.K)
    assert w.shape == (N, K)
    f = fmt_of(p)
    codes = np.empty((N, K) if f in ("fp8", "fp8h") else (N, K // 4) if f == "int2" else (N, K // 2), np.uint8)
    scales = None
    if f in ("int4", "int2"):
        scales = np.empty((K // p.group_size, N), np.uint16)
    elif f == "nf4":
        scales = np.empty(16 + (K // p.group_size) * N, np.uint16)
    elif f == "fp4":
        scales = np.empty((N, K // 16), np.uint8)
    alpha = ctypes.c_float(0.0)
    _check(_lib.qgemm_quantize(ctypes.byref(p), w.ctypes.data, codes.ctypes.data,
                               None if scales is None else scales.ctypes.data, ctypes.byref(alpha)))
    return codes, scales, float(alpha.value)


def packed_sizes(p):
    wb, sb = _sz(0), _sz(0)
    _check(_lib.qgemm_pack(ctypes.byref(p), None, None, None, ctypes.byref(wb), None, ctypes.byref(sb)))
    return wb.value, sb.value


def pack(p, codes, scales):
    """Canonical codes / scales (host) -> packed device-layout bytes (host numpy uint8)."""
    wsz, ssz = packed_sizes(p)
    codes = np.ascontiguousarray(codes)
    wpk = np.empty(wsz, np.uint8)
    spk = np.empty(max(ssz, 0), np.uint8)
    if scales is not None:
        scales = np.ascontiguousarray(scales)
    wb, sb = _sz(wsz), _sz(ssz)
    _check(_lib.qgemm_pack(ctypes.byref(p), codes.ctypes.data,
                           None if scales is None else scales.ctypes.data,
                           wpk.ctypes.data, ctypes.byref(wb),
                           spk.ctypes.data if ssz else None, ctypes.byref(sb)))
    return wpk, (spk if ssz else None)


def workspace_bytes(p):
    n = _sz(0)
    _check(_lib.qgemm_workspace_bytes(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def plan_describe(p):
    """The launch qgemm_run would make for this problem, as one line of text."""
    buf = ctypes.create_string_buffer(512)
    _check(_lib.qgemm_plan_describe(ctypes.byref(p), buf, 512))
    return buf.value.decode()


def plan_fields(p):
    """plan_describe as a dict: {"kernel": ..., key: value, ...} (values as text)."""
    head, *rest = plan_describe(p).split()
    return {"kernel": head, **dict(f.split("=", 1) for f in rest)}


# ----------------------------------------------------------------------------- device calls
def alloc_workspace(p, device="cuda"):
    """A zero-filled workspace of the size qgemm_workspace_bytes reports (or None)."""
    import torch
    n = workspace_bytes(p)
    if n == 0:
        return None
    return torch.zeros(n, dtype=torch.uint8, device=device)


def run(p, A, w_packed, s_packed, alpha, out, workspace=None, stream=None, bias=None):
    """Enqueue out = A . dequant(W) (* alpha) (+ bias) on `stream` (default: torch's current
    stream); qgemm_run, or qgemm_run_bias when a bias is given."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if bias is None:
        _check(_lib.qgemm_run(ctypes.byref(p), _ptr(A), _ptr(w_packed), _ptr(s_packed), _ptr(alpha),
                              _ptr(out), _ptr(workspace), ws_bytes, stream))
    else:
        _check(_lib.qgemm_run_bias(ctypes.byref(p), _ptr(A), _ptr(w_packed), _ptr(s_packed), _ptr(alpha),
                                   _ptr(bias), _ptr(out), _ptr(workspace), ws_bytes, stream))


def run_no_alloc(p, A, w_packed, s_packed, alpha, out, stream=None, bias=None):
    """qgemm_run_no_alloc: as run(), with the library's static per-GPU scratch as the split-K
    workspace (no workspace argument; nothing is allocated).  Calls that overlap in time on
    one GPU race."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    _check(_lib.qgemm_run_no_alloc(ctypes.byref(p), _ptr(A), _ptr(w_packed), _ptr(s_packed), _ptr(alpha),
                                   _ptr(bias), _ptr(out), stream))


def run_raw(p, A, w_packed, s_packed, alpha, out, workspace, workspace_bytes_, stream):
    """qgemm_run on raw integer addresses; returns the status (no exception)."""
    return _lib.qgemm_run(ctypes.byref(p), A, w_packed, s_packed, alpha, out, workspace,
                          workspace_bytes_, stream)


def run_bias_raw(p, A, w_packed, s_packed, alpha, bias, out, workspace, workspace_bytes_, stream):
    """qgemm_run_bias on raw integer addresses; returns the status (no exception)."""
    return _lib.qgemm_run_bias(ctypes.byref(p), A, w_packed, s_packed, alpha, bias, out, workspace,
                               workspace_bytes_, stream)


def last_error():
    return _lib.qgemm_last_error().decode()


def status_string(st):
    return _lib.qgemm_status_string(st).decode()


def version():
    return int(_lib.qgemm_version())
