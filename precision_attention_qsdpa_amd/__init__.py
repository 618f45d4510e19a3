"""Python binding of ``libqsdpa.so``: quantized scaled-dot-product attention
for MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/qsdpa.h``.  PyTorch supplies
device memory and the stream.  There is no fallback: if the library is not
built, ``load()`` raises.
"""
from __future__ import annotations

import ctypes
import math
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libqsdpa.so")

QSDPA_OK = 0
QSDPA_ERR_INVALID_ARG = -1
QSDPA_ERR_UNSUPPORTED = -2
QSDPA_ERR_ALIGNMENT = -3
QSDPA_ERR_WORKSPACE_TOO_SMALL = -4
QSDPA_ERR_ALIAS = -5
QSDPA_ERR_HIP = -6
QSDPA_ERR_SCRATCH_TOO_SMALL = -7
QSDPA_SCRATCH_BYTES = 96 << 20   # the static scratch array of qsdpa_forward_noalloc, per GPU
MAX_SEQ_LEN = 1 << 22             # QSDPA_MAX_SEQ_LEN: longest sequence accepted
MAX_BH = 65535                    # QSDPA_MAX_BH: largest B*H accepted
MAX_ELEMS = 1 << 36               # QSDPA_MAX_ELEMS: largest B*H*round_up(N, 128)*128
QSDPA_QK_FP8_E4M3 = 0
QSDPA_QK_FP4_E2M1 = 1
QSDPA_QK_MXFP4_E2M1 = 2
QK_FORMATS = {"fp8": QSDPA_QK_FP8_E4M3, "fp4": QSDPA_QK_FP4_E2M1, "mxfp4": QSDPA_QK_MXFP4_E2M1}
HEAD_DIM = 128

EXPORTS = ("qsdpa_abi_version", "qsdpa_status_string", "qsdpa_validate_params", "qsdpa_workspace_bytes",
           "qsdpa_workspace_layout", "qsdpa_quantize", "qsdpa_attention", "qsdpa_forward",
           "qsdpa_forward_noalloc", "qsdpa_attention_bf16q", "qsdpa_vc_workspace_bytes",
           "qsdpa_vc_workspace_layout", "qsdpa_forward_vc")


class QsdpaParams(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_q", ctypes.c_int32), ("block_k", ctypes.c_int32),
                ("qk_format", ctypes.c_int32), ("fp4_group", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float)]


ABI_VERSION = 7   # QSDPA_ABI_VERSION of include/qsdpa.h (the layout struct below)


class QsdpaLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in ("q_codes", "q_scales", "k_codes", "k_scales", "k_mean",
                                               "v_codes", "v_scales", "v_amax", "stats", "k_expanded",
                                               "total")] + \
               [(n, ctypes.c_int32) for n in ("n_pad", "code_row_bytes", "q_scale_count", "k_scale_count",
                                              "stats_splits")] + [("reserved", ctypes.c_int32 * 3)]


class QsdpaVcLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in ("token_error", "selected", "partials", "total")] + \
               [(n, ctypes.c_int32) for n in ("count", "count_pad", "chunks", "chunk_keys")]


VC_RHO = 0.005   # the fraction of tokens VC-Attention FP8 corrects on the VisualGen page


class QsdpaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


_LIB = None


def load() -> ctypes.CDLL:
    """Load the in-tree library (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m precision_attention_qsdpa_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(QsdpaParams)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.qsdpa_abi_version.restype = ctypes.c_int
    lib.qsdpa_abi_version.argtypes = []
    lib.qsdpa_status_string.restype = ctypes.c_char_p
    lib.qsdpa_status_string.argtypes = [ctypes.c_int]
    lib.qsdpa_validate_params.restype = ctypes.c_int
    lib.qsdpa_validate_params.argtypes = [P]
    lib.qsdpa_workspace_bytes.restype = sz
    lib.qsdpa_workspace_bytes.argtypes = [P]
    lib.qsdpa_workspace_layout.restype = ctypes.c_int
    lib.qsdpa_workspace_layout.argtypes = [P, ctypes.POINTER(QsdpaLayout)]
    lib.qsdpa_quantize.restype = ctypes.c_int
    lib.qsdpa_quantize.argtypes = [P, vp, vp, vp, vp, sz, vp]
    lib.qsdpa_attention.restype = ctypes.c_int
    lib.qsdpa_attention.argtypes = [P, vp, sz, vp, vp]
    lib.qsdpa_forward.restype = ctypes.c_int
    lib.qsdpa_forward.argtypes = [P, vp, vp, vp, vp, vp, sz, vp]
    lib.qsdpa_vc_workspace_bytes.restype = sz
    lib.qsdpa_vc_workspace_bytes.argtypes = [P, ctypes.c_float]
    lib.qsdpa_vc_workspace_layout.restype = ctypes.c_int
    lib.qsdpa_vc_workspace_layout.argtypes = [P, ctypes.c_float, ctypes.POINTER(QsdpaVcLayout)]
    lib.qsdpa_forward_vc.restype = ctypes.c_int
    lib.qsdpa_forward_vc.argtypes = [P, ctypes.c_float, vp, vp, vp, vp, vp, sz, vp]
    lib.qsdpa_attention_bf16q.restype = ctypes.c_int
    lib.qsdpa_attention_bf16q.argtypes = [P, vp, vp, sz, vp, vp]
    lib.qsdpa_forward_noalloc.restype = ctypes.c_int
    lib.qsdpa_forward_noalloc.argtypes = [P, vp, vp, vp, vp, vp]
    if lib.qsdpa_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{LIB_PATH} has ABI version {lib.qsdpa_abi_version()}, this binding expects "
                           f"{ABI_VERSION}: rebuild it with `python -m precision_attention_qsdpa_amd.build`")
    _LIB = lib
    return lib


def status_string(status: int) -> str:
    return load().qsdpa_status_string(int(status)).decode()


def make_params(batch: int, heads: int, seq_len: int, *, fmt: str = "fp8", block_q: int = 128,
                block_k: int = 64, softmax_scale: float | None = None, head_dim: int = HEAD_DIM,
                fp4_group: int = 16) -> QsdpaParams:
    if fmt not in QK_FORMATS:
        raise ValueError(f"fmt must be one of {sorted(QK_FORMATS)}, not {fmt!r}")
    tau = 1.0 / math.sqrt(head_dim) if softmax_scale is None else softmax_scale
    return QsdpaParams(batch, heads, seq_len, head_dim, block_q, block_k, QK_FORMATS[fmt], fp4_group, tau)


def qsdpa_validate_params(params: QsdpaParams) -> int:
    return load().qsdpa_validate_params(ctypes.byref(params))


def qsdpa_workspace_bytes(params: QsdpaParams) -> int:
    return int(load().qsdpa_workspace_bytes(ctypes.byref(params)))


def qsdpa_workspace_layout(params: QsdpaParams) -> QsdpaLayout:
    out = QsdpaLayout()
    st = load().qsdpa_workspace_layout(ctypes.byref(params), ctypes.byref(out))
    if st != QSDPA_OK:
        raise QsdpaError(st, "qsdpa_workspace_layout")
    return out


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _torch_stream(stream, device):
    """The torch stream object the kernels will run on (the current stream of
    ``device`` if None; a raw hipStream_t handle is wrapped)."""
    import torch
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def _check_qkv(t, params: QsdpaParams, name: str, device):
    import torch
    shape = (params.batch, params.heads, params.seq_len, params.head_dim)
    if (t.dtype != torch.bfloat16 or not t.is_cuda or t.device != device or not t.is_contiguous()
            or tuple(t.shape) != shape):
        raise ValueError(f"{name} must be a contiguous CUDA bfloat16 tensor of shape {shape} on {device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


def _check_workspace(ws, device):
    """The workspace must be contiguous device memory on the tensors' GPU:
    the library takes its address as a device pointer."""
    if not ws.is_cuda or ws.device != device or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous CUDA tensor on {device}, got one on {ws.device}"
                         f"{'' if ws.is_contiguous() else ' (not contiguous)'}")


def empty_workspace(params: QsdpaParams, device=None):
    """A uint8 device tensor big enough for ``params`` (256-byte aligned)."""
    import torch
    n = qsdpa_workspace_bytes(params)
    if n == 0:
        raise QsdpaError(qsdpa_validate_params(params), "qsdpa_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def qsdpa_quantize(q, k, v, workspace, params: QsdpaParams, stream=None) -> None:
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check_qkv(t, params, n, q.device)
    _check_workspace(workspace, q.device)
    import torch
    with torch.cuda.device(q.device):
        st = load().qsdpa_quantize(ctypes.byref(params), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                   workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                   _stream(stream))
    if st != QSDPA_OK:
        raise QsdpaError(st, "qsdpa_quantize")


def qsdpa_attention(workspace, out, params: QsdpaParams, stream=None) -> None:
    _check_qkv(out, params, "out", out.device)
    _check_workspace(workspace, out.device)
    import torch
    with torch.cuda.device(out.device):
        st = load().qsdpa_attention(ctypes.byref(params), workspace.data_ptr(),
                                    workspace.numel() * workspace.element_size(), out.data_ptr(), _stream(stream))
    if st != QSDPA_OK:
        raise QsdpaError(st, "qsdpa_attention")


def qsdpa_attention_bf16q(q, workspace, out, params: QsdpaParams, stream=None) -> None:
    """Attention of bf16 ``q`` on the K/V codes in ``workspace`` (filled by
    qsdpa_quantize or qsdpa_forward with the same params); the kernel
    quantizes Q itself."""
    _check_qkv(q, params, "q", q.device)
    _check_qkv(out, params, "out", q.device)
    _check_workspace(workspace, q.device)
    import torch
    with torch.cuda.device(q.device):
        st = load().qsdpa_attention_bf16q(ctypes.byref(params), q.data_ptr(), workspace.data_ptr(),
                                          workspace.numel() * workspace.element_size(), out.data_ptr(),
                                          _stream(stream))
    if st != QSDPA_OK:
        raise QsdpaError(st, "qsdpa_attention_bf16q")


def qsdpa_forward(q, k, v, out=None, workspace=None, *, fmt: str = "fp8", block_q: int = 128,
                  block_k: int = 64, softmax_scale: float | None = None, params: QsdpaParams | None = None,
                  stream=None):
    """O = quantized SDPA(q, k, v) for bf16 [B, H, N, 128] CUDA tensors."""
    import torch
    if params is None:
        B, H, N, Dh = q.shape
        params = make_params(B, H, N, fmt=fmt, block_q=block_q, block_k=block_k,
                             softmax_scale=softmax_scale, head_dim=Dh)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check_qkv(t, params, n, q.device)
    if out is None or workspace is None:
        # allocated on the stream the kernels run on: the caching allocator
        # then hands these blocks to no other stream's work while the kernels
        # may still use them (the workspace is freed when this call returns)
        with torch.cuda.stream(_torch_stream(stream, q.device)):
            if out is None:
                out = torch.empty_like(q)
            if workspace is None:
                workspace = empty_workspace(params, q.device)
    _check_qkv(out, params, "out", q.device)
    _check_workspace(workspace, q.device)
    with torch.cuda.device(q.device):   # the library launches on the current device
        st = load().qsdpa_forward(ctypes.byref(params), q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                  workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                  _stream(stream))
    if st != QSDPA_OK:
        raise QsdpaError(st, "qsdpa_forward")
    return out


def qsdpa_forward_noalloc(q, k, v, out, params: QsdpaParams, stream=None):
    """qsdpa_forward with the workspace in the library's static scratch array
    (no allocation by the library or here; ``out`` is the caller's).  Calls
    whose work may overlap on one GPU share that array and must not overlap."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _check_qkv(t, params, n, q.device)
    import torch
    with torch.cuda.device(q.device):
        st = load().qsdpa_forward_noalloc(ctypes.byref(params), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                          out.data_ptr(), _stream(stream))
    if st != QSDPA_OK:
        raise QsdpaError(st, "qsdpa_forward_noalloc")
    return out


def qsdpa_vc_workspace_bytes(params: QsdpaParams, rho: float = VC_RHO) -> int:
    return int(load().qsdpa_vc_workspace_bytes(ctypes.byref(params), ctypes.c_float(rho)))


def qsdpa_vc_workspace_layout(params: QsdpaParams, rho: float = VC_RHO) -> QsdpaVcLayout:
    out = QsdpaVcLayout()
    st = load().qsdpa_vc_workspace_layout(ctypes.byref(params), ctypes.c_float(rho), ctypes.byref(out))
    if st != QSDPA_OK:
        raise QsdpaError(st, "qsdpa_vc_workspace_layout")
    return out


def qsdpa_forward_vc(q, k, v, out=None, workspace=None, *, rho: float = VC_RHO, params: QsdpaParams | None = None,
                     stream=None):
    """FP8 quantized SDPA with the selective correction: the ceil(rho N)
    query tokens of each (b, h) with the largest own quantization error get
    unquantized attention.  Returns (out, workspace); the workspace holds the
    tokens' errors and the corrected rows (qsdpa_vc_workspace_layout)."""
    import torch
    if params is None:
        B, H, N, Dh = q.shape
        params = make_params(B, H, N, fmt="fp8", head_dim=Dh)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check_qkv(t, params, n, q.device)
    nbytes = qsdpa_vc_workspace_bytes(params, rho)
    if nbytes == 0:
        qsdpa_vc_workspace_layout(params, rho)   # raises with the reason
    if out is None or workspace is None:
        with torch.cuda.stream(_torch_stream(stream, q.device)):
            if out is None:
                out = torch.empty_like(q)
            if workspace is None:
                workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    _check_qkv(out, params, "out", q.device)
    _check_workspace(workspace, q.device)
    with torch.cuda.device(q.device):
        st = load().qsdpa_forward_vc(ctypes.byref(params), ctypes.c_float(rho), q.data_ptr(), k.data_ptr(),
                                     v.data_ptr(), out.data_ptr(), workspace.data_ptr(),
                                     workspace.numel() * workspace.element_size(), _stream(stream))
    if st != QSDPA_OK:
        raise QsdpaError(st, "qsdpa_forward_vc")
    return out, workspace
