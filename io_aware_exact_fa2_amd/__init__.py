"""FA2-order exact attention (forward and backward) for AMD MI355X (gfx950).

Thin Python binding of the C ABI in ``include/fa.h`` (``libfa.so``, built from
``csrc/`` by ``build.py``). It only marshals arguments: every step of the
computation runs in the HIP kernel. PyTorch supplies device buffers and the
stream. There is no fallback: if the library is missing, every call raises.

Functions with the C names (``fa_fwd``, ``fa_fwd_fp16``, ``fa_fwd_ex``,
``fa_bwd``, ``fa_bwd_fp16``, ``fa_fwd_supported``, ``fa_strerror``,
``fa_last_hip_error``, ``fa_version``) map 1:1 onto the C entry points;
``forward`` and ``backward`` are the tensor-level conveniences that allocate the
outputs and raise ``FAError`` on a nonzero status.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "FA_OK", "FA_ERR_NULL", "FA_ERR_SHAPE", "FA_ERR_UNSUPPORTED", "FA_ERR_ALIAS",
    "FA_ERR_ALIGN", "FA_ERR_HIP", "FA_DTYPE_BF16", "FA_DTYPE_FP16", "FAError",
    "library_path", "lib", "fa_fwd", "fa_fwd_fp16", "fa_fwd_ex", "fa_fwd_supported",
    "fa_bwd", "fa_bwd_fp16", "backward", "fa_fwd_splitkv", "fa_fwd_splitkv_workspace_size",
    "fa_fwd_fa1", "fa_fwd_fa1_workspace_size", "forward_splitkv", "forward_fa1", "FA_MAX_SPLITS",
    "fa_fwd_fp8", "forward_fp8", "fa_device_supported", "fa_device_info", "fa_fwd_splitkv_static",
    "FA_ERR_SCRATCH", "FA_STATIC_SCRATCH_BYTES",
    "fa_strerror", "FA_DEFAULT_RESCALE_LOG2", "FA_MAX_RESCALE_LOG2",
    "fa_last_hip_error", "fa_version", "forward", "EXPORTS",
]

FA_OK = 0
FA_ERR_NULL = -1
FA_ERR_SHAPE = -2
FA_ERR_UNSUPPORTED = -3
FA_ERR_ALIAS = -4
FA_ERR_ALIGN = -5
FA_ERR_HIP = -6
FA_ERR_SCRATCH = -7
FA_DTYPE_BF16 = 0
FA_DTYPE_FP16 = 1

EXPORTS = ("fa_fwd", "fa_fwd_fp16", "fa_fwd_ex", "fa_fwd_fp8", "fa_fwd_splitkv", "fa_fwd_splitkv_workspace_size",
           "fa_fwd_splitkv_static",
           "fa_fwd_fa1", "fa_fwd_fa1_workspace_size", "fa_bwd", "fa_bwd_fp16", "fa_fwd_supported",
           "fa_device_supported", "fa_device_info",
           "fa_strerror", "fa_last_hip_error", "fa_version")
FA_MAX_SPLITS = 64
FA_STATIC_SCRATCH_BYTES = 64 << 20
FA_DEFAULT_RESCALE_LOG2 = 8.0
FA_MAX_RESCALE_LOG2 = 15.0

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, where: str = "fa_fwd"):
        self.status = status
        msg = f"{where} failed: {status} ({fa_strerror(status)})"
        if status == FA_ERR_HIP:
            msg += f", hipError {fa_last_hip_error()}"
        super().__init__(msg)


def library_path() -> str:
    return os.environ.get("FA355_LIB", os.path.join(_HERE, "libfa.so"))


def lib() -> ctypes.CDLL:
    """Load libfa.so once. Raises ImportError when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m io_aware_exact_fa2_amd.build` "
            "(there is no CPU fallback)")
    L = ctypes.CDLL(path)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    for name in ("fa_fwd", "fa_fwd_fp16"):
        fn = getattr(L, name)
        fn.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
        fn.restype = i
    L.fa_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, f, vp]
    L.fa_fwd_ex.restype = i
    sz = ctypes.c_size_t
    L.fa_fwd_fp8.argtypes = [vp, vp, vp, f, f, f, vp, vp, i, i, i, i, f, i, vp]
    L.fa_fwd_fp8.restype = i
    L.fa_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, i, i, vp]
    L.fa_fwd_splitkv.restype = i
    L.fa_fwd_splitkv_static.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, i, vp]
    L.fa_fwd_splitkv_static.restype = i
    L.fa_fwd_splitkv_workspace_size.argtypes = [i, i, i, i, i]
    L.fa_fwd_splitkv_workspace_size.restype = sz
    L.fa_fwd_fa1.argtypes = [vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, i, vp]
    L.fa_fwd_fa1.restype = i
    L.fa_fwd_fa1_workspace_size.argtypes = [i, i, i, i]
    L.fa_fwd_fa1_workspace_size.restype = sz
    for name in ("fa_bwd", "fa_bwd_fp16"):
        fn = getattr(L, name)
        fn.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
        fn.restype = i
    L.fa_device_supported.argtypes = [i]
    L.fa_device_supported.restype = i
    L.fa_device_info.argtypes = [i, ctypes.POINTER(i), ctypes.POINTER(i)]
    L.fa_device_info.restype = i
    L.fa_fwd_supported.argtypes = [i, i, i]
    L.fa_fwd_supported.restype = i
    L.fa_strerror.argtypes = [i]
    L.fa_strerror.restype = ctypes.c_char_p
    L.fa_last_hip_error.argtypes = []
    L.fa_last_hip_error.restype = i
    L.fa_version.argtypes = []
    L.fa_version.restype = ctypes.c_char_p
    _lib = L
    return L


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is None or isinstance(s, int):
        return s
    return s.cuda_stream


def fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, stream=None) -> int:
    """C ``fa_fwd`` (bfloat16). Pointers may be tensors or raw integers."""
    return lib().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                        float(scale), int(causal), _stream(stream))


def fa_fwd_fp16(q, k, v, o, lse, B, H, N, d, scale, causal, stream=None) -> int:
    """C ``fa_fwd_fp16`` (float16). Pointers may be tensors or raw integers."""
    return lib().fa_fwd_fp16(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                             float(scale), int(causal), _stream(stream))


def fa_fwd_ex(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, rescale_log2,
              stream=None) -> int:
    """C ``fa_fwd_ex``: explicit dtype code and rescale threshold (log2 units)."""
    return lib().fa_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                           float(scale), int(causal), int(dtype), float(rescale_log2),
                           _stream(stream))


def fa_fwd_fp8(q, k, v, q_scale, k_scale, v_scale, o, lse, B, H, N, d, scale, causal,
               stream=None) -> int:
    """C ``fa_fwd_fp8``: E4M3 codes with per-tensor scales in, bfloat16 O out."""
    return lib().fa_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), float(q_scale), float(k_scale),
                            float(v_scale), _ptr(o), _ptr(lse), B, H, N, d, float(scale),
                            int(causal), _stream(stream))


def fa_fwd_splitkv(q, k, v, o, lse, workspace, workspace_bytes, B, H, N, d, scale, causal,
                   n_splits, dtype, stream=None) -> int:
    """C ``fa_fwd_splitkv``: key ranges in separate workgroups, then an LSE merge."""
    return lib().fa_fwd_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(workspace),
                                int(workspace_bytes), B, H, N, d, float(scale), int(causal),
                                int(n_splits), int(dtype), _stream(stream))


def fa_fwd_splitkv_static(q, k, v, o, lse, B, H, N, d, scale, causal, n_splits, dtype,
                          stream=None) -> int:
    """C ``fa_fwd_splitkv_static``: ``fa_fwd_splitkv`` on the library's own device scratch
    (no workspace argument; nothing allocated)."""
    return lib().fa_fwd_splitkv_static(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N,
                                       d, float(scale), int(causal), int(n_splits), int(dtype),
                                       _stream(stream))


def fa_fwd_splitkv_workspace_size(B, H, N, d, n_splits) -> int:
    return lib().fa_fwd_splitkv_workspace_size(B, H, N, d, n_splits)


def fa_fwd_fa1(q, k, v, o, lse, workspace, workspace_bytes, B, H, N, d, scale, causal, dtype,
               stream=None) -> int:
    """C ``fa_fwd_fa1``: the FA1 loop order (ablation)."""
    return lib().fa_fwd_fa1(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(workspace),
                            int(workspace_bytes), B, H, N, d, float(scale), int(causal),
                            int(dtype), _stream(stream))


def fa_fwd_fa1_workspace_size(B, H, N, d) -> int:
    return lib().fa_fwd_fa1_workspace_size(B, H, N, d)


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal, stream=None) -> int:
    """C ``fa_bwd`` (bfloat16). Pointers may be tensors or raw integers."""
    return lib().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                        _ptr(dk), _ptr(dv), B, H, N, d, float(scale), int(causal),
                        _stream(stream))


def fa_bwd_fp16(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal,
                stream=None) -> int:
    """C ``fa_bwd_fp16`` (float16). Pointers may be tensors or raw integers."""
    return lib().fa_bwd_fp16(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                             _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, float(scale),
                             int(causal), _stream(stream))


def fa_device_supported(device: int = 0) -> int:
    """C ``fa_device_supported``: 1 for a gfx950 device, else 0."""
    return lib().fa_device_supported(int(device))


def fa_device_info(device: int = 0) -> tuple[int, int]:
    """C ``fa_device_info``: (compute-unit count, peak engine clock in kHz) of a device;
    raises FAError if the runtime cannot report them."""
    cus, khz = ctypes.c_int(0), ctypes.c_int(0)
    st = lib().fa_device_info(int(device), ctypes.byref(cus), ctypes.byref(khz))
    if st != FA_OK:
        raise FAError(st, "fa_device_info")
    return cus.value, khz.value


def fa_fwd_supported(d: int, dtype: int, causal: int) -> int:
    return lib().fa_fwd_supported(d, dtype, causal)


def fa_strerror(status: int) -> str:
    return lib().fa_strerror(status).decode()


def fa_last_hip_error() -> int:
    return lib().fa_last_hip_error()


def fa_version() -> str:
    return lib().fa_version().decode()


def forward(q, k, v, causal: bool = False, scale: float | None = None,
            out=None, lse=None, stream=None, rescale_log2: float | None = None):
    """O, L for contiguous [B, H, N, d] bf16/fp16 CUDA tensors q, k, v.

    scale defaults to 1/sqrt(d). O has q's dtype; L is float32 [B, H, N]. The
    launch goes on ``stream`` (default: the current stream of q's device).
    rescale_log2 selects the running-max rescale threshold (``fa_fwd_ex``); None
    uses the library default (``fa_fwd`` / ``fa_fwd_fp16``).
    """
    import torch

    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("q, k, v must share dtype bfloat16 or float16")
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must have the same [B, H, N, d] shape")
    if not (q.is_cuda and k.device == q.device and v.device == q.device):
        raise ValueError("q, k, v must be on the same GPU")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        if rescale_log2 is None:
            fn = fa_fwd if q.dtype == torch.bfloat16 else fa_fwd_fp16
            st = fn(q, k, v, out, lse, B, H, N, d, scale, causal, stream)
            name = fn.__name__
        else:
            dt = FA_DTYPE_BF16 if q.dtype == torch.bfloat16 else FA_DTYPE_FP16
            st = fa_fwd_ex(q, k, v, out, lse, B, H, N, d, scale, causal, dt, rescale_log2,
                           stream)
            name = "fa_fwd_ex"
    if st != FA_OK:
        raise FAError(st, name)
    return out, lse


def backward(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None,
             dq=None, dk=None, dv=None, stream=None):
    """dQ, dK, dV for contiguous [B, H, N, d] bf16/fp16 CUDA tensors (d = 64 or 128).

    o and lse are ``forward``'s outputs for the same q, k, v, causal and scale; dout
    is the gradient of the loss with respect to o. The gradients have q's dtype.
    """
    import torch

    ts = (q, k, v, o, dout)
    if any(t.dtype != q.dtype for t in ts) or q.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("q, k, v, o, dout must share dtype bfloat16 or float16")
    if q.dim() != 4 or any(t.shape != q.shape for t in ts):
        raise ValueError("q, k, v, o, dout must have the same [B, H, N, d] shape")
    if not q.is_cuda or any(t.device != q.device for t in (*ts, lse)):
        raise ValueError("all tensors must be on the same GPU")
    if not all(t.is_contiguous() for t in (*ts, lse)):
        raise ValueError("all tensors must be contiguous")
    B, H, N, d = q.shape
    if lse.shape != (B, H, N) or lse.dtype != torch.float32:
        raise ValueError("lse must be a float32 [B, H, N] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    outs = []
    for t in (dq, dk, dv):
        if t is None:
            t = torch.empty_like(q)
        elif t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous():
            raise ValueError("dq, dk, dv must be contiguous tensors like q")
        outs.append(t)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    fn = fa_bwd if q.dtype == torch.bfloat16 else fa_bwd_fp16
    with torch.cuda.device(q.device):
        st = fn(q, k, v, o, lse, dout, *outs, B, H, N, d, scale, causal, stream)
    if st != FA_OK:
        raise FAError(st, fn.__name__)
    return tuple(outs)


def _workspace_call(name, size_fn, call_fn, q, k, v, causal, scale, stream, extra, workspace):
    import torch

    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("q, k, v must share dtype bfloat16 or float16")
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must have the same [B, H, N, d] shape")
    if not (q.is_cuda and k.device == q.device and v.device == q.device):
        raise ValueError("q, k, v must be on the same GPU")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = size_fn(B, H, N, d, *extra)
    if need == 0:
        raise FAError(FA_ERR_SHAPE if d in (64, 128) else FA_ERR_UNSUPPORTED, name)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    dt = FA_DTYPE_BF16 if q.dtype == torch.bfloat16 else FA_DTYPE_FP16
    with torch.cuda.device(q.device):
        st = call_fn(q, k, v, out, lse, workspace, workspace.numel() * workspace.element_size(),
                     B, H, N, d, scale, causal, *extra, dt, stream)
    if st != FA_OK:
        raise FAError(st, name)
    return out, lse


def forward_splitkv(q, k, v, causal: bool = False, scale: float | None = None,
                    n_splits: int = 4, stream=None, workspace=None):
    """O, L by the split-KV path (``fa_fwd_splitkv``); d = 64 or 128. The workspace
    (a uint8 CUDA tensor of at least ``fa_fwd_splitkv_workspace_size`` bytes) is
    allocated here unless given."""
    return _workspace_call("fa_fwd_splitkv", fa_fwd_splitkv_workspace_size, fa_fwd_splitkv,
                           q, k, v, causal, scale, stream, (int(n_splits),), workspace)


def forward_fa1(q, k, v, causal: bool = False, scale: float | None = None, stream=None,
                workspace=None):
    """O, L in the FA1 loop order (``fa_fwd_fa1``, an ablation); d = 64 or 128."""
    return _workspace_call("fa_fwd_fa1", fa_fwd_fa1_workspace_size, fa_fwd_fa1,
                           q, k, v, causal, scale, stream, (), workspace)


def forward_fp8(q8, k8, v8, q_scale: float, k_scale: float, v_scale: float,
                causal: bool = False, scale: float | None = None, stream=None):
    """O (bfloat16), L for contiguous [B, H, N, d] uint8 (or float8_e4m3fn) CUDA tensors of
    E4M3 codes with per-tensor scales (``fa_fwd_fp8``); d = 64 or 128."""
    import torch

    ts = (q8, k8, v8)
    if any(t.element_size() != 1 for t in ts):
        raise ValueError("q8, k8, v8 must be 1-byte tensors of E4M3 codes")
    if q8.dim() != 4 or any(t.shape != q8.shape for t in ts):
        raise ValueError("q8, k8, v8 must have the same [B, H, N, d] shape")
    if not q8.is_cuda or any(t.device != q8.device for t in ts):
        raise ValueError("q8, k8, v8 must be on the same GPU")
    if not all(t.is_contiguous() for t in ts):
        raise ValueError("q8, k8, v8 must be contiguous")
    B, H, N, d = q8.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    if stream is None:
        stream = torch.cuda.current_stream(q8.device)
    with torch.cuda.device(q8.device):
        st = fa_fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, out, lse, B, H, N, d, scale,
                        causal, stream)
    if st != FA_OK:
        raise FAError(st, "fa_fwd_fp8")
    return out, lse
