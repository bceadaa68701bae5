"""ctypes binding of libfa.so (include/fa.h), with the same names as the C ABI.

Argument marshalling only: every step of the attention forward/backward runs
in the library's HIP kernels.  The library is loaded on first use from this
package directory; if it is missing the call raises (there is no fallback).

Low level: fa_abi_version, fa_status_string, fa_fwd, fa_bwd_preprocess,
fa_bwd_workspace_bytes, fa_bwd, fa_bwd_noalloc, fa_debug_dropout_mask take FaParams /
FaTensor structures and raw device pointers, exactly like the C functions.
High level: forward(...) and backward(...) take [B, H, N, d] torch tensors
on the GPU (queries and keys may differ in N), forward_varlen(...) and
backward_varlen(...) packed [total, H, d] tensors with cumulative sequence
offsets; they allocate the outputs with torch and enqueue on torch's
current stream (or on the stream passed as `stream=`, on which they then
also allocate).
"""

import ctypes
import math
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libfa.so")

FA_DTYPE_F32 = 0
FA_DTYPE_BF16 = 1
FA_DTYPE_F16 = 2
ABI_VERSION = 3

STATUS_NAMES = {
    0: "FA_SUCCESS",
    1: "FA_ERR_INVALID_VALUE",
    2: "FA_ERR_NOT_SUPPORTED",
    3: "FA_ERR_MISALIGNED",
    4: "FA_ERR_LAUNCH_FAILED",
    5: "FA_ERR_HIP",
    6: "FA_ERR_TOO_LARGE",
}

STATIC_WORKSPACE_BYTES = 128 * 1024 * 1024  # FA_STATIC_WORKSPACE_BYTES

EXPORTS = ("fa_abi_version", "fa_last_hip_error", "fa_status_string", "fa_fwd", "fa_bwd_preprocess",
           "fa_bwd_workspace_bytes", "fa_bwd", "fa_bwd_noalloc", "fa_debug_dropout_mask")


class FaTensor(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("stride_b", ctypes.c_int64),
                ("stride_h", ctypes.c_int64), ("stride_n", ctypes.c_int64)]


class FaParams(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("seqlen", ctypes.c_int32), ("seqlen_k", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("sm_scale", ctypes.c_float),
                ("causal", ctypes.c_int32), ("window_left", ctypes.c_int32),
                ("window_right", ctypes.c_int32), ("deterministic", ctypes.c_int32),
                ("dropout_p", ctypes.c_double), ("seed", ctypes.c_uint64),
                ("offset", ctypes.c_uint64), ("cu_seqlens_q", ctypes.c_void_p),
                ("cu_seqlens_k", ctypes.c_void_p)]


class FaError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        hip = fa_last_hip_error() if status in (4, 5) else 0
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({fa_status_string(status)})"
                         + (f", hipError_t {hip}" if hip else ""))


_lib = None


def load_library(path=LIB_PATH):
    """Load libfa.so once and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m flashattention_backward_pass_fa_amd.build`")
    # torch ships its own HIP runtime under the same soname.  Loading torch
    # first makes libfa.so bind to that copy, so one runtime (and one set of
    # streams and allocations) serves both; loading libfa.so first would pull
    # in a second runtime whose handles torch's streams are not.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P, T, vp, fp = ctypes.POINTER(FaParams), FaTensor, ctypes.c_void_p, ctypes.c_void_p
    lib.fa_abi_version.restype = ctypes.c_int
    lib.fa_abi_version.argtypes = []
    lib.fa_last_hip_error.restype = ctypes.c_int
    lib.fa_last_hip_error.argtypes = []
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_status_string.argtypes = [ctypes.c_int]
    lib.fa_fwd.restype = ctypes.c_int
    lib.fa_fwd.argtypes = [P, T, T, T, T, fp, vp]
    lib.fa_bwd_preprocess.restype = ctypes.c_int
    lib.fa_bwd_preprocess.argtypes = [P, T, T, fp, fp, vp]
    lib.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_bwd_workspace_bytes.argtypes = [P]
    lib.fa_bwd.restype = ctypes.c_int
    lib.fa_bwd.argtypes = [P, T, T, T, T, fp, fp, T, T, T, fp, vp]
    lib.fa_bwd_noalloc.restype = ctypes.c_int
    lib.fa_bwd_noalloc.argtypes = [P, T, T, T, T, fp, fp, T, T, T, vp]
    lib.fa_debug_dropout_mask.restype = ctypes.c_int
    lib.fa_debug_dropout_mask.argtypes = [P, ctypes.c_int32, ctypes.c_int32, vp, vp]
    if lib.fa_abi_version() != ABI_VERSION:
        raise RuntimeError(f"libfa.so ABI {lib.fa_abi_version()} != binding ABI {ABI_VERSION}")
    _lib = lib
    return lib


# ----------------------------------------------------------- the C ABI, 1:1

def fa_abi_version():
    return load_library().fa_abi_version()


def fa_last_hip_error():
    return load_library().fa_last_hip_error()


def fa_status_string(status):
    return load_library().fa_status_string(int(status)).decode()


def fa_fwd(params, q, k, v, o, lse, stream):
    return load_library().fa_fwd(ctypes.byref(params), q, k, v, o, lse, stream)


def fa_bwd_preprocess(params, o, dout, delta, dq_acc, stream):
    return load_library().fa_bwd_preprocess(ctypes.byref(params), o, dout, delta, dq_acc, stream)


def fa_bwd_workspace_bytes(params):
    return load_library().fa_bwd_workspace_bytes(ctypes.byref(params))


def fa_bwd(params, q, k, v, dout, lse, delta, dq, dk, dv, dq_acc, stream):
    return load_library().fa_bwd(ctypes.byref(params), q, k, v, dout, lse, delta, dq, dk, dv,
                                 dq_acc, stream)


def fa_bwd_noalloc(params, q, k, v, dout, lse, delta, dq, dk, dv, stream):
    return load_library().fa_bwd_noalloc(ctypes.byref(params), q, k, v, dout, lse, delta, dq, dk, dv,
                                         stream)


def fa_debug_dropout_mask(params, b, h, mask, stream):
    return load_library().fa_debug_dropout_mask(ctypes.byref(params), b, h, mask, stream)


# ------------------------------------------------------ torch-facing helpers

def make_params(shape, dtype, sm_scale=None, causal=False, window=(-1, -1), dropout_p=0.0,
                seed=0, offset=0, deterministic=False, seqlen_k=None, cu_seqlens_q=None,
                cu_seqlens_k=None):
    """FaParams for a [B, H, Nq, d] problem with Nk = seqlen_k keys (default Nq).

    sm_scale None means 1/sqrt(d).  cu_seqlens_q / cu_seqlens_k: device
    addresses (ints) of the varlen offset arrays, or None.
    """
    bsz, nh, n, d = shape
    return FaParams(dtype=dtype, batch=bsz, heads=nh, seqlen=n,
                    seqlen_k=n if seqlen_k is None else int(seqlen_k), head_dim=d,
                    sm_scale=(1.0 / math.sqrt(d)) if sm_scale is None else float(sm_scale),
                    causal=1 if causal else 0, window_left=int(window[0]),
                    window_right=int(window[1]), deterministic=1 if deterministic else 0,
                    dropout_p=float(dropout_p), seed=int(seed), offset=int(offset),
                    cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k)


def tensor_arg(t):
    """FaTensor view of a [B, H, N, d] tensor or a packed [total, H, d] one.

    The d-stride must be 1.  A packed tensor gets batch stride 0 (varlen
    mode ignores it).
    """
    if t.dim() == 3 and t.stride(2) == 1:
        return FaTensor(t.data_ptr(), 0, t.stride(1), t.stride(0))
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("expected a [B, H, N, d] or [total, H, d] tensor with unit stride on d")
    return FaTensor(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return FA_DTYPE_BF16
    if t.dtype == torch.float16:
        return FA_DTYPE_F16
    if t.dtype == torch.float32:
        return FA_DTYPE_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _validate(q, k, v, o=None, dout=None, lse=None, lse_shape=None, varlen=False):
    """Host-side checks of the helpers' tensors, before anything is launched.

    The C ABI receives raw pointers and cannot see sizes, so a tensor that
    disagrees with q's shape would be read or written out of bounds there.
    """
    want_dim = 3 if varlen else 4
    if q.dim() != want_dim or k.dim() != want_dim or v.dim() != want_dim:
        raise ValueError(f"q, k, v must be {want_dim}-D ({'[total, H, d]' if varlen else '[B, H, N, d]'})")
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout)):
        if t is None:
            continue
        if t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must have q's dtype and device")
    if k.shape != v.shape:
        raise ValueError(f"k {tuple(k.shape)} and v {tuple(v.shape)} must have the same shape")
    same = (1, 2) if varlen else (0, 1, 3)  # heads and d; batch too when not packed
    if any(q.shape[i] != k.shape[i] for i in same):
        raise ValueError(f"q {tuple(q.shape)} and k {tuple(k.shape)} disagree")
    for name, t in (("o", o), ("dout", dout)):
        if t is not None and t.shape != q.shape:
            raise ValueError(f"{name} {tuple(t.shape)} must have q's shape {tuple(q.shape)}")
    if lse is not None:
        _check_f32(lse, "lse", lse_shape, q.device)
    if not q.is_cuda:
        raise ValueError("the tensors must be on a GPU")


def _check_f32(t, name, shape, device):
    import torch
    if t.dtype != torch.float32 or t.device != device or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be a contiguous float32 tensor of shape {tuple(shape)} on {device}")


def _stream(stream, device):
    """The caller's stream, else the current stream of the tensors' device
    (which need not be the current device); it must belong to that device."""
    import torch
    s = torch.cuda.current_stream(device) if stream is None else stream
    if s.device != torch.device(device) and torch.device(device).index is not None:
        raise ValueError(f"stream is on {s.device}, the tensors on {device}")
    return ctypes.c_void_p(s.cuda_stream)


def _alloc_on(stream):
    """Context in which the helpers allocate: the caller's stream when one
    is given, so that the caching allocator ties every output and temporary
    to the stream the kernels run on (a temporary freed on return is then
    reused only by later work on that same stream)."""
    import contextlib
    import torch
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _check(status, where):
    if status != 0:
        raise FaError(status, where)


def forward(q, k, v, sm_scale=None, causal=False, window=(-1, -1), dropout_p=0.0, seed=0,
            offset=0, stream=None):
    """O (dtype of q) and L (fp32 [B, H, N]) of softmax attention on q, k, v."""
    import torch
    _validate(q, k, v)
    params = make_params(tuple(q.shape), _dtype_code(q), sm_scale, causal, window, dropout_p,
                         seed, offset, seqlen_k=k.shape[2])
    with _alloc_on(stream):
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):  # the library launches on the current device
        _check(fa_fwd(params, tensor_arg(q), tensor_arg(k), tensor_arg(v), tensor_arg(o),
                      ctypes.c_void_p(lse.data_ptr()), _stream(stream, q.device)), "fa_fwd")
    return o, lse


def backward(q, k, v, o, dout, lse, sm_scale=None, causal=False, window=(-1, -1), dropout_p=0.0,
             seed=0, offset=0, deterministic=False, stream=None, workspace=None, delta=None):
    """dQ, dK, dV (dtype of q): the pre-pass for D, then the backward kernels.

    workspace: optional fp32 tensor of at least fa_bwd_workspace_bytes bytes
    (atomic mode); allocated here when None.  delta: optional fp32 [B, H, N]
    output for D.  Returns (dq, dk, dv, delta).
    """
    _validate(q, k, v, o, dout, lse, tuple(q.shape[:3]))
    params = make_params(tuple(q.shape), _dtype_code(q), sm_scale, causal, window, dropout_p,
                         seed, offset, deterministic, seqlen_k=k.shape[2])
    return _backward(params, q, k, v, o, dout, lse, q.shape[:3], stream, workspace, delta)


def _backward(params, q, k, v, o, dout, lse, delta_shape, stream, workspace, delta):
    import torch
    st = _stream(stream, q.device)
    ws_bytes = fa_bwd_workspace_bytes(params)
    if delta is not None:
        _check_f32(delta, "delta", delta_shape, q.device)
    if ws_bytes and workspace is not None and (
            workspace.dtype != torch.float32 or workspace.device != q.device
            or not workspace.is_contiguous() or workspace.numel() * 4 < ws_bytes):
        raise ValueError(f"workspace must be a contiguous float32 tensor of at least {ws_bytes} bytes on {q.device}")
    with _alloc_on(stream):
        if delta is None:
            delta = torch.empty(delta_shape, dtype=torch.float32, device=q.device)
        if ws_bytes and workspace is None:
            workspace = torch.empty(ws_bytes // 4, dtype=torch.float32, device=q.device)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if ws_bytes else ctypes.c_void_p(0)
    with torch.cuda.device(q.device):
        _check(fa_bwd_preprocess(params, tensor_arg(o), tensor_arg(dout),
                                 ctypes.c_void_p(delta.data_ptr()), ws_ptr, st), "fa_bwd_preprocess")
        _check(fa_bwd(params, tensor_arg(q), tensor_arg(k), tensor_arg(v), tensor_arg(dout),
                      ctypes.c_void_p(lse.data_ptr()), ctypes.c_void_p(delta.data_ptr()),
                      tensor_arg(dq), tensor_arg(dk), tensor_arg(dv), ws_ptr, st), "fa_bwd")
    return dq, dk, dv, delta


def _varlen_params(q, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, sm_scale, causal,
                   window, dropout_p, seed, offset, deterministic=False):
    import torch
    for cu in (cu_seqlens_q, cu_seqlens_k):
        if cu.dtype != torch.int32 or cu.dim() != 1 or not cu.is_contiguous() or cu.device != q.device:
            raise ValueError("cu_seqlens must be contiguous int32 vectors on the tensors' device")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k need the same B + 1 >= 2 entries")
    bsz = cu_seqlens_q.numel() - 1
    return make_params((bsz, q.shape[1], int(max_seqlen_q), q.shape[2]), _dtype_code(q), sm_scale,
                       causal, window, dropout_p, seed, offset, deterministic,
                       seqlen_k=int(max_seqlen_k), cu_seqlens_q=cu_seqlens_q.data_ptr(),
                       cu_seqlens_k=cu_seqlens_k.data_ptr())


def forward_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, sm_scale=None,
                   causal=False, window=(-1, -1), dropout_p=0.0, seed=0, offset=0, stream=None):
    """Packed variable-length forward.

    q: [total_q, H, d]; k, v: [total_k, H, d]; sequence b owns rows
    cu_seqlens_q[b]:cu_seqlens_q[b+1] of q (int32 device tensors of B + 1
    entries).  Returns O [total_q, H, d] and L [B, H, max_seqlen_q] (entries
    past a sequence's length are not written).
    """
    import torch
    _validate(q, k, v, varlen=True)
    params = _varlen_params(q, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, sm_scale,
                            causal, window, dropout_p, seed, offset)
    with _alloc_on(stream):
        o = torch.empty_like(q)
        lse = torch.empty((params.batch, q.shape[1], params.seqlen), dtype=torch.float32,
                          device=q.device)
    with torch.cuda.device(q.device):
        _check(fa_fwd(params, tensor_arg(q), tensor_arg(k), tensor_arg(v), tensor_arg(o),
                      ctypes.c_void_p(lse.data_ptr()), _stream(stream, q.device)), "fa_fwd")
    return o, lse


def backward_varlen(q, k, v, o, dout, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                    sm_scale=None, causal=False, window=(-1, -1), dropout_p=0.0, seed=0, offset=0,
                    deterministic=False, stream=None, workspace=None, delta=None):
    """Packed variable-length backward; tensors as in forward_varlen.

    Returns (dq, dk, dv, delta) with delta [B, H, max_seqlen_q].  The offset
    values themselves stay on the device unread here: the caller guarantees
    that they rise from 0 to at most the packed row count (the kernels clamp
    each length to the longest one).
    """
    params = _varlen_params(q, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, sm_scale,
                            causal, window, dropout_p, seed, offset, deterministic)
    shape_l = (params.batch, q.shape[1], params.seqlen)
    _validate(q, k, v, o, dout, lse, shape_l, varlen=True)
    return _backward(params, q, k, v, o, dout, lse, shape_l, stream, workspace, delta)


def debug_dropout_mask(shape, b, h, dropout_p, seed, offset=0, device="cuda", stream=None,
                       seqlen_k=None):
    """The Nq x Nk keep mask (uint8) of head (b, h), computed on the GPU."""
    import torch
    params = make_params(shape, FA_DTYPE_F32, None, False, (-1, -1), dropout_p, seed, offset,
                         seqlen_k=seqlen_k)
    n = shape[2]
    with _alloc_on(stream):
        mask = torch.empty((n, params.seqlen_k), dtype=torch.uint8, device=device)
    with torch.cuda.device(mask.device):
        _check(fa_debug_dropout_mask(params, b, h, ctypes.c_void_p(mask.data_ptr()),
                                     _stream(stream, mask.device)), "fa_debug_dropout_mask")
    return mask
