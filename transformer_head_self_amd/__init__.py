"""MI355X (gfx950) multi-head attention forward: Python binding of libmha.so.

The functions here only marshal arguments: they turn torch tensors into
device pointers and sizes, allocate outputs and scratch with torch, and call
the C ABI declared in ``include/mha.h`` on torch's current HIP stream.  Every
step of the computation runs in the library's HIP kernels; there is no
fallback, and every call raises if the library is missing or returns an error.

Entry points (same names as the C ABI):
* ``mha_forward``  projections, fused attention, concatenation, W^O.
* ``attn_core``    fused attention on already projected heads.
* ``attn_core_split``  the same with the key axis cut into partitions whose
  summaries are merged afterwards (few query rows, many keys).
* ``attn_split_workspace_bytes``.
* ``attn_core_split_noalloc``  the key-split form with the library's static
  scratch instead of a workspace (for callers that cannot allocate).
* ``attn_core_backward``  gradients of the attention core from the forward's
  row statistics; ``attn_backward_workspace_bytes``.
* ``mha_backward``  gradients of the whole layer (inputs, weights, biases)
  from the forward's workspace and row statistics;
  ``mha_backward_workspace_bytes``.
* ``mha_workspace_bytes``, ``mha_status_string``.
"""

from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "MhaError", "MhaDims", "MhaMask", "MhaBias", "MhaBiasGrad", "lib", "mha_backward",
    "mha_backward_workspace_bytes", "mha_forward", "attn_core", "attn_core_split",
    "attn_split_workspace_bytes", "attn_core_split_noalloc", "attn_core_backward",
    "attn_bias_backward", "attn_backward_workspace_bytes",
    "mha_workspace_bytes", "mha_status_string", "MHA_F32", "MHA_BF16", "MHA_F16",
    "MHA_MASK_CAUSAL", "MHA_MASK_KEY_PADDING", "MHA_MASK_BOOL", "MHA_MASK_ADDITIVE",
]

# The library to load: the in-tree build, or the file named by
# TRANSFORMER_HEAD_SELF_AMD_LIB (an instrumented build of the same sources).
LIB_PATH = (os.environ.get("TRANSFORMER_HEAD_SELF_AMD_LIB") or
            os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmha.so"))

MHA_F32, MHA_BF16, MHA_F16 = 0, 1, 2
MHA_ERR_SCRATCH = -10
MHA_STATIC_SCRATCH_BYTES = 16 << 20   # the static scratch of attn_core_split_noalloc
MHA_MASK_CAUSAL, MHA_MASK_KEY_PADDING, MHA_MASK_BOOL, MHA_MASK_ADDITIVE = 1, 2, 4, 8


class MhaError(RuntimeError):
    def __init__(self, status, where=""):
        self.status = int(status)
        super().__init__(f"{where}: {mha_status_string(status)} ({status})")


class MhaDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "h", "n_q", "n_k", "d_q", "d_k", "d_v", "d_h", "d_vh", "d_o")] + [
        ("scale", ctypes.c_float), ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("work_dtype", ctypes.c_int32)]


class MhaMask(ctypes.Structure):
    _fields_ = [("flags", ctypes.c_uint32), ("key_len", ctypes.c_void_p),
                ("allowed", ctypes.c_void_p), ("allowed_batch_stride", ctypes.c_int64),
                ("add", ctypes.c_void_p), ("add_batch_stride", ctypes.c_int64)]


class MhaBiasGrad(ctypes.Structure):
    _fields_ = [("db_Q", ctypes.c_void_p), ("db_K", ctypes.c_void_p), ("db_V", ctypes.c_void_p),
                ("db_O", ctypes.c_void_p)]


class MhaBias(ctypes.Structure):
    _fields_ = [("b_Q", ctypes.c_void_p), ("b_K", ctypes.c_void_p), ("b_V", ctypes.c_void_p),
                ("b_O", ctypes.c_void_p)]


_LIB = None


def lib():
    """The loaded libmha.so (ctypes), with argument types declared."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                "(hipcc, gfx950) before calling the library")
        L = ctypes.CDLL(LIB_PATH)
        vp, P = ctypes.c_void_p, ctypes.POINTER
        L.mha_workspace_bytes.argtypes = [P(MhaDims)]
        L.mha_workspace_bytes.restype = ctypes.c_size_t
        L.mha_forward.argtypes = ([P(MhaDims), P(MhaMask)] + [vp] * 7 + [P(MhaBias)] +
                                  [vp] * 4 + [ctypes.c_size_t, vp])
        L.mha_forward.restype = ctypes.c_int
        L.attn_core.argtypes = [P(MhaDims), P(MhaMask), vp, vp, vp, vp, vp, vp, vp]
        L.attn_core.restype = ctypes.c_int
        L.attn_split_workspace_bytes.argtypes = [P(MhaDims), ctypes.c_int32]
        L.attn_split_workspace_bytes.restype = ctypes.c_size_t
        L.attn_core_split.argtypes = [P(MhaDims), P(MhaMask), vp, vp, vp, vp, vp, vp,
                                      ctypes.c_int32, vp, ctypes.c_size_t, vp]
        L.attn_core_split.restype = ctypes.c_int
        L.attn_core_split_noalloc.argtypes = [P(MhaDims), P(MhaMask), vp, vp, vp, vp, vp, vp,
                                              ctypes.c_int32, vp]
        L.attn_core_split_noalloc.restype = ctypes.c_int
        L.attn_backward_workspace_bytes.argtypes = [P(MhaDims)]
        L.attn_backward_workspace_bytes.restype = ctypes.c_size_t
        L.attn_core_backward.argtypes = [P(MhaDims), P(MhaMask)] + [vp] * 11 + [ctypes.c_size_t,
                                                                                vp]
        L.attn_core_backward.restype = ctypes.c_int
        L.attn_bias_backward.argtypes = [P(MhaDims), P(MhaMask)] + [vp] * 9 + [ctypes.c_size_t,
                                                                               vp]
        L.attn_bias_backward.restype = ctypes.c_int
        L.mha_backward_workspace_bytes.argtypes = [P(MhaDims)]
        L.mha_backward_workspace_bytes.restype = ctypes.c_size_t
        L.mha_backward.argtypes = ([P(MhaDims), P(MhaMask)] + [vp] * 11 + [ctypes.c_size_t] +
                                   [vp] * 7 + [P(MhaBiasGrad), vp, ctypes.c_size_t, vp])
        L.mha_backward.restype = ctypes.c_int
        L.mha_status_string.argtypes = [ctypes.c_int]
        L.mha_status_string.restype = ctypes.c_char_p
        L.mha_max_head_dim.argtypes = []
        L.mha_max_head_dim.restype = ctypes.c_int32
        _LIB = L
    return _LIB


def mha_status_string(status):
    return lib().mha_status_string(int(status)).decode()


def mha_workspace_bytes(dims: MhaDims):
    return int(lib().mha_workspace_bytes(ctypes.byref(dims)))


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t == torch.float32:
        return MHA_F32
    if t == torch.bfloat16:
        return MHA_BF16
    if t == torch.float16:
        return MHA_F16
    raise TypeError(f"unsupported element type {t}; use float32, bfloat16 or float16")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _mask(B, n_q, n_k, causal, key_len, allowed, device, add=None):
    torch = _torch()
    m = MhaMask()
    m.flags = 0
    keep = []
    if causal:
        m.flags |= MHA_MASK_CAUSAL
    if key_len is not None:
        kl = torch.as_tensor(key_len, dtype=torch.int32, device=device).contiguous()
        keep.append(kl)
        m.flags |= MHA_MASK_KEY_PADDING
        m.key_len = kl.data_ptr()
    if allowed is not None:
        G = torch.as_tensor(allowed, device=device)
        # a bool tensor is one byte per entry (0 / 1): reinterpreted, not copied
        G = (G.view(torch.uint8) if G.dtype == torch.bool else G.to(torch.uint8)).contiguous()
        if G.dim() != 3 or G.shape[1:] != (n_q, n_k) or G.shape[0] not in (1, B):
            raise ValueError("allowed must have shape [B or 1, n_q, n_k]")
        keep.append(G)
        m.flags |= MHA_MASK_BOOL
        m.allowed = G.data_ptr()
        m.allowed_batch_stride = 0 if G.shape[0] == 1 else n_q * n_k
    if add is not None:
        M = torch.as_tensor(add, device=device).to(torch.float32).contiguous()
        if M.dim() != 3 or M.shape[1:] != (n_q, n_k) or M.shape[0] not in (1, B):
            raise ValueError("add must have shape [B or 1, n_q, n_k]")
        keep.append(M)
        m.flags |= MHA_MASK_ADDITIVE
        m.add = M.data_ptr()
        m.add_batch_stride = 0 if M.shape[0] == 1 else n_q * n_k
    return m, keep


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _launch_stream(stream):
    """The torch stream the kernels will run on (torch's current stream by
    default)."""
    torch = _torch()
    return torch.cuda.current_stream() if stream is None else stream


def _used_on(stream, tensors):
    """Mark tensors allocated here (outputs, workspace, converted masks) as
    used by the launches on ``stream``: torch's caching allocator then keeps
    their memory out of reuse until that stream's work has finished, also
    when ``stream`` is not the stream they were allocated on."""
    torch = _torch()
    if stream is None or stream == torch.cuda.current_stream():
        return
    for t in tensors:
        if t is not None and t.is_cuda:
            t.record_stream(stream)


def default_work_dtype(in_dtype):
    """Intermediate element type used when the caller does not choose one."""
    torch = _torch()
    return torch.float16 if in_dtype in (torch.bfloat16, torch.float16) else torch.float32


def mha_forward(Q, K, V, W_Q, W_K, W_V, W_O, h, d_h, d_vh, *, scale=None, causal=False,
                key_len=None, allowed=None, add=None, b_Q=None, b_K=None, b_V=None, b_O=None,
                out_dtype=None, work_dtype=None, Y=None, row_m=None, row_l=None,
                workspace=None, stream=None):
    """Y [B, n_q, d_o] = MHA(Q, K, V) for Q [B,n_q,d_q], K [B,n_k,d_k], V [B,n_k,d_v].

    Weights are combined (head r in column block r): W_Q [d_q, h*d_h],
    W_K [d_k, h*d_h], W_V [d_v, h*d_vh], W_O [h*d_vh, d_o]; optional
    projection biases b_Q [h*d_h], b_K [h*d_h], b_V [h*d_vh], b_O [d_o] in
    the weights' element type; optional additive score bias ``add``
    [B or 1, n_q, n_k] (float32, -inf forbids a key).  ``scale`` defaults
    to 1/sqrt(d_h); ``out_dtype`` to float32; ``work_dtype`` (the
    intermediates' element type) to float16 for 2-byte inputs, else float32.
    """
    torch = _torch()
    B, n_q, d_q = Q.shape
    n_k, d_k = K.shape[1], K.shape[2]
    d_v = V.shape[2]
    d_o = W_O.shape[1]
    in_code = _dtype_code(Q.dtype)
    for t in (K, V, W_Q, W_K, W_V, W_O, b_Q, b_K, b_V, b_O):
        if t is not None and t.dtype != Q.dtype:
            raise TypeError("Q, K, V, the weights and the biases must share one element type")
    for t, n in ((b_Q, h * d_h), (b_K, h * d_h), (b_V, h * d_vh), (b_O, d_o)):
        if t is not None and t.numel() != n:
            raise ValueError("a projection bias has the wrong length")
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    work_dtype = default_work_dtype(Q.dtype) if work_dtype is None else work_dtype
    dims = MhaDims(B=B, h=h, n_q=n_q, n_k=n_k, d_q=d_q, d_k=d_k, d_v=d_v, d_h=d_h, d_vh=d_vh,
                   d_o=d_o, scale=(1.0 / math.sqrt(d_h)) if scale is None else float(scale),
                   in_dtype=in_code, out_dtype=_dtype_code(out_dtype),
                   work_dtype=_dtype_code(work_dtype))
    m, keep = _mask(B, n_q, n_k, causal, key_len, allowed, Q.device, add)
    bias = MhaBias(b_Q=_ptr(b_Q), b_K=_ptr(b_K), b_V=_ptr(b_V), b_O=_ptr(b_O))
    if Y is None:
        Y = torch.empty((B, n_q, d_o), dtype=out_dtype, device=Q.device)
    need = mha_workspace_bytes(dims)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=Q.device)
    st = lib().mha_forward(ctypes.byref(dims), ctypes.byref(m), _ptr(Q), _ptr(K), _ptr(V),
                           _ptr(W_Q), _ptr(W_K), _ptr(W_V), _ptr(W_O), ctypes.byref(bias),
                           _ptr(Y), _ptr(row_m),
                           _ptr(row_l), _ptr(workspace), workspace.numel(), _stream(stream))
    _used_on(stream, keep + [Y, workspace])
    del keep
    if st != 0:
        raise MhaError(st, "mha_forward")
    return Y


def _core_dims(Qh, Kh, Vh, scale, out_dtype):
    B, h, n_q, d_h = Qh.shape
    n_k = Kh.shape[2]
    d_vh = Vh.shape[3]
    if Kh.dtype != Qh.dtype or Vh.dtype != Qh.dtype:
        raise TypeError("Qh, Kh and Vh must share one element type")
    return MhaDims(B=B, h=h, n_q=n_q, n_k=n_k, d_q=1, d_k=1, d_v=1, d_h=d_h, d_vh=d_vh, d_o=1,
                   scale=(1.0 / math.sqrt(d_h)) if scale is None else float(scale),
                   in_dtype=_dtype_code(Qh.dtype), out_dtype=_dtype_code(out_dtype),
                   work_dtype=_dtype_code(Qh.dtype))


def attn_core(Qh, Kh, Vh, *, scale=None, causal=False, key_len=None, allowed=None,
              add=None, out_dtype=None, Z=None, row_m=None, row_l=None, stream=None):
    """Z [B, n_q, h*d_vh] from heads Qh [B,h,n_q,d_h], Kh [B,h,n_k,d_h], Vh [B,h,n_k,d_vh]."""
    torch = _torch()
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    dims = _core_dims(Qh, Kh, Vh, scale, out_dtype)
    B, h, n_q, n_k, d_vh = dims.B, dims.h, dims.n_q, dims.n_k, dims.d_vh
    m, keep = _mask(B, n_q, n_k, causal, key_len, allowed, Qh.device, add)
    if Z is None:
        Z = torch.empty((B, n_q, h * d_vh), dtype=out_dtype, device=Qh.device)
    st = lib().attn_core(ctypes.byref(dims), ctypes.byref(m), _ptr(Qh), _ptr(Kh), _ptr(Vh),
                         _ptr(Z), _ptr(row_m), _ptr(row_l), _stream(stream))
    _used_on(stream, keep + [Z])
    del keep
    if st != 0:
        raise MhaError(st, "attn_core")
    return Z


def attn_split_workspace_bytes(dims: MhaDims, splits=0):
    return lib().attn_split_workspace_bytes(ctypes.byref(dims) if dims is not None else None,
                                            int(splits))


def attn_core_split(Qh, Kh, Vh, *, splits=0, scale=None, causal=False, key_len=None,
                    allowed=None, add=None, out_dtype=None, Z=None, row_m=None, row_l=None,
                    workspace=None, stream=None):
    """attn_core with the key axis cut into partitions merged afterwards
    (``splits`` partitions requested, 0 = library's choice)."""
    torch = _torch()
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    dims = _core_dims(Qh, Kh, Vh, scale, out_dtype)
    B, h, n_q, n_k, d_vh = dims.B, dims.h, dims.n_q, dims.n_k, dims.d_vh
    m, keep = _mask(B, n_q, n_k, causal, key_len, allowed, Qh.device, add)
    if Z is None:
        Z = torch.empty((B, n_q, h * d_vh), dtype=out_dtype, device=Qh.device)
    if workspace is None:
        nbytes = attn_split_workspace_bytes(dims, splits)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=Qh.device)
    st = lib().attn_core_split(ctypes.byref(dims), ctypes.byref(m), _ptr(Qh), _ptr(Kh),
                               _ptr(Vh), _ptr(Z), _ptr(row_m), _ptr(row_l), int(splits),
                               _ptr(workspace), workspace.numel(), _stream(stream))
    _used_on(stream, keep + [Z, workspace])
    del keep
    if st != 0:
        raise MhaError(st, "attn_core_split")
    return Z


def attn_core_split_noalloc(Qh, Kh, Vh, *, splits=0, scale=None, causal=False, key_len=None,
                            allowed=None, add=None, out_dtype=None, Z=None, row_m=None,
                            row_l=None, stream=None):
    """attn_core_split with the partitions' summaries in the library's static
    scratch (MHA_STATIC_SCRATCH_BYTES per GPU) instead of a workspace: the C
    call allocates nothing.  Calls that overlap in time on one GPU share that
    scratch and race; calls ordered on one stream are safe."""
    torch = _torch()
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    dims = _core_dims(Qh, Kh, Vh, scale, out_dtype)
    B, h, n_q, n_k, d_vh = dims.B, dims.h, dims.n_q, dims.n_k, dims.d_vh
    m, keep = _mask(B, n_q, n_k, causal, key_len, allowed, Qh.device, add)
    if Z is None:
        Z = torch.empty((B, n_q, h * d_vh), dtype=out_dtype, device=Qh.device)
    st = lib().attn_core_split_noalloc(ctypes.byref(dims), ctypes.byref(m), _ptr(Qh), _ptr(Kh),
                                       _ptr(Vh), _ptr(Z), _ptr(row_m), _ptr(row_l), int(splits),
                                       _stream(stream))
    _used_on(stream, keep + [Z])
    del keep
    if st != 0:
        raise MhaError(st, "attn_core_split_noalloc")
    return Z


def attn_backward_workspace_bytes(dims: MhaDims):
    return int(lib().attn_backward_workspace_bytes(ctypes.byref(dims) if dims is not None
                                                   else None))


def attn_core_backward(Qh, Kh, Vh, Z, dZ, row_m, row_l, *, scale=None, causal=False,
                       key_len=None, allowed=None, add=None, dQh=None, dKh=None, dVh=None,
                       workspace=None, stream=None):
    """Gradients (dQh, dKh, dVh) of a loss with upstream gradient dZ for the
    attention core; Z, row_m and row_l come from the same forward call (same
    masks and scale).  Gradients have the element type of Z and dZ.  Heads
    may be bf16, fp16 or fp32."""
    torch = _torch()
    if dZ.dtype != Z.dtype:
        raise TypeError("Z and dZ must share one element type")
    dims = _core_dims(Qh, Kh, Vh, scale, Z.dtype)
    B, h, n_q, n_k, d_h, d_vh = dims.B, dims.h, dims.n_q, dims.n_k, dims.d_h, dims.d_vh
    m, keep = _mask(B, n_q, n_k, causal, key_len, allowed, Qh.device, add)
    if dQh is None:
        dQh = torch.empty((B, h, n_q, d_h), dtype=Z.dtype, device=Qh.device)
    if dKh is None:
        dKh = torch.empty((B, h, n_k, d_h), dtype=Z.dtype, device=Qh.device)
    if dVh is None:
        dVh = torch.empty((B, h, n_k, d_vh), dtype=Z.dtype, device=Qh.device)
    if workspace is None:
        workspace = torch.empty(max(attn_backward_workspace_bytes(dims), 1), dtype=torch.uint8,
                                device=Qh.device)
    st = lib().attn_core_backward(ctypes.byref(dims), ctypes.byref(m), _ptr(Qh), _ptr(Kh),
                                  _ptr(Vh), _ptr(Z), _ptr(dZ), _ptr(row_m), _ptr(row_l),
                                  _ptr(dQh), _ptr(dKh), _ptr(dVh), _ptr(workspace),
                                  workspace.numel(), _stream(stream))
    _used_on(stream, keep + [dQh, dKh, dVh, workspace])
    del keep
    if st != 0:
        raise MhaError(st, "attn_core_backward")
    return dQh, dKh, dVh


def attn_bias_backward(Qh, Kh, Vh, Z, dZ, row_m, row_l, add, *, scale=None, causal=False,
                       key_len=None, allowed=None, dM=None, workspace=None, stream=None):
    """Gradient dM (fp32, the shape of ``add``: [B or 1, n_q, n_k]) of a loss
    with upstream gradient dZ with respect to the additive score bias of
    the attention core: dS summed over heads (and items for a shared bias).
    Same arguments as ``attn_core_backward``."""
    torch = _torch()
    if dZ.dtype != Z.dtype:
        raise TypeError("Z and dZ must share one element type")
    dims = _core_dims(Qh, Kh, Vh, scale, Z.dtype)
    B, n_q, n_k = dims.B, dims.n_q, dims.n_k
    m, keep = _mask(B, n_q, n_k, causal, key_len, allowed, Qh.device, add)
    Bo = 1 if m.add_batch_stride == 0 else B
    if dM is None:
        dM = torch.empty((Bo, n_q, n_k), dtype=torch.float32, device=Qh.device)
    if dM.dtype != torch.float32 or not dM.is_contiguous() or tuple(dM.shape) != (Bo, n_q, n_k):
        raise ValueError(f"dM must be a contiguous float32 [{Bo}, {n_q}, {n_k}] tensor")
    if workspace is None:
        workspace = torch.empty(max(attn_backward_workspace_bytes(dims), 1), dtype=torch.uint8,
                                device=Qh.device)
    st = lib().attn_bias_backward(ctypes.byref(dims), ctypes.byref(m), _ptr(Qh), _ptr(Kh),
                                  _ptr(Vh), _ptr(Z), _ptr(dZ), _ptr(row_m), _ptr(row_l),
                                  _ptr(dM), _ptr(workspace), workspace.numel(), _stream(stream))
    _used_on(stream, keep + [dM, workspace])
    del keep
    if st != 0:
        raise MhaError(st, "attn_bias_backward")
    return dM


def mha_backward_workspace_bytes(dims: MhaDims):
    return int(lib().mha_backward_workspace_bytes(ctypes.byref(dims) if dims is not None
                                                  else None))


def mha_backward(Q, K, V, W_Q, W_K, W_V, W_O, h, d_h, d_vh, dY, row_m, row_l, fwd_workspace, *,
                 scale=None, causal=False, key_len=None, allowed=None, add=None, work_dtype=None,
                 bias_grads=False, workspace=None, stream=None):
    """Gradients of the layer for the upstream gradient dY, after
    ``mha_forward`` was called with the same arguments, ``workspace=
    fwd_workspace`` and ``row_m``/``row_l`` requested.  Returns a dict with
    dQ, dK, dV, dW_Q, dW_K, dW_V, dW_O (and db_Q, db_K, db_V, db_O if
    ``bias_grads``), all of dY's element type."""
    torch = _torch()
    B, n_q, d_q = Q.shape
    n_k, d_k = K.shape[1], K.shape[2]
    d_v = V.shape[2]
    d_o = W_O.shape[1]
    work_dtype = default_work_dtype(Q.dtype) if work_dtype is None else work_dtype
    dims = MhaDims(B=B, h=h, n_q=n_q, n_k=n_k, d_q=d_q, d_k=d_k, d_v=d_v, d_h=d_h, d_vh=d_vh,
                   d_o=d_o, scale=(1.0 / math.sqrt(d_h)) if scale is None else float(scale),
                   in_dtype=_dtype_code(Q.dtype), out_dtype=_dtype_code(dY.dtype),
                   work_dtype=_dtype_code(work_dtype))
    m, keep = _mask(B, n_q, n_k, causal, key_len, allowed, Q.device, add)
    dev, od = Q.device, dY.dtype
    out = {"dQ": torch.empty((B, n_q, d_q), dtype=od, device=dev),
           "dK": torch.empty((B, n_k, d_k), dtype=od, device=dev),
           "dV": torch.empty((B, n_k, d_v), dtype=od, device=dev),
           "dW_Q": torch.empty(tuple(W_Q.shape), dtype=od, device=dev),
           "dW_K": torch.empty(tuple(W_K.shape), dtype=od, device=dev),
           "dW_V": torch.empty(tuple(W_V.shape), dtype=od, device=dev),
           "dW_O": torch.empty(tuple(W_O.shape), dtype=od, device=dev)}
    db = MhaBiasGrad()
    if bias_grads:
        for k, n in (("db_Q", h * d_h), ("db_K", h * d_h), ("db_V", h * d_vh), ("db_O", d_o)):
            out[k] = torch.empty(n, dtype=od, device=dev)
            setattr(db, k, out[k].data_ptr())
    if workspace is None:
        workspace = torch.empty(max(mha_backward_workspace_bytes(dims), 1), dtype=torch.uint8,
                                device=dev)
    st = lib().mha_backward(ctypes.byref(dims), ctypes.byref(m), _ptr(Q), _ptr(K), _ptr(V),
                            _ptr(W_Q), _ptr(W_K), _ptr(W_V), _ptr(W_O), _ptr(dY), _ptr(row_m),
                            _ptr(row_l), _ptr(fwd_workspace), fwd_workspace.numel(),
                            _ptr(out["dQ"]), _ptr(out["dK"]), _ptr(out["dV"]), _ptr(out["dW_Q"]),
                            _ptr(out["dW_K"]), _ptr(out["dW_V"]), _ptr(out["dW_O"]),
                            ctypes.byref(db), _ptr(workspace), workspace.numel(),
                            _stream(stream))
    _used_on(stream, keep + list(out.values()) + [workspace])
    del keep
    if st != 0:
        raise MhaError(st, "mha_backward")
    return out
