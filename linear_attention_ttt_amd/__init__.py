"""Python binding of libttt_la (TTT-with-KV-binding forward pass on MI355X).

Argument marshalling only: PyTorch supplies device memory and the current
stream; every step of the computation runs in the library's HIP kernels.
There is no CPU fallback: if ``libttt_la.so`` is missing the calls raise.

    O, W_out = forward(Q, K, V, eta, W0, chunk, mode)

``mode`` is "per_token_linear", "large_chunk_linear" or
"large_chunk_swiglu", or an ordering variant ("per_token_linear_exclusive",
"large_chunk_linear_update_first", "large_chunk_swiglu_update_first"), or
the integer constant.  Shapes, layouts and the
supported set are those of ``include/ttt_la.h``.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["forward", "forward_muon", "forward_muon_raw", "muon_workspace_bytes", "forward_noalloc_raw", "NOALLOC_SCRATCH_BYTES", "forward_momentum", "forward_momentum_raw", "backward", "backward_raw", "backward_workspace_bytes", "forward_timed_raw", "TimingEvent", "workspace_bytes", "TTTLAError", "MODES", "Desc", "lib", "library_path",
           "PER_TOKEN_LINEAR", "LARGE_CHUNK_LINEAR", "LARGE_CHUNK_SWIGLU", "PER_TOKEN_LINEAR_EXCLUSIVE",
           "LARGE_CHUNK_LINEAR_UPDATE_FIRST", "LARGE_CHUNK_SWIGLU_UPDATE_FIRST", "LARGE_CHUNK_SWIGLU_LAST_LAYER",
           "O_AS_INPUT", "O_FP32", "make_desc"]

PER_TOKEN_LINEAR = 0
LARGE_CHUNK_LINEAR = 1
LARGE_CHUNK_SWIGLU = 2
PER_TOKEN_LINEAR_EXCLUSIVE = 3
LARGE_CHUNK_LINEAR_UPDATE_FIRST = 4
LARGE_CHUNK_SWIGLU_UPDATE_FIRST = 5
LARGE_CHUNK_SWIGLU_LAST_LAYER = 6
MODES = {"per_token_linear": PER_TOKEN_LINEAR, "large_chunk_linear": LARGE_CHUNK_LINEAR,
         "large_chunk_swiglu": LARGE_CHUNK_SWIGLU, "per_token_linear_exclusive": PER_TOKEN_LINEAR_EXCLUSIVE,
         "large_chunk_linear_update_first": LARGE_CHUNK_LINEAR_UPDATE_FIRST,
         "large_chunk_swiglu_update_first": LARGE_CHUNK_SWIGLU_UPDATE_FIRST,
         "large_chunk_swiglu_last_layer": LARGE_CHUNK_SWIGLU_LAST_LAYER}
FP32, BF16 = 0, 1
O_AS_INPUT, O_FP32 = 0, 1      # ttt_la_desc.o_dtype

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libttt_la.so")


class TTTLAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"ttt_la error {status}: {msg}")
        self.status = status


class Desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("T", ctypes.c_int64),
                ("d_k", ctypes.c_int64), ("d_v", ctypes.c_int64), ("d_h", ctypes.c_int64),
                ("io_dtype", ctypes.c_int32), ("o_dtype", ctypes.c_int32)]


_LIB = None


def lib() -> ctypes.CDLL:
    """Load libttt_la.so (built in-tree); raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(library_path):
            raise RuntimeError(f"{library_path} is missing: build it with "
                               "`python -m linear_attention_ttt_amd.build` (needs ROCm hipcc)")
        L = ctypes.CDLL(library_path)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        L.ttt_la_forward.argtypes = [vp, vp, vp, vp, vp, i64, i32, ctypes.POINTER(Desc), vp, vp, vp,
                                     ctypes.c_size_t, vp]
        L.ttt_la_forward.restype = ctypes.c_int
        L.ttt_la_forward_timed.argtypes = [vp, vp, vp, vp, vp, i64, i32, ctypes.POINTER(Desc), vp, vp, vp,
                                           ctypes.c_size_t, vp, vp, vp]
        L.ttt_la_forward_timed.restype = ctypes.c_int
        L.ttt_la_forward_momentum.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_float, i64, i32, ctypes.POINTER(Desc),
                                              vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.ttt_la_forward_momentum.restype = ctypes.c_int
        L.ttt_la_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i32, ctypes.POINTER(Desc), vp, vp, vp]
        L.ttt_la_forward_noalloc.restype = ctypes.c_int
        L.ttt_la_forward_muon.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_float, ctypes.c_float, i64, i32,
                                          ctypes.POINTER(Desc), vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.ttt_la_forward_muon.restype = ctypes.c_int
        L.ttt_la_muon_workspace_bytes.argtypes = [ctypes.POINTER(Desc), i64, i32]
        L.ttt_la_muon_workspace_bytes.restype = ctypes.c_size_t
        L.ttt_la_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i32, ctypes.POINTER(Desc), vp, vp, vp, vp,
                                      vp, vp, ctypes.c_size_t, vp]
        L.ttt_la_backward.restype = ctypes.c_int
        L.ttt_la_backward_workspace_bytes.argtypes = [ctypes.POINTER(Desc), i64, i32]
        L.ttt_la_backward_workspace_bytes.restype = ctypes.c_size_t
        L.ttt_la_workspace_bytes.argtypes = [ctypes.POINTER(Desc), i64, i32]
        L.ttt_la_workspace_bytes.restype = ctypes.c_size_t
        L.ttt_la_status_string.argtypes = [ctypes.c_int]
        L.ttt_la_status_string.restype = ctypes.c_char_p
        L.ttt_la_abi_version.argtypes = []
        L.ttt_la_abi_version.restype = ctypes.c_int
        L.ttt_la_event_create.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        L.ttt_la_event_create.restype = ctypes.c_int
        L.ttt_la_event_record.argtypes = [vp, vp]
        L.ttt_la_event_record.restype = ctypes.c_int
        L.ttt_la_event_elapsed_ms.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_float)]
        L.ttt_la_event_elapsed_ms.restype = ctypes.c_int
        L.ttt_la_event_destroy.argtypes = [vp]
        L.ttt_la_event_destroy.restype = ctypes.c_int
        _LIB = L
    return _LIB


def _mode(mode) -> int:
    return MODES[mode] if isinstance(mode, str) else int(mode)


def make_desc(B, H, T, d_k, d_v, d_h=0, io_dtype=BF16, o_dtype=O_AS_INPUT) -> Desc:
    return Desc(B, H, T, d_k, d_v, d_h, io_dtype, o_dtype)


def _o_dtype(out_dtype, in_dtype):
    """(torch dtype of O, o_dtype code) for the requested output dtype (None: the input dtype)."""
    import torch
    if out_dtype is None or out_dtype == in_dtype:
        return in_dtype, O_AS_INPUT
    if out_dtype == torch.float32:
        return torch.float32, O_FP32
    raise ValueError("out_dtype must be None, the input dtype or torch.float32")


def workspace_bytes(desc: Desc, chunk: int, mode) -> int:
    return int(lib().ttt_la_workspace_bytes(ctypes.byref(desc), int(chunk), _mode(mode)))


def backward_workspace_bytes(desc: Desc, chunk: int, mode) -> int:
    return int(lib().ttt_la_backward_workspace_bytes(ctypes.byref(desc), int(chunk), _mode(mode)))


def backward_raw(Q, K, V, eta, W0, dO, dW_out, chunk, mode, desc: Desc, dQ, dK, dV, deta, dW0, workspace,
                 workspace_bytes_, stream) -> int:
    """ttt_la_backward on raw device addresses (ints or None); returns the status code."""
    return lib().ttt_la_backward(Q, K, V, eta, W0, dO, dW_out, int(chunk), _mode(mode), ctypes.byref(desc), dQ, dK,
                                 dV, deta, dW0, workspace, workspace_bytes_, stream)


def forward_momentum_raw(Q, K, V, eta, W0, M0, momentum, chunk, mode, desc: Desc, O, W_out, M_out, workspace,
                         workspace_bytes_, stream) -> int:
    """ttt_la_forward_momentum on raw device addresses (ints or None); returns the status code."""
    return lib().ttt_la_forward_momentum(Q, K, V, eta, W0, M0, float(momentum), int(chunk), _mode(mode),
                                         ctypes.byref(desc), O, W_out, M_out, workspace, workspace_bytes_, stream)


def status_string(status: int) -> str:
    return lib().ttt_la_status_string(int(status)).decode()


def forward_raw(Q, K, V, eta, W0, chunk, mode, desc: Desc, O, W_out, workspace, workspace_bytes_,
                stream) -> int:
    """Call ttt_la_forward with raw integer device addresses; returns the status."""
    return int(lib().ttt_la_forward(Q, K, V, eta, W0, int(chunk), _mode(mode), ctypes.byref(desc), O, W_out,
                                    workspace, int(workspace_bytes_), stream))


def forward_noalloc_raw(Q, K, V, eta, W0, chunk, mode, desc: Desc, O, W_out, stream) -> int:
    """ttt_la_forward_noalloc (the library's own device scratch instead of a workspace) with raw
    integer device addresses; returns the status."""
    return int(lib().ttt_la_forward_noalloc(Q, K, V, eta, W0, int(chunk), _mode(mode), ctypes.byref(desc), O, W_out,
                                            stream))


NOALLOC_SCRATCH_BYTES = 128 << 20     # TTT_LA_NOALLOC_SCRATCH_BYTES


def forward_timed_raw(Q, K, V, eta, W0, chunk, mode, desc: Desc, O, W_out, workspace, workspace_bytes_,
                      stream, ev_start, ev_stop) -> int:
    """ttt_la_forward_timed with raw addresses and raw hipEvent_t handles; returns the status."""
    return int(lib().ttt_la_forward_timed(Q, K, V, eta, W0, int(chunk), _mode(mode), ctypes.byref(desc), O, W_out,
                                          workspace, int(workspace_bytes_), stream, ev_start, ev_stop))


class TimingEvent:
    """A fence-free timing event from ttt_la_event_create (a raw hipEvent_t in ``.handle``)."""

    def __init__(self):
        h = ctypes.c_void_p()
        st = int(lib().ttt_la_event_create(ctypes.byref(h)))
        if st != 0:
            raise TTTLAError(st, status_string(st))
        self.handle = h.value

    def record(self, stream) -> None:
        st = int(lib().ttt_la_event_record(self.handle, stream))
        if st != 0:
            raise TTTLAError(st, status_string(st))

    def elapsed_ms(self, stop: "TimingEvent") -> float:
        ms = ctypes.c_float()
        st = int(lib().ttt_la_event_elapsed_ms(self.handle, stop.handle, ctypes.byref(ms)))
        if st != 0:
            raise TTTLAError(st, status_string(st))
        return float(ms.value)

    def __del__(self):
        if getattr(self, "handle", None) and _LIB is not None:
            _LIB.ttt_la_event_destroy(self.handle)
            self.handle = None


def forward(Q, K, V, eta, W0, chunk: int, mode, *, out=None, W_out=None, workspace=None, stream=None,
            timing=None, out_dtype=None):
    """Run the TTT forward pass.

    Q, K ``[B,H,T,d_k]`` and V ``[B,H,T,d_v]`` (bfloat16 or float32, same
    dtype), eta ``[B,H,T]`` float32, W0 float32 (``[B,H,d_k,d_v]`` for the
    linear modes, ``[B,H,3*d*d_h]`` packed W1|W3|W2 for SwiGLU), all
    contiguous CUDA tensors on one device.  Returns ``(O, W_out)``.
    Passing ``W_out=W0`` updates the state in place.  ``timing=(start, stop)``
    (two ``TimingEvent`` or two ``torch.cuda.Event(enable_timing=True)``)
    has the library record them around the call's dominant kernel;
    ``start.elapsed_ms(stop)`` (``elapsed_time`` for torch events) then gives
    that kernel's duration.  ``stream`` is a raw hipStream_t (default: torch's
    current stream).  ``out_dtype=torch.float32`` returns O in float32 for
    bfloat16 inputs (``TTT_LA_O_FP32``: no final rounding of the outputs)."""
    import torch

    m = _mode(mode)
    tensors = dict(Q=Q, K=K, V=V, eta=eta, W0=W0)
    dev = Q.device
    for name, t in tensors.items():
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device != dev or dev.type != "cuda":
            raise ValueError(f"{name} must be on the same CUDA device as Q")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if Q.dtype not in (torch.bfloat16, torch.float32) or K.dtype != Q.dtype or V.dtype != Q.dtype:
        raise ValueError("Q, K, V must share dtype bfloat16 or float32")
    if eta.dtype != torch.float32 or W0.dtype != torch.float32:
        raise ValueError("eta and W0 must be float32")
    if Q.dim() != 4 or K.shape != Q.shape or V.dim() != 4 or V.shape[:3] != Q.shape[:3]:
        raise ValueError("Q, K must be [B,H,T,d_k] and V [B,H,T,d_v]")
    B, H, T, dk = Q.shape
    dv = V.shape[3]
    if tuple(eta.shape) != (B, H, T):
        raise ValueError("eta must be [B,H,T]")
    dh = 0
    if m in (LARGE_CHUNK_SWIGLU, LARGE_CHUNK_SWIGLU_UPDATE_FIRST, LARGE_CHUNK_SWIGLU_LAST_LAYER):
        if W0.dim() != 3 or tuple(W0.shape[:2]) != (B, H) or W0.shape[2] % (3 * dk) != 0:
            raise ValueError("SwiGLU W0 must be [B,H,3*d*d_h]")
        dh = W0.shape[2] // (3 * dk)
    elif tuple(W0.shape) != (B, H, dk, dv):
        raise ValueError("W0 must be [B,H,d_k,d_v]")
    odt, ocode = _o_dtype(out_dtype, Q.dtype)
    desc = make_desc(B, H, T, dk, dv, dh, BF16 if Q.dtype == torch.bfloat16 else FP32, ocode)
    if out is not None and (out.dtype != odt or tuple(out.shape) != (B, H, T, dv) or not out.is_contiguous()
                            or out.device != dev):
        raise ValueError("out must be a contiguous [B,H,T,d_v] tensor of the output dtype on Q's device")
    O = out if out is not None else torch.empty((B, H, T, dv), dtype=odt, device=dev)
    Wo = W_out if W_out is not None else torch.empty_like(W0)
    nbytes = workspace_bytes(desc, chunk, m)
    ws = workspace
    if nbytes > 0 and (ws is None or ws.numel() * ws.element_size() < nbytes):
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    ws_ptr = ws.data_ptr() if (ws is not None and nbytes > 0) else None
    ws_len = ws.numel() * ws.element_size() if ws_ptr else 0
    st = stream if stream is not None else torch.cuda.current_stream(dev).cuda_stream
    if timing is None:
        status = forward_raw(Q.data_ptr(), K.data_ptr(), V.data_ptr(), eta.data_ptr(), W0.data_ptr(), chunk, m,
                             desc, O.data_ptr(), Wo.data_ptr(), ws_ptr, ws_len, st)
    else:
        e0, e1 = timing
        if isinstance(e0, TimingEvent) and isinstance(e1, TimingEvent):
            h0, h1 = e0.handle, e1.handle
        else:
            sobj = torch.cuda.ExternalStream(st) if stream is not None else torch.cuda.current_stream(dev)
            for ev in (e0, e1):      # torch creates its events lazily, on the first record
                if not ev.cuda_event:
                    ev.record(sobj)
            h0, h1 = e0.cuda_event, e1.cuda_event
        status = forward_timed_raw(Q.data_ptr(), K.data_ptr(), V.data_ptr(), eta.data_ptr(), W0.data_ptr(), chunk,
                                   m, desc, O.data_ptr(), Wo.data_ptr(), ws_ptr, ws_len, st, h0, h1)
    if status != 0:
        raise TTTLAError(status, status_string(status))
    return O, Wo


def backward(Q, K, V, eta, W0, dO, dW_out, chunk: int, mode="per_token_linear", *, workspace=None, stream=None):
    """Gradients of the forward (with O in the input dtype) in every mode: per-token and large-chunk
    linear (both read orders) and the three SwiGLU modes (``W0`` and ``dW_out`` packed like the
    forward's state): given the inputs of ``forward``,
    ``dO`` (gradient of O, like V) and ``dW_out`` (gradient of the final
    memory, float32 like W0), return ``(dQ, dK, dV, deta, dW0)``, all
    float32.  Argument checks as in ``forward``."""
    import torch

    m = _mode(mode)
    tensors = dict(Q=Q, K=K, V=V, eta=eta, W0=W0, dO=dO, dW_out=dW_out)
    dev = Q.device
    for name, t in tensors.items():
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device != dev or dev.type != "cuda":
            raise ValueError(f"{name} must be on the same CUDA device as Q")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if Q.dtype not in (torch.bfloat16, torch.float32) or K.dtype != Q.dtype or V.dtype != Q.dtype or \
            dO.dtype != Q.dtype:
        raise ValueError("Q, K, V, dO must share dtype bfloat16 or float32")
    if eta.dtype != torch.float32 or W0.dtype != torch.float32 or dW_out.dtype != torch.float32:
        raise ValueError("eta, W0 and dW_out must be float32")
    if Q.dim() != 4 or K.shape != Q.shape or V.dim() != 4 or V.shape[:3] != Q.shape[:3] or dO.shape != V.shape:
        raise ValueError("Q, K must be [B,H,T,d_k], V and dO [B,H,T,d_v]")
    B, H, T, dk = Q.shape
    dv = V.shape[3]
    dh = 0
    if m in (LARGE_CHUNK_SWIGLU, LARGE_CHUNK_SWIGLU_UPDATE_FIRST, LARGE_CHUNK_SWIGLU_LAST_LAYER):
        if W0.dim() != 3 or tuple(W0.shape[:2]) != (B, H) or W0.shape[2] % (3 * dk) != 0 or dv != dk:
            raise ValueError("SwiGLU W0 must be [B,H,3*d*d_h] with d = d_k = d_v")
        dh = W0.shape[2] // (3 * dk)
        if tuple(eta.shape) != (B, H, T) or dW_out.shape != W0.shape:
            raise ValueError("eta must be [B,H,T] and dW_out shaped like W0")
    elif tuple(eta.shape) != (B, H, T) or tuple(W0.shape) != (B, H, dk, dv) or dW_out.shape != W0.shape:
        raise ValueError("eta must be [B,H,T], W0 and dW_out [B,H,d_k,d_v]")
    desc = make_desc(B, H, T, dk, dv, dh, BF16 if Q.dtype == torch.bfloat16 else FP32)
    f32 = dict(dtype=torch.float32, device=dev)
    dQ, dK, dV = torch.empty(Q.shape, **f32), torch.empty(K.shape, **f32), torch.empty(V.shape, **f32)
    deta, dW0 = torch.empty_like(eta), torch.empty_like(W0)
    nbytes = backward_workspace_bytes(desc, chunk, m)
    ws = workspace
    if ws is None or ws.numel() * ws.element_size() < nbytes:
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    st = stream if stream is not None else torch.cuda.current_stream(dev).cuda_stream

    def p(t):
        return t.data_ptr() if t.numel() > 0 else None

    status = backward_raw(p(Q), p(K), p(V), p(eta), W0.data_ptr(), p(dO), dW_out.data_ptr(), chunk, m, desc, p(dQ),
                          p(dK), p(dV), p(deta), dW0.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(), st)
    if status != 0:
        raise TTTLAError(status, status_string(status))
    return dQ, dK, dV, deta, dW0


def muon_workspace_bytes(desc: Desc, chunk: int, mode) -> int:
    return int(lib().ttt_la_muon_workspace_bytes(ctypes.byref(desc), int(chunk), _mode(mode)))


def forward_muon_raw(Q, K, V, eta, W0, M0, momentum, muon_scale, chunk, mode, desc: Desc, O, W_out, M_out, workspace,
                     workspace_bytes_, stream) -> int:
    """ttt_la_forward_muon on raw device addresses (ints or None); returns the status code."""
    return lib().ttt_la_forward_muon(Q, K, V, eta, W0, M0, float(momentum), float(muon_scale), int(chunk),
                                     _mode(mode), ctypes.byref(desc), O, W_out, M_out, workspace, workspace_bytes_,
                                     stream)


def forward_muon(Q, K, V, eta, W0, chunk: int, muon_scale: float, momentum: float = 0.0, M0=None,
                 mode="large_chunk_swiglu", *, workspace=None, stream=None, out_dtype=None):
    """SwiGLU forward with Muon as the update rule (``ttt_la_forward_muon``): returns
    ``(O, W_out, M_out)`` (``M_out`` None without momentum and ``M0``).  Same tensor checks as
    ``forward``."""
    import torch

    m = _mode(mode)
    if m not in (LARGE_CHUNK_SWIGLU, LARGE_CHUNK_SWIGLU_UPDATE_FIRST):
        raise ValueError("Muon is defined for the SwiGLU modes (read-first and update-first)")
    for name, t in dict(Q=Q, K=K, V=V, eta=eta, W0=W0).items():
        if not isinstance(t, torch.Tensor) or t.device != Q.device or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor on Q's device")
    if M0 is not None and (M0.shape != W0.shape or M0.dtype != torch.float32 or not M0.is_contiguous()):
        raise ValueError("M0 must be a contiguous float32 tensor shaped like W0")
    if Q.dtype != torch.bfloat16 or K.dtype != Q.dtype or V.dtype != Q.dtype:
        raise ValueError("Q, K, V must be bfloat16")
    B, H, T, dk = Q.shape
    if W0.dim() != 3 or tuple(W0.shape[:2]) != (B, H) or W0.shape[2] % (3 * dk) != 0:
        raise ValueError("SwiGLU W0 must be [B,H,3*d*d_h]")
    dh = W0.shape[2] // (3 * dk)
    odt, ocode = _o_dtype(out_dtype, Q.dtype)
    desc = make_desc(B, H, T, dk, dk, dh, BF16, ocode)
    O = torch.empty((B, H, T, dk), dtype=odt, device=Q.device)
    Wo = torch.empty_like(W0)
    Mo = torch.empty_like(W0) if (momentum != 0.0 or M0 is not None) else None
    nbytes = muon_workspace_bytes(desc, chunk, m)
    ws = workspace
    if nbytes > 0 and (ws is None or ws.numel() * ws.element_size() < nbytes):
        ws = torch.empty(nbytes, dtype=torch.uint8, device=Q.device)
    ws_len = ws.numel() * ws.element_size() if ws is not None else 0
    st = stream if stream is not None else torch.cuda.current_stream(Q.device).cuda_stream

    def p(t):
        return t.data_ptr() if t is not None and t.numel() > 0 else None

    status = forward_muon_raw(p(Q), p(K), p(V), p(eta), W0.data_ptr(), p(M0), momentum, muon_scale, chunk, m, desc,
                              p(O), Wo.data_ptr(), p(Mo), p(ws), ws_len, st)
    if status != 0:
        raise TTTLAError(status, status_string(status))
    return O, Wo, Mo


def forward_momentum(Q, K, V, eta, W0, chunk: int, momentum: float, M0=None, mode="large_chunk_linear", *,
                     workspace=None, stream=None, out_dtype=None):
    """Large-chunk forward (linear or SwiGLU memory) with a momentum buffer
    (``ttt_la_forward_momentum``): returns ``(O, W_out, M_out)``.  ``M0`` (float32 like W0) is
    the buffer before the first chunk, zeros when None.  Same tensor checks as ``forward``."""
    import torch

    m = _mode(mode)
    if m not in (LARGE_CHUNK_LINEAR, LARGE_CHUNK_LINEAR_UPDATE_FIRST, LARGE_CHUNK_SWIGLU,
                 LARGE_CHUNK_SWIGLU_UPDATE_FIRST):
        raise ValueError("momentum is defined for the large-chunk linear and SwiGLU modes (not last-layer)")
    for name, t in dict(Q=Q, K=K, V=V, eta=eta, W0=W0).items():
        if not isinstance(t, torch.Tensor) or t.device != Q.device or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor on Q's device")
    if M0 is not None and (M0.shape != W0.shape or M0.dtype != torch.float32 or not M0.is_contiguous()):
        raise ValueError("M0 must be a contiguous float32 tensor shaped like W0")
    if Q.dtype != torch.bfloat16 or K.dtype != Q.dtype or V.dtype != Q.dtype:
        raise ValueError("Q, K, V must be bfloat16")
    B, H, T, dk = Q.shape
    dv = V.shape[3]
    if m in (LARGE_CHUNK_SWIGLU, LARGE_CHUNK_SWIGLU_UPDATE_FIRST):
        if W0.dim() != 3 or tuple(W0.shape[:2]) != (B, H) or W0.shape[2] % (3 * dk) != 0 or dv != dk:
            raise ValueError("SwiGLU W0 must be [B,H,3*d*d_h] with d = d_k = d_v")
    elif tuple(W0.shape) != (B, H, dk, dv):
        raise ValueError("W0 must be [B,H,d_k,d_v]")
    dh = W0.shape[2] // (3 * dk) if m in (LARGE_CHUNK_SWIGLU, LARGE_CHUNK_SWIGLU_UPDATE_FIRST) else 0
    odt, ocode = _o_dtype(out_dtype, Q.dtype)
    desc = make_desc(B, H, T, dk, dv, dh, BF16, ocode)
    O = torch.empty((B, H, T, dv), dtype=odt, device=Q.device)
    Wo, Mo = torch.empty_like(W0), torch.empty_like(W0)
    nbytes = workspace_bytes(desc, chunk, m)
    ws = workspace
    if nbytes > 0 and (ws is None or ws.numel() * ws.element_size() < nbytes):
        ws = torch.empty(nbytes, dtype=torch.uint8, device=Q.device)
    ws_ptr = ws.data_ptr() if (ws is not None and nbytes > 0) else None
    ws_len = ws.numel() * ws.element_size() if ws_ptr else 0
    st = stream if stream is not None else torch.cuda.current_stream(Q.device).cuda_stream

    def p(t):
        return t.data_ptr() if t is not None and t.numel() > 0 else None

    status = forward_momentum_raw(p(Q), p(K), p(V), p(eta), W0.data_ptr(), p(M0), momentum, chunk, m, desc, p(O),
                                  Wo.data_ptr(), Mo.data_ptr(), ws_ptr, ws_len, st)
    if status != 0:
        raise TTTLAError(status, status_string(status))
    return O, Wo, Mo
