"""ctypes binding of libipttt (include/ipttt.h): argument marshalling only.

Every step of the prefill runs in the library's HIP kernels; PyTorch only owns
device memory and supplies the HIP stream. The functions keep the C names.
Loading fails loudly if libipttt.so has not been built (there is no fallback).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libipttt.so")

IPTTT_OK = 0
IPTTT_E_INVALID = -1
IPTTT_E_UNSUPPORTED = -2
IPTTT_E_HIP = -3
IPTTT_E_STATE = -4
IPTTT_E_WORKSPACE = -5

IPTTT_F32 = 0
IPTTT_BF16 = 1
IPTTT_UPDATE_LINEAR = 0
IPTTT_UPDATE_MSE = 1
IPTTT_FLAG_GENERIC_KERNELS = 1

IPTTT_NOALLOC_SCRATCH_BYTES = 256 << 20

EXPORTS = (
    "ipttt_workspace_bytes", "ipttt_init", "ipttt_prefill_layer", "ipttt_prefill_layer_noalloc",
    "ipttt_prefill_packed", "ipttt_decode_step", "ipttt_backward_workspace_bytes",
    "ipttt_backward_layer", "ipttt_reset_fast_weights", "ipttt_profile_begin",
    "ipttt_profile_end", "ipttt_destroy", "ipttt_status_str", "ipttt_last_error",
)

KERNELS = ("gateup", "conv", "proj", "update", "apply", "snapshot", "gram",  # ipttt_kernel order
           "bw_scan", "bw_dz", "bw_dv", "bw_dx", "bw_dw", "bw_small", "bw_misc",
           "mse_fix")


class LayerDesc(ctypes.Structure):
    _fields_ = [
        ("d", ctypes.c_int32),
        ("d_ff", ctypes.c_int32),
        ("conv_k", ctypes.c_int32),
        ("chunk", ctypes.c_int32),
        ("max_batch", ctypes.c_int32),
        ("eta", ctypes.c_float),
        ("update", ctypes.c_int),
        ("in_dtype", ctypes.c_int),
        ("flags", ctypes.c_uint32),
        ("group_chunks", ctypes.c_int32),
        ("w_gate", ctypes.c_void_p),
        ("w_up", ctypes.c_void_p),
        ("proj", ctypes.c_void_p),
        ("conv_w", ctypes.c_void_p),
        ("w0", ctypes.c_void_p),
        ("w_state", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class Grads(ctypes.Structure):
    _fields_ = [(k, ctypes.c_void_p) for k in
                ("dx", "de", "dw_gate", "dw_up", "dproj", "dconv_w", "dw0")]


class IptttError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads libipttt.so once; raises if it is missing (build it first)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with chunked_weight_mlp_amd/build.py "
                          "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    pdesc = ctypes.POINTER(LayerDesc)
    lib.ipttt_workspace_bytes.argtypes = [pdesc, i32, i32]
    lib.ipttt_workspace_bytes.restype = ctypes.c_size_t
    lib.ipttt_init.argtypes = [pdesc, ctypes.POINTER(vp)]
    lib.ipttt_init.restype = ctypes.c_int
    lib.ipttt_prefill_layer.argtypes = [vp, vp, vp, vp, i32, i64, vp]
    lib.ipttt_prefill_layer.restype = ctypes.c_int
    lib.ipttt_prefill_layer_noalloc.argtypes = [vp, vp, vp, vp, i32, i64, vp]
    lib.ipttt_prefill_layer_noalloc.restype = ctypes.c_int
    lib.ipttt_prefill_packed.argtypes = [vp, vp, vp, vp, i32, i64, ctypes.POINTER(i64), i32, vp]
    lib.ipttt_prefill_packed.restype = ctypes.c_int
    lib.ipttt_decode_step.argtypes = [vp, vp, vp, i64, i32, vp, i32, vp]
    lib.ipttt_decode_step.restype = ctypes.c_int
    lib.ipttt_backward_workspace_bytes.argtypes = [pdesc, i32, i64]
    lib.ipttt_backward_workspace_bytes.restype = ctypes.c_size_t
    lib.ipttt_backward_layer.argtypes = [vp, vp, vp, vp, vp, i32, i64, ctypes.POINTER(Grads), vp,
                                         ctypes.c_size_t, vp]
    lib.ipttt_backward_layer.restype = ctypes.c_int
    lib.ipttt_reset_fast_weights.argtypes = [vp, i32, i32, vp]
    lib.ipttt_reset_fast_weights.restype = ctypes.c_int
    lib.ipttt_profile_begin.argtypes = [vp]
    lib.ipttt_profile_begin.restype = ctypes.c_int
    lib.ipttt_profile_end.argtypes = [vp, ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_double)]
    lib.ipttt_profile_end.restype = ctypes.c_int
    lib.ipttt_destroy.argtypes = [vp]
    lib.ipttt_destroy.restype = None
    lib.ipttt_status_str.argtypes = [ctypes.c_int]
    lib.ipttt_status_str.restype = ctypes.c_char_p
    lib.ipttt_last_error.argtypes = []
    lib.ipttt_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != IPTTT_OK:
        raise IptttError(status, ipttt_last_error() or ipttt_status_str(status))


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to libipttt must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    return stream if isinstance(stream, int) else stream.cuda_stream


def ipttt_status_str(status: int) -> str:
    return load().ipttt_status_str(status).decode()


def ipttt_last_error() -> str:
    return load().ipttt_last_error().decode()


def ipttt_workspace_bytes(desc: LayerDesc, batch: int, slab_chunks: int) -> int:
    return load().ipttt_workspace_bytes(ctypes.byref(desc), batch, slab_chunks)


def ipttt_init(desc: LayerDesc) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(load().ipttt_init(ctypes.byref(desc), ctypes.byref(h)))
    return h


def ipttt_prefill_layer(h, x, e, o, batch: int, seq_len: int, stream=None) -> None:
    _check(load().ipttt_prefill_layer(h, _ptr(x), _ptr(e), _ptr(o), batch, seq_len, _stream(stream)))


def ipttt_prefill_layer_noalloc(h, x, e, o, batch: int, seq_len: int, stream=None) -> None:
    _check(load().ipttt_prefill_layer_noalloc(h, _ptr(x), _ptr(e), _ptr(o), batch, seq_len,
                                              _stream(stream)))


def ipttt_prefill_packed(h, x, e, o, slot: int, seq_len: int, doc_starts, stream=None) -> None:
    starts = [int(p) for p in doc_starts]
    arr = (ctypes.c_int64 * max(1, len(starts)))(*starts)
    _check(load().ipttt_prefill_packed(h, _ptr(x), _ptr(e), _ptr(o), slot, seq_len, arr,
                                       len(starts), _stream(stream)))


def ipttt_decode_step(h, x, e, seq_stride: int, pos: int, o, batch: int, stream=None) -> None:
    _check(load().ipttt_decode_step(h, _ptr(x), _ptr(e), seq_stride, pos, _ptr(o), batch,
                                    _stream(stream)))


def ipttt_backward_workspace_bytes(desc: LayerDesc, batch: int, seq_len: int) -> int:
    return load().ipttt_backward_workspace_bytes(ctypes.byref(desc), batch, seq_len)


def ipttt_backward_layer(h, x, e, d_o, d_wfinal, batch: int, seq_len: int, grads: dict,
                         workspace, workspace_bytes: int, stream=None) -> None:
    """grads: {"dx", "de", "dw_gate", "dw_up", "dproj", "dconv_w", "dw0"} -> fp32 buffers."""
    g = None if grads is None else Grads(**{k: _ptr(grads[k]) for k, _ in Grads._fields_})
    _check(load().ipttt_backward_layer(h, _ptr(x), _ptr(e), _ptr(d_o), _ptr(d_wfinal), batch,
                                       seq_len, None if g is None else ctypes.byref(g),
                                       _ptr(workspace), workspace_bytes, _stream(stream)))


def ipttt_reset_fast_weights(h, first_seq: int, n_seq: int, stream=None) -> None:
    _check(load().ipttt_reset_fast_weights(h, first_seq, n_seq, _stream(stream)))


def ipttt_profile_begin(h) -> None:
    _check(load().ipttt_profile_begin(h))


def ipttt_profile_end(h) -> dict:
    """Returns {kernel: (launches, total_ms)} for the launches recorded since begin."""
    n = (ctypes.c_int32 * len(KERNELS))()
    ms = (ctypes.c_double * len(KERNELS))()
    _check(load().ipttt_profile_end(h, n, ms))
    return {k: (n[i], ms[i]) for i, k in enumerate(KERNELS)}


def ipttt_destroy(h) -> None:
    if h:
        load().ipttt_destroy(h)


_DT = {torch.float32: IPTTT_F32, torch.bfloat16: IPTTT_BF16}


class Layer:
    """One fast-weight MLP layer: owns w_state and the workspace (torch device
    tensors) and keeps the borrowed weight tensors alive for the handle.

    Weights use the library's output-major layout (see include/ipttt.h):
    w_gate / w_up [d_ff, d], proj [d, d], conv_w [d, conv_k], w0 [d, d_ff] fp32.
    """

    def __init__(self, *, w_gate, w_up, proj, conv_w, w0, chunk: int, eta: float,
                 update: str = "linear", max_batch: int = 1, workspace_bytes: int | None = None,
                 slab_chunks: int | None = None, max_seq_len: int | None = None,
                 flags: int = 0, group_chunks: int = 0):
        d_ff, d = w_gate.shape
        dtype = w_gate.dtype
        if dtype not in _DT:
            raise ValueError(f"unsupported weight dtype {dtype}")
        dev = w_gate.device
        self.tensors = dict(w_gate=w_gate, w_up=w_up, proj=proj, conv_w=conv_w, w0=w0)
        self.w_state = torch.empty((max_batch, d, d_ff), dtype=torch.float32, device=dev)
        desc = LayerDesc(d=d, d_ff=d_ff, conv_k=conv_w.shape[1], chunk=chunk, max_batch=max_batch,
                         eta=eta, update=IPTTT_UPDATE_MSE if update == "mse" else IPTTT_UPDATE_LINEAR,
                         in_dtype=_DT[dtype], flags=flags, group_chunks=group_chunks)
        if workspace_bytes is None:
            if slab_chunks is None:
                slab_chunks = 1 if max_seq_len is None else -(-max_seq_len // chunk)
            workspace_bytes = ipttt_workspace_bytes(desc, max_batch, slab_chunks)
            if workspace_bytes == 0:
                raise IptttError(IPTTT_E_INVALID, "invalid layer sizes")
        self.workspace = torch.empty(workspace_bytes, dtype=torch.uint8, device=dev)
        for k, t in self.tensors.items():
            setattr(desc, k, _ptr(t))
        desc.w_state = _ptr(self.w_state)
        desc.workspace = _ptr(self.workspace)
        desc.workspace_bytes = workspace_bytes
        self.desc = desc
        self.d, self.d_ff, self.chunk, self.dtype = d, d_ff, chunk, dtype
        self.handle = ipttt_init(desc)

    def reset(self, first_seq: int = 0, n_seq: int | None = None, stream=None) -> None:
        n = self.desc.max_batch - first_seq if n_seq is None else n_seq
        ipttt_reset_fast_weights(self.handle, first_seq, n, stream)

    def prefill(self, x, e, o=None, stream=None):
        """x, e: [batch, seq_len, d] (or [seq_len, d]); returns o fp32 of the same shape."""
        squeeze = x.dim() == 2
        x3 = x.unsqueeze(0) if squeeze else x
        e3 = e.unsqueeze(0) if squeeze else e
        if o is None:
            o = torch.empty(x3.shape, dtype=torch.float32, device=x.device)
        ipttt_prefill_layer(self.handle, x3, e3, o, x3.shape[0], x3.shape[1], stream)
        return o[0] if squeeze and o.dim() == 3 else o

    def prefill_packed(self, x, e, doc_starts, slot: int = 0, o=None, stream=None):
        """One sequence [seq_len, d] of packed documents; W resets at each start."""
        if o is None:
            o = torch.empty(x.shape, dtype=torch.float32, device=x.device)
        ipttt_prefill_packed(self.handle, x, e, o, slot, x.shape[0], doc_starts, stream)
        return o

    def decode_step(self, x_chunk, e_chunk, pos: int, o=None, stream=None):
        """x_chunk, e_chunk: [batch, B, d] buffers of the chunk in progress whose
        rows 0..pos are filled (the new token at row pos); returns o [batch, d]."""
        if o is None:
            o = torch.empty((x_chunk.shape[0], x_chunk.shape[2]), dtype=torch.float32,
                            device=x_chunk.device)
        ipttt_decode_step(self.handle, x_chunk, e_chunk, x_chunk.shape[1] * x_chunk.shape[2], pos, o,
                          x_chunk.shape[0], stream)
        return o

    def backward(self, x, e, d_o, d_wfinal=None, workspace=None, grads=None, stream=None):
        """Gradients through the scan of a prefill of x, e ([batch, seq_len, d]) that
        starts from w0, for dL/dO = d_o and dL/dW_final = d_wfinal ([batch, d, d_ff]
        fp32 or None). Returns the fp32 gradients as a dict (layouts of the inputs
        and weights); workspace / grads may be passed in to reuse buffers."""
        batch, seq_len, d = x.shape
        dev = x.device
        need = ipttt_backward_workspace_bytes(self.desc, batch, seq_len)
        if need == 0:
            raise IptttError(IPTTT_E_UNSUPPORTED, "backward unsupported for this layer or size")
        if workspace is None or workspace.numel() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        if grads is None:
            f32 = dict(dtype=torch.float32, device=dev)
            kc = self.tensors["conv_w"].shape[1]
            grads = dict(dx=torch.empty(x.shape, **f32), de=torch.empty(x.shape, **f32),
                         dw_gate=torch.empty((self.d_ff, d), **f32),
                         dw_up=torch.empty((self.d_ff, d), **f32), dproj=torch.empty((d, d), **f32),
                         dconv_w=torch.empty((d, kc), **f32), dw0=torch.empty((d, self.d_ff), **f32))
        ipttt_backward_layer(self.handle, x, e, d_o, d_wfinal, batch, seq_len, grads, workspace,
                             workspace.numel(), stream)
        return grads

    def close(self) -> None:
        if getattr(self, "handle", None):
            ipttt_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
