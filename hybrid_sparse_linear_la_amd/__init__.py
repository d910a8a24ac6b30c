"""MI355X (gfx950) causal linear-attention ("Lightning Attention") layer.

A thin ctypes binding over ``liblightning_la.so`` (C ABI in
``include/lightning_la.h``).  This module only marshals arguments: it checks
dtypes/shapes, allocates outputs and workspace with torch on the tensors' device
and passes raw pointers plus the current HIP stream.  Every step of the layer
runs in the library's HIP kernels; there is no fallback path.  If the library
is missing, every call raises.

    o, S_out = prefill(q, k, v, gate, S_in=None, pos0=0)
    o, S_out = prefill_noalloc(q, k, v, gate, S_in=None, pos0=0)   # no workspace
    o = decode_step(q, k, v, gate, S, pos)        # S updated in place
    o, S_out = prefill_varlen(q, k, v, gate, cu_seqlens, pos0=None, S_in=None)
    y = linear(x, w)                              # y = x w^T
    y, S_out = layer_forward(x, w_qkvg, w_o, S_in=None, pos0=0)
    grads = backward(q, k, v, gate, d_o, S_in=None, dS_out=None, pos0=0)
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["prefill", "prefill_noalloc", "decode_step", "prefill_varlen", "linear", "layer_forward", "backward",
           "prefill_workspace_bytes", "backward_workspace_bytes",
           "layer_workspace_bytes",
           "prefill_varlen_workspace_bytes", "LAError", "library", "lib_path",
           "STATUS", "HEAD_DIM", "DEFAULT_CHUNK", "SUPPORTED_CHUNKS",
           "sparse_prefill", "sparse_prefill_workspace_bytes", "sparse_block_means", "sparse_decode",
           "SPARSE_BLOCK"]

_PKG = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_PKG, "liblightning_la.so")

HEAD_DIM = 128
DEFAULT_CHUNK = 64
SUPPORTED_CHUNKS = (0, 64, 128, 256)
SPARSE_BLOCK = 64
STATUS = {
    0: "LA_OK", 1: "LA_ERR_NULL_PTR", 2: "LA_ERR_BAD_SHAPE", 3: "LA_ERR_UNSUPPORTED",
    4: "LA_ERR_ALIGNMENT", 5: "LA_ERR_ALIASING", 6: "LA_ERR_WORKSPACE", 7: "LA_ERR_HIP",
    8: "LA_ERR_CAPTURING",
}

_vp = ctypes.c_void_p
_lib = None


class LAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def library():
    """Load liblightning_la.so (built by ``__graft_entry__.build()``); raise if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise ImportError(f"{lib_path} is not built; run __graft_entry__.build() first")
        lib = ctypes.CDLL(lib_path)
        lib.la_version.restype = ctypes.c_int
        lib.la_status_string.restype = ctypes.c_char_p
        lib.la_status_string.argtypes = [ctypes.c_int]
        lib.la_prefill_workspace_bytes.restype = ctypes.c_size_t
        lib.la_prefill_workspace_bytes.argtypes = [ctypes.c_int] * 5
        lib.la_prefill.restype = ctypes.c_int
        lib.la_prefill.argtypes = [_vp] * 7 + [ctypes.c_int] * 4 + [
            ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_float, _vp, _vp, _vp,
            ctypes.c_size_t, _vp]
        lib.la_prefill_profiled.restype = ctypes.c_int
        lib.la_prefill_profiled.argtypes = lib.la_prefill.argtypes + [ctypes.POINTER(ctypes.c_void_p),
                                                                      ctypes.c_int]
        lib.la_prefill_noalloc.restype = ctypes.c_int
        lib.la_prefill_noalloc.argtypes = [_vp] * 7 + [ctypes.c_int] * 4 + [
            ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_float, _vp, _vp, _vp]
        lib.la_prefill_varlen_workspace_bytes.restype = ctypes.c_size_t
        lib.la_prefill_varlen_workspace_bytes.argtypes = [ctypes.c_int, _vp, ctypes.c_int, ctypes.c_int,
                                                          ctypes.c_int]
        lib.la_prefill_varlen.restype = ctypes.c_int
        lib.la_prefill_varlen.argtypes = [_vp] * 9 + [ctypes.c_int] * 5 + [
            ctypes.c_float, ctypes.c_float, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        lib.la_linear.restype = ctypes.c_int
        lib.la_linear.argtypes = [_vp, _vp, _vp, ctypes.c_int64, ctypes.c_int, ctypes.c_int, _vp]
        lib.la_layer_workspace_bytes.restype = ctypes.c_size_t
        lib.la_layer_workspace_bytes.argtypes = [ctypes.c_int] * 5
        lib.la_layer_forward.restype = ctypes.c_int
        lib.la_layer_forward.argtypes = [_vp] * 6 + [ctypes.c_int] * 5 + [
            ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_float, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        lib.la_backward_workspace_bytes.restype = ctypes.c_size_t
        lib.la_backward_workspace_bytes.argtypes = [ctypes.c_int] * 5
        lib.la_backward.restype = ctypes.c_int
        lib.la_backward.argtypes = [_vp] * 14 + [ctypes.c_int] * 4 + [
            ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_float, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        lib.la_backward_saved.restype = ctypes.c_int
        lib.la_backward_saved.argtypes = lib.la_backward.argtypes[:-1] + [_vp, ctypes.c_size_t, _vp]
        lib.la_decode_step.restype = ctypes.c_int
        lib.la_decode_step.argtypes = [_vp] * 6 + [ctypes.c_int] * 3 + [
            ctypes.c_int64, ctypes.c_float, ctypes.c_float, _vp, _vp, _vp]
        lib.la_sparse_prefill_workspace_bytes.restype = ctypes.c_size_t
        lib.la_sparse_prefill_workspace_bytes.argtypes = [ctypes.c_int] * 6
        lib.la_sparse_prefill.restype = ctypes.c_int
        lib.la_sparse_prefill.argtypes = [_vp] * 6 + [ctypes.c_int] * 6 + [_vp, ctypes.c_size_t, _vp]
        lib.la_sparse_block_means.restype = ctypes.c_int
        lib.la_sparse_block_means.argtypes = [_vp, _vp] + [ctypes.c_int] * 7 + [_vp]
        lib.la_sparse_decode.restype = ctypes.c_int
        lib.la_sparse_decode.argtypes = [_vp] * 8 + [ctypes.c_int] * 6 + [_vp]
        _lib = lib
    return _lib


def _check(status: int):
    if status != 0:
        msg = library().la_status_string(status).decode()
        raise LAError(status, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _on_gpu(t) -> bool:
    return t.is_cuda


def _act(name, t, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if t.dim() != ndim or t.shape[-1] != HEAD_DIM:
        raise ValueError(f"{name} must have {ndim} dims with last dim {HEAD_DIM}, got {tuple(t.shape)}")
    if not _on_gpu(t) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous GPU tensor")


def _like(name, t, ref, dtype=torch.bfloat16):
    """An output the caller supplies: the library writes as many bytes as ``ref``
    describes, so its dtype, shape and device must be exactly ``ref``'s."""
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or tuple(t.shape) != tuple(ref.shape) \
            or t.device != ref.device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(ref.shape)} "
                         f"on {ref.device}")


def _f32(name, t, shape, device):
    if t is None:
        return
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or tuple(t.shape) != tuple(shape) \
            or not _on_gpu(t) or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous fp32 tensor of shape {tuple(shape)} on {device}")


def _workspace(t, need, device):
    """The caller's workspace if it is a large enough contiguous buffer on the
    device, else a new one."""
    if t is None:
        return torch.empty(need, dtype=torch.uint8, device=device)
    if not isinstance(t, torch.Tensor) or t.device != device or not t.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")
    if t.numel() * t.element_size() < need:
        return torch.empty(need, dtype=torch.uint8, device=device)
    return t


def prefill_workspace_bytes(B: int, T: int, H: int, D: int = HEAD_DIM, chunk: int = 0) -> int:
    return int(library().la_prefill_workspace_bytes(B, T, H, D, chunk))


def prefill(q, k, v, gate, S_in=None, pos0: int = 0, chunk: int = 0, rope_base: float = 10000.0,
            rms_eps: float = 1e-6, q_norm_w=None, k_norm_w=None, out=None, S_out=None,
            workspace=None, events=None):
    """Chunked prefill.  q, k, v, gate: bf16 [B, T, H, 128] on the GPU.

    Returns (o bf16 [B, T, H, 128], S_out fp32 [B, H, 128, 128]).  ``S_out`` may be
    given (and may be ``S_in`` itself, for an in-place carry).  ``events``: four raw
    hipEvent_t handles recorded around the library's three kernels (profiling)."""
    lib = library()
    for n, t in (("q", q), ("k", k), ("v", v), ("gate", gate)):
        _act(n, t, 4)
        if t.shape != q.shape or t.device != q.device:
            raise ValueError(f"{n} must match q's shape and device")
    B, T, H, D = q.shape
    dev = q.device
    _f32("S_in", S_in, (B, H, D, D), dev)
    _f32("q_norm_w", q_norm_w, (D,), dev)
    _f32("k_norm_w", k_norm_w, (D,), dev)
    if out is None:
        out = torch.empty_like(q)
    else:
        _like("out", out, q)
    if S_out is None:
        S_out = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    else:
        _f32("S_out", S_out, (B, H, D, D), dev)
    need = int(lib.la_prefill_workspace_bytes(B, T, H, D, chunk))
    if need == 0:
        status = 3 if (D != HEAD_DIM or chunk not in SUPPORTED_CHUNKS) else 2
        raise LAError(status, lib.la_status_string(status).decode())
    workspace = _workspace(workspace, need, dev)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(S_in), _ptr(S_out), _ptr(out),
            B, T, H, D, int(pos0), int(chunk), float(rope_base), float(rms_eps),
            _ptr(q_norm_w), _ptr(k_norm_w), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(q.device))
    if events is None:
        _check(lib.la_prefill(*args))
    else:
        arr = (ctypes.c_void_p * len(events))(*events)
        _check(lib.la_prefill_profiled(*args, arr, len(events)))
    return out, S_out


def prefill_noalloc(q, k, v, gate, S_in=None, pos0: int = 0, chunk: int = 0, rope_base: float = 10000.0,
                    rms_eps: float = 1e-6, q_norm_w=None, k_norm_w=None, out=None, S_out=None):
    """``prefill`` through la_prefill_noalloc: no workspace, the library's static
    device scratch instead.  Pass ``out`` and ``S_out`` to make the call allocate
    nothing at all (e.g. under graph capture).  Calls that overlap in time on one
    GPU share that scratch and race."""
    lib = library()
    for n, t in (("q", q), ("k", k), ("v", v), ("gate", gate)):
        _act(n, t, 4)
        if t.shape != q.shape or t.device != q.device:
            raise ValueError(f"{n} must match q's shape and device")
    B, T, H, D = q.shape
    dev = q.device
    _f32("S_in", S_in, (B, H, D, D), dev)
    _f32("q_norm_w", q_norm_w, (D,), dev)
    _f32("k_norm_w", k_norm_w, (D,), dev)
    if out is None:
        out = torch.empty_like(q)
    else:
        _like("out", out, q)
    if S_out is None:
        S_out = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    else:
        _f32("S_out", S_out, (B, H, D, D), dev)
    _check(lib.la_prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(S_in), _ptr(S_out), _ptr(out),
                                  B, T, H, D, int(pos0), int(chunk), float(rope_base), float(rms_eps),
                                  _ptr(q_norm_w), _ptr(k_norm_w), _stream(dev)))
    return out, S_out


def _host_array(name, values, ctype, n):
    """Host copy of a length-n integer sequence as a ctypes array."""
    if isinstance(values, torch.Tensor):
        values = values.detach().cpu().tolist()
    values = [int(x) for x in values]
    if len(values) != n:
        raise ValueError(f"{name} must have {n} entries, got {len(values)}")
    return (ctype * n)(*values)


def prefill_varlen_workspace_bytes(cu_seqlens, H: int, D: int = HEAD_DIM, chunk: int = 0) -> int:
    cu = _host_array("cu_seqlens", cu_seqlens, ctypes.c_int32, len(cu_seqlens))
    return int(library().la_prefill_varlen_workspace_bytes(len(cu) - 1, cu, H, D, chunk))


def prefill_varlen(q, k, v, gate, cu_seqlens, pos0=None, S_in=None, chunk: int = 0,
                   rope_base: float = 10000.0, rms_eps: float = 1e-6, q_norm_w=None, k_norm_w=None,
                   out=None, S_out=None, workspace=None):
    """Variable-length batch.  q, k, v, gate: bf16 [total_T, H, 128] holding the
    sequences back to back; cu_seqlens: nseq + 1 offsets (host list or CPU tensor);
    pos0: nseq start positions or None; S_in/S_out: fp32 [nseq, H, 128, 128].

    Returns (o bf16 [total_T, H, 128], S_out)."""
    lib = library()
    for n, t in (("q", q), ("k", k), ("v", v), ("gate", gate)):
        _act(n, t, 3)
        if t.shape != q.shape or t.device != q.device:
            raise ValueError(f"{n} must match q's shape and device")
    total_T, H, D = q.shape
    nseq = len(cu_seqlens) - 1
    cu = _host_array("cu_seqlens", cu_seqlens, ctypes.c_int32, nseq + 1)
    p0 = None if pos0 is None else _host_array("pos0", pos0, ctypes.c_int64, nseq)
    dev = q.device
    _f32("S_in", S_in, (nseq, H, D, D), dev)
    _f32("q_norm_w", q_norm_w, (D,), dev)
    _f32("k_norm_w", k_norm_w, (D,), dev)
    if out is None:
        out = torch.empty_like(q)
    else:
        _like("out", out, q)
    if S_out is None:
        S_out = torch.empty((nseq, H, D, D), dtype=torch.float32, device=dev)
    else:
        _f32("S_out", S_out, (nseq, H, D, D), dev)
    need = int(lib.la_prefill_varlen_workspace_bytes(nseq, cu, H, D, chunk))
    if need == 0:
        status = 3 if (D != HEAD_DIM or chunk not in SUPPORTED_CHUNKS) else 2
        raise LAError(status, lib.la_status_string(status).decode())
    workspace = _workspace(workspace, need, dev)
    _check(lib.la_prefill_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), cu, p0, _ptr(S_in), _ptr(S_out),
                                 _ptr(out), nseq, total_T, H, D, int(chunk), float(rope_base),
                                 float(rms_eps), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(q.device)))
    return out, S_out


def _bf16_2d(name, t):
    if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or not _on_gpu(t) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous bf16 GPU tensor")


def linear(x, w, out=None):
    """y = x w^T.  x: bf16 [..., K] (contiguous), w: bf16 [N, K].  Returns bf16 [..., N]."""
    _bf16_2d("x", x)
    _bf16_2d("w", w)
    if w.dim() != 2 or x.shape[-1] != w.shape[1]:
        raise ValueError(f"x [..., K] and w [N, K] do not match: {tuple(x.shape)}, {tuple(w.shape)}")
    if w.device != x.device:
        raise ValueError("x and w must be on the same device")
    N, K = w.shape
    M = x.numel() // K
    if out is None:
        out = torch.empty(tuple(x.shape[:-1]) + (N,), dtype=torch.bfloat16, device=x.device)
    else:
        _bf16_2d("out", out)
        if out.numel() != M * N or out.shape[-1] != N or out.device != x.device:
            raise ValueError(f"out must hold [..., {N}] with {M * N} elements on {x.device}")
    _check(library().la_linear(_ptr(x), _ptr(w), _ptr(out), M, N, K, _stream(x.device)))
    return out


def layer_workspace_bytes(B: int, T: int, H: int, D: int = HEAD_DIM, chunk: int = 0) -> int:
    return int(library().la_layer_workspace_bytes(B, T, H, D, chunk))


def layer_forward(x, w_qkvg, w_o, S_in=None, pos0: int = 0, chunk: int = 0, rope_base: float = 10000.0,
                  rms_eps: float = 1e-6, q_norm_w=None, k_norm_w=None, out=None, S_out=None, workspace=None):
    """One layer: [q|k|v|g] = x w_qkvg^T, la_prefill, y = o w_o^T.  x: bf16 [B, T, hidden];
    w_qkvg: bf16 [4 H 128, hidden]; w_o: bf16 [hidden, H 128].  Returns (y, S_out)."""
    lib = library()
    _bf16_2d("x", x)
    _bf16_2d("w_qkvg", w_qkvg)
    _bf16_2d("w_o", w_o)
    if x.dim() != 3:
        raise ValueError("x must be [B, T, hidden]")
    B, T, hidden = x.shape
    HD = w_o.shape[1]
    if HD % HEAD_DIM or tuple(w_qkvg.shape) != (4 * HD, hidden) or tuple(w_o.shape) != (hidden, HD):
        raise ValueError("weights must be w_qkvg [4 H 128, hidden] and w_o [hidden, H 128]")
    H, D = HD // HEAD_DIM, HEAD_DIM
    dev = x.device
    if w_qkvg.device != dev or w_o.device != dev:
        raise ValueError("x and the weights must be on the same device")
    _f32("S_in", S_in, (B, H, D, D), dev)
    _f32("q_norm_w", q_norm_w, (D,), dev)
    _f32("k_norm_w", k_norm_w, (D,), dev)
    if out is None:
        out = torch.empty_like(x)
    else:
        _like("out", out, x)
    if S_out is None:
        S_out = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    else:
        _f32("S_out", S_out, (B, H, D, D), dev)
    need = int(lib.la_layer_workspace_bytes(B, T, H, D, chunk))
    if need == 0:
        raise LAError(2, lib.la_status_string(2).decode())
    workspace = _workspace(workspace, need, dev)
    _check(lib.la_layer_forward(_ptr(x), _ptr(w_qkvg), _ptr(w_o), _ptr(S_in), _ptr(S_out), _ptr(out), B, T,
                                hidden, H, D, int(pos0), int(chunk), float(rope_base), float(rms_eps),
                                _ptr(q_norm_w), _ptr(k_norm_w), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(x.device)))
    return out, S_out


def backward_workspace_bytes(B: int, T: int, H: int, D: int = HEAD_DIM, chunk: int = 0) -> int:
    return int(library().la_backward_workspace_bytes(B, T, H, D, chunk))


def backward(q, k, v, gate, d_o, S_in=None, dS_out=None, pos0: int = 0, chunk: int = 0,
             rope_base: float = 10000.0, rms_eps: float = 1e-6, q_norm_w=None, k_norm_w=None,
             weight_grads: bool = False, workspace=None, fwd_workspace=None):
    """Gradients of la_prefill for output gradient d_o (bf16 [B, T, H, 128]) and
    final-state gradient dS_out (fp32 [B, H, 128, 128] or None).  Returns a dict
    with dq, dk, dv, dgate (bf16), dS_in (fp32) and, with weight_grads, dq_norm_w
    and dk_norm_w (fp32 [128]; at weights of one when none are given).
    ``fwd_workspace``: the workspace of the ``prefill`` call that computed this
    forward (la_backward_saved: its segment states are reused)."""
    lib = library()
    for n, t in (("q", q), ("k", k), ("v", v), ("gate", gate), ("d_o", d_o)):
        _act(n, t, 4)
        if t.shape != q.shape or t.device != q.device:
            raise ValueError(f"{n} must match q's shape and device")
    B, T, H, D = q.shape
    dev = q.device
    _f32("S_in", S_in, (B, H, D, D), dev)
    _f32("dS_out", dS_out, (B, H, D, D), dev)
    _f32("q_norm_w", q_norm_w, (D,), dev)
    _f32("k_norm_w", k_norm_w, (D,), dev)
    out = {n: torch.empty_like(q) for n in ("dq", "dk", "dv", "dgate")}
    out["dS_in"] = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
    if weight_grads:
        out["dq_norm_w"] = torch.empty(D, dtype=torch.float32, device=q.device)
        out["dk_norm_w"] = torch.empty(D, dtype=torch.float32, device=q.device)
    need = int(lib.la_backward_workspace_bytes(B, T, H, D, chunk))
    if need == 0:
        status = 3 if (D != HEAD_DIM or chunk not in (0, 64)) else 2
        raise LAError(status, lib.la_status_string(status).decode())
    workspace = _workspace(workspace, need, dev)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(S_in), _ptr(d_o), _ptr(dS_out),
            _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dgate"]),
            _ptr(out["dS_in"]), _ptr(out.get("dq_norm_w")), _ptr(out.get("dk_norm_w")), B, T, H, D,
            int(pos0), int(chunk), float(rope_base), float(rms_eps), _ptr(q_norm_w),
            _ptr(k_norm_w), _ptr(workspace), workspace.numel() * workspace.element_size())
    if fwd_workspace is None:
        _check(lib.la_backward(*args, _stream(q.device)))
    else:
        if not isinstance(fwd_workspace, torch.Tensor) or fwd_workspace.device != dev or \
                not fwd_workspace.is_contiguous():
            raise ValueError(f"fwd_workspace must be a contiguous tensor on {dev}")
        _check(lib.la_backward_saved(*args, _ptr(fwd_workspace),
                                     fwd_workspace.numel() * fwd_workspace.element_size(), _stream(q.device)))
    return out


def decode_step(q, k, v, gate, S, pos: int, rope_base: float = 10000.0, rms_eps: float = 1e-6,
                q_norm_w=None, k_norm_w=None, out=None):
    """One decode step.  q, k, v, gate: bf16 [B, H, 128]; S: fp32 [B, H, 128, 128],
    updated in place.  Returns o bf16 [B, H, 128]."""
    lib = library()
    for n, t in (("q", q), ("k", k), ("v", v), ("gate", gate)):
        _act(n, t, 3)
        if t.shape != q.shape or t.device != q.device:
            raise ValueError(f"{n} must match q's shape and device")
    B, H, D = q.shape
    dev = q.device
    if S is None:
        raise ValueError("S must be given (it is updated in place)")
    _f32("S", S, (B, H, D, D), dev)
    _f32("q_norm_w", q_norm_w, (D,), dev)
    _f32("k_norm_w", k_norm_w, (D,), dev)
    if out is None:
        out = torch.empty_like(q)
    else:
        _like("out", out, q)
    _check(lib.la_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(S), _ptr(out), B, H, D,
                              int(pos), float(rope_base), float(rms_eps), _ptr(q_norm_w),
                              _ptr(k_norm_w), _stream(q.device)))
    return out


# ---- sparse attention layers (block selection, NoPE, output gate)

def sparse_prefill_workspace_bytes(B: int, T: int, H: int, D: int = HEAD_DIM, topk: int = 16) -> int:
    return int(library().la_sparse_prefill_workspace_bytes(B, T, H, D, 0, topk))


def sparse_prefill(q, k, v, gate, topk: int = 16, return_sel: bool = False, out=None, workspace=None):
    """Sparse layer over whole sequences.  q, k, v, gate: bf16 [B, T, H, 128] on the
    GPU.  Returns o (bf16, shaped as q), and with ``return_sel`` also the chosen key
    blocks (int32 [B, H, ceil(T / 64), topk], increasing, then -1)."""
    lib = library()
    for n, t in (("q", q), ("k", k), ("v", v), ("gate", gate)):
        _act(n, t, 4)
        if t.shape != q.shape or t.device != q.device:
            raise ValueError(f"{n} must match q's shape and device")
    B, T, H, D = q.shape
    o = torch.empty_like(q) if out is None else out
    _like("out", o, q)
    nqb = -(-T // SPARSE_BLOCK)
    sel = torch.empty((B, H, nqb, topk), dtype=torch.int32, device=q.device) if return_sel else None
    need = int(lib.la_sparse_prefill_workspace_bytes(B, T, H, D, 0, topk))
    if need == 0:
        raise LAError(3, lib.la_status_string(3).decode())
    workspace = _workspace(workspace, need, q.device)
    _check(lib.la_sparse_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(o), _ptr(sel), B, T, H, D, 0,
                                 int(topk), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _stream(q.device)))
    return (o, sel) if return_sel else o


def sparse_block_means(k_cache, means=None, first_block: int = 0, nblocks=None):
    """Block means (fp32 [B, H, Tmax / 64, 128]) of a key cache [B, Tmax, H, 128];
    only blocks [first_block, first_block + nblocks) are (re)computed."""
    lib = library()
    _act("k_cache", k_cache, 4)
    B, Tmax, H, D = k_cache.shape
    shape = (B, H, Tmax // SPARSE_BLOCK, D)
    if means is None:
        means = torch.zeros(shape, dtype=torch.float32, device=k_cache.device)
    _f32("means", means, shape, k_cache.device)
    if nblocks is None:
        nblocks = Tmax // SPARSE_BLOCK - first_block
    _check(lib.la_sparse_block_means(_ptr(k_cache), _ptr(means), B, Tmax, H, D, 0, int(first_block), int(nblocks),
                                     _stream(k_cache.device)))
    return means


def sparse_decode(q, k_cache, v_cache, means, gate, lens, topk: int = 16, return_sel: bool = False, out=None):
    """One decode step of the sparse layer.  q, gate: bf16 [B, H, 128] (the newest
    token's query; its k, v already in the caches); k_cache, v_cache: bf16
    [B, Tmax, H, 128]; means: their block means; lens: int32 [B] on the GPU (valid
    tokens, the newest included).  Returns o bf16 [B, H, 128] (and the chosen blocks,
    int32 [B, H, topk], with ``return_sel``)."""
    lib = library()
    _act("q", q, 3)
    _act("gate", gate, 3)
    _act("k_cache", k_cache, 4)
    _act("v_cache", v_cache, 4)
    B, Tmax, H, D = k_cache.shape
    dev = q.device
    if v_cache.shape != k_cache.shape or q.shape != (B, H, D) or gate.shape != q.shape:
        raise ValueError("shapes of q, gate, k_cache, v_cache disagree")
    if any(t.device != dev for t in (gate, k_cache, v_cache)):
        raise ValueError("q, gate, k_cache and v_cache must be on the same device")
    _f32("means", means, (B, H, Tmax // SPARSE_BLOCK, D), dev)
    if not isinstance(lens, torch.Tensor) or lens.dtype != torch.int32 or tuple(lens.shape) != (B,) \
            or lens.device != dev or not lens.is_contiguous():
        raise ValueError(f"lens must be a contiguous int32 tensor of shape [{B}] on {dev}")
    o = torch.empty_like(q) if out is None else out
    _like("out", o, q)
    sel = torch.empty((B, H, topk), dtype=torch.int32, device=q.device) if return_sel else None
    _check(lib.la_sparse_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(means), _ptr(gate), _ptr(lens),
                                _ptr(o), _ptr(sel), B, Tmax, H, D, 0, int(topk), _stream(q.device)))
    return (o, sel) if return_sel else o
