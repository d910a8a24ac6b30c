"""fp64 CPU oracle of the causal linear-attention (Lightning Attention) layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The HIP library never
imports, links or calls it, and it shares no code with the HIP library.

The arithmetic lives in ``la_oracle.c`` (plain C, double precision, OpenMP over
independent (batch, head, value-column block) tasks); this module only builds
and loads it and marshals numpy arrays.  Every function takes inputs as float32
arrays (exact images of bf16 or fp32 data) and returns float64 results.

What each function follows (pages cited by title and section):
  * ``rmsnorm_row`` / ``rope_row`` / ``prologue`` -- QK-normalization and RoPE of
    the linear layers: "創新Transformer！面壁基於稀疏-線性混合架構SALA訓練9B模型"
    (MiniCPM-SALA technical-report rendering), 02 模型架構 (3) 線性注意力模塊 and
    (4) 混合位置編碼 (HyPE).
  * ``forward`` -- the state update S_t = S_{t-1} + k_t v_t^T of "MiniCPM-SALA:
    Hybridizing Sparse and Linear Attention for Efficient Long-Context Modeling"
    (paper digest), 前置知识 > 线性注意力, read out as o_t = sigmoid(g_t) * (q_t S_t).
  * ``chunked`` -- the same sum regrouped by chunks (for the chunk invariance check).
  * ``decode_step`` -- ``forward`` with one token.
  * ``backward`` -- the gradients of ``forward`` (reverse mode of the same
    recurrence, through the gate, RoPE and RMSNorm) for given output and
    final-state gradients; what training the converted linear layers needs
    (technical-report page, 03 模型訓練: the linear layers are trained after
    conversion).
  * ``linear`` / ``layer_forward`` -- the projections around the layer (one
    fused q/k/v/gate projection and the output projection; hidden 4096, 32 heads
    of 128, MHA): the technical-report rendering above, 02 模型架構 (3)
    線性注意力模塊.  ``linear`` is a float64 matrix product (numpy); the layer
    composes it with ``forward`` and, like the GPU path, rounds the projected
    q, k, v, g and the layer output o to bfloat16 (nearest-even) where they are
    handed on, so the comparison measures the layer's arithmetic rather than the
    hand-over format.
  * ``sparse_forward`` / ``sparse_decode`` -- the sparse attention layers of the
    same hybrid (block selection, NoPE, output gate): technical-report rendering,
    02 模型架構 (2) 稀疏注意力模塊 and (4) 混合位置編碼, and "9B端側開源模型跑通百萬上下文，
    面壁全新稀疏-線性混合注意力" (architecture section).  The arithmetic is in
    ``sparse_oracle.c`` (own library), whose header lists the readings taken where
    the pages are silent.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_DIR, "la_oracle.c")
_LIB = os.path.join(_DIR, "liblaoracle.so")
_lib = None

_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)


def build(force: bool = True) -> str:
    """Compile la_oracle.c into liblaoracle.so with gcc (-O2 -fopenmp)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _bind(lib):
    lib.lao_set_threads.argtypes = [ctypes.c_int]
    lib.lao_get_threads.restype = ctypes.c_int
    lib.lao_rmsnorm_row.argtypes = [_f64p, ctypes.c_int, ctypes.c_double, _f32p, _f64p]
    lib.lao_rope_row.argtypes = [_f64p, ctypes.c_int, ctypes.c_int64, ctypes.c_double, _f64p]
    lib.lao_prologue.argtypes = [_f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_int64, ctypes.c_double, ctypes.c_double, _f32p, _f64p]
    common = [_f32p, _f32p, _f32p, _f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
              ctypes.c_int64, ctypes.c_double, ctypes.c_double, _f32p, _f32p]
    lib.lao_forward.argtypes = common + [_f64p, _f64p]
    lib.lao_chunked.argtypes = common + [ctypes.c_int, _f64p, _f64p]
    if hasattr(lib, "lao_backward"):
        lib.lao_backward.argtypes = [_f32p] * 5 + [ctypes.c_int] * 4 + [
            ctypes.c_int64, ctypes.c_double, ctypes.c_double, _f32p, _f32p, _f64p, _f64p] + [_f64p] * 7
    return lib


_SPARSE_SRC = os.path.join(_DIR, "sparse_oracle.c")
_SPARSE_LIB = os.path.join(_DIR, "libsparseoracle.so")
_slib = None
_i32p = ctypes.POINTER(ctypes.c_int32)


def build_sparse(force: bool = True) -> str:
    """Compile sparse_oracle.c into libsparseoracle.so with gcc (-O2 -fopenmp)."""
    if force or not os.path.exists(_SPARSE_LIB) or os.path.getmtime(_SPARSE_LIB) < os.path.getmtime(_SPARSE_SRC):
        tmp = _SPARSE_LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", _SPARSE_SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _SPARSE_LIB)
    return _SPARSE_LIB


def _bind_sparse(lib):
    lib.lso_set_threads.argtypes = [ctypes.c_int]
    lib.lso_sparse_forward.argtypes = [_f32p] * 4 + [ctypes.c_int] * 6 + [_i32p, ctypes.c_int, _f64p, _f64p]
    lib.lso_sparse_decode.argtypes = [_f32p] * 4 + [_i32p] + [ctypes.c_int] * 6 + [_i32p, ctypes.c_int, _f64p,
                                                                                       _f64p]
    return lib


def _load_sparse():
    global _slib
    if _slib is None:
        if not os.path.exists(_SPARSE_LIB) or os.path.getmtime(_SPARSE_LIB) < os.path.getmtime(_SPARSE_SRC):
            build_sparse(force=True)
        _slib = _bind_sparse(ctypes.CDLL(_SPARSE_LIB))
    return _slib


@contextlib.contextmanager
def use_sparse_library(path: str):
    """Temporarily route the sparse-layer calls to another build of sparse_oracle.c."""
    global _slib
    saved = _load_sparse()
    _slib = _bind_sparse(ctypes.CDLL(path))
    try:
        yield
    finally:
        _slib = saved


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


@contextlib.contextmanager
def use_library(path: str):
    """Temporarily route every call of this module to another build of la_oracle.c
    (used by the tests that plant mistakes in a copy of the oracle)."""
    global _lib
    saved = _load()
    _lib = _bind(ctypes.CDLL(path))
    try:
        yield
    finally:
        _lib = saved


def set_threads(n: int) -> None:
    _load().lao_set_threads(int(n))


def get_threads() -> int:
    return int(_load().lao_get_threads())


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _p32(a):
    return None if a is None else a.ctypes.data_as(_f32p)


def _p64(a):
    return None if a is None else a.ctypes.data_as(_f64p)


def rmsnorm_row(x, eps: float = 1e-6, w=None) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    w = None if w is None else _f32(w)
    out = np.empty_like(x)
    _load().lao_rmsnorm_row(_p64(x), x.shape[-1], float(eps), _p32(w), _p64(out))
    return out


def rope_row(x, pos: int, base: float = 10000.0) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty_like(x)
    _load().lao_rope_row(_p64(x), x.shape[-1], int(pos), float(base), _p64(out))
    return out


def prologue(x, pos0: int = 0, base: float = 10000.0, eps: float = 1e-6, w=None) -> np.ndarray:
    """RMSNorm then RoPE on a [B, T, H, D] tensor (token t at position pos0 + t)."""
    x = _f32(x)
    B, T, H, D = x.shape
    w = None if w is None else _f32(w)
    out = np.empty(x.shape, dtype=np.float64)
    _load().lao_prologue(_p32(x), B, T, H, D, int(pos0), float(base), float(eps), _p32(w), _p64(out))
    return out


def _prep(q, k, v, g, S):
    q, k, v, g = _f32(q), _f32(k), _f32(v), _f32(g)
    B, T, H, D = q.shape
    for a in (k, v, g):
        assert a.shape == q.shape, (a.shape, q.shape)
    St = np.zeros((B, H, D, D), np.float64) if S is None else np.array(S, dtype=np.float64, order="C")
    assert St.shape == (B, H, D, D)
    return q, k, v, g, St, (B, T, H, D)


def forward(q, k, v, g, S=None, pos0: int = 0, base: float = 10000.0, eps: float = 1e-6,
            q_w=None, k_w=None):
    """Token-by-token recurrence.  Returns (o [B,T,H,D] f64, S_out [B,H,D,D] f64)."""
    q, k, v, g, St, (B, T, H, D) = _prep(q, k, v, g, S)
    q_w = None if q_w is None else _f32(q_w)
    k_w = None if k_w is None else _f32(k_w)
    o = np.empty((B, T, H, D), np.float64)
    _load().lao_forward(_p32(q), _p32(k), _p32(v), _p32(g), B, T, H, D, int(pos0), float(base),
                        float(eps), _p32(q_w), _p32(k_w), _p64(St), _p64(o))
    return o, St


def chunked(q, k, v, g, C: int, S=None, pos0: int = 0, base: float = 10000.0, eps: float = 1e-6,
            q_w=None, k_w=None):
    """Chunk-by-chunk form of the same layer.  Returns (o, S_out) in f64."""
    q, k, v, g, St, (B, T, H, D) = _prep(q, k, v, g, S)
    q_w = None if q_w is None else _f32(q_w)
    k_w = None if k_w is None else _f32(k_w)
    o = np.empty((B, T, H, D), np.float64)
    _load().lao_chunked(_p32(q), _p32(k), _p32(v), _p32(g), B, T, H, D, int(pos0), float(base),
                        float(eps), _p32(q_w), _p32(k_w), int(C), _p64(St), _p64(o))
    return o, St


def decode_step(q, k, v, g, S, pos: int, base: float = 10000.0, eps: float = 1e-6,
                q_w=None, k_w=None):
    """One token per sequence: q, k, v, g are [B, H, D]; S is [B, H, D, D].

    Returns (o [B, H, D] f64, S_new [B, H, D, D] f64)."""
    q, k, v, g = (np.asarray(a)[:, None] for a in (q, k, v, g))
    o, S_new = forward(q, k, v, g, S=S, pos0=pos, base=base, eps=eps, q_w=q_w, k_w=k_w)
    return o[:, 0], S_new


def linear(x, w) -> np.ndarray:
    """y = x w^T in float64: x [..., K], w [N, K] (the nn.Linear weight layout)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    return x @ w.T


def round_bf16(a) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even), returned as float32."""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32).copy()
    nan = np.isnan(a)
    out[nan] = a[nan]
    return out


def layer_forward(x, w_qkvg, w_o, S=None, pos0: int = 0, base: float = 10000.0, eps: float = 1e-6,
                  q_w=None, k_w=None):
    """[q | k | v | g] = x w_qkvg^T (column blocks of H * D), then ``forward``, then
    y = o w_o^T.  x [B, T, hidden]; returns (y [B, T, hidden] f64, S_out f64)."""
    x = np.asarray(x, dtype=np.float64)
    B, T, hidden = x.shape
    HD = np.asarray(w_o).shape[1]
    D = 128
    H = HD // D
    proj = linear(x, w_qkvg)
    q, k, v, g = (round_bf16(proj[..., i * HD:(i + 1) * HD]).reshape(B, T, H, D) for i in range(4))
    o, S_out = forward(q, k, v, g, S=S, pos0=pos0, base=base, eps=eps, q_w=q_w, k_w=k_w)
    y = linear(round_bf16(o.reshape(B, T, HD)), w_o)
    return y, S_out


def backward(q, k, v, g, do, S=None, dS_out=None, pos0: int = 0, base: float = 10000.0,
             eps: float = 1e-6, q_w=None, k_w=None) -> dict:
    """Gradients of the loss L with dL/do = do and dL/dS_out = dS_out (None = 0).

    Returns dq, dk, dv, dg ([B, T, H, D] f64), dS_in ([B, H, D, D] f64) and, when
    weights are given, dq_w, dk_w ([D] f64)."""
    q, k, v, g, St, (B, T, H, D) = _prep(q, k, v, g, S)
    do = _f32(do)
    dSo = None if dS_out is None else np.ascontiguousarray(np.asarray(dS_out, dtype=np.float64))
    q_w = None if q_w is None else _f32(q_w)
    k_w = None if k_w is None else _f32(k_w)
    out = {n: np.empty((B, T, H, D), np.float64) for n in ("dq", "dk", "dv", "dg")}
    dS_in = np.empty((B, H, D, D), np.float64)
    dqw = np.empty((B * H, D), np.float64) if q_w is not None else None
    dkw = np.empty((B * H, D), np.float64) if k_w is not None else None
    _load().lao_backward(_p32(q), _p32(k), _p32(v), _p32(g), _p32(do), B, T, H, D, int(pos0), float(base),
                         float(eps), _p32(q_w), _p32(k_w), _p64(St), _p64(dSo), _p64(out["dq"]),
                         _p64(out["dk"]), _p64(out["dv"]), _p64(out["dg"]), _p64(dS_in), _p64(dqw), _p64(dkw))
    out["dS_in"] = dS_in
    if dqw is not None:
        out["dq_w"] = dqw.sum(axis=0)
    if dkw is not None:
        out["dk_w"] = dkw.sum(axis=0)
    return out


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def sparse_forward(q, k, v, g, block: int = 64, topk: int = 16, sel=None, threads: int = 0):
    """Sparse layer over whole sequences from position 0 (readings in sparse_oracle.c).
    q, k, v, g: [B, T, H, D].  With ``sel`` ([B, H, ceil(T / block), topk] int32, -1 =
    unused) those blocks are attended instead of the computed choice.  Returns
    (o [B, T, H, D] float64, sel int32, scores [B, H, nqb, T // block] float64)."""
    q, k, v, g = (_f32(x) for x in (q, k, v, g))
    B, T, H, D = q.shape
    assert D <= 1024 and block >= 1 and topk >= 1
    nqb, nkb = -(-T // block), T // block
    use = sel is not None
    s = _i32(sel).copy() if use else np.empty((B, H, nqb, topk), np.int32)
    assert s.shape == (B, H, nqb, topk)
    scores = np.zeros((B, H, nqb, max(nkb, 1)), np.float64)
    o = np.empty((B, T, H, D), np.float64)
    lib = _load_sparse()
    lib.lso_set_threads(int(threads))
    lib.lso_sparse_forward(_p32(q), _p32(k), _p32(v), _p32(g), B, T, H, D, int(block), int(topk),
                           s.ctypes.data_as(_i32p), int(use), _p64(scores), _p64(o))
    return o, s, scores[..., :nkb]


def sparse_decode(q, k_cache, v_cache, g, lens, block: int = 64, topk: int = 16, sel=None, threads: int = 0):
    """One decode step of the sparse layer.  q, g: [B, H, D] (the query of each cache's
    last valid token); k_cache, v_cache: [B, Tmax, H, D]; lens: [B] valid tokens (>= 1).
    Returns (o [B, H, D] float64, sel [B, H, topk] int32, scores [B, H, Tmax // block])."""
    q, k_cache, v_cache, g = (_f32(x) for x in (q, k_cache, v_cache, g))
    B, Tmax, H, D = k_cache.shape
    lens = _i32(lens)
    assert lens.shape == (B,) and np.all(lens >= 1) and np.all(lens <= Tmax) and D <= 1024
    use = sel is not None
    s = _i32(sel).copy() if use else np.empty((B, H, topk), np.int32)
    nkb = Tmax // block
    scores = np.zeros((B, H, max(nkb, 1)), np.float64)
    o = np.empty((B, H, D), np.float64)
    lib = _load_sparse()
    lib.lso_set_threads(int(threads))
    lib.lso_sparse_decode(_p32(q), _p32(k_cache), _p32(v_cache), _p32(g), lens.ctypes.data_as(_i32p), B, Tmax, H,
                          D, int(block), int(topk), s.ctypes.data_as(_i32p), int(use), _p64(scores), _p64(o))
    return o, s, scores[..., :nkb]
