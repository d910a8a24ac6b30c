"""The C-ABI library loads, exports every function include/lightning_la.h declares,
and rejects bad arguments before touching the GPU.  CPU only: every call here
fails validation, so no kernel is launched and no pointer is dereferenced."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lightning_la.h")


@pytest.fixture(scope="module")
def lib():
    import hybrid_sparse_linear_la_amd as la
    return la.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(la_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(
        ["la_version", "la_status_string", "la_prefill_workspace_bytes", "la_prefill", "la_prefill_profiled",
         "la_prefill_noalloc",
         "la_prefill_varlen_workspace_bytes", "la_prefill_varlen", "la_linear", "la_layer_workspace_bytes",
         "la_layer_forward", "la_backward_workspace_bytes", "la_backward", "la_backward_saved", "la_decode_step",
         "la_sparse_prefill_workspace_bytes", "la_sparse_prefill", "la_sparse_block_means", "la_sparse_decode"])


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.la_version() == 200


def test_status_strings(lib):
    for s, name in ((0, b"LA_OK"), (1, b"LA_ERR_NULL_PTR"), (2, b"LA_ERR_BAD_SHAPE"), (3, b"LA_ERR_UNSUPPORTED"),
                    (4, b"LA_ERR_ALIGNMENT"), (5, b"LA_ERR_ALIASING"), (6, b"LA_ERR_WORKSPACE"), (7, b"LA_ERR_HIP"),
                    (8, b"LA_ERR_CAPTURING")):
        assert lib.la_status_string(s).startswith(name)
    assert lib.la_status_string(99) == b"unknown la_status"


def test_workspace_bytes(lib):
    # one fp32 128x128 state per (b, h, segment). One round of 256 workgroups while
    # segments stay within 128 chunks of 64; then 128-chunk segments up to 1024
    # workgroups; then longer segments. When the B * H sequence-heads fill the
    # device by themselves (or the input is one chunk), one segment per (b, h) and
    # no states: 256 bytes.
    st = 128 * 128 * 4
    assert lib.la_prefill_workspace_bytes(1, 262144, 32, 128, 0) == 32 * 32 * st
    assert lib.la_prefill_workspace_bytes(1, 32768, 32, 128, 64) == 32 * 8 * st     # 64-chunk segments
    assert lib.la_prefill_workspace_bytes(1, 65536, 32, 128, 0) == 32 * 8 * st      # 128-chunk segments
    assert lib.la_prefill_workspace_bytes(1, 131072, 32, 128, 0) == 32 * 16 * st    # 512 workgroups
    assert lib.la_prefill_workspace_bytes(1, 1 << 20, 32, 128, 0) == 32 * 32 * st   # 512-chunk segments
    assert lib.la_prefill_workspace_bytes(4, 8192, 32, 128, 0) == 128 * 2 * st
    assert lib.la_prefill_workspace_bytes(1, 300, 2, 128, 0) == 2 * 5 * 128 * 128 * 4
    assert lib.la_prefill_workspace_bytes(1, 300, 2, 64, 0) == 0
    assert lib.la_prefill_workspace_bytes(1, 300, 2, 128, 96) == 0
    # wider chunks: segments hold whole chunks (5 sub-chunks of 64 -> 3 or 2 segments)
    assert lib.la_prefill_workspace_bytes(1, 300, 2, 128, 128) == 2 * 3 * 128 * 128 * 4
    assert lib.la_prefill_workspace_bytes(1, 300, 2, 128, 256) == 2 * 2 * 128 * 128 * 4
    assert lib.la_prefill_workspace_bytes(1, 262144, 32, 128, 256) == 32 * 32 * 128 * 128 * 4
    assert lib.la_prefill_workspace_bytes(0, 300, 2, 128, 0) == 0
    # one segment per (b, h): one chunk, or enough sequence-heads
    for B, T, H, C in ((1, 64, 2, 0), (1, 200, 3, 256), (8, 32768, 32, 0), (2, 5000, 128, 128),
                       (1, 100, 1000, 0), (3, 1000, 100, 0)):
        assert lib.la_prefill_workspace_bytes(B, T, H, 128, C) == 256, (B, T, H, C)
    # 300 sequence-heads leave the second round of 256 mostly empty: segments
    assert lib.la_prefill_workspace_bytes(1, 65536, 300, 128, 0) == 300 * 4 * st


# fake, never-dereferenced device addresses (validation fails before any use)
A = 1 << 40
MB = 1 << 20


def _prefill(lib, q=A, k=A + 64 * MB, v=A + 128 * MB, g=A + 192 * MB, S_in=None, S_out=A + 256 * MB,
             o=A + 320 * MB, B=1, T=64, H=2, D=128, pos0=0, chunk=0, base=10000.0, eps=1e-6, qw=None,
             kw=None, ws=A + 384 * MB, ws_bytes=1 << 30):
    vp = ctypes.c_void_p
    return lib.la_prefill(vp(q), vp(k), vp(v), vp(g), vp(S_in), vp(S_out), vp(o), B, T, H, D, pos0, chunk,
                          base, eps, vp(qw), vp(kw), vp(ws), ws_bytes, None)


def test_prefill_validation(lib):
    import hybrid_sparse_linear_la_amd  # noqa: F401  (argtypes set by library())
    assert _prefill(lib, q=None) == 1
    assert _prefill(lib, ws=None) == 1
    assert _prefill(lib, S_out=None) == 1
    assert _prefill(lib, B=0) == 2
    assert _prefill(lib, T=0) == 2
    assert _prefill(lib, H=-1) == 2
    assert _prefill(lib, D=64) == 3
    assert _prefill(lib, chunk=32) == 3
    assert _prefill(lib, chunk=96) == 3
    assert _prefill(lib, chunk=512) == 3
    assert _prefill(lib, base=0.0) == 3
    assert _prefill(lib, eps=-1.0) == 3
    assert _prefill(lib, eps=float("nan")) == 3
    assert _prefill(lib, q=A + 8) == 4
    assert _prefill(lib, qw=A + 1000 * MB + 4) == 4
    assert _prefill(lib, o=A + 32) == 5                  # o overlaps q
    assert _prefill(lib, S_out=A + 64 * MB + 1024) == 5  # S_out overlaps k
    assert _prefill(lib, S_in=A + 256 * MB + 16, S_out=A + 256 * MB) == 5  # partial overlap
    assert _prefill(lib, ws=A + 320 * MB + 64) == 5      # workspace overlaps o
    assert _prefill(lib, ws_bytes=255) == 6


def _cu(values):
    return (ctypes.c_int32 * len(values))(*values)


def _varlen(lib, q=A, k=A + 64 * MB, v=A + 128 * MB, g=A + 192 * MB, cu=(0, 5, 5, 70), pos0=None,
            S_in=None, S_out=A + 256 * MB, o=A + 320 * MB, nseq=None, total_T=None, H=2, D=128, chunk=0,
            base=10000.0, eps=1e-6, qw=None, ws=A + 1024 * MB, ws_bytes=1 << 30):
    vp = ctypes.c_void_p
    cu_arr = None if cu is None else _cu(list(cu))
    nseq = len(cu) - 1 if nseq is None else nseq
    total_T = cu[-1] if total_T is None else total_T
    p0 = None if pos0 is None else (ctypes.c_int64 * len(pos0))(*pos0)
    return lib.la_prefill_varlen(vp(q), vp(k), vp(v), vp(g), cu_arr, p0, vp(S_in), vp(S_out), vp(o), nseq,
                                 total_T, H, D, chunk, base, eps, vp(qw), None, vp(ws), ws_bytes, None)


def test_varlen_workspace_bytes(lib):
    import hybrid_sparse_linear_la_amd as la
    f = lib.la_prefill_varlen_workspace_bytes
    # one 2-token sequence: one segment per head after a 256-byte table area
    assert f(1, _cu([0, 2]), 2, 128, 0) == 256 + 2 * 128 * 128 * 4
    # single-token and empty sequences need no segment states
    assert f(3, _cu([0, 1, 1, 2]), 2, 128, 0) == 256
    # equal lengths: the same 10 segments as la_prefill, after 10 x 24 + 2 x 16 bytes of
    # tables rounded up to 512
    assert f(2, _cu([0, 300, 600]), 2, 128, 0) - 512 == lib.la_prefill_workspace_bytes(2, 300, 2, 128, 0)
    assert f(2, _cu([0, 3, 2]), 2, 128, 0) == 0   # decreasing offsets
    assert f(1, _cu([1, 3]), 2, 128, 0) == 0      # does not start at 0
    assert f(1, _cu([0, 3]), 2, 64, 0) == 0
    assert f(1, _cu([0, 3]), 2, 128, 96) == 0
    assert la.prefill_varlen_workspace_bytes([0, 1, 300, 300, 5000], 32) > 0


def test_varlen_validation(lib):
    import hybrid_sparse_linear_la_amd  # noqa: F401
    assert _varlen(lib, q=None) == 1
    assert _varlen(lib, cu=None, nseq=3, total_T=70) == 1
    assert _varlen(lib, ws=None) == 1
    assert _varlen(lib, nseq=0, total_T=0) == 2
    assert _varlen(lib, cu=(0, 5, 4, 70)) == 2          # decreasing
    assert _varlen(lib, cu=(2, 5, 5, 70)) == 2          # first offset not 0
    assert _varlen(lib, total_T=71) == 2                # last offset != total_T
    assert _varlen(lib, D=64) == 3
    assert _varlen(lib, chunk=96) == 3
    assert _varlen(lib, eps=-1.0) == 3
    assert _varlen(lib, k=A + 64 * MB + 8) == 4
    assert _varlen(lib, o=A + 64) == 5                  # o overlaps q
    assert _varlen(lib, S_in=A + 256 * MB + 16) == 5    # S_in partly overlaps S_out
    assert _varlen(lib, ws=A + 320 * MB + 256) == 5     # workspace overlaps o
    assert _varlen(lib, ws_bytes=16) == 6


def _decode(lib, q=A, k=A + MB, v=A + 2 * MB, g=A + 3 * MB, S=A + 4 * MB, o=A + 512 * MB, B=2, H=2,
            D=128, pos=0, base=10000.0, eps=1e-6):
    vp = ctypes.c_void_p
    return lib.la_decode_step(vp(q), vp(k), vp(v), vp(g), vp(S), vp(o), B, H, D, pos, base, eps, None, None,
                              None)


def test_decode_validation(lib):
    import hybrid_sparse_linear_la_amd  # noqa: F401
    assert _decode(lib, S=None) == 1
    assert _decode(lib, B=0) == 2
    assert _decode(lib, D=256) == 3
    assert _decode(lib, base=-2.0) == 3
    assert _decode(lib, v=A + 2 * MB + 2) == 4
    assert _decode(lib, o=A + 256) == 5        # o overlaps q
    assert _decode(lib, S=A + 3 * MB) == 5     # S overlaps g


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    import hybrid_sparse_linear_la_amd as la
    monkeypatch.setattr(la, "_lib", None)
    monkeypatch.setattr(la, "lib_path", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        la.library()


def test_linear_and_layer_validation(lib):
    vp = ctypes.c_void_p
    lin = lambda x=A, w=A + 64 * MB, y=A + 128 * MB, M=4, N=256, K=64: lib.la_linear(  # noqa: E731
        vp(x), vp(w), vp(y), M, N, K, None)
    assert lin(x=None) == 1
    assert lin(M=0) == 2
    assert lin(K=96) == 3
    assert lin(N=384) == 3
    assert lin(w=A + 64 * MB + 2) == 4
    assert lin(y=A) == 5                     # y overlaps x
    assert lin(y=A + 64 * MB) == 5           # y overlaps w
    assert lib.la_layer_workspace_bytes(1, 300, 2, 128, 0) == 5 * 153600 + lib.la_prefill_workspace_bytes(
        1, 300, 2, 128, 0)
    assert lib.la_layer_workspace_bytes(1, 300, 2, 64, 0) == 0

    def layer(x=A, wq=A + 64 * MB, wo=A + 128 * MB, S_in=None, S_out=A + 192 * MB, y=A + 256 * MB, B=1, T=300,
              hidden=256, H=2, D=128, ws=A + 512 * MB, ws_bytes=1 << 30):
        return lib.la_layer_forward(vp(x), vp(wq), vp(wo), vp(S_in), vp(S_out), vp(y), B, T, hidden, H, D, 0, 0,
                                    10000.0, 1e-6, None, None, vp(ws), ws_bytes, None)
    assert layer(wq=None) == 1
    assert layer(T=0) == 2
    assert layer(hidden=320) == 3
    assert layer(H=3) == 3                   # H * D = 384 is not a multiple of 256
    assert layer(y=A + 256 * MB + 8) == 4
    assert layer(y=A + 1024) == 5            # y overlaps x
    assert layer(y=A) == 5                   # y is x itself
    assert layer(ws=A + 256 * MB) == 5       # workspace overlaps y
    assert layer(ws_bytes=4096) == 6


def test_backward_validation(lib):
    vp = ctypes.c_void_p
    assert lib.la_backward_workspace_bytes(1, 300, 2, 128, 128) == 0   # chunk 64 only
    assert lib.la_backward_workspace_bytes(1, 300, 2, 128, 0) > 2 * lib.la_prefill_workspace_bytes(1, 300, 2, 128, 0)

    def bwd(q=A, k=A + MB, v=A + 2 * MB, g=A + 3 * MB, S_in=None, d_o=A + 4 * MB, dS_out=None, dq=A + 8 * MB,
            dk=A + 9 * MB, dv=A + 10 * MB, dg=A + 11 * MB, dS_in=A + 12 * MB, B=1, T=300, H=2, D=128, chunk=0,
            ws=A + 64 * MB, ws_bytes=1 << 30):
        return lib.la_backward(vp(q), vp(k), vp(v), vp(g), vp(S_in), vp(d_o), vp(dS_out), vp(dq), vp(dk), vp(dv),
                               vp(dg), vp(dS_in), None, None, B, T, H, D, 0, chunk, 10000.0, 1e-6, None, None,
                               vp(ws), ws_bytes, None)
    assert bwd(d_o=None) == 1
    assert bwd(dS_in=None) == 1
    assert bwd(T=0) == 2
    assert bwd(chunk=128) == 3
    assert bwd(D=64) == 3
    assert bwd(dq=A + 8 * MB + 4) == 4
    assert bwd(dq=A + 1024) == 5          # dq overlaps q
    assert bwd(dk=A + 8 * MB + 64) == 5   # dk overlaps dq
    assert bwd(ws=A + 12 * MB) == 5       # workspace overlaps dS_in
    assert bwd(ws_bytes=4096) == 6


def test_backward_saved_validation(lib):
    """la_backward_saved checks the forward workspace before anything is launched:
    alignment, size (la_prefill's for the shape) and overlap with the outputs."""
    vp = ctypes.c_void_p
    B, T, H = 1, 20000, 2             # la_prefill keeps segment states for this shape
    fwd_need = lib.la_prefill_workspace_bytes(B, T, H, 128, 0)
    assert fwd_need > 4096
    act = B * T * H * 128 * 2

    def bwd(fwd=A + 512 * MB, fwd_bytes=fwd_need, dq=A + 100 * MB, ws_bytes=1 << 30):
        return lib.la_backward_saved(vp(A), vp(A + 20 * MB), vp(A + 40 * MB), vp(A + 60 * MB), None,
                                     vp(A + 80 * MB), None, vp(dq), vp(A + 120 * MB), vp(A + 140 * MB),
                                     vp(A + 160 * MB), vp(A + 180 * MB), None, None, B, T, H, 128, 0, 0, 10000.0,
                                     1e-6, None, None, vp(A + 200 * MB), ws_bytes, vp(fwd) if fwd else None,
                                     fwd_bytes, None)
    assert act < 20 * MB
    assert bwd(fwd=A + 512 * MB + 8) == 4               # misaligned forward workspace
    assert bwd(fwd_bytes=fwd_need - 256) == 6           # smaller than la_prefill's
    assert bwd(dq=A + 512 * MB + 4096) == 5             # an output inside the forward workspace
    assert bwd(ws_bytes=4096) == 6                      # the backward's own workspace still checked


def test_sparse_validation(lib):
    vp = ctypes.c_void_p
    # workspace: fp32 means of the complete 64-token key blocks
    # key means, then the block choice [B, H, ceil(T / 64), topk] int32, each rounded to 256 bytes
    assert lib.la_sparse_prefill_workspace_bytes(1, 32768, 32, 128, 0, 16) == 32 * 512 * 128 * 4 + 32 * 512 * 16 * 4
    assert lib.la_sparse_prefill_workspace_bytes(1, 300, 2, 128, 64, 16) == 2 * 4 * 128 * 4 + 768
    assert lib.la_sparse_prefill_workspace_bytes(1, 300, 2, 128, 32, 16) == 0     # block 64 only
    assert lib.la_sparse_prefill_workspace_bytes(1, 300, 2, 128, 0, 0) == 0       # topk in [1, 64]
    assert lib.la_sparse_prefill_workspace_bytes(1, 300, 2, 128, 0, 65) == 0
    assert lib.la_sparse_prefill_workspace_bytes(1, 300, 2, 64, 0, 16) == 0
    assert lib.la_sparse_prefill_workspace_bytes(1, 64 * 8192 + 64, 1, 128, 0, 16) == 0   # > 8192 key blocks

    def pre(q=A, k=A + MB, v=A + 2 * MB, g=A + 3 * MB, o=A + 4 * MB, sel=None, B=1, T=300, H=2, D=128, block=0,
            topk=16, ws=A + 8 * MB, ws_bytes=1 << 20):
        return lib.la_sparse_prefill(vp(q), vp(k), vp(v), vp(g), vp(o), vp(sel), B, T, H, D, block, topk, vp(ws),
                                     ws_bytes, None)
    assert pre(k=None) == 1
    assert pre(ws=None) == 1
    assert pre(T=0) == 2
    assert pre(topk=0) == 3
    assert pre(block=128) == 3
    assert pre(o=A + 4 * MB + 8) == 4
    assert pre(o=A + 1024) == 5              # o overlaps q
    assert pre(sel=A + 4 * MB + 256) == 5    # sel overlaps o
    assert pre(ws=A + 3 * MB) == 5           # workspace overlaps gate
    assert pre(ws_bytes=1024) == 6

    def means(k=A, m=A + 64 * MB, B=1, Tmax=1024, H=2, D=128, block=0, first=0, n=16):
        return lib.la_sparse_block_means(vp(k), vp(m), B, Tmax, H, D, block, first, n, None)
    assert means(m=None) == 1
    assert means(n=17) == 2                  # past the cache
    assert means(first=-1) == 2
    assert means(D=96) == 3
    assert means(m=A + 4) == 4
    assert means(m=A + 1024) == 5

    def dec(q=A, kc=A + MB, vc=A + 64 * MB, m=A + 128 * MB, g=A + 129 * MB, lens=A + 130 * MB, o=A + 131 * MB,
            sel=None, B=2, Tmax=4096, H=2, D=128, block=0, topk=16):
        return lib.la_sparse_decode(vp(q), vp(kc), vp(vc), vp(m), vp(g), vp(lens), vp(o), vp(sel), B, Tmax, H, D,
                                    block, topk, None)
    assert dec(lens=None) == 1
    assert dec(m=None) == 1
    assert dec(B=0) == 2
    assert dec(topk=65) == 3
    assert dec(o=A + 131 * MB + 2) == 4
    assert dec(o=A + 2 * MB) == 5            # o inside the key cache
    assert dec(sel=A + 130 * MB) == 5        # sel overlaps lens
