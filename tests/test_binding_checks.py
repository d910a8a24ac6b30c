"""The Python binding rejects caller-supplied outputs, states, weights and
workspaces that do not match the inputs' shape, dtype or device, before any
library call.  The C ABI sees only pointers and sizes, so an undersized output
would be written past its end: the binding is where such a mistake is caught.

CPU only: the tensors live on torch's "meta" device (shape and dtype, no memory)
and on the CPU, with the binding's GPU test widened to accept both, so every
check runs and every call stops at a ValueError before reaching the library."""
import pytest
import torch

import hybrid_sparse_linear_la_amd as la

D = 128


@pytest.fixture(autouse=True)
def meta_is_gpu(monkeypatch):
    la.library()
    monkeypatch.setattr(la, "_on_gpu", lambda t: t.device.type in ("meta", "cpu"))


def act(*shape, dtype=torch.bfloat16, device="meta"):
    return torch.empty(shape, dtype=dtype, device=device)


def f32(*shape, device="meta"):
    return torch.empty(shape, dtype=torch.float32, device=device)


def qkvg(*shape):
    return [act(*shape) for _ in range(4)]


BAD_OUTS_4D = [act(1, 63, 2, D), act(1, 64, 1, D), act(1, 64, 2, D, dtype=torch.float32),
               act(1, 64, 2, D, device="cpu"), act(1, 128, 2, D)[:, ::2], act(1, 64, 2, 2 * D)[..., :D]]


@pytest.mark.parametrize("bad", range(len(BAD_OUTS_4D)))
def test_prefill_rejects_bad_out(bad):
    with pytest.raises(ValueError):
        la.prefill(*qkvg(1, 64, 2, D), out=BAD_OUTS_4D[bad])


def test_prefill_rejects_bad_states_weights_workspace():
    x = qkvg(1, 64, 2, D)
    for kw in (dict(S_in=f32(1, 2, D, D, device="cpu")), dict(S_in=f32(1, 1, D, D)),
               dict(S_out=f32(2, 2, D, D)), dict(S_out=f32(1, 2, D, D, device="cpu")),
               dict(q_norm_w=f32(D, device="cpu")), dict(k_norm_w=f32(D + 1)),
               dict(workspace=torch.empty(1 << 20, dtype=torch.uint8, device="cpu"))):
        with pytest.raises(ValueError):
            la.prefill(*x, **kw)
    with pytest.raises(ValueError):   # an input on another device
        la.prefill(*x[:3], act(1, 64, 2, D, device="cpu"))


def test_varlen_rejects_bad_out_and_states():
    x = qkvg(300, 2, D)
    cu = [0, 100, 300]
    for kw in (dict(out=act(299, 2, D)), dict(out=act(300, 2, D, device="cpu")),
               dict(S_in=f32(3, 2, D, D)), dict(S_out=f32(2, 2, D, D, device="cpu"))):
        with pytest.raises(ValueError):
            la.prefill_varlen(*x, cu, **kw)


def test_decode_rejects_bad_out_and_state():
    x = qkvg(4, 2, D)
    S = f32(4, 2, D, D)
    for kw in (dict(out=act(3, 2, D)), dict(out=act(4, 2, D, device="cpu")),
               dict(out=act(4, 2, D, dtype=torch.float16))):
        with pytest.raises(ValueError):
            la.decode_step(*x, S, 0, **kw)
    for bad_S in (f32(4, 2, D, D, device="cpu"), f32(4, 1, D, D), None):
        with pytest.raises(ValueError):
            la.decode_step(*x, bad_S, 0)


def test_linear_rejects_bad_out():
    x, w = act(64, 256), act(512, 256)
    for out in (act(64, 256), act(64, 512, device="cpu"), act(32, 1024)):
        with pytest.raises(ValueError):
            la.linear(x, w, out=out)
    with pytest.raises(ValueError):
        la.linear(x, act(512, 256, device="cpu"))


def test_layer_forward_rejects_bad_out():
    x = act(1, 64, 256)
    w_qkvg, w_o = act(4 * 256, 256), act(256, 256)
    for out in (act(1, 63, 256), act(64, 256), act(1, 64, 256, device="cpu")):
        with pytest.raises(ValueError):
            la.layer_forward(x, w_qkvg, w_o, out=out)
    with pytest.raises(ValueError):
        la.layer_forward(x, w_qkvg, act(256, 256, device="cpu"))


def test_backward_rejects_bad_states_and_weights():
    x = qkvg(1, 64, 2, D)
    d_o = act(1, 64, 2, D)
    for kw in (dict(S_in=f32(1, 2, D, D, device="cpu")), dict(dS_out=f32(1, 3, D, D)),
               dict(q_norm_w=f32(D, device="cpu"))):
        with pytest.raises(ValueError):
            la.backward(*x, d_o, **kw)


def test_sparse_entry_points_reject_bad_outputs():
    x = qkvg(1, 256, 2, D)
    for out in (act(1, 255, 2, D), act(1, 256, 2, D, device="cpu")):
        with pytest.raises(ValueError):
            la.sparse_prefill(*x, out=out)
    kc, vc = act(2, 256, 2, D), act(2, 256, 2, D)
    q, g = act(2, 2, D), act(2, 2, D)
    means = f32(2, 2, 4, D)
    lens = torch.empty(2, dtype=torch.int32, device="meta")
    for kw in (dict(out=act(1, 2, D)), dict(out=act(2, 2, D, device="cpu"))):
        with pytest.raises(ValueError):
            la.sparse_decode(q, kc, vc, means, g, lens, **kw)
    with pytest.raises(ValueError):
        la.sparse_decode(q, kc, vc, f32(2, 2, 4, D, device="cpu"), g, lens)
    with pytest.raises(ValueError):
        la.sparse_decode(q, kc, vc, means, g, torch.empty(2, dtype=torch.int32, device="cpu"))
    with pytest.raises(ValueError):
        la.sparse_block_means(kc, means=f32(2, 2, 4, D, device="cpu"))
