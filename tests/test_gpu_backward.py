"""GPU parity of la_backward (gradients of the prefill) against the fp64 oracle's
reverse mode: dq, dk, dv, dgate per (b, t, h) row, dS_in per (b, h), the
norm-weight gradients, on ragged and multi-segment shapes."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import assert_o_close, assert_S_close, to_np, to_np32

pytestmark = pytest.mark.gpu
D = 128


@pytest.fixture(scope="module")
def la():
    import hybrid_sparse_linear_la_amd as la
    la.library()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return la


def _inputs(B, T, H, seed, S_std, dS_std, weights):
    gen = workloads.generator(seed, "cuda")
    q, k, v, g = workloads.activations(B, T, H, D, seed, "cuda", gen=gen)
    d_o = torch.randn((B, T, H, D), generator=gen, device="cuda").to(torch.bfloat16)
    S_in = workloads.state(B, H, D, S_std, gen, "cuda") if S_std else None
    dS_out = workloads.state(B, H, D, dS_std, gen, "cuda") if dS_std else None
    qw = kw = None
    if weights:
        qw = torch.rand(D, generator=gen, device="cuda") + 0.5
        kw = torch.rand(D, generator=gen, device="cuda") + 0.5
    return q, k, v, g, d_o, S_in, dS_out, qw, kw


def _check(grads, q, k, v, g, d_o, S_in, dS_out, pos0, qw, kw, weight_grads):
    ref = oracle.backward(to_np32(q), to_np32(k), to_np32(v), to_np32(g), to_np32(d_o),
                          S=None if S_in is None else to_np(S_in),
                          dS_out=None if dS_out is None else to_np(dS_out), pos0=pos0,
                          q_w=to_np32(qw) if qw is not None else (np.ones(D, np.float32) if weight_grads else None),
                          k_w=to_np32(kw) if kw is not None else (np.ones(D, np.float32) if weight_grads else None))
    errs = {}
    for name, key in (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dgate", "dg")):
        errs[name] = assert_o_close(to_np(grads[name]), ref[key], what=name)["max"]
    errs["dS_in"] = assert_S_close(to_np(grads["dS_in"]), ref["dS_in"], what="dS_in")["fro"]
    if weight_grads:
        for name, key in (("dq_norm_w", "dq_w"), ("dk_norm_w", "dk_w")):
            got, want = to_np(grads[name]), ref[key]
            rel = np.linalg.norm(got - want) / np.linalg.norm(want)
            assert rel <= 1e-2, f"{name}: relative error {rel:.2e}"
            errs[name] = rel
    return errs


CASES = [
    # B, T, H, pos0, S_std, dS_std, weights, weight_grads
    (1, 1, 1, 0, 0.0, 0.0, False, False),
    (1, 2, 2, 0, 0.0, 0.0, False, False),
    (1, 63, 2, 0, 0.0, 0.0, False, False),
    (1, 64, 1, 0, 0.0, 0.0, False, False),
    (2, 65, 2, 5, 0.5, 0.3, False, False),
    (1, 129, 2, 7, 0.0, 0.0, False, False),
    (1, 300, 3, 262144, 0.2, 0.5, True, True),
    (2, 1000, 4, 1000, 0.0, 0.0, False, True),
    (1, 4096, 32, 0, 0.0, 0.0, False, False),       # several segments per head
    (2, 5000, 8, 1048000, 0.1, 0.1, True, True),    # ragged last chunk, several segments
    (1, 300, 3, 262144, 0.2, 0.5, True, False),     # norm weights, prologue backward inside the chunk kernel
    (2, 5000, 8, 1048000, 0.1, 0.1, True, False),
]


@pytest.mark.parametrize("B,T,H,pos0,S_std,dS_std,weights,weight_grads", CASES)
def test_backward_matches_oracle(la, B, T, H, pos0, S_std, dS_std, weights, weight_grads):
    print(f"backward case B={B} T={T} H={H} pos0={pos0} weights={weights}", flush=True)
    q, k, v, g, d_o, S_in, dS_out, qw, kw = _inputs(B, T, H, 500 + T, S_std, dS_std, weights)
    grads = la.backward(q, k, v, g, d_o, S_in=S_in, dS_out=dS_out, pos0=pos0, q_norm_w=qw, k_norm_w=kw,
                        weight_grads=weight_grads)
    torch.cuda.synchronize()
    errs = _check(grads, q, k, v, g, d_o, S_in, dS_out, pos0, qw, kw, weight_grads)
    print(f"  errors {errs}", flush=True)


def test_backward_is_deterministic(la):
    q, k, v, g, d_o, S_in, dS_out, qw, kw = _inputs(1, 3000, 16, 7, 0.1, 0.1, True)
    a = la.backward(q, k, v, g, d_o, S_in=S_in, dS_out=dS_out, q_norm_w=qw, k_norm_w=kw, weight_grads=True)
    b = la.backward(q, k, v, g, d_o, S_in=S_in, dS_out=dS_out, q_norm_w=qw, k_norm_w=kw, weight_grads=True)
    torch.cuda.synchronize()
    for n in a:
        assert torch.equal(a[n], b[n]), n


def test_backward_rejects_bad_arguments(la):
    q, k, v, g, d_o, _, _, _, _ = _inputs(1, 64, 2, 9, 0.0, 0.0, False)
    with pytest.raises(la.LAError):
        la.backward(q, k, v, g, d_o, chunk=128)
    with pytest.raises(ValueError):
        la.backward(q, k, v, g, d_o[:, :32].contiguous())


@pytest.mark.parametrize("given", ["q", "k"])
@pytest.mark.parametrize("weight_grads", [False, True])
def test_backward_with_one_norm_weight(la, given, weight_grads):
    """Only one of the two norm weights given: the other acts as ones (the chunk
    kernel keeps both vectors in LDS and fills the absent one with ones)."""
    B, T, H = 1, 700, 4
    print(f"backward case B={B} T={T} H={H} only {given}_norm_w weight_grads={weight_grads}", flush=True)
    q, k, v, g, d_o, S_in, dS_out, qw, kw = _inputs(B, T, H, 95, 0.2, 0.3, True)
    if given == "q":
        kw = None
    else:
        qw = None
    grads = la.backward(q, k, v, g, d_o, S_in=S_in, dS_out=dS_out, pos0=33, q_norm_w=qw, k_norm_w=kw,
                        weight_grads=weight_grads)
    torch.cuda.synchronize()
    ref_qw = qw if qw is not None else torch.ones(D, device="cuda")
    ref_kw = kw if kw is not None else torch.ones(D, device="cuda")
    _check(grads, q, k, v, g, d_o, S_in, dS_out, 33, ref_qw, ref_kw, weight_grads)


def test_backward_with_more_workgroups_than_weight_parts(la):
    """More (b, h, segment) workgroups than per-workgroup weight-gradient parts
    (2048): the prologue backward runs in its own kernel."""
    B, T, H = 17, 100, 128
    print(f"backward case B={B} T={T} H={H} (separate prologue kernel)", flush=True)
    q, k, v, g, d_o, S_in, dS_out, qw, kw = _inputs(B, T, H, 93, 0.1, 0.1, True)
    grads = la.backward(q, k, v, g, d_o, S_in=S_in, dS_out=dS_out, pos0=11, q_norm_w=qw, k_norm_w=kw,
                        weight_grads=True)
    torch.cuda.synchronize()
    _check(grads, q, k, v, g, d_o, S_in, dS_out, 11, qw, kw, True)


@pytest.mark.parametrize("weights", [False, True])
def test_backward_with_and_without_weight_gradients_agree(la, weights):
    """Asking for the norm-weight gradients changes how the chunk kernel is
    compiled (norm weights of one are then applied explicitly), not what it
    computes; the compiler may contract the row arithmetic into fused multiply-adds
    differently, so a rare element lands one bf16 step away: per row the two agree
    to one bf16 step (2^-8), and few elements differ at all."""
    B, T, H = 2, 3000, 4
    q, k, v, g, d_o, S_in, dS_out, qw, kw = _inputs(B, T, H, 91, 0.1, 0.2, weights)
    fused = la.backward(q, k, v, g, d_o, S_in=S_in, dS_out=dS_out, pos0=77, q_norm_w=qw, k_norm_w=kw)
    separate = la.backward(q, k, v, g, d_o, S_in=S_in, dS_out=dS_out, pos0=77, q_norm_w=qw, k_norm_w=kw,
                           weight_grads=True)
    torch.cuda.synchronize()
    for name in ("dq", "dk", "dv", "dgate", "dS_in"):
        a, b = fused[name].double(), separate[name].double()
        rel = (a - b).norm(dim=-1) / b.norm(dim=-1).clamp_min(1e-30)
        assert rel.max().item() <= 2.0 ** -8, f"{name}: row difference {rel.max().item():.2e}"
        frac = (a != b).double().mean().item()
        assert frac <= 1e-4, f"{name}: {frac:.2e} of the elements differ"


def _random_cases(n, seed):
    """Seeded random shapes for the backward: batch, length, heads, start position,
    initial state, final-state gradient, norm weights and their gradients."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B = int(rng.integers(1, 3))
        T = int(rng.choice([rng.integers(1, 130), rng.integers(130, 1200), rng.integers(1200, 4000)]))
        H = int(rng.integers(1, 7))
        pos0 = int(rng.choice([0, rng.integers(1, 3000), rng.integers(200000, 1000000)]))
        S_std, dS_std = (float(rng.choice([0.0, 0.3])) for _ in range(2))
        weights = bool(rng.integers(0, 2))
        out.append((B, T, H, pos0, S_std, dS_std, weights, bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("B,T,H,pos0,S_std,dS_std,weights,weight_grads", _random_cases(8, 515))
def test_backward_random_shapes_match_oracle(la, B, T, H, pos0, S_std, dS_std, weights, weight_grads):
    print(f"random backward case B={B} T={T} H={H} pos0={pos0} weights={weights} wgrad={weight_grads}",
          flush=True)
    q, k, v, g, d_o, S_in, dS_out, qw, kw = _inputs(B, T, H, 700 + T, S_std, dS_std, weights)
    grads = la.backward(q, k, v, g, d_o, S_in=S_in, dS_out=dS_out, pos0=pos0, q_norm_w=qw, k_norm_w=kw,
                        weight_grads=weight_grads)
    torch.cuda.synchronize()
    _check(grads, q, k, v, g, d_o, S_in, dS_out, pos0, qw, kw, weight_grads)


@pytest.mark.parametrize("B,T,H,pos0,S_std,weights,weight_grads", [
    (1, 5000, 4, 0, 0.0, False, False),     # many segments per (b, h)
    (2, 777, 3, 9000, 0.02, True, True),     # ragged tail, initial state, norm weights and their gradients
    (2, 200, 128, 0, 0.02, False, False),    # 256 (b, h): la_prefill keeps no states, they are recomputed
])
def test_backward_with_saved_forward_states(la, B, T, H, pos0, S_std, weights, weight_grads):
    """la_backward_saved, given the workspace of the la_prefill call that computed the
    forward, reuses its segment states: the gradients equal la_backward's bit for bit
    (the same kernels form the same states), and the oracle's within tolerance."""
    print(f"backward saved states B={B} T={T} H={H}", flush=True)
    q, k, v, g, d_o, S_in, dS_out, qw, kw = _inputs(B, T, H, 4242 + T, S_std, 0.01, weights)
    kw_args = dict(S_in=S_in, pos0=pos0, q_norm_w=qw, k_norm_w=kw)
    fws = torch.full((la.prefill_workspace_bytes(B, T, H),), 0xFF, dtype=torch.uint8, device="cuda")
    la.prefill(q, k, v, g, workspace=fws, **kw_args)
    ref = la.backward(q, k, v, g, d_o, dS_out=dS_out, weight_grads=weight_grads, **kw_args)
    got = la.backward(q, k, v, g, d_o, dS_out=dS_out, weight_grads=weight_grads, fwd_workspace=fws, **kw_args)
    torch.cuda.synchronize()
    for name in ref:
        assert torch.equal(ref[name].view(torch.int8) if ref[name].dtype == torch.bfloat16 else ref[name],
                           got[name].view(torch.int8) if got[name].dtype == torch.bfloat16 else got[name]), name
    _check(got, q, k, v, g, d_o, S_in, dS_out, pos0, qw, kw, weight_grads)
