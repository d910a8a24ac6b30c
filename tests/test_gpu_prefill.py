"""GPU parity of la_prefill against the fp64 oracle on small and ragged shapes,
plus invariants of the HIP path (determinism, in-place carry, what S ignores)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import assert_o_close, assert_S_close, o_row_errors, to_np, to_np32

pytestmark = pytest.mark.gpu
D = 128


@pytest.fixture(scope="module")
def la():
    import hybrid_sparse_linear_la_amd as la
    la.library()  # raises if the HIP library is not built
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return la


def _inputs(B, T, H, seed, S_std=0.0, weights=False):
    gen = workloads.generator(seed, "cuda")
    q, k, v, g = workloads.activations(B, T, H, D, seed, "cuda", gen=gen)
    S_in = workloads.state(B, H, D, S_std, gen, "cuda") if S_std else None
    qw = kw = None
    if weights:
        qw = torch.rand(D, generator=gen, device="cuda") + 0.5
        kw = torch.rand(D, generator=gen, device="cuda") + 0.5
    return q, k, v, g, S_in, qw, kw


def _oracle(q, k, v, g, S_in, pos0, qw=None, kw=None):
    return oracle.forward(to_np32(q), to_np32(k), to_np32(v), to_np32(g),
                          S=None if S_in is None else to_np(S_in), pos0=pos0,
                          q_w=None if qw is None else to_np32(qw), k_w=None if kw is None else to_np32(kw))


CASES = [
    # B, T, H, pos0, S_std, weights
    (1, 1, 1, 0, 0.0, False),
    (1, 2, 2, 0, 0.0, False),
    (1, 63, 3, 0, 0.0, False),
    (2, 64, 2, 5, 0.5, False),
    (1, 65, 1, 0, 0.0, True),
    (2, 127, 3, 1000, 0.0, False),
    (1, 300, 2, 262144, 1.0, False),
    (3, 1000, 4, 7, 0.2, True),
    (1, 4096, 32, 0, 0.0, False),       # several segments per head: exercises the state scan
    (2, 5000, 8, 1048000, 0.1, False),  # ragged last chunk inside the last segment
]


@pytest.mark.parametrize("B,T,H,pos0,S_std,weights", CASES)
def test_prefill_matches_oracle(la, B, T, H, pos0, S_std, weights):
    print(f"prefill case B={B} T={T} H={H} pos0={pos0} S_std={S_std} weights={weights}", flush=True)
    q, k, v, g, S_in, qw, kw = _inputs(B, T, H, seed=11 + T, S_std=S_std, weights=weights)
    o, S = la.prefill(q, k, v, g, S_in=S_in, pos0=pos0, q_norm_w=qw, k_norm_w=kw)
    torch.cuda.synchronize()
    o_ref, S_ref = _oracle(q, k, v, g, S_in, pos0, qw, kw)
    assert_o_close(to_np(o), o_ref)
    assert_S_close(to_np(S), S_ref)


WIDE_CASES = [
    # chunk, B, T, H, pos0, S_std, weights
    (128, 1, 1, 1, 0, 0.0, False),
    (128, 1, 63, 3, 0, 0.0, False),       # one partial sub-block
    (128, 2, 200, 2, 5, 0.5, False),      # second chunk ragged inside its first sub-block
    (128, 1, 700, 4, 262144, 1.0, True),
    (128, 1, 4096, 32, 0, 0.0, False),    # several segments per head
    (256, 1, 100, 2, 0, 0.0, False),
    (256, 2, 300, 3, 1000, 0.2, False),   # second chunk: one full and a partial sub-block
    (256, 1, 1000, 4, 7, 0.0, True),      # last chunk: three sub-blocks, the last ragged
    (256, 1, 4096, 32, 0, 0.0, False),
]


@pytest.mark.parametrize("chunk,B,T,H,pos0,S_std,weights", WIDE_CASES)
def test_wide_chunk_matches_oracle(la, chunk, B, T, H, pos0, S_std, weights):
    print(f"wide-chunk case C={chunk} B={B} T={T} H={H} pos0={pos0}", flush=True)
    q, k, v, g, S_in, qw, kw = _inputs(B, T, H, seed=21 + T + chunk, S_std=S_std, weights=weights)
    o, S = la.prefill(q, k, v, g, S_in=S_in, pos0=pos0, chunk=chunk, q_norm_w=qw, k_norm_w=kw)
    torch.cuda.synchronize()
    o_ref, S_ref = _oracle(q, k, v, g, S_in, pos0, qw, kw)
    assert_o_close(to_np(o), o_ref)
    assert_S_close(to_np(S), S_ref)


DIRECT_CASES = [
    # chunk, B, T, H, pos0, S_std, weights: enough sequence-heads that each (b, h) is
    # one segment (no state pass; the output kernel starts from S_in)
    (64, 8, 1000, 32, 0, 0.0, False),
    (64, 2, 777, 512, 262144, 0.3, True),
    (128, 8, 1000, 32, 5, 0.2, False),
    (256, 4, 613, 64, 1000, 0.0, True),
]


@pytest.mark.parametrize("chunk,B,T,H,pos0,S_std,weights", DIRECT_CASES)
def test_one_segment_per_head_matches_oracle(la, chunk, B, T, H, pos0, S_std, weights):
    print(f"one-segment case C={chunk} B={B} T={T} H={H} pos0={pos0}", flush=True)
    assert la.prefill_workspace_bytes(B, T, H, D, chunk) == 256  # the direct form
    q, k, v, g, S_in, qw, kw = _inputs(B, T, H, seed=41 + T + chunk, S_std=S_std, weights=weights)
    o, S = la.prefill(q, k, v, g, S_in=S_in, pos0=pos0, chunk=chunk, q_norm_w=qw, k_norm_w=kw)
    torch.cuda.synchronize()
    # every head's final state, and the outputs of sampled (b, h)
    bs = sorted({0, B - 1})
    hs = sorted({0, H // 2, H - 1})
    sel = lambda t: t[bs][:, :, hs]  # noqa: E731
    o_ref, S_ref = _oracle(sel(q), sel(k), sel(v), sel(g), None if S_in is None else S_in[bs][:, hs], pos0, qw, kw)
    assert_o_close(to_np(sel(o)), o_ref)
    assert_S_close(to_np(S[bs][:, hs]), S_ref)
    _, S_all = _oracle(q, k, v, g, S_in, pos0, qw, kw)
    assert_S_close(to_np(S), S_all, what="every final state")


def test_one_segment_in_place_carry(la):
    """S_in == S_out with one segment per (b, h): each workgroup reads its state
    before it writes it."""
    q, k, v, g, S, _, _ = _inputs(4, 300, 64, seed=43, S_std=0.2)
    S_ref_in = to_np(S)
    o, S_out = la.prefill(q, k, v, g, S_in=S, S_out=S, pos0=17)
    torch.cuda.synchronize()
    assert S_out.data_ptr() == S.data_ptr()
    o_ref, S_ref = oracle.forward(to_np32(q), to_np32(k), to_np32(v), to_np32(g), S=S_ref_in, pos0=17)
    assert_o_close(to_np(o), o_ref)
    assert_S_close(to_np(S), S_ref)


def test_chunk_sizes_agree(la):
    """Every chunk size evaluates the same closed form: the outputs agree with each
    other within the tolerance to the oracle (the typical row far inside it), and
    the final state (the same fp32 sums, grouped into segments of whole chunks)
    agrees to rounding."""
    q, k, v, g, S_in, _, _ = _inputs(1, 2000, 4, seed=31, S_std=0.1)
    outs = {c: la.prefill(q, k, v, g, S_in=S_in, pos0=123, chunk=c) for c in (64, 128, 256)}
    torch.cuda.synchronize()
    o64, S64 = outs[64]
    for c in (128, 256):
        o, S = outs[c]
        e = o_row_errors(to_np(o), to_np(o64))
        # each side carries ~1e-3 of bf16 output rounding per row
        assert e["max"] <= 2e-2 and e["median"] <= 5e-3 and e["fro"] <= 5e-3, (c, e)
        rel = float(torch.linalg.norm(S - S64) / torch.linalg.norm(S64))
        assert rel <= 1e-5, (c, rel)


def test_prefill_in_place_state_carry(la):
    q, k, v, g, S, _, _ = _inputs(1, 200, 4, seed=3, S_std=0.3)
    S_ref_in = to_np(S)
    o, S_out = la.prefill(q, k, v, g, S_in=S, S_out=S, pos0=17)
    torch.cuda.synchronize()
    assert S_out.data_ptr() == S.data_ptr()
    o_ref, S_ref = oracle.forward(to_np32(q), to_np32(k), to_np32(v), to_np32(g), S=S_ref_in, pos0=17)
    assert_o_close(to_np(o), o_ref)
    assert_S_close(to_np(S), S_ref)


def test_prefill_is_deterministic(la):
    q, k, v, g, S_in, _, _ = _inputs(1, 3000, 16, seed=4, S_std=0.1)
    o1, S1 = la.prefill(q, k, v, g, S_in=S_in, pos0=9)
    o2, S2 = la.prefill(q, k, v, g, S_in=S_in, pos0=9)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_state_ignores_q_and_gate(la):
    q, k, v, g, _, _, _ = _inputs(1, 700, 4, seed=5)
    q2, _, _, g2, _, _, _ = _inputs(1, 700, 4, seed=6)
    _, S1 = la.prefill(q, k, v, g)
    _, S2 = la.prefill(q2, k, v, g2)
    torch.cuda.synchronize()
    assert torch.equal(S1, S2)


def test_output_invariant_to_position_shift(la):
    # with S_in = 0 RoPE makes o depend only on position differences
    q, k, v, g, _, _, _ = _inputs(1, 513, 2, seed=7)
    o0, _ = la.prefill(q, k, v, g, pos0=0)
    o1, _ = la.prefill(q, k, v, g, pos0=999_983)
    torch.cuda.synchronize()
    e = o_row_errors(to_np(o1), to_np(o0))
    assert e["max"] <= 2e-2, e


def test_nan_stays_in_its_head(la):
    q, k, v, g, _, _, _ = _inputs(1, 256, 3, seed=8)
    k[0, 100, 1, 5] = float("nan")
    o, S = la.prefill(q, k, v, g)
    torch.cuda.synchronize()
    assert torch.isfinite(o[:, :, 0]).all() and torch.isfinite(o[:, :, 2]).all()
    assert torch.isfinite(S[:, 0]).all() and torch.isfinite(S[:, 2]).all()
    assert not torch.isfinite(S[:, 1]).all()


def test_binding_rejects_bad_arguments(la):
    q, k, v, g, _, _, _ = _inputs(1, 64, 2, seed=9)
    with pytest.raises(TypeError):
        la.prefill(q.float(), k, v, g)
    with pytest.raises(la.LAError) as ei:
        la.prefill(q, k, v, g, chunk=48)
    assert ei.value.status == 3
    with pytest.raises(ValueError):
        la.prefill(q, k[:, :32], v, g)


def _random_cases(n, seed):
    """Seeded random shapes: batch, length (any remainder modulo 64, several
    segments for the longer ones), heads, start position, chunk, initial state and
    norm weights."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B = int(rng.integers(1, 4))
        T = int(rng.choice([rng.integers(1, 130), rng.integers(130, 1500), rng.integers(1500, 6000)]))
        H = int(rng.integers(1, 9))
        pos0 = int(rng.choice([0, rng.integers(1, 5000), rng.integers(200000, 1100000)]))
        chunk = int(rng.choice([0, 64, 128, 256]))
        S_std = float(rng.choice([0.0, 0.3]))
        out.append((B, T, H, pos0, chunk, S_std, bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("B,T,H,pos0,chunk,S_std,weights", _random_cases(12, 2024))
def test_random_shapes_match_oracle(la, B, T, H, pos0, chunk, S_std, weights):
    print(f"random case B={B} T={T} H={H} pos0={pos0} C={chunk} S_std={S_std} weights={weights}", flush=True)
    q, k, v, g, S_in, qw, kw = _inputs(B, T, H, seed=31 + T + H, S_std=S_std, weights=weights)
    o, S = la.prefill(q, k, v, g, S_in=S_in, pos0=pos0, chunk=chunk, q_norm_w=qw, k_norm_w=kw)
    torch.cuda.synchronize()
    o_ref, S_ref = _oracle(q, k, v, g, S_in, pos0, qw, kw)
    assert_o_close(to_np(o), o_ref)
    assert_S_close(to_np(S), S_ref)
