"""GPU parity of la_decode_step against the fp64 oracle, and decode = prefill."""
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


@pytest.mark.parametrize("B,H,steps,pos,S_std,weights", [
    (1, 1, 1, 0, 0.0, False),
    (3, 5, 4, 262144, 0.02, False),
    (2, 32, 3, 1048575, 1.0, True),
])
def test_decode_matches_oracle(la, B, H, steps, pos, S_std, weights):
    print(f"decode case B={B} H={H} steps={steps} pos={pos}", flush=True)
    gen = workloads.generator(100 + B * H, "cuda")
    S = workloads.state(B, H, D, S_std, gen, "cuda") if S_std else torch.zeros(B, H, D, D, device="cuda")
    q, k, v, g = workloads.activations(steps, B, H, D, 0, "cuda", gen=gen)
    qw = kw = None
    if weights:
        qw = torch.rand(D, generator=gen, device="cuda") + 0.5
        kw = torch.rand(D, generator=gen, device="cuda") + 0.5
    S_ref = to_np(S)
    for n in range(steps):
        o = la.decode_step(q[n], k[n], v[n], g[n], S, pos + n, q_norm_w=qw, k_norm_w=kw)
        torch.cuda.synchronize()
        o_ref, S_ref = oracle.decode_step(to_np32(q[n]), to_np32(k[n]), to_np32(v[n]), to_np32(g[n]),
                                          S_ref, pos + n, q_w=None if qw is None else to_np32(qw),
                                          k_w=None if kw is None else to_np32(kw))
        assert_o_close(to_np(o), o_ref, what=f"o step {n}")
        assert_S_close(to_np(S), S_ref, what=f"S step {n}")


def test_decode_batch_beyond_the_cache(la):
    """A batch whose states exceed 192 MiB (100 x 32 heads: 200 MiB) is written back
    with non-temporal stores: the same step split into two halves (100 MiB each,
    plain stores) gives bit-identical o and S, and sampled sequences match the
    oracle."""
    B, H, steps, pos = 100, 32, 2, 262144
    gen = workloads.generator(4242, "cuda")
    S = workloads.state(B, H, D, 0.02, gen, "cuda")
    q, k, v, g = workloads.activations(steps, B, H, D, 0, "cuda", gen=gen)
    S_half = S.clone()
    picks = (0, 37, 99)
    S_ref = {b: to_np(S[b:b + 1]) for b in picks}
    for n in range(steps):
        o = la.decode_step(q[n], k[n], v[n], g[n], S, pos + n)
        halves = [la.decode_step(q[n][h0:h0 + 50].contiguous(), k[n][h0:h0 + 50].contiguous(),
                                 v[n][h0:h0 + 50].contiguous(), g[n][h0:h0 + 50].contiguous(),
                                 S_half[h0:h0 + 50], pos + n) for h0 in (0, 50)]
        torch.cuda.synchronize()
        assert torch.equal(o, torch.cat(halves)), f"o step {n}"
        assert torch.equal(S, S_half), f"S step {n}"
        for b in picks:
            o_ref, S_ref[b] = oracle.decode_step(to_np32(q[n][b:b + 1]), to_np32(k[n][b:b + 1]),
                                                 to_np32(v[n][b:b + 1]), to_np32(g[n][b:b + 1]), S_ref[b], pos + n)
            assert_o_close(to_np(o[b:b + 1]), o_ref, what=f"o step {n} sequence {b}")
            assert_S_close(to_np(S[b:b + 1]), S_ref[b], what=f"S step {n} sequence {b}")


def test_decode_steps_equal_prefill(la):
    B, H, N, pos0 = 2, 4, 24, 4000
    gen = workloads.generator(55, "cuda")
    S0 = workloads.state(B, H, D, 0.05, gen, "cuda")
    q, k, v, g = workloads.activations(B, N, H, D, 0, "cuda", gen=gen)
    o_pre, S_pre = la.prefill(q, k, v, g, S_in=S0, pos0=pos0)
    S = S0.clone()
    outs = []
    for n in range(N):
        outs.append(la.decode_step(q[:, n].contiguous(), k[:, n].contiguous(), v[:, n].contiguous(),
                                   g[:, n].contiguous(), S, pos0 + n))
    torch.cuda.synchronize()
    o_dec = torch.stack(outs, dim=1)
    # both are approximations of the same exact result: compare each to the oracle and to each other
    o_ref, S_ref = oracle.forward(to_np32(q), to_np32(k), to_np32(v), to_np32(g), S=to_np(S0), pos0=pos0)
    assert_o_close(to_np(o_dec), o_ref, what="decode")
    assert_o_close(to_np(o_pre), o_ref, what="prefill")
    assert_o_close(to_np(o_dec), to_np(o_pre), what="decode vs prefill")
    assert_S_close(to_np(S), S_ref, what="decode S")
    assert_S_close(to_np(S_pre), S_ref, what="prefill S")
    # prefill rounds kh to bf16 for the MFMA (relative 2^-9), decode keeps fp32
    assert_S_close(to_np(S_pre), to_np(S), what="prefill S vs decode S")


def test_decode_rejects_bad_arguments(la):
    q = torch.zeros(2, 3, D, dtype=torch.bfloat16, device="cuda")
    S = torch.zeros(2, 3, D, D, device="cuda")
    with pytest.raises(ValueError):
        la.decode_step(q, q, q, q, S[:1], 0)
    with pytest.raises(TypeError):
        la.decode_step(q.float(), q, q, q, S, 0)


def _random_decode(n, seed):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 70)), int(rng.integers(1, 40)), int(rng.integers(1, 4)),
             int(rng.choice([0, rng.integers(1, 5000), rng.integers(200000, 1 << 21)])),
             float(rng.choice([0.0, 0.02, 0.5])), bool(rng.integers(0, 2))) for _ in range(n)]


@pytest.mark.parametrize("B,H,steps,pos,S_std,weights", _random_decode(8, 717))
def test_decode_random_shapes_match_oracle(la, B, H, steps, pos, S_std, weights):
    """Seeded random batches, heads, positions (up to 2^21), states and norm weights."""
    test_decode_matches_oracle(la, B, H, steps, pos, S_std, weights)
