"""GPU parity of la_prefill_varlen (packed variable-length batches, including
single-token decode steps and empty sequences) against the fp64 oracle run on
each sequence alone, and its agreement with la_prefill / la_decode_step."""
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
    la.library()  # raises if the HIP library is not built
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return la


def _packed(lengths, H, seed, S_std=0.0, weights=False):
    total = int(sum(lengths))
    gen = workloads.generator(seed, "cuda")
    q, k, v, g = workloads.activations(1, max(total, 1), H, D, seed, "cuda", gen=gen)
    q, k, v, g = (x[0, :total].contiguous() for x in (q, k, v, g))
    S_in = workloads.state(len(lengths), H, D, S_std, gen, "cuda") if S_std else None
    qw = kw = None
    if weights:
        qw = torch.rand(D, generator=gen, device="cuda") + 0.5
        kw = torch.rand(D, generator=gen, device="cuda") + 0.5
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64).tolist()
    return q, k, v, g, S_in, qw, kw, cu


def _check_against_oracle(o, S_out, q, k, v, g, S_in, cu, pos0, qw=None, kw=None):
    o_np, S_np = to_np(o), to_np(S_out)
    for b in range(len(cu) - 1):
        t0, t1 = cu[b], cu[b + 1]
        S_ref_in = None if S_in is None else to_np(S_in[b:b + 1])
        if t1 == t0:
            want = np.zeros((1,) + S_np.shape[1:]) if S_ref_in is None else S_ref_in
            assert np.array_equal(S_np[b:b + 1], want), f"empty sequence {b}: S_out != S_in"
            continue
        sl = lambda x: to_np32(x[t0:t1])[None]  # noqa: E731
        o_ref, S_ref = oracle.forward(sl(q), sl(k), sl(v), sl(g), S=S_ref_in, pos0=pos0[b],
                                      q_w=None if qw is None else to_np32(qw),
                                      k_w=None if kw is None else to_np32(kw))
        assert_o_close(o_np[t0:t1][None], o_ref, what=f"o of sequence {b} (T={t1 - t0})")
        assert_S_close(S_np[b:b + 1], S_ref, what=f"S of sequence {b} (T={t1 - t0})")


CASES = [
    # lengths, H, S_std, weights, chunk
    ([0, 1, 2, 63, 64, 65, 300, 1, 1000], 4, 0.3, False, 0),
    ([1, 1, 1, 1, 1], 2, 0.5, True, 0),               # decode steps only
    ([0, 0, 0], 3, 0.2, False, 0),                     # empty sequences only: S_out = S_in
    ([5000, 1, 37, 1, 2048], 8, 0.0, False, 0),        # several segments per head in the long ones
    ([129, 1, 700, 256], 4, 0.1, True, 128),
    ([300, 1, 1000, 257], 2, 0.1, False, 256),
]


@pytest.mark.parametrize("lengths,H,S_std,weights,chunk", CASES)
def test_varlen_matches_oracle(la, lengths, H, S_std, weights, chunk):
    print(f"varlen case lengths={lengths} H={H} chunk={chunk}", flush=True)
    q, k, v, g, S_in, qw, kw, cu = _packed(lengths, H, seed=41 + len(lengths) + H, S_std=S_std,
                                           weights=weights)
    pos0 = [1000 * b + 7 * (b % 3) for b in range(len(lengths))]
    pos0[-1] = 262144
    o, S_out = la.prefill_varlen(q, k, v, g, cu, pos0=pos0, S_in=S_in, chunk=chunk, q_norm_w=qw, k_norm_w=kw)
    torch.cuda.synchronize()
    _check_against_oracle(o, S_out, q, k, v, g, S_in, cu, pos0, qw, kw)


def test_varlen_without_initial_state_and_in_place(la):
    lengths = [1, 200, 0, 65, 1]
    q, k, v, g, S_in, _, _, cu = _packed(lengths, 3, seed=51, S_std=0.4)
    pos0 = [5, 0, 9, 100000, 3]
    o0, S0 = la.prefill_varlen(q, k, v, g, cu, pos0=pos0)           # S_in = zeros
    S = S_in.clone()
    o1, S1 = la.prefill_varlen(q, k, v, g, cu, pos0=pos0, S_in=S, S_out=S)  # carried in place
    torch.cuda.synchronize()
    assert S1.data_ptr() == S.data_ptr()
    _check_against_oracle(o0, S0, q, k, v, g, None, cu, pos0)
    _check_against_oracle(o1, S1, q, k, v, g, S_in, cu, pos0)


def test_varlen_equal_lengths_is_prefill(la):
    """Equal lengths give the segments la_prefill uses, so the results are identical."""
    B, T, H = 3, 777, 4
    gen = workloads.generator(61, "cuda")
    q, k, v, g = workloads.activations(B, T, H, D, 61, "cuda", gen=gen)
    S_in = workloads.state(B, H, D, 0.1, gen, "cuda")
    o_ref, S_ref = la.prefill(q, k, v, g, S_in=S_in, pos0=4242)
    flat = lambda x: x.reshape(B * T, H, D)  # noqa: E731
    o, S = la.prefill_varlen(flat(q), flat(k), flat(v), flat(g), [0, T, 2 * T, 3 * T], pos0=[4242] * B,
                             S_in=S_in)
    torch.cuda.synchronize()
    assert torch.equal(o, flat(o_ref))
    assert torch.equal(S, S_ref)


def test_varlen_decode_rows_are_decode_steps(la):
    """Single-token sequences run the decode kernel: identical to la_decode_step."""
    B, H = 6, 4
    gen = workloads.generator(71, "cuda")
    q, k, v, g = workloads.activations(1, B, H, D, 71, "cuda", gen=gen)
    q, k, v, g = (x[0].contiguous() for x in (q, k, v, g))
    S_in = workloads.state(B, H, D, 0.05, gen, "cuda")
    pos = 262144
    S_dec = S_in.clone()
    o_dec = la.decode_step(q, k, v, g, S_dec, pos)
    o, S = la.prefill_varlen(q, k, v, g, list(range(B + 1)), pos0=[pos] * B, S_in=S_in)
    torch.cuda.synchronize()
    assert torch.equal(o, o_dec)
    assert torch.equal(S, S_dec)


def test_varlen_rejects_bad_arguments(la):
    q, k, v, g, _, _, _, cu = _packed([3, 4], 2, seed=81)
    with pytest.raises(la.LAError):
        la.prefill_varlen(q, k, v, g, [0, 3, 8])      # last offset != total tokens
    with pytest.raises(la.LAError):
        la.prefill_varlen(q, k, v, g, [0, 4, 3])      # decreasing offsets
    with pytest.raises(ValueError):
        la.prefill_varlen(q, k, v, g, cu, pos0=[0])   # pos0 of the wrong length


def _random_batches(n, seed):
    """Seeded random packed batches: 1-40 sequences mixing empty ones, decode steps
    and prompts up to a few thousand tokens, random positions, heads and chunk."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        nseq = int(rng.integers(1, 41))
        kinds = rng.integers(0, 4, nseq)
        lengths = [int([0, 1, rng.integers(2, 200), rng.integers(200, 3000)][kd]) for kd in kinds]
        pos0 = [int(rng.choice([0, rng.integers(1, 5000), rng.integers(200000, 900000)])) for _ in range(nseq)]
        out.append((lengths, pos0, int(rng.integers(1, 7)), float(rng.choice([0.0, 0.3])),
                    bool(rng.integers(0, 2)), int(rng.choice([0, 128, 256]))))
    return out


@pytest.mark.parametrize("lengths,pos0,H,S_std,weights,chunk", _random_batches(6, 99))
def test_varlen_random_batches_match_oracle(la, lengths, pos0, H, S_std, weights, chunk):
    print(f"random varlen case nseq={len(lengths)} total={sum(lengths)} H={H} chunk={chunk}", flush=True)
    q, k, v, g, S_in, qw, kw, cu = _packed(lengths, H, seed=61 + len(lengths) + H, S_std=S_std,
                                           weights=weights)
    o, S_out = la.prefill_varlen(q, k, v, g, cu, pos0=pos0, S_in=S_in, chunk=chunk, q_norm_w=qw, k_norm_w=kw)
    torch.cuda.synchronize()
    _check_against_oracle(o, S_out, q, k, v, g, S_in, cu, pos0, qw, kw)
