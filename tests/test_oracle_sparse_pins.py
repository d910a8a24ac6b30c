"""Pins of the sparse-layer oracle (oracle.sparse_forward / sparse_decode) against
what the pages and plain mathematics fix, independent of the oracle itself:

* dense fallback: with no more than topk earlier blocks per query block the layer is
  ordinary causal softmax attention with the output gate, written here as numpy
  matrix products with an explicit mask;
* attention over a given block selection equals the same brute force with that
  selection's mask;
* planted selections: keys built so that known blocks score highest are the ones
  chosen (and ties go to the lower block);
* a decode step equals the last row of a prefill whose last query block is that
  single token;
* closed forms: identical keys average the attended values; g = 0 halves the output.

The layer's readings (block means, candidates, scale) are listed in
oracle/sparse_oracle.c.  CPU only.
"""
import numpy as np
import pytest

import oracle


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _masked_attention(q, k, v, g, allowed):
    """o[b, t, h] = sigmoid(g) * softmax over keys s with allowed[b, h, t, s] of
    q_t . k_s / sqrt(D), times v; numpy in float64."""
    q, k, v, g = (np.asarray(x, np.float64) for x in (q, k, v, g))
    B, T, H, D = q.shape
    o = np.empty((B, T, H, D))
    for b in range(B):
        for h in range(H):
            logits = q[b, :, h] @ k[b, :, h].T / np.sqrt(D)
            logits = np.where(allowed[b, h], logits, -np.inf)
            logits -= logits.max(axis=1, keepdims=True)
            p = np.exp(logits)
            p /= p.sum(axis=1, keepdims=True)
            o[b, :, h] = _sigmoid(g[b, :, h]) * (p @ v[b, :, h])
    return o


def _causal_mask(B, H, T):
    return np.broadcast_to(np.tril(np.ones((T, T), bool)), (B, H, T, T))


def _selection_mask(sel, T, block):
    """Allowed keys from a selection: the selected blocks plus the own block up to t."""
    B, H, nqb, _ = sel.shape
    allowed = np.zeros((B, H, T, T), bool)
    for b in range(B):
        for h in range(H):
            for i in range(nqb):
                r0, r1 = i * block, min(i * block + block, T)
                for t in range(r0, r1):
                    for j in sel[b, h, i]:
                        if j >= 0:
                            allowed[b, h, t, j * block:(j + 1) * block] = True
                    allowed[b, h, t, r0:t + 1] = True
    return allowed


def _inputs(B, T, H, D, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, T, H, D)).astype(np.float32) for _ in range(4)]


@pytest.mark.parametrize("B,T,H,D,block,topk", [(1, 70, 2, 16, 16, 4), (2, 33, 1, 8, 8, 4),
                                                (1, 50, 3, 32, 4, 100), (1, 1, 1, 8, 16, 1)])
def test_dense_fallback_is_causal_softmax_attention(B, T, H, D, block, topk):
    """At most topk earlier blocks per query block: every earlier block is attended."""
    assert -(-T // block) - 1 <= topk
    q, k, v, g = _inputs(B, T, H, D, seed=T + D)
    o, sel, _ = oracle.sparse_forward(q, k, v, g, block=block, topk=topk)
    want = _masked_attention(q, k, v, g, _causal_mask(B, H, T))
    np.testing.assert_allclose(o, want, rtol=1e-12, atol=1e-13)
    # every query block selects every earlier block, in increasing order
    for i in range(sel.shape[2]):
        assert list(sel[0, 0, i][sel[0, 0, i] >= 0]) == list(range(min(i, T // block)))


@pytest.mark.parametrize("T,block,topk", [(200, 16, 3), (130, 8, 5)])
def test_attention_over_its_selection_is_masked_softmax(T, block, topk):
    """The output is attention restricted to the chosen blocks plus the own block up
    to the query, both for the oracle's own choice and for an imposed one."""
    B, H, D = 1, 2, 16
    q, k, v, g = _inputs(B, T, H, D, seed=5)
    o, sel, _ = oracle.sparse_forward(q, k, v, g, block=block, topk=topk)
    np.testing.assert_allclose(o, _masked_attention(q, k, v, g, _selection_mask(sel, T, block)),
                               rtol=1e-12, atol=1e-13)
    # an imposed selection (lowest-index blocks, some slots unused)
    nqb = sel.shape[2]
    imposed = np.full_like(sel, -1)
    for i in range(nqb):
        m = min(i, T // block, topk - 1)
        imposed[:, :, i, :m] = np.arange(m)
    o2, sel2, _ = oracle.sparse_forward(q, k, v, g, block=block, topk=topk, sel=imposed)
    assert np.array_equal(sel2, imposed)
    np.testing.assert_allclose(o2, _masked_attention(q, k, v, g, _selection_mask(imposed, T, block)),
                               rtol=1e-12, atol=1e-13)


def test_planted_blocks_are_selected():
    """Query-block means are exactly e0; key block j has alpha_j in dim 0 plus a
    pattern in the other dims, which e0 does not see, so the scores are alpha_j: the
    chosen blocks are the topk largest alphas among the earlier blocks, and of three
    equal alphas the lower blocks win."""
    B, H, D, block, topk = 1, 1, 8, 4, 2
    nblk = 10
    T = nblk * block
    rng = np.random.default_rng(3)
    alpha = rng.permutation(np.arange(1, nblk + 1)).astype(np.float64)
    alpha[2] = alpha[5] = alpha[7] = 20.0     # a three-way tie at the top
    k = np.zeros((B, T, H, D), np.float32)
    for j in range(nblk):
        for u in range(block):
            k[0, j * block + u, 0, 0] = alpha[j]
            k[0, j * block + u, 0, 1 + u % (D - 1)] = (-1.0) ** u * 5.0
    q = np.zeros((B, T, H, D), np.float32)
    q[..., 0] = 1.0
    q[..., 1:] = rng.standard_normal((B, T, H, D - 1)) * 0.1
    # make every query block's mean exactly e0 * (row count): pair up the noise rows
    for i in range(nblk):
        q[0, i * block + 1, 0, 1:] = -q[0, i * block, 0, 1:]
        q[0, i * block + 3, 0, 1:] = -q[0, i * block + 2, 0, 1:]
    v, g = _inputs(B, T, H, D, seed=9)[:2]
    _, sel, scores = oracle.sparse_forward(q, k, v, g, block=block, topk=topk)
    for i in range(nblk):
        cand = list(range(i))
        order = sorted(cand, key=lambda j: (-alpha[j], j))[:topk]
        got = sorted(x for x in sel[0, 0, i] if x >= 0)
        assert got == sorted(order), f"query block {i}: {got} != {sorted(order)}"
        np.testing.assert_allclose(scores[0, 0, i, :i], alpha[:i], rtol=1e-12)


def test_decode_step_is_the_last_row_of_a_prefill():
    """When the last token opens a new block its query block is that token alone, so
    its selection and output are the decode step's."""
    B, H, D, block, topk = 2, 2, 16, 8, 3
    T = 6 * block + 1
    q, k, v, g = _inputs(B, T, H, D, seed=21)
    o, sel, _ = oracle.sparse_forward(q, k, v, g, block=block, topk=topk)
    Tmax = T + 5
    kc = np.zeros((B, Tmax, H, D), np.float32)
    vc = np.zeros((B, Tmax, H, D), np.float32)
    kc[:, :T], vc[:, :T] = k, v
    od, seld, _ = oracle.sparse_decode(q[:, T - 1], kc, vc, g[:, T - 1], np.full(B, T), block=block, topk=topk)
    np.testing.assert_allclose(od, o[:, T - 1], rtol=1e-12, atol=1e-13)
    assert np.array_equal(seld, sel[:, :, -1])


def test_decode_matches_masked_attention_at_ragged_lengths():
    B, H, D, block, topk, Tmax = 3, 2, 16, 8, 2, 90
    rng = np.random.default_rng(31)
    kc, vc = (rng.standard_normal((B, Tmax, H, D)).astype(np.float32) for _ in range(2))
    q, g = (rng.standard_normal((B, H, D)).astype(np.float32) for _ in range(2))
    lens = np.array([1, 37, 90])
    o, sel, scores = oracle.sparse_decode(q, kc, vc, g, lens, block=block, topk=topk)
    for b in range(B):
        t = lens[b] - 1
        own = t // block
        for h in range(H):
            kmean = kc[b, :own * block, h].reshape(own, block, D).astype(np.float64).mean(axis=1)
            sc = kmean @ q[b, h].astype(np.float64)
            np.testing.assert_allclose(scores[b, h, :own], sc, rtol=1e-12, atol=1e-12)
            best = sorted(sorted(range(own), key=lambda j: (-sc[j], j))[:topk])
            assert list(sel[b, h][sel[b, h] >= 0]) == best
            keys = [j * block + u for j in best for u in range(block)] + list(range(own * block, t + 1))
            logits = kc[b, keys, h].astype(np.float64) @ q[b, h].astype(np.float64) / np.sqrt(D)
            p = np.exp(logits - logits.max())
            p /= p.sum()
            want = _sigmoid(g[b, h].astype(np.float64)) * (p @ vc[b, keys, h].astype(np.float64))
            np.testing.assert_allclose(o[b, h], want, rtol=1e-12, atol=1e-13)


def test_identical_keys_average_the_values_and_zero_gate_halves():
    B, T, H, D, block, topk = 1, 40, 1, 8, 8, 2
    rng = np.random.default_rng(2)
    q, v = (rng.standard_normal((B, T, H, D)).astype(np.float32) for _ in range(2))
    k = np.broadcast_to(rng.standard_normal(D).astype(np.float32), (B, T, H, D)).copy()
    g = np.zeros((B, T, H, D), np.float32)
    o, sel, _ = oracle.sparse_forward(q, k, v, g, block=block, topk=topk)
    for t in range(T):
        i = t // block
        keys = [j * block + u for j in sel[0, 0, i] if j >= 0 for u in range(block)] + list(range(i * block, t + 1))
        np.testing.assert_allclose(o[0, t, 0], 0.5 * v[0, keys, 0].astype(np.float64).mean(axis=0),
                                   rtol=1e-12, atol=1e-13)
