"""GPU parity of the sparse layer (la_sparse_prefill, la_sparse_block_means,
la_sparse_decode) against the fp64 oracle.

The block choice is an integer decision taken from fp32 scores on the GPU and fp64
scores in the oracle, so near-ties may resolve differently: the GPU's choice is
checked for validity (the right number of blocks, all of them candidates, none
scoring below an unchosen candidate by more than the fp32 rounding of a 128-term
dot product), and the outputs are compared with the oracle evaluated on the GPU's
choice, to the layer's row tolerance (2e-2 relative)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import assert_o_close, to_np, to_np32

pytestmark = pytest.mark.gpu
D = 128
BLK = 64
kMaxT = 8192 * BLK  # the most key blocks a sequence may have


@pytest.fixture(scope="module")
def la():
    import hybrid_sparse_linear_la_amd as la
    la.library()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return la


def _check_choice(sel, scores, ncand, topk, what):
    """sel: [..., topk] chosen blocks (increasing, then -1); scores: [..., nkb] fp64
    oracle scores; ncand: candidates per entry (same leading shape)."""
    sel = np.asarray(sel)
    flat_sel = sel.reshape(-1, sel.shape[-1])
    flat_sc = scores.reshape(-1, scores.shape[-1]) if scores.shape[-1] else np.zeros((flat_sel.shape[0], 0))
    flat_n = np.broadcast_to(ncand, sel.shape[:-1]).reshape(-1)
    differ = 0
    for e in range(flat_sel.shape[0]):
        n = int(flat_n[e])
        chosen = [int(x) for x in flat_sel[e] if x >= 0]
        assert len(chosen) == min(topk, n), f"{what} entry {e}: {len(chosen)} blocks for {n} candidates"
        assert chosen == sorted(set(chosen)) and all(0 <= x < n for x in chosen), f"{what} entry {e}: {chosen}"
        assert all(x == -1 for x in flat_sel[e][len(chosen):]), f"{what} entry {e}: padding"
        if n > topk:
            sc = flat_sc[e, :n]
            rest = np.setdiff1d(np.arange(n), chosen)
            tol = 1e-4 * np.abs(sc).max() + 1e-6
            assert sc[chosen].min() >= sc[rest].max() - tol, f"{what} entry {e}: a better block was left out"
            best = sorted(np.lexsort((np.arange(n), -sc))[:topk].tolist())
            differ += best != chosen
    return differ


def _prefill_case(la, B, T, H, topk, seed):
    q, k, v, g = workloads.activations(B, T, H, D, seed, "cuda")
    o, sel = la.sparse_prefill(q, k, v, g, topk=topk, return_sel=True)
    torch.cuda.synchronize()
    f = [to_np32(x) for x in (q, k, v, g)]
    # the oracle evaluated on the GPU's choice; its scores do not depend on the choice
    o_ref, _, scores = oracle.sparse_forward(*f, block=BLK, topk=topk, sel=sel.cpu().numpy())
    nqb = -(-T // BLK)
    ncand = np.minimum(np.arange(nqb), T // BLK)
    differ = _check_choice(sel.cpu().numpy(), scores, ncand[None, None, :], topk, f"prefill T={T}")
    err = assert_o_close(to_np(o), o_ref, what=f"sparse prefill B={B} T={T} H={H} topk={topk}")
    return err, differ


PREFILL_CASES = [
    # B, T, H, topk
    (1, 1, 1, 16),            # one token
    (1, 64, 2, 16),           # one full block
    (2, 300, 3, 16),          # dense regime (at most 4 earlier blocks)
    (1, 65 * 64 + 17, 2, 4),  # sparse: 65 full blocks and a ragged tail
    (2, 40 * 64, 2, 1),       # topk 1
    (1, 30 * 64 + 1, 1, 64),  # topk 64 (dense up to block 64), last block a single token
]


@pytest.mark.parametrize("B,T,H,topk", PREFILL_CASES)
def test_sparse_prefill_matches_oracle(la, B, T, H, topk):
    print(f"sparse prefill B={B} T={T} H={H} topk={topk}", flush=True)
    err, differ = _prefill_case(la, B, T, H, topk, seed=100 + T % 97 + topk)
    print(f"  row error max {err['max']:.2e}, choices differing from the fp64 order: {differ}", flush=True)


def _caches(B, Tmax, H, seed):
    gen = workloads.generator(seed, "cuda")
    kc, vc = (torch.randn((B, Tmax, H, D), generator=gen, device="cuda").to(torch.bfloat16) for _ in range(2))
    q, g = (torch.randn((B, H, D), generator=gen, device="cuda").to(torch.bfloat16) for _ in range(2))
    return q, kc, vc, g


@pytest.mark.parametrize("lens,H,topk", [([1, 63, 64, 65, 1000, 4096], 2, 16), ([4096, 2000], 3, 4),
                                         ([129, 3000], 2, 64)])
def test_sparse_decode_matches_oracle(la, lens, H, topk):
    print(f"sparse decode lens={lens} H={H} topk={topk}", flush=True)
    B, Tmax = len(lens), 4096
    q, kc, vc, g = _caches(B, Tmax, H, seed=200 + topk)
    means = la.sparse_block_means(kc)
    lt = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o, sel = la.sparse_decode(q, kc, vc, means, g, lt, topk=topk, return_sel=True)
    torch.cuda.synchronize()
    f = [to_np32(x) for x in (q, kc, vc, g)]
    o_ref, _, scores = oracle.sparse_decode(*f, np.array(lens), block=BLK, topk=topk, sel=sel.cpu().numpy())
    ncand = np.array([(n - 1) // BLK for n in lens])
    _check_choice(sel.cpu().numpy(), scores, ncand[:, None], topk, "decode")
    assert_o_close(to_np(o)[:, None], o_ref[:, None], what=f"sparse decode lens={lens}")


def test_block_means_match_and_update_in_place(la):
    B, Tmax, H = 2, 1024, 3
    _, kc, _, _ = _caches(B, Tmax, H, seed=7)
    means = la.sparse_block_means(kc)
    ref = to_np32(kc).astype(np.float64).reshape(B, Tmax // BLK, BLK, H, D).mean(axis=2).transpose(0, 2, 1, 3)
    np.testing.assert_allclose(to_np(means), ref, rtol=1e-5, atol=1e-6)
    # recompute two blocks after changing them
    kc[:, 3 * BLK:5 * BLK] = 0
    la.sparse_block_means(kc, means, first_block=3, nblocks=2)
    torch.cuda.synchronize()
    ref[:, :, 3:5] = 0
    np.testing.assert_allclose(to_np(means), ref, rtol=1e-5, atol=1e-6)


def test_decode_is_the_last_row_of_prefill(la):
    """When the newest token opens a block, decode and prefill take the same choice
    (the query block is that token); outputs agree to the rounding of each path."""
    B, H, topk = 1, 2, 4
    T = 40 * BLK + 1
    q, k, v, g = workloads.activations(B, T, H, D, 17, "cuda")
    o, sel = la.sparse_prefill(q, k, v, g, topk=topk, return_sel=True)
    means = la.sparse_block_means(k)
    od, seld = la.sparse_decode(q[:, -1].contiguous(), k, v, means, g[:, -1].contiguous(),
                                torch.tensor([T], dtype=torch.int32, device="cuda"), topk=topk, return_sel=True)
    torch.cuda.synchronize()
    assert torch.equal(seld, sel[:, :, -1])
    a, b = to_np(od), to_np(o[:, -1])
    rel = np.linalg.norm(a - b, axis=-1) / np.linalg.norm(b, axis=-1)
    assert rel.max() <= 2e-2, rel.max()


def test_sparse_prefill_32k_sampled_heads(la):
    """The 32K workload (B 1, T 32768, H 32, topk 16) as the bench runs it; the
    oracle checks two heads (all 512 query blocks each)."""
    w = workloads.SPARSE_32K
    q, k, v, g = workloads.activations(w.B, w.T, w.H, D, w.seed, "cuda")
    o, sel = la.sparse_prefill(q, k, v, g, topk=w.topk, return_sel=True)
    torch.cuda.synchronize()
    for h in (0, 29):
        f = [to_np32(x[:, :, h:h + 1]) for x in (q, k, v, g)]
        s = sel[:, h:h + 1].cpu().numpy()
        o_ref, _, scores = oracle.sparse_forward(*f, block=BLK, topk=w.topk, sel=s)
        differ = _check_choice(s, scores, np.arange(w.T // BLK)[None, None, :], w.topk, f"32K head {h}")
        e = assert_o_close(to_np(o[:, :, h:h + 1]), o_ref, what=f"32K head {h}")
        print(f"head {h}: row error max {e['max']:.2e}, choices differing from the fp64 order: {differ}",
              flush=True)


def test_tied_scores_choose_the_lowest_blocks(la):
    """Identical keys give every key block the same mean and every candidate the
    same score: each query block must take the topk lowest blocks."""
    B, T, H, topk = 1, 40 * BLK + 7, 2, 4
    q, k, v, g = workloads.activations(B, T, H, D, 23, "cuda")
    k = k[:, :1].expand(B, T, H, D).contiguous()
    o, sel = la.sparse_prefill(q, k, v, g, topk=topk, return_sel=True)
    torch.cuda.synchronize()
    s = sel.cpu().numpy()
    for i in range(s.shape[2]):
        want = list(range(min(i, topk))) + [-1] * (topk - min(i, topk))
        assert list(s[0, 0, i]) == want and list(s[0, 1, i]) == want, (i, s[0, :, i])
    f = [to_np32(x) for x in (q, k, v, g)]
    o_ref, sel_ref, _ = oracle.sparse_forward(*f, block=BLK, topk=topk)
    assert np.array_equal(sel_ref, s)
    assert_o_close(to_np(o), o_ref, what="tied scores")


def test_sparse_rejects_bad_arguments(la):
    q, k, v, g = workloads.activations(1, 100, 2, D, 3, "cuda")
    with pytest.raises(la.LAError):
        la.sparse_prefill(q, k, v, g, topk=0)
    with pytest.raises(la.LAError):
        la.sparse_prefill(q, k, v, g, topk=65)
    with pytest.raises(ValueError):
        la.sparse_prefill(q, k[:, :50].contiguous(), v, g)


def test_blocks_far_above_the_own_block_restart_the_pass(la):
    """Keys of block 3 (6 q) and block 7 (9 q) give logits about 98 and 147 base-2
    units above the own blocks' (small random keys): the attention must restart its
    pass with a raised reference (twice for query blocks that choose both) and still
    match the fp64 softmax."""
    B, T, H, topk = 1, 20 * BLK, 1, 4
    gen = workloads.generator(41, "cuda")
    q = torch.ones((B, T, H, D), device="cuda")
    k = 0.05 * torch.randn((B, T, H, D), generator=gen, device="cuda")
    k[:, 3 * BLK:4 * BLK] = 6.0
    k[:, 7 * BLK:8 * BLK] = 9.0
    v, g = (torch.randn((B, T, H, D), generator=gen, device="cuda") for _ in range(2))
    q, k, v, g = (x.to(torch.bfloat16) for x in (q, k, v, g))
    o, sel = la.sparse_prefill(q, k, v, g, topk=topk, return_sel=True)
    torch.cuda.synchronize()
    s = sel.cpu().numpy()
    for i in range(8, T // BLK):
        assert 3 in s[0, 0, i] and 7 in s[0, 0, i], (i, s[0, 0, i])
    assert torch.isfinite(o.float()).all()
    f = [to_np32(x) for x in (q, k, v, g)]
    o_ref, _, _ = oracle.sparse_forward(*f, block=BLK, topk=topk, sel=s)
    assert_o_close(to_np(o), o_ref, what="restarted passes")


def _attend_rows(q, k, v, g, rows, keys, allowed):
    """fp64 softmax attention of query rows over key rows (token indices), restricted
    to allowed[row, key], gated: o = sigmoid(g) * softmax(q k / sqrt(D)) v."""
    qd, kd, vd = (x.astype(np.float64) for x in (q, k, v))
    logits = np.where(allowed, qd[rows] @ kd[keys].T / np.sqrt(D), -np.inf)
    logits -= logits.max(axis=1, keepdims=True)
    pr = np.exp(logits)
    pr /= pr.sum(axis=1, keepdims=True)
    return 1.0 / (1.0 + np.exp(-g[rows].astype(np.float64))) * (pr @ vd[keys])


def test_sparse_prefill_at_the_largest_supported_length(la):
    """8192 key blocks (T = 524288, one head), where the full fp64 oracle takes minutes:
    on sampled query blocks (the last ones included) the GPU's choice is checked
    against fp64 block scores and its output against fp64 softmax attention over that
    choice, causal in the own block."""
    B, T, H, topk = 1, kMaxT, 1, 16
    q, k, v, g = workloads.activations(B, T, H, D, 61, "cuda")
    o, sel = la.sparse_prefill(q, k, v, g, topk=topk, return_sel=True)
    torch.cuda.synchronize()
    qn, kn, vn, gn = (to_np32(x)[0, :, 0] for x in (q, k, v, g))
    on, s = to_np(o)[0, :, 0], sel.cpu().numpy()[0, 0]
    kmean = kn.astype(np.float64).reshape(T // BLK, BLK, D).mean(axis=1)
    nqb = T // BLK
    for i in (1, 17, 1000, 4097, nqb - 2, nqb - 1):
        qmean = qn[i * BLK:(i + 1) * BLK].astype(np.float64).mean(axis=0)
        scores = (kmean[:i] @ qmean)[None, None, None, :]
        _check_choice(s[i][None, None, None, :], scores, np.array([i]), topk, f"query block {i}")
        rows = np.arange(i * BLK, (i + 1) * BLK)
        keys = np.array([int(j) * BLK + u for j in s[i] if j >= 0 for u in range(BLK)] + list(rows))
        allowed = (keys[None, :] < i * BLK) | (keys[None, :] <= rows[:, None])  # own block: causal
        ref = _attend_rows(qn, kn, vn, gn, rows, keys, allowed)
        assert_o_close(on[rows][None, :, None], ref[None, :, None], what=f"query block {i} of {nqb}")


def test_sparse_decode_at_the_largest_supported_cache(la):
    """A full 524288-token cache (8191 candidate blocks): the choice against fp64
    scores, the output against fp64 softmax attention over it."""
    B, Tmax, H, topk = 1, kMaxT, 2, 16
    q, kc, vc, g = _caches(B, Tmax, H, seed=62)
    means = la.sparse_block_means(kc)
    lens = torch.tensor([Tmax], dtype=torch.int32, device="cuda")
    o, sel = la.sparse_decode(q, kc, vc, means, g, lens, topk=topk, return_sel=True)
    torch.cuda.synchronize()
    t = Tmax - 1
    own = t // BLK
    for h in range(H):
        qn, gn = to_np32(q)[0, h], to_np32(g)[0, h]
        kn, vn = to_np32(kc)[0, :, h], to_np32(vc)[0, :, h]
        kmean = kn[:own * BLK].astype(np.float64).reshape(own, BLK, D).mean(axis=1)
        s = sel.cpu().numpy()[0, h]
        _check_choice(s[None, :], (kmean @ qn.astype(np.float64))[None, :], np.array([own]), topk, f"head {h}")
        keys = [int(j) * BLK + u for j in s if j >= 0 for u in range(BLK)] + list(range(own * BLK, t + 1))
        logits = kn[keys].astype(np.float64) @ qn.astype(np.float64) / np.sqrt(D)
        pr = np.exp(logits - logits.max())
        pr /= pr.sum()
        ref = (pr @ vn[keys].astype(np.float64)) / (1.0 + np.exp(-gn.astype(np.float64)))
        assert_o_close(to_np(o)[0, h][None, None, None], ref[None, None, None], what=f"decode head {h}")


def _random_sparse_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B = int(rng.integers(1, 3))
        T = int(rng.choice([rng.integers(1, 200), rng.integers(200, 3000), rng.integers(3000, 9000)]))
        H = int(rng.integers(1, 5))
        topk = int(rng.choice([1, 2, 7, 16, 33, 64]))
        out.append((B, T, H, topk))
    return out


@pytest.mark.parametrize("B,T,H,topk", _random_sparse_cases(8, 77))
def test_sparse_random_shapes_match_oracle(la, B, T, H, topk):
    print(f"random sparse case B={B} T={T} H={H} topk={topk}", flush=True)
    err, differ = _prefill_case(la, B, T, H, topk, seed=300 + T % 101 + topk)
    print(f"  row error max {err['max']:.2e}, choices differing from the fp64 order: {differ}", flush=True)
