"""The library holds no mutable state: calls issued at the same time from several
host threads, each on its own stream, give the same results, bit for bit, as the
same calls made one after another."""
import threading

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu
D = 128


@pytest.fixture(scope="module")
def la():
    import hybrid_sparse_linear_la_amd as la
    la.library()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return la


def _work(la, seed):
    """One thread's calls: a prefill, a varlen batch, three decode steps and a sparse
    prefill on inputs of its own."""
    B, T, H = 1, 3000 + 97 * seed, 4
    q, k, v, g = workloads.activations(B, T, H, D, 120 + seed, "cuda")
    S = torch.zeros((B, H, D, D), device="cuda")

    def run():
        o, S_out = la.prefill(q, k, v, g, pos0=seed)
        cu = [0, 1, 700, 700 + 1500, T]
        ov, Sv = la.prefill_varlen(q[0], k[0], v[0], g[0], cu, pos0=[5, 6, 7, 8])
        Sd = S_out.clone()
        od = [la.decode_step(q[:, n], k[:, n], v[:, n], g[:, n], Sd, T + n) for n in range(3)]
        os_ = la.sparse_prefill(q, k, v, g, topk=8)
        return [o, S_out, ov, Sv, Sd, *od, os_]
    del S
    return run


def test_concurrent_threads_match_sequential_calls(la):
    runs = [_work(la, s) for s in range(4)]
    torch.cuda.synchronize()
    expected = [r() for r in runs]
    torch.cuda.synchronize()

    results = [None] * len(runs)
    errors = []

    def worker(i):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                for _ in range(3):
                    results[i] = runs[i]()
            stream.synchronize()
        except Exception as e:  # reported below, in the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(runs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    torch.cuda.synchronize()
    for i, (got, want) in enumerate(zip(results, expected)):
        for n, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a, b), f"thread {i}: output {n} differs from the sequential run"
