"""The library's calls captured in HIP graphs: every replay (three, with the
program's own eager work and synchronizations between them) must reproduce the
eager result bit for bit (the kernels are deterministic and read nothing that a
replay changes).  Graphs hold kernel launches only: none of these calls records a
memset or a host copy."""
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


def _replays(graph, reset, outputs, expected, what):
    for rep in range(3):
        reset()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("first", "second", "third", "fourth"), outputs, expected):
            assert torch.equal(got, want), f"{what}: replay {rep}, {name} output differs from the eager run"
        # eager work between replays
        torch.randn(1 << 20, device="cuda").sum().item()


def test_decode_steps_in_a_graph(la):
    B, H, steps, pos = 8, 32, 6, 262144
    gen = workloads.generator(91, "cuda")
    S0 = workloads.state(B, H, D, 0.02, gen, "cuda")
    q, k, v, g = workloads.activations(steps, B, H, D, 0, "cuda", gen=gen)
    S_e, o_e = S0.clone(), torch.empty_like(q)
    for n in range(steps):
        la.decode_step(q[n], k[n], v[n], g[n], S_e, pos + n, out=o_e[n])
    S_g, o_g = S0.clone(), torch.empty_like(q)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for n in range(steps):
            la.decode_step(q[n], k[n], v[n], g[n], S_g, pos + n, out=o_g[n])
    _replays(graph, lambda: S_g.copy_(S0), (o_g, S_g), (o_e, S_e), "decode")


def test_prefill_in_a_graph(la):
    B, T, H = 1, 5000, 8
    gen = workloads.generator(92, "cuda")
    q, k, v, g = workloads.activations(B, T, H, D, 92, "cuda", gen=gen)
    S_in = workloads.state(B, H, D, 0.3, gen, "cuda")
    ws = torch.empty(la.prefill_workspace_bytes(B, T, H), dtype=torch.uint8, device="cuda")
    o_e, S_e = la.prefill(q, k, v, g, S_in=S_in, pos0=77, workspace=ws)
    o_g, S_g = torch.empty_like(o_e), torch.empty_like(S_e)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        la.prefill(q, k, v, g, S_in=S_in, pos0=77, out=o_g, S_out=S_g, workspace=ws)
    _replays(graph, lambda: None, (o_g, S_g), (o_e, S_e), "prefill")


def test_sparse_prefill_and_decode_in_a_graph(la):
    B, T, H, topk = 1, 40 * 64 + 9, 4, 8
    q, k, v, g = workloads.activations(B, T, H, D, 93, "cuda")
    ws = torch.empty(la.sparse_prefill_workspace_bytes(B, T, H, topk=topk), dtype=torch.uint8, device="cuda")
    o_e = la.sparse_prefill(q, k, v, g, topk=topk, workspace=ws)
    means = la.sparse_block_means(k)
    lens = torch.tensor([T], dtype=torch.int32, device="cuda")
    od_e = la.sparse_decode(q[:, -1].contiguous(), k, v, means, g[:, -1].contiguous(), lens, topk=topk)
    o_g, od_g = torch.empty_like(o_e), torch.empty_like(od_e)
    q1, g1 = q[:, -1].contiguous(), g[:, -1].contiguous()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        la.sparse_prefill(q, k, v, g, topk=topk, out=o_g, workspace=ws)
        la.sparse_decode(q1, k, v, means, g1, lens, topk=topk, out=od_g)
    _replays(graph, lambda: None, (o_g, od_g), (o_e, od_e), "sparse")
