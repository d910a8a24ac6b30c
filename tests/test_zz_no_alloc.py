"""la_prefill_noalloc (the workspace-free prefill, for callers that cannot
allocate) through the C ABI, against la_prefill: two calls in a row, the second
smaller, each bit-identical to la_prefill on the same inputs (both use the same
segment plan); a shape whose plan needs more states than the static scratch
holds, cut into longer segments and checked against la_prefill and the oracle;
and the B * H limit refused before anything runs."""
import ctypes

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
    la.library()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return la


def _noalloc(la, q, k, v, g, S_in, o, S_out, pos0, chunk):
    """Direct C-ABI call with caller-owned outputs."""
    B, T, H, _ = q.shape
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    return la.library().la_prefill_noalloc(p(q), p(k), p(v), p(g), p(S_in), p(S_out), p(o), B, T, H, D,
                                           pos0, chunk, 10000.0, 1e-6, None, None,
                                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("chunk", (0, 128))
def test_noalloc_equals_prefill_two_calls(la, chunk):
    print(f"no-alloc prefill, chunk {chunk}: a large call then a smaller one", flush=True)
    gen = workloads.generator(501, "cuda")
    for (B, T, H, pos0) in ((2, 9000, 16, 3), (1, 300, 4, 262144)):
        q, k, v, g = workloads.activations(B, T, H, D, 0, "cuda", gen=gen)
        S_in = workloads.state(B, H, D, 0.1, gen, "cuda")
        o_ref, S_ref = la.prefill(q, k, v, g, S_in=S_in, pos0=pos0, chunk=chunk)
        o = torch.full_like(q, float("nan"))
        S = torch.full_like(S_in, float("nan"))
        assert _noalloc(la, q, k, v, g, S_in, o, S, pos0, chunk) == 0
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(S, S_ref), (B, T, H)
        print(f"  B={B} T={T} H={H}: bit-identical to la_prefill", flush=True)


def test_noalloc_capped_plan(la):
    """300 heads x 65536 tokens: la_prefill cuts each head into 4 segments (1200
    states, 75 MiB), more than the scratch's 1024, so the call uses 3 longer ones."""
    print("no-alloc prefill with a capped plan (B*H = 300)", flush=True)
    B, T, H = 1, 65536, 300
    assert la.prefill_workspace_bytes(B, T, H) > 1024 * D * D * 4
    gen = workloads.generator(502, "cuda")
    q, k, v, g = workloads.activations(B, T, H, D, 0, "cuda", gen=gen)
    o_ref, S_ref = la.prefill(q, k, v, g, pos0=11)
    o = torch.empty_like(q)
    S = torch.empty_like(S_ref)
    assert _noalloc(la, q, k, v, g, None, o, S, 11, 0) == 0
    torch.cuda.synchronize()
    e = o_row_errors(to_np(o[:, -4096:]), to_np(o_ref[:, -4096:]))
    assert e["max"] <= 2e-2 and e["median"] <= 2e-3, e
    rel = float(torch.linalg.norm(S - S_ref) / torch.linalg.norm(S_ref))
    assert rel <= 1e-5, rel
    for h in (0, 299):
        sl = lambda t: to_np32(t[:, :, h:h + 1])  # noqa: E731
        o_or, S_or = oracle.forward(sl(q), sl(k), sl(v), sl(g), pos0=11)
        assert_o_close(to_np(o[:, :, h:h + 1]), o_or, what=f"head {h}")
        assert_S_close(to_np(S[:, h:h + 1]), S_or, what=f"head {h}")


@pytest.mark.parametrize("chunk", (0, 128, 256))
def test_noalloc_many_heads(la, chunk):
    """1100 sequence-heads: one segment each (no states kept) for every chunk size,
    bit-identical to la_prefill, which takes the same one-segment plan."""
    print(f"no-alloc prefill, 1100 heads, chunk {chunk}", flush=True)
    gen = workloads.generator(503, "cuda")
    q, k, v, g = workloads.activations(1, 300, 1100, D, 0, "cuda", gen=gen)
    S_in = workloads.state(1, 1100, D, 0.05, gen, "cuda")
    o_ref, S_ref = la.prefill(q, k, v, g, S_in=S_in, chunk=chunk)
    o = torch.empty_like(q)
    S = torch.empty_like(S_ref)
    assert _noalloc(la, q, k, v, g, S_in, o, S, 0, chunk) == 0
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
