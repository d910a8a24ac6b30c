"""GPU parity at the layer's full workload sizes, in the launch configuration the
benchmark times (default chunk, B = 1, 32 heads x 128):

  * 32K-token prefill: every output and the final state against the oracle;
  * 256K-token prefill at chunk 64, 128 and 256: every output row and every
    head's final state against the oracle (the oracle is chunk independent, so it
    runs once);
  * 1M tokens streamed as 16 segments of 65536 with S carried in place: equal to
    one single-shot call, and sampled heads against the oracle streamed segment by
    segment;
  * batched decode (64 sequences x 32 heads, 1000 steps from position 262144):
    o at every step and S after steps 1, 10 and 1000 against the oracle;
  * a packed serving batch (4 prompts of 16384 tokens and 60 decode steps) in one
    variable-length call: every decode row and sampled prompt heads;
  * the backward of the 32K-token prefill: every gradient row against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import assert_o_close, assert_S_close, o_row_errors, s_errors, to_np, to_np32

pytestmark = pytest.mark.gpu
D = 128


@pytest.fixture(scope="module")
def la():
    import hybrid_sparse_linear_la_amd as la
    la.library()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return la


def _head(t, h):
    """[B, T, H, D] GPU tensor -> float32 numpy [B, T, 1, D] of head h."""
    return to_np32(t[:, :, h:h + 1])


def test_prefill_32k_all_heads(la):
    w = workloads.PREFILL_32K
    print(f"workload {w.name}", flush=True)
    q, k, v, g = workloads.activations(w.B, w.T, w.H, D, w.seed, "cuda")
    o, S = la.prefill(q, k, v, g)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.forward(to_np32(q), to_np32(k), to_np32(v), to_np32(g))
    eo = assert_o_close(to_np(o), o_ref)
    es = assert_S_close(to_np(S), S_ref)
    print(f"32K parity o {eo} S {es}", flush=True)


@pytest.fixture(scope="module")
def ref_256k(la):
    """The 256K-token workload on the GPU and the oracle on all 32 heads (about a
    minute of host work); the oracle does not depend on the chunk size, so the
    three chunk sizes share it."""
    w = workloads.PREFILL_256K
    print(f"workload {w.name}: oracle on all {w.H} heads", flush=True)
    q, k, v, g = workloads.activations(w.B, w.T, w.H, D, w.seed, "cuda")
    o_ref, S_ref = oracle.forward(to_np32(q), to_np32(k), to_np32(v), to_np32(g))
    print("oracle done", flush=True)
    return q, k, v, g, o_ref, S_ref


@pytest.mark.timeout(900)
@pytest.mark.parametrize("chunk", (64, 128, 256))
def test_prefill_256k_all_heads(la, ref_256k, chunk):
    """Every output row and every head's final state of the 256K-token prefill, at
    each chunk size the benchmark sweeps, against the oracle."""
    q, k, v, g, o_ref, S_ref = ref_256k
    o, S = la.prefill(q, k, v, g, chunk=chunk)
    torch.cuda.synchronize()
    es = assert_S_close(to_np(S), S_ref, what=f"S C={chunk}")
    worst = {"max": 0.0}
    for h in range(q.shape[2]):
        e = assert_o_close(to_np(o[:, :, h:h + 1]), o_ref[:, :, h:h + 1], what=f"o C={chunk} head {h}")
        if e["max"] > worst["max"]:
            worst = dict(e, head=h)
    print(f"256K C={chunk} parity: worst head o {worst}, S {es}", flush=True)


def test_stream_1m_segmented_equals_single_shot(la):
    w = workloads.STREAM_1M
    print(f"workload {w.name}", flush=True)
    q, k, v, g = workloads.activations(w.B, w.T, w.H, D, w.seed, "cuda")
    o1, S1 = la.prefill(q, k, v, g)
    seg = w.T // w.segments
    S = torch.zeros((w.B, w.H, D, D), dtype=torch.float32, device="cuda")
    o2 = torch.empty_like(q)
    ws = torch.empty(la.prefill_workspace_bytes(w.B, seg, w.H), dtype=torch.uint8, device="cuda")
    for s in range(w.segments):
        sl = slice(s * seg, (s + 1) * seg)
        la.prefill(q[:, sl], k[:, sl], v[:, sl], g[:, sl], S_in=S, S_out=S, pos0=s * seg, out=o2[:, sl],
                   workspace=ws)
    torch.cuda.synchronize()
    # segmented and single-shot differ only in fp32 summation order of the carried state
    e = o_row_errors(to_np(o2[:, -seg:]), to_np(o1[:, -seg:]))
    assert e["max"] <= 2e-2, e
    es = s_errors(to_np(S), to_np(S1))
    assert es["fro"] <= 1e-3, es
    print(f"1M segmented vs single-shot: o {e} S {es}", flush=True)
    # sampled head against the oracle, streamed segment by segment (host memory bounded)
    h = 5
    S_ref = None
    worst = 0.0
    for s in range(w.segments):
        sl = slice(s * seg, (s + 1) * seg)
        o_ref, S_ref = oracle.forward(to_np32(q[:, sl, h:h + 1]), to_np32(k[:, sl, h:h + 1]),
                                      to_np32(v[:, sl, h:h + 1]), to_np32(g[:, sl, h:h + 1]),
                                      S=S_ref, pos0=s * seg)
        eo = assert_o_close(to_np(o2[:, sl, h:h + 1]), o_ref, what=f"o segment {s}")
        worst = max(worst, eo["max"])
    es = assert_S_close(to_np(S[:, h:h + 1]), S_ref, what="S after 1M tokens")
    print(f"1M head {h} vs oracle: worst segment o row error {worst:.3e}, S {es}", flush=True)


def test_decode_b64_1000_steps(la):
    w = workloads.DECODE_B64
    print(f"workload {w.name}", flush=True)
    S0, q, k, v, g = workloads.decode_inputs(w, device="cuda")
    S = S0.clone()
    outs = torch.empty_like(q)
    snaps = {}
    for n in range(w.steps):
        la.decode_step(q[n], k[n], v[n], g[n], S, w.pos0 + n, out=outs[n])
        if n + 1 in (1, 10):
            snaps[n + 1] = to_np(S)
    torch.cuda.synchronize()
    snaps[w.steps] = None
    S0_np = to_np(S0)
    # S after 1 and 10 steps: every sequence
    for n in (1, 10):
        _, S_ref = oracle.forward(to_np32(q[:n].transpose(0, 1)), to_np32(k[:n].transpose(0, 1)),
                                  to_np32(v[:n].transpose(0, 1)), to_np32(g[:n].transpose(0, 1)),
                                  S=S0_np, pos0=w.pos0)
        assert_S_close(snaps[n], S_ref, what=f"S after step {n}")
    # o at every step and S after 1000 steps: sampled sequences
    bs = [0, 31, 63]
    sel = lambda t: to_np32(t[:, bs].transpose(0, 1))  # noqa: E731  [3, steps, H, D]
    o_ref, S_ref = oracle.forward(sel(q), sel(k), sel(v), sel(g), S=S0_np[bs], pos0=w.pos0)
    eo = assert_o_close(to_np(outs[:, bs].transpose(0, 1)), o_ref, what="o over 1000 steps")
    es = assert_S_close(to_np(S[bs]), S_ref, what="S after 1000 steps")
    print(f"decode parity o {eo} S {es}", flush=True)


def test_serving_mix_varlen(la):
    """The packed serving batch the benchmark times (4 x 16384-token prompts from
    position 0 and 60 decode steps at position 262144, one la_prefill_varlen call):
    every decode row and its state, and sampled heads of the prompts, against the
    oracle."""
    w = workloads.SERVING_MIX
    print(f"workload {w.name}", flush=True)
    q, k, v, g, S_in, cu = workloads.mixed_inputs(w, "cuda")
    o, S_out = la.prefill_varlen(q, k, v, g, cu, pos0=list(w.pos0), S_in=S_in)
    torch.cuda.synchronize()
    n_pre = sum(1 for n in w.lengths if n > 1)
    # decode rows: all sequences and heads, one oracle step each
    t_dec = cu[n_pre:-1]
    row = lambda t: to_np32(t[t_dec][:, None])  # noqa: E731  [n_dec, 1, H, D]
    S_dec = to_np(S_in[n_pre:])
    o_ref, S_ref = oracle.forward(row(q), row(k), row(v), row(g), S=S_dec, pos0=w.pos0[-1])
    assert_o_close(to_np(o[t_dec][:, None]), o_ref, what="decode rows")
    assert_S_close(to_np(S_out[n_pre:]), S_ref, what="decode states")
    # prompts: heads 0 and 21 of the first and last prompt
    for b in (0, n_pre - 1):
        t0, t1 = cu[b], cu[b + 1]
        for h in (0, 21):
            sl = lambda t: to_np32(t[t0:t1, h:h + 1][None])  # noqa: E731
            o_ref, S_ref = oracle.forward(sl(q), sl(k), sl(v), sl(g), S=to_np(S_in[b:b + 1, h:h + 1]),
                                          pos0=w.pos0[b])
            eo = assert_o_close(to_np(o[t0:t1, h:h + 1][None]), o_ref, what=f"prompt {b} head {h}")
            assert_S_close(to_np(S_out[b:b + 1, h:h + 1]), S_ref, what=f"prompt {b} head {h} state")
            print(f"serving mix prompt {b} head {h}: o {eo}", flush=True)


def test_backward_32k_all_heads(la):
    """Gradients of the 32K-token prefill (32 heads x 128) for a seeded output
    gradient and final-state gradient: every row of dq, dk, dv, dgate and every
    dS_in against the oracle's reverse mode."""
    w = workloads.PREFILL_32K
    print(f"workload {w.name} backward", flush=True)
    gen = workloads.generator(w.seed, "cuda")
    q, k, v, g = workloads.activations(w.B, w.T, w.H, w.D, w.seed, "cuda", gen=gen)
    d_o = torch.randn(q.shape, generator=gen, device="cuda").to(torch.bfloat16)
    dS_out = workloads.state(w.B, w.H, w.D, 0.02, gen, "cuda")
    grads = la.backward(q, k, v, g, d_o, dS_out=dS_out)
    torch.cuda.synchronize()
    ref = oracle.backward(to_np32(q), to_np32(k), to_np32(v), to_np32(g), to_np32(d_o), dS_out=to_np(dS_out))
    for name, key in (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dgate", "dg")):
        e = assert_o_close(to_np(grads[name]), ref[key], what=f"32K {name}")
        print(f"32K backward {name}: {e}", flush=True)
    assert_S_close(to_np(grads["dS_in"]), ref["dS_in"], what="32K dS_in")
