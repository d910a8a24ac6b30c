"""GPU parity of the projections around the layer: la_linear against a float64
matrix product, and la_layer_forward (projection, layer, output projection)
against the oracle's layer."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import assert_o_close, assert_S_close, o_row_errors, to_np, to_np32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def la():
    import hybrid_sparse_linear_la_amd as la
    la.library()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return la


def _linear_close(y, ref, what):
    """bf16 output: every element within one bf16 rounding (2^-8 relative, with a
    floor of 2^-8 of the row's rms for entries that cancel); rows within 4e-3."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref ** 2, axis=-1, keepdims=True))
    bound = 2.0 ** -8 * np.maximum(np.abs(ref), rms)
    worst = float(np.max(np.abs(y - ref) / bound))
    assert worst <= 1.0, f"{what}: element error {worst:.2f} x the bf16 bound"
    rel = np.linalg.norm(y - ref, axis=-1) / np.maximum(np.linalg.norm(ref, axis=-1), 1e-30)
    assert rel.max() <= 4e-3, f"{what}: row error {rel.max():.2e}"


LINEAR_CASES = [(1, 256, 64), (77, 512, 128), (300, 256, 4096), (1000, 768, 192), (513, 1024, 1024)]


@pytest.mark.parametrize("M,N,K", LINEAR_CASES)
def test_linear_matches_float64(la, M, N, K):
    print(f"linear case M={M} N={N} K={K}", flush=True)
    gen = workloads.generator(100 + M, "cuda")
    x = torch.randn((M, K), generator=gen, device="cuda").to(torch.bfloat16)
    w = (torch.randn((N, K), generator=gen, device="cuda") / K ** 0.5).to(torch.bfloat16)
    y = la.linear(x, w)
    torch.cuda.synchronize()
    _linear_close(to_np(y), oracle.linear(to_np(x), to_np(w)), f"linear {M}x{N}x{K}")


def test_linear_full_width_sampled_rows(la):
    """The fused q/k/v/gate projection of a 32K-token prompt (M 32768, N 16384,
    K 4096): 64 sampled rows against float64, every column."""
    w = workloads.LAYER_32K
    x, w_qkvg, _ = workloads.layer_inputs(w.B, w.T, w.hidden, w.H, w.D, w.seed, "cuda")
    y = la.linear(x, w_qkvg)
    torch.cuda.synchronize()
    rows = torch.tensor([0, 1, 255, 256, 4097, 32767] + list(range(1000, 32768, 558)), device="cuda")
    xs = to_np(x[0, rows])
    _linear_close(to_np(y[0, rows]), oracle.linear(xs, to_np(w_qkvg)), "projection rows")


LAYER_CASES = [
    # B, T, hidden, H, pos0, S_std, weights
    (1, 1, 256, 2, 0, 0.0, False),
    (2, 300, 256, 2, 5, 0.3, True),
    (1, 1000, 512, 4, 262144, 0.0, False),
]


@pytest.mark.parametrize("B,T,hidden,H,pos0,S_std,weights", LAYER_CASES)
def test_layer_forward_matches_oracle(la, B, T, hidden, H, pos0, S_std, weights):
    print(f"layer case B={B} T={T} hidden={hidden} H={H}", flush=True)
    x, w_qkvg, w_o = workloads.layer_inputs(B, T, hidden, H, 128, seed=200 + T, device="cuda")
    gen = workloads.generator(300 + T, "cuda")
    S_in = workloads.state(B, H, 128, S_std, gen, "cuda") if S_std else None
    qw = kw = None
    if weights:
        qw = torch.rand(128, generator=gen, device="cuda") + 0.5
        kw = torch.rand(128, generator=gen, device="cuda") + 0.5
    y, S = la.layer_forward(x, w_qkvg, w_o, S_in=S_in, pos0=pos0, q_norm_w=qw, k_norm_w=kw)
    torch.cuda.synchronize()
    y_ref, S_ref = oracle.layer_forward(to_np32(x), to_np32(w_qkvg), to_np32(w_o),
                                        S=None if S_in is None else to_np(S_in), pos0=pos0,
                                        q_w=None if qw is None else to_np32(qw),
                                        k_w=None if kw is None else to_np32(kw))
    assert_o_close(to_np(y), y_ref, what="layer output")
    assert_S_close(to_np(S), S_ref, what="layer state")


def test_layer_full_width(la):
    """hidden 4096, 32 heads x 128, 4096 tokens: every output row and the state."""
    x, w_qkvg, w_o = workloads.layer_inputs(1, 4096, 4096, 32, 128, seed=6, device="cuda")
    y, S = la.layer_forward(x, w_qkvg, w_o, pos0=123)
    torch.cuda.synchronize()
    y_ref, S_ref = oracle.layer_forward(to_np32(x), to_np32(w_qkvg), to_np32(w_o), pos0=123)
    e = assert_o_close(to_np(y), y_ref, what="layer output (full width)")
    assert_S_close(to_np(S), S_ref, what="layer state (full width)")
    print(f"full-width layer: {e}", flush=True)


def test_layer_is_its_parts(la):
    """la_layer_forward equals la_linear -> la_prefill -> la_linear bit for bit."""
    B, T, hidden, H = 2, 500, 512, 4
    x, w_qkvg, w_o = workloads.layer_inputs(B, T, hidden, H, 128, seed=77, device="cuda")
    y, S = la.layer_forward(x, w_qkvg, w_o, pos0=9)
    proj = la.linear(x, w_qkvg)
    q, k, v, g = (proj[..., i * H * 128:(i + 1) * H * 128].reshape(B, T, H, 128).contiguous() for i in range(4))
    o, S2 = la.prefill(q, k, v, g, pos0=9)
    y2 = la.linear(o.reshape(B, T, H * 128), w_o)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    assert torch.equal(S, S2)


def test_linear_rejects_bad_shapes(la):
    x = torch.zeros((4, 100), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(la.LAError):
        la.linear(x, torch.zeros((256, 100), dtype=torch.bfloat16, device="cuda"))   # K % 64
    x = torch.zeros((4, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(la.LAError):
        la.linear(x, torch.zeros((100, 128), dtype=torch.bfloat16, device="cuda"))   # N % 256
    with pytest.raises(ValueError):
        la.linear(x, torch.zeros((256, 64), dtype=torch.bfloat16, device="cuda"))    # K mismatch


def _random_linear(n, seed):
    rng = np.random.default_rng(seed)
    return [(int(rng.choice([rng.integers(1, 64), rng.integers(64, 700), rng.integers(700, 3000)])),
             256 * int(rng.integers(1, 9)), 64 * int(rng.integers(1, 40))) for _ in range(n)]


@pytest.mark.parametrize("M,N,K", _random_linear(8, 313))
def test_linear_random_shapes_match_float64(la, M, N, K):
    """Seeded random shapes: any M (ragged last row tile), N a multiple of 256, K of 64."""
    print(f"random linear case M={M} N={N} K={K}", flush=True)
    gen = workloads.generator(200 + M + K, "cuda")
    x = torch.randn((M, K), generator=gen, device="cuda").to(torch.bfloat16)
    w = (torch.randn((N, K), generator=gen, device="cuda") / K ** 0.5).to(torch.bfloat16)
    y = la.linear(x, w)
    torch.cuda.synchronize()
    _linear_close(to_np(y), oracle.linear(to_np(x), to_np(w)), f"linear {M}x{N}x{K}")
