"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Each test fixes one part of what the oracle computes against mathematics that the
pages (or their plainest reading) determine: closed forms of RMSNorm and RoPE, the
brute-force masked quadratic form of causal linear attention without softmax, the
chunk-size invariance of the chunked form, gate special cases, a hand-worked
example, and the invariants of the recurrence (segmenting, decode = prefill,
relative-position property of RoPE).  CPU only.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_inputs(rng, B, T, H, D, scale=1.0):
    q, k, v, g = (rng.standard_normal((B, T, H, D)).astype(np.float32) * scale for _ in range(4))
    return q, k, v, g


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _quadratic(qh, kh, v, g, S_in):
    """Brute-force causal linear attention without softmax:
    U = ((Qh Kh^T) * M) V + Qh S_in with M[t, s] = [s <= t]; o = sigmoid(g) * U.
    Per (b, h); written with an explicit mask matrix and numpy matmuls."""
    B, T, H, D = qh.shape
    o = np.empty((B, T, H, D))
    S_out = np.empty((B, H, D, D))
    M = np.tril(np.ones((T, T)))
    for b in range(B):
        for h in range(H):
            Q, K, V = qh[b, :, h], kh[b, :, h], v[b, :, h].astype(np.float64)
            U = ((Q @ K.T) * M) @ V + Q @ S_in[b, h]
            o[b, :, h] = _sigmoid(g[b, :, h].astype(np.float64)) * U
            S_out[b, h] = S_in[b, h] + K.T @ V
    return o, S_out


# ---------------------------------------------------------------- RMSNorm


def test_rmsnorm_closed_forms():
    # (3, 4): mean square 12.5 -> (3, 4) / sqrt(12.5) with eps = 0
    out = oracle.rmsnorm_row([3.0, 4.0], eps=0.0)
    np.testing.assert_allclose(out, np.array([3.0, 4.0]) / math.sqrt(12.5), rtol=1e-15)
    # a constant vector c * 1 maps to c / sqrt(c^2 + eps) * 1
    c, eps = -2.5, 1e-3
    out = oracle.rmsnorm_row(np.full(16, c), eps=eps)
    np.testing.assert_allclose(out, np.full(16, c / math.sqrt(c * c + eps)), rtol=1e-14)
    # weights multiply elementwise
    w = np.arange(1, 9, dtype=np.float32) / 4
    x = np.linspace(-1, 2, 8)
    np.testing.assert_allclose(oracle.rmsnorm_row(x, eps=0.0, w=w),
                               w * x / math.sqrt(np.mean(x * x)), rtol=1e-14)


def test_rmsnorm_invariants():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(128)
    eps = 1e-6
    n = oracle.rmsnorm_row(x, eps=eps)
    ms = np.mean(x * x)
    # RMS of the output is sqrt(ms / (ms + eps))
    assert abs(math.sqrt(np.mean(n * n)) - math.sqrt(ms / (ms + eps))) < 1e-14
    # scale invariance for eps = 0
    np.testing.assert_allclose(oracle.rmsnorm_row(7.25 * x, eps=0.0), oracle.rmsnorm_row(x, eps=0.0),
                               rtol=1e-13)


# ---------------------------------------------------------------- RoPE


def test_rope_d2_is_complex_rotation():
    # D = 2: theta_0 = 1, so RoPE is multiplication of x0 + i x1 by e^{i p}
    for p in (0, 1, 5, 262144, 1048575):
        x = np.array([0.3, -1.7])
        z = complex(x[0], x[1]) * np.exp(1j * p)
        np.testing.assert_allclose(oracle.rope_row(x, p), [z.real, z.imag], rtol=0, atol=1e-12)


def test_rope_d4_basis_vectors_fix_frequencies_and_pairing():
    # D = 4, base 10000: theta_0 = 1, theta_1 = 10000^(-2/4) = 1/100; pairs are (0, 2) and (1, 3)
    p = 37
    e0 = oracle.rope_row([1.0, 0, 0, 0], p, base=10000.0)
    np.testing.assert_allclose(e0, [math.cos(p), 0, math.sin(p), 0], atol=1e-15)
    e1 = oracle.rope_row([0, 1.0, 0, 0], p, base=10000.0)
    np.testing.assert_allclose(e1, [0, math.cos(p / 100), 0, math.sin(p / 100)], atol=1e-15)
    e2 = oracle.rope_row([0, 0, 1.0, 0], p, base=10000.0)
    np.testing.assert_allclose(e2, [-math.sin(p), 0, math.cos(p), 0], atol=1e-15)
    # D = 8: theta_3 = base^(-6/8)
    e3 = oracle.rope_row([0, 0, 0, 1.0, 0, 0, 0, 0], p, base=500.0)
    a = p * 500.0 ** (-6 / 8)
    np.testing.assert_allclose(e3, [0, 0, 0, math.cos(a), 0, 0, 0, math.sin(a)], atol=1e-13)


def test_rope_identity_norm_and_relative_property():
    rng = np.random.default_rng(2)
    x, y = rng.standard_normal(128), rng.standard_normal(128)
    np.testing.assert_array_equal(oracle.rope_row(x, 0), x)
    r = oracle.rope_row(x, 123457)
    assert abs(np.linalg.norm(r) - np.linalg.norm(x)) < 1e-12
    # (R_m x) . (R_n y) depends only on n - m
    for m, n in ((0, 5), (1000, 1005), (262144, 262149)):
        assert abs(oracle.rope_row(x, m) @ oracle.rope_row(y, n)
                   - x @ oracle.rope_row(y, n - m)) < 1e-9


# ---------------------------------------------------------------- recurrence


@pytest.mark.parametrize("B,T,H,D,pos0,nonzero_S", [
    (1, 256, 2, 16, 0, False),     # tiny oracle-check workload: batch 1, 2 heads, dim 16, 256 tokens
    (2, 37, 3, 8, 1000, True),
    (1, 64, 1, 128, 262144, True),
])
def test_recurrence_equals_bruteforce_quadratic(B, T, H, D, pos0, nonzero_S):
    rng = np.random.default_rng(0)
    q, k, v, g = _rand_inputs(rng, B, T, H, D)
    S_in = rng.standard_normal((B, H, D, D)) * 0.1 if nonzero_S else np.zeros((B, H, D, D))
    o, S_out = oracle.forward(q, k, v, g, S=S_in, pos0=pos0)
    qh = oracle.prologue(q, pos0=pos0)
    kh = oracle.prologue(k, pos0=pos0)
    o_ref, S_ref = _quadratic(qh, kh, v, g, S_in)
    assert np.max(np.abs(o - o_ref)) <= 1e-10 * max(1.0, np.max(np.abs(o_ref)))
    assert np.max(np.abs(S_out - S_ref)) <= 1e-10 * max(1.0, np.max(np.abs(S_ref)))


def test_chunked_equals_recurrence_for_every_chunk_size():
    # tiny workload: B = 1, H = 2, D = 16, T = 256, fp32 inputs, every C in 1..256
    rng = np.random.default_rng(0)
    q, k, v, g = _rand_inputs(rng, 1, 256, 2, 16)
    o_rec, S_rec = oracle.forward(q, k, v, g)
    scale_o, scale_S = np.max(np.abs(o_rec)), np.max(np.abs(S_rec))
    for C in range(1, 257):
        o_c, S_c = oracle.chunked(q, k, v, g, C)
        assert np.max(np.abs(o_c - o_rec)) <= 1e-11 * scale_o, C
        assert np.max(np.abs(S_c - S_rec)) <= 1e-11 * scale_S, C


def test_hand_worked_example():
    with open(os.path.join(GOLDEN, "hand_d2_t2.json")) as f:
        fx = json.load(f)
    env = {"sin": math.sin, "cos": math.cos, "sqrt": math.sqrt, "log": math.log}

    def ev(a):
        return np.array([[eval(str(e), {"__builtins__": {}}, env) for e in row] for row in a])

    inp = {n: ev(fx["inputs"][n]).reshape(1, 2, 1, 2) for n in "qkvg"}
    o, S = oracle.forward(inp["q"], inp["k"], inp["v"], inp["g"], pos0=0, eps=0.0)
    np.testing.assert_allclose(o[0, :, 0], ev(fx["expected"]["o"]), rtol=1e-7, atol=1e-12)
    np.testing.assert_allclose(S[0, 0], ev(fx["expected"]["S_out"]), rtol=1e-12)


def test_state_closed_form_and_independence_from_q_and_gate():
    rng = np.random.default_rng(3)
    q, k, v, g = _rand_inputs(rng, 2, 40, 2, 16)
    S_in = rng.standard_normal((2, 2, 16, 16))
    _, S1 = oracle.forward(q, k, v, g, S=S_in, pos0=7)
    q2, g2 = _rand_inputs(rng, 2, 40, 2, 16)[:2]
    _, S2 = oracle.forward(q2, k, v, g2, S=S_in, pos0=7)
    np.testing.assert_array_equal(S1, S2)
    kh = oracle.prologue(k, pos0=7)
    S_ref = S_in + np.einsum("bthi,bthj->bhij", kh, v.astype(np.float64))
    np.testing.assert_allclose(S1, S_ref, rtol=1e-12, atol=1e-12)


def test_gate_special_cases():
    rng = np.random.default_rng(4)
    q, k, v, _ = _rand_inputs(rng, 1, 20, 2, 8)
    o_half, _ = oracle.forward(q, k, v, np.zeros_like(q))
    o_open, _ = oracle.forward(q, k, v, np.full_like(q, 60.0))    # sigmoid(60) == 1 in double
    np.testing.assert_allclose(o_half, 0.5 * o_open, rtol=1e-15)
    o_shut, _ = oracle.forward(q, k, v, np.full_like(q, -800.0))  # sigmoid(-800) == 0
    assert np.all(o_shut == 0.0)


def test_output_is_linear_in_v():
    rng = np.random.default_rng(5)
    q, k, v1, g = _rand_inputs(rng, 1, 30, 2, 8)
    v2 = rng.standard_normal(v1.shape).astype(np.float32)
    o1, _ = oracle.forward(q, k, v1, g)
    o2, _ = oracle.forward(q, k, v2, g)
    o12, _ = oracle.forward(q, k, v1 + v2, g)   # v1 + v2 exact enough in fp32 for this check
    np.testing.assert_allclose(o12, o1 + o2, rtol=1e-6, atol=1e-6)


def test_segmented_equals_single_shot():
    rng = np.random.default_rng(6)
    q, k, v, g = _rand_inputs(rng, 1, 96, 2, 16)
    o_full, S_full = oracle.forward(q, k, v, g, pos0=500)
    S = None
    outs = []
    for s0 in (0, 32, 64):
        o_s, S = oracle.forward(q[:, s0:s0 + 32], k[:, s0:s0 + 32], v[:, s0:s0 + 32],
                                g[:, s0:s0 + 32], S=S, pos0=500 + s0)
        outs.append(o_s)
    np.testing.assert_allclose(np.concatenate(outs, axis=1), o_full, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, S_full, rtol=1e-12, atol=1e-12)


def test_decode_steps_equal_prefill():
    rng = np.random.default_rng(7)
    B, N, H, D = 3, 5, 2, 16
    q, k, v, g = _rand_inputs(rng, B, N, H, D)
    S0 = rng.standard_normal((B, H, D, D)) * 0.02
    o_pre, S_pre = oracle.forward(q, k, v, g, S=S0, pos0=262144)
    S = S0
    for n in range(N):
        o_n, S = oracle.decode_step(q[:, n], k[:, n], v[:, n], g[:, n], S, pos=262144 + n)
        np.testing.assert_allclose(o_n, o_pre[:, n], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S, S_pre, rtol=1e-12, atol=1e-13)


def test_output_invariant_to_position_shift_when_state_starts_empty():
    # RoPE's relative property: with S_in = 0, o depends only on position differences
    rng = np.random.default_rng(8)
    q, k, v, g = _rand_inputs(rng, 1, 48, 2, 32)
    o0, S0 = oracle.forward(q, k, v, g, pos0=0)
    o1, S1 = oracle.forward(q, k, v, g, pos0=1000003)
    np.testing.assert_allclose(o1, o0, rtol=1e-7, atol=1e-9)
    assert np.max(np.abs(S1 - S0)) > 1e-2   # the state itself is position dependent


def test_threads_do_not_change_results():
    rng = np.random.default_rng(9)
    q, k, v, g = _rand_inputs(rng, 1, 50, 4, 32)
    n = oracle.get_threads()
    oracle.set_threads(1)
    try:
        o1, S1 = oracle.forward(q, k, v, g)
    finally:
        oracle.set_threads(0)
    o2, S2 = oracle.forward(q, k, v, g)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(S1, S2)
    assert n >= 1


# ---------------------------------------------------------------------------
# Projections around the layer (oracle.linear, oracle.round_bf16, oracle.layer_forward)

def test_linear_hand_example():
    """y = x w^T with w in the nn.Linear [out, in] layout, worked by hand."""
    x = np.array([[1.0, 2.0], [3.0, 4.0]])
    w = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    assert np.array_equal(oracle.linear(x, w), np.array([[1.0, 2.0, 3.0], [3.0, 4.0, 7.0]]))


def test_round_bf16_ties_to_even():
    """bfloat16 keeps 8 significant bits: at 1.0 the spacing is 2^-7."""
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -9, -(1 + 2 ** -8), 2 ** -8 * 3], np.float32)
    want = np.array([1.0, 1 + 2 ** -6, 1.0, -1.0, 2 ** -8 * 3], np.float32)
    assert np.array_equal(oracle.round_bf16(x), want)


def test_layer_with_identity_projections_is_the_layer():
    """w_qkvg = [I; I; I; 0] (q = k = v = x, gate logits 0) and w_o = I reduce the
    layer to half of the bare recurrence (sigmoid(0) = 1/2), rounded to bf16."""
    rng = np.random.default_rng(7)
    T, HD = 40, 128
    x = oracle.round_bf16(rng.standard_normal((1, T, HD)))
    eye = np.eye(HD)
    w_qkvg = np.concatenate([eye, eye, eye, np.zeros((HD, HD))])
    y, S = oracle.layer_forward(x, w_qkvg, eye, pos0=11)
    xs = x.reshape(1, T, 1, HD)
    o, S_ref = oracle.forward(xs, xs, xs, np.zeros_like(xs), pos0=11)
    np.testing.assert_allclose(y, oracle.round_bf16(o.reshape(1, T, HD)), rtol=0, atol=0)
    np.testing.assert_allclose(S, S_ref, rtol=0, atol=0)


# ---------------------------------------------------------------------------
# Gradients (oracle.backward) against central finite differences of the forward

def _loss(q, k, v, g, S, do, dSo, pos0, qw, kw):
    o, S_out = oracle.forward(q, k, v, g, S=S, pos0=pos0, q_w=qw, k_w=kw)
    return float(np.sum(o * do) + np.sum(S_out * dSo))


@pytest.mark.parametrize("weights", [False, True])
def test_backward_matches_finite_differences(weights):
    """Every gradient element of a tiny layer (B 1, T 5, H 2, D 8) against central
    differences of L = <o, do> + <S_out, dS_out>.  The perturbed inputs are float32,
    so the step actually taken is used as the denominator."""
    rng = np.random.default_rng(11)
    B, T, H, D, pos0 = 1, 5, 2, 8, 3
    q, k, v, g = (rng.standard_normal((B, T, H, D)).astype(np.float32) for _ in range(4))
    S = rng.standard_normal((B, H, D, D)) * 0.3
    do = rng.standard_normal((B, T, H, D)).astype(np.float32)  # the oracle takes do as float32
    dSo = rng.standard_normal((B, H, D, D))
    qw = (rng.random(D) + 0.5).astype(np.float32) if weights else None
    kw = (rng.random(D) + 0.5).astype(np.float32) if weights else None
    grads = oracle.backward(q, k, v, g, do, S=S, dS_out=dSo, pos0=pos0, q_w=qw, k_w=kw)
    inputs = {"dq": q, "dk": k, "dv": v, "dg": g}
    if weights:
        inputs["dq_w"] = qw
        inputs["dk_w"] = kw
    h = 1e-3
    for name, arr in inputs.items():
        fd = np.zeros(arr.shape)
        for idx in np.ndindex(arr.shape):
            x0 = arr[idx]
            arr[idx] = np.float32(x0 + h)
            xp = float(arr[idx])
            lp = _loss(q, k, v, g, S, do, dSo, pos0, qw, kw)
            arr[idx] = np.float32(x0 - h)
            xm = float(arr[idx])
            lm = _loss(q, k, v, g, S, do, dSo, pos0, qw, kw)
            arr[idx] = x0
            fd[idx] = (lp - lm) / (xp - xm)
        np.testing.assert_allclose(grads[name], fd, rtol=1e-4, atol=1e-5 * np.abs(fd).max(), err_msg=name)
    # dS_in: S is float64, so a plain central difference
    fd = np.zeros(S.shape)
    for idx in np.ndindex(S.shape):
        s0 = S[idx]
        S[idx] = s0 + h
        lp = _loss(q, k, v, g, S, do, dSo, pos0, qw, kw)
        S[idx] = s0 - h
        lm = _loss(q, k, v, g, S, do, dSo, pos0, qw, kw)
        S[idx] = s0
        fd[idx] = (lp - lm) / (2 * h)
    np.testing.assert_allclose(grads["dS_in"], fd, rtol=1e-6, atol=1e-9, err_msg="dS_in")


def test_backward_is_linear_in_the_output_gradients():
    rng = np.random.default_rng(12)
    B, T, H, D = 1, 7, 1, 8
    q, k, v, g = (rng.standard_normal((B, T, H, D)).astype(np.float32) for _ in range(4))
    # dyadic values, so 2 a - b is exact in the float32 the oracle takes do in
    do1, do2 = np.round(rng.standard_normal((2, B, T, H, D)) * 16) / 16
    dS1, dS2 = np.round(rng.standard_normal((2, B, H, D, D)) * 16) / 16
    a = oracle.backward(q, k, v, g, do1, dS_out=dS1)
    b = oracle.backward(q, k, v, g, do2, dS_out=dS2)
    c = oracle.backward(q, k, v, g, 2 * do1 - do2, dS_out=2 * dS1 - dS2)
    for n in ("dq", "dk", "dv", "dg", "dS_in"):
        np.testing.assert_allclose(c[n], 2 * a[n] - b[n], rtol=1e-10, atol=1e-12, err_msg=n)
