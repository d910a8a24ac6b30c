"""Seeded synthetic inputs for the linear-attention layer.

This module only draws random numbers; it holds none of the layer's arithmetic.
Both the HIP path's tests/benchmark and the oracle's checks take their inputs
from here, so the two sides see identical data.

Recipe (the pages measure whole-model latency on long prompts and quality on
public suites; i.i.d. Gaussian tensors at the layer's real shapes stand in for
them, since the layer has no data-dependent control flow):
  * q, k, v, gate logits ~ N(0, 1), drawn in that order from one
    ``torch.Generator`` seeded with the workload's seed, in float32, then rounded
    to nearest-even bfloat16 (or kept float32 where the workload says so);
  * the decode state S ~ N(0, 0.02^2) in float32, drawn after the activations;
  * layout [B, T, H, D] for activations, [B, H, D, D] for states.
"""
from __future__ import annotations

import dataclasses

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    D: int
    seed: int
    dtype: torch.dtype = torch.bfloat16
    chunk: int = 0
    pos0: int = 0
    segments: int = 1
    steps: int = 1
    state_std: float = 0.0


# The five workloads of the layer (tiny CPU check, 32K prefill, 256K prefill,
# 1M streamed prefill, batched decode).  Seeds 0..4.
TINY = Workload("tiny_b1_h2_d16_t256_fp32", 1, 256, 2, 16, seed=0, dtype=torch.float32, chunk=32)
PREFILL_32K = Workload("prefill_b1_h32_d128_t32768", 1, 32768, 32, 128, seed=1)
PREFILL_256K = Workload("prefill_b1_h32_d128_t262144", 1, 262144, 32, 128, seed=2)
STREAM_1M = Workload("stream_b1_h32_d128_t1048576_seg65536", 1, 1048576, 32, 128, seed=3,
                     segments=16)
DECODE_B64 = Workload("decode_b64_h32_d128_pos262144", 64, 1, 32, 128, seed=4, pos0=262144,
                      steps=1000, state_std=0.02)

ALL = (TINY, PREFILL_32K, PREFILL_256K, STREAM_1M, DECODE_B64)

# Beside those: a batch of 8 prompts of 32K tokens (as many tokens as the 256K
# prefill, spread over 256 sequence-heads), and the batched decode at 256
# sequences, whose 512 MiB of states exceed the GPU's 256 MB memory-side cache.
PREFILL_B8_32K = Workload("prefill_b8_h32_d128_t32768", 8, 32768, 32, 128, seed=10)
DECODE_B256 = Workload("decode_b256_h32_d128_pos262144", 256, 1, 32, 128, seed=11, pos0=262144,
                       steps=200, state_std=0.02)
# 384 sequences: 768 MiB of states, three times that cache.
DECODE_B384 = Workload("decode_b384_h32_d128_pos262144", 384, 1, 32, 128, seed=12, pos0=262144,
                       steps=100, state_std=0.02)


@dataclasses.dataclass(frozen=True)
class MixedBatch:
    """A packed variable-length batch: prefill sequences and single-token decode
    steps side by side, as a serving step schedules them."""
    name: str
    lengths: tuple
    pos0: tuple
    H: int
    D: int
    seed: int
    state_std: float


# Serving mix: four 16K-token prompts being prefilled from position 0 while 60
# sequences decode one token each at position 262144 (their states ~ N(0, 0.02^2)).
SERVING_MIX = MixedBatch("mixed_4x16384_prefill_60x1_decode_h32_d128", (16384,) * 4 + (1,) * 60,
                         (0,) * 4 + (262144,) * 60, 32, 128, seed=5, state_std=0.02)


def mixed_inputs(w: MixedBatch, device="cpu"):
    """(q, k, v, g [total_T, H, D] bf16, S_in [nseq, H, D, D] fp32, cu_seqlens list)."""
    gen = generator(w.seed, device)
    total = sum(w.lengths)
    q, k, v, g = (x[0] for x in activations(1, total, w.H, w.D, w.seed, device, gen=gen))
    S = state(len(w.lengths), w.H, w.D, w.state_std, gen, device)
    cu = [0]
    for n in w.lengths:
        cu.append(cu[-1] + n)
    return q, k, v, g, S, cu


def generator(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def activations(B: int, T: int, H: int, D: int, seed: int, device="cpu",
                dtype=torch.bfloat16, gen: torch.Generator | None = None):
    """q, k, v, gate logits: [B, T, H, D], N(0, 1) drawn in fp32 then cast to ``dtype``."""
    gen = gen if gen is not None else generator(seed, device)
    out = []
    for _ in range(4):
        x = torch.randn((B, T, H, D), generator=gen, device=device, dtype=torch.float32)
        out.append(x.to(dtype))
        del x
    return tuple(out)


def state(B: int, H: int, D: int, std: float, gen: torch.Generator, device="cpu"):
    """fp32 state [B, H, D, D] ~ N(0, std^2)."""
    return torch.randn((B, H, D, D), generator=gen, device=device, dtype=torch.float32) * std


def decode_inputs(w: Workload, steps: int | None = None, device="cpu"):
    """(S0, q, k, v, g) for the batched-decode workload.

    S0 [B, H, D, D] fp32 is drawn first, then q, k, v, g as [steps, B, H, D]
    tensors (one token per sequence per step), each drawn whole, in that order."""
    steps = w.steps if steps is None else steps
    gen = generator(w.seed, device)
    S0 = state(w.B, w.H, w.D, w.state_std, gen, device)
    toks = activations(steps, w.B, w.H, w.D, w.seed, device, w.dtype, gen=gen)
    return (S0,) + tuple(toks)


@dataclasses.dataclass(frozen=True)
class LayerWorkload:
    """Inputs of one layer forward: x [B, T, hidden] ~ N(0, 1) and the fused
    q/k/v/gate and output projection weights ~ N(0, 1 / fan_in), all bf16."""
    name: str
    B: int
    T: int
    hidden: int
    H: int
    D: int
    seed: int


# One layer of the model's shape (hidden 4096, 32 heads x 128) on a 32K-token prompt.
LAYER_32K = LayerWorkload("layer_b1_t32768_hidden4096_h32_d128", 1, 32768, 4096, 32, 128, seed=6)


def layer_inputs(B: int, T: int, hidden: int, H: int, D: int, seed: int, device="cpu"):
    """(x, w_qkvg [4 H D, hidden], w_o [hidden, H D]), drawn in that order."""
    gen = generator(seed, device)
    x = torch.randn((B, T, hidden), generator=gen, device=device).to(torch.bfloat16)
    w_qkvg = (torch.randn((4 * H * D, hidden), generator=gen, device=device) / hidden ** 0.5).to(torch.bfloat16)
    w_o = (torch.randn((hidden, H * D), generator=gen, device=device) / (H * D) ** 0.5).to(torch.bfloat16)
    return x, w_qkvg, w_o


@dataclasses.dataclass(frozen=True)
class SparseWorkload:
    """Sparse-layer inputs: q, k, v, gate logits ~ N(0, 1) bf16 drawn as by
    ``activations`` (prefill: [B, T, H, D]); decode draws the caches [B, T, H, D]
    and then q, gate [B, H, D], every sequence full (T valid tokens)."""
    name: str
    B: int
    T: int
    H: int
    D: int
    topk: int
    seed: int


# A 32K-token prompt through one sparse layer (32 heads x 128, 16 chosen blocks of 64).
SPARSE_32K = SparseWorkload("sparse_prefill_b1_t32768_h32_d128_top16", 1, 32768, 32, 128, 16, seed=8)
# Batched decode against 128K-token caches (8 sequences, 32 heads).
SPARSE_DECODE = SparseWorkload("sparse_decode_b8_ctx131072_h32_d128_top16", 8, 131072, 32, 128, 16, seed=9)


def sparse_decode_inputs(w: SparseWorkload, device="cpu"):
    """(q, k_cache, v_cache, gate) of one decode step; the caches hold T tokens."""
    gen = generator(w.seed, device)
    kc, vc = (torch.randn((w.B, w.T, w.H, w.D), generator=gen, device=device).to(torch.bfloat16)
              for _ in range(2))
    q, g = (torch.randn((w.B, w.H, w.D), generator=gen, device=device).to(torch.bfloat16) for _ in range(2))
    return q, kc, vc, g
