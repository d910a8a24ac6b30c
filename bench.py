#!/usr/bin/env python3
"""Benchmark of the MI355X linear-attention layer (one GPU).

One timed step = one la_prefill over the 256K-token workload (B = 1, 32 heads x
128, bf16 q/k/v/gate, fp32 state, S0 = 0): QK-RMSNorm + RoPE prologue,
intra-chunk masked scores and P V, inter-chunk Qh S_pre, the state scan and the
sigmoid gate epilogue.  After the K timed prefill steps, the batched decode
workload (64 sequences x 32 heads, 1000 consecutive steps from position 262144)
is timed too and reported under "decode".  Inputs are generated on the GPU
before any timed region; nothing is skipped inside it.

Prints one JSON line (rank 0, N = 1):
  value     prefill tokens/s (B * T * K / wall time of the K steps)
  roofline  the dominant kernel (the chunk-output kernel) against HBM bandwidth,
            from HIP events recorded on the library's stream around each kernel
  cpu_baseline  the fp64 oracle timed on this host on a bounded sample
  prefill_detail.chunk_sweep  the same prefill at chunk 64, 128 and 256
  varlen    a packed serving batch (4 x 16K-token prompts + 60 decode steps) in
            one la_prefill_varlen call, beside the same work as two calls
  layer     one layer on a 32K-token prompt (hidden 4096): q/k/v/gate projection,
            the layer, output projection; the projections against bf16 MFMA peak
  backward  la_backward over the 256K-token input
"""
from __future__ import annotations

import argparse
import ctypes
import glob
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 (256 CU x 2.4 GHz x 4096 flop/clk)
TOKEN_HEAD_BYTES = 1280         # read q, k, v, gate (4 x 256 B) + write o (256 B)
STATE_BYTES = 128 * 128 * 4     # one fp32 D x D state
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_prefill_output_kernel.json")
KERNEL_SOURCES = [os.path.join(ROOT, "hybrid_sparse_linear_la_amd", "csrc", f)
                  for f in ("la_prefill.hip", "la_tiles.hpp", "la_device.hpp", "la_internal.hpp")]


class HipEvents:
    """hipEvent_t helpers through the HIP runtime torch already loaded."""

    def __init__(self):
        path = None
        for line in open("/proc/self/maps"):
            if "libamdhip64" in line:
                path = line.split()[-1]
                break
        self.hip = ctypes.CDLL(path or "libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            ev = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(ev)) == 0
            out.append(ev.value)
        return out

    def record(self, ev, stream):
        assert self.hip.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream)) == 0

    def ms(self, a, b):
        assert self.hip.hipEventSynchronize(ctypes.c_void_p(b)) == 0
        out = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return float(out.value)

    def destroy(self, evs):
        for ev in evs:
            self.hip.hipEventDestroy(ctypes.c_void_p(ev))


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(launch_tokens: int):
    """HBM bytes per output-kernel launch from committed rocprofv3 counters, if they
    were taken on the current kernel source; else None."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha") != kernel_source_hash() or rec.get("tokens") != launch_tokens:
        return None
    return rec.get("hbm_bytes_per_launch")


def bench_prefill(la, torch, workloads, hip, args):
    w = workloads.PREFILL_256K
    B, T, H, D = w.B, w.T, w.H, w.D
    q, k, v, g = workloads.activations(B, T, H, D, w.seed, "cuda")
    o = torch.empty_like(q)
    S_out = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(la.prefill_workspace_bytes(B, T, H, D, args.chunk), dtype=torch.uint8, device="cuda")
    plan_nseg = ws.numel() // (B * H * STATE_BYTES)
    chunk = args.chunk or la.DEFAULT_CHUNK

    for _ in range(args.warmup):
        la.prefill(q, k, v, g, chunk=args.chunk, out=o, S_out=S_out, workspace=ws)
    evs = [hip.create(4) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        la.prefill(q, k, v, g, chunk=args.chunk, out=o, S_out=S_out, workspace=ws, events=evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    names = ("chunk_state", "state_scan", "chunk_output")
    per = {n: sum(hip.ms(e[i], e[i + 1]) for e in evs) / args.steps for i, n in enumerate(names)}
    step_ms = [hip.ms(e[0], e[3]) for e in evs]
    gpu_ms = sum(step_ms) / args.steps
    for e in evs:
        hip.destroy(e)

    tokens = B * T
    step_s = wall / args.steps
    comp_bytes = TOKEN_HEAD_BYTES * B * T * H
    # the state pass sums every segment but a sequence's last (whose output workgroup
    # writes S_out from its carried state); segments are whole 64-token chunks
    seg_tokens = -(-(-(-T // 64)) // plan_nseg) * 64
    state_tokens = min(T, (plan_nseg - 1) * seg_tokens)
    out_bytes = comp_bytes + STATE_BYTES * B * H * (plan_nseg + 1)  # output kernel: + prefix states, S_out
    state_bytes = 512 * B * state_tokens * H + STATE_BYTES * B * H * (plan_nseg - 1)  # k, v -> segment sums
    scan_bytes = 2 * STATE_BYTES * B * H * plan_nseg  # S_in and the sums in, the prefixes out
    flops = (4 * D * D + 2 * D * (chunk + 1)) * B * T * H
    out_s = per["chunk_output"] / 1e3
    traffic = measured_traffic(tokens) if chunk == la.DEFAULT_CHUNK else None
    roofline = {
        "bound": "hbm",
        "kernel": "la_chunk_output_kernel" if chunk == la.DEFAULT_CHUNK else "la_chunk_output_wide_kernel",
        "achieved": round(out_bytes / out_s / 1e9, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(out_bytes / out_s / 1e9 / HBM_PEAK_GBS, 4),
        "traffic": traffic,
        "algorithmic_bytes_per_launch": out_bytes,
        "avg_launch_ms": round(per["chunk_output"], 4),
    }
    t_roof = comp_bytes / (HBM_PEAK_GBS * 1e9)
    detail = {
        "kernels_ms": {n: round(x, 4) for n, x in per.items()},
        "kernels_GBps": {"chunk_state": round(state_bytes / (per["chunk_state"] / 1e3) / 1e9, 1),
                         "state_scan": round(scan_bytes / (per["state_scan"] / 1e3) / 1e9, 1),
                         "chunk_output": roofline["achieved"]},
        "gpu_ms_per_step_events": round(gpu_ms, 4),
        "gpu_ms_per_step_median": round(statistics.median(step_ms), 4),
        "path_roofline": {"t_roof_ms": round(t_roof * 1e3, 4), "frac": round(t_roof / step_s, 4),
                          "compulsory_bytes": comp_bytes,
                          "achieved_GBps": round(comp_bytes / step_s / 1e9, 1)},
        "mfma": {"algorithmic_tflop": round(flops / 1e12, 4),
                 "achieved_tflops": round(flops / step_s / 1e12, 2),
                 "frac_of_bf16_peak": round(flops / step_s / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                 "ceiling_frac_at_hbm_roof": round(flops / t_roof / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)},
        "segments_per_head": plan_nseg,
        "chunk": chunk,
    }
    if not args.no_chunk_sweep:
        detail["chunk_sweep"] = chunk_sweep(la, torch, hip, (q, k, v, g), o, S_out)
    return w, tokens * args.steps / wall, step_s, roofline, detail, (q, k, v, g)


def chunk_sweep(la, torch, hip, tensors, o, S_out, steps=3):
    """GPU time of the same 256K prefill at every supported chunk size (events
    around each kernel, one warm-up call, `steps` timed calls)."""
    q, k, v, g = tensors
    B, T, H, D = q.shape
    res = {}
    for c in (64, 128, 256):
        ws = torch.empty(la.prefill_workspace_bytes(B, T, H, D, c), dtype=torch.uint8, device="cuda")
        la.prefill(q, k, v, g, chunk=c, out=o, S_out=S_out, workspace=ws)
        evs = [hip.create(4) for _ in range(steps)]
        for e in evs:
            la.prefill(q, k, v, g, chunk=c, out=o, S_out=S_out, workspace=ws, events=e)
        torch.cuda.synchronize()
        ms = sum(hip.ms(e[0], e[3]) for e in evs) / steps
        out_ms = sum(hip.ms(e[2], e[3]) for e in evs) / steps
        for e in evs:
            hip.destroy(e)
        del ws
        res[str(c)] = {"gpu_ms": round(ms, 4), "output_kernel_ms": round(out_ms, 4),
                       "tokens_per_s": round(B * T / (ms / 1e3), 1),
                       "kernel": "la_chunk_output_kernel" if c == 64 else "la_chunk_output_wide_kernel"}
    return res


def bench_decode(la, torch, workloads, hip, args):
    w = workloads.DECODE_B64
    steps = args.decode_steps
    S0, q, k, v, g = workloads.decode_inputs(w, steps=steps, device="cuda")
    out = torch.empty_like(q)
    S = S0.clone()
    for n in range(min(3, steps)):  # warm-up on a scratch copy of the state
        la.decode_step(q[n], k[n], v[n], g[n], S, w.pos0 + n, out=out[n])
    S.copy_(S0)
    stream = torch.cuda.current_stream().cuda_stream
    ev = hip.create(2)
    torch.cuda.synchronize()
    hip.record(ev[0], stream)
    for n in range(steps):
        la.decode_step(q[n], k[n], v[n], g[n], S, w.pos0 + n, out=out[n])
    hip.record(ev[1], stream)
    ms = hip.ms(ev[0], ev[1])
    hip.destroy(ev)
    us = ms * 1e3 / steps
    bytes_step = 2 * w.B * w.H * STATE_BYTES + 5 * w.B * w.H * w.D * 2
    # the same steps captured in one HIP graph
    graph_us = None
    if not args.no_graph:
        S.copy_(S0)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for n in range(steps):
                la.decode_step(q[n], k[n], v[n], g[n], S, w.pos0 + n, out=out[n])
        S.copy_(S0)
        torch.cuda.synchronize()
        ev = hip.create(2)
        stream = torch.cuda.current_stream().cuda_stream
        hip.record(ev[0], stream)
        graph.replay()
        hip.record(ev[1], stream)
        graph_us = hip.ms(ev[0], ev[1]) * 1e3 / steps
        hip.destroy(ev)
        del graph
    best = min(us, graph_us) if graph_us else us
    return {
        "workload": w.name, "steps": steps, "us_per_step": round(us, 3),
        "us_per_step_hipgraph": None if graph_us is None else round(graph_us, 3),
        "GB_per_s": round(bytes_step / (best * 1e-6) / 1e9, 1),
        "roofline": {"bound": "hbm", "kernel": "la_decode_kernel",
                     "achieved": round(bytes_step / (best * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(bytes_step / (best * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes_per_launch": bytes_step,
                     "note": ("the 128 MiB of states can stay in the 256 MB memory-side cache between steps, so this "
                              "rate may be cache-assisted at any value; the b384 entry (768 MiB) is DRAM-bound")},
    }


def cpu_baseline(tensors, args):
    """The oracle, untuned, on the first `cpu_tokens` tokens of the same input (all heads)."""
    import oracle
    q, k, v, g = tensors
    n = args.cpu_tokens
    host = [t[:, :n].float().cpu().numpy() for t in (q, k, v, g)]
    t0 = time.perf_counter()
    oracle.forward(*host)
    dt = time.perf_counter() - t0
    return {"value": round(n / dt, 1), "unit": "tokens/s", "cores": oracle.get_threads(), "kind": "oracle",
            "sample": f"first {n} tokens x {q.shape[2]} heads of the 256K-token prefill input "
                      f"(fp64 token-by-token recurrence, {dt:.1f} s)"}


def cpu_decode_baseline(workloads, steps=5):
    """The oracle's decode step on the batched-decode workload (64 sequences x 32
    heads), a few consecutive steps timed on the host."""
    import oracle
    w = workloads.DECODE_B64
    S0, q, k, v, g = (t.double().numpy() for t in workloads.decode_inputs(w, steps=steps, device="cpu"))
    S = S0
    t0 = time.perf_counter()
    for n in range(steps):
        _, S = oracle.decode_step(q[n], k[n], v[n], g[n], S, w.pos0 + n)
    dt = time.perf_counter() - t0
    return {"value": round(dt / steps * 1e6, 1), "unit": "us/step", "cores": oracle.get_threads(),
            "kind": "oracle", "sample": f"{steps} consecutive steps of the {w.B} x {w.H}-head batch ({dt:.1f} s)"}


def bench_varlen(la, torch, workloads, hip, args, steps=5):
    """The serving mix as one la_prefill_varlen call, and the same work as one
    equal-length la_prefill over the prompts plus one la_decode_step."""
    w = workloads.SERVING_MIX
    q, k, v, g, S_in, cu = workloads.mixed_inputs(w, "cuda")
    n_pre = sum(1 for n in w.lengths if n > 1)
    T_pre = w.lengths[0]
    o = torch.empty_like(q)
    S_out = torch.empty_like(S_in)
    ws = torch.empty(la.prefill_varlen_workspace_bytes(cu, w.H), dtype=torch.uint8, device="cuda")

    def one_call():
        la.prefill_varlen(q, k, v, g, cu, pos0=list(w.pos0), S_in=S_in, out=o, S_out=S_out, workspace=ws)

    # the same work as two calls: prompts [n_pre, T_pre] and decode rows [n_dec]
    pre = [x[:n_pre * T_pre].view(n_pre, T_pre, w.H, w.D) for x in (q, k, v, g)]
    dec = [x[n_pre * T_pre:] for x in (q, k, v, g)]
    S_pre_in, S_dec = S_in[:n_pre].contiguous(), S_in[n_pre:].clone()
    ws2 = torch.empty(la.prefill_workspace_bytes(n_pre, T_pre, w.H), dtype=torch.uint8, device="cuda")
    o_pre = torch.empty_like(pre[0])
    S_pre_out = torch.empty_like(S_pre_in)

    def two_calls():
        la.prefill(*pre, S_in=S_pre_in, pos0=0, out=o_pre, S_out=S_pre_out, workspace=ws2)
        la.decode_step(*dec, S_dec, w.pos0[-1])

    res = {}
    for name, fn in (("varlen_one_call", one_call), ("prefill_plus_decode_calls", two_calls)):
        fn()
        e = hip.create(2)
        stream = torch.cuda.current_stream().cuda_stream
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        hip.record(e[0], stream)
        for _ in range(steps):
            fn()
        hip.record(e[1], stream)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
        ms = hip.ms(e[0], e[1]) / steps
        hip.destroy(e)
        res[name] = {"gpu_ms": round(ms, 4), "wall_ms": round(wall * 1e3, 4)}
    tokens = sum(w.lengths)
    n_dec = len(w.lengths) - n_pre
    # compulsory bytes: activations in/out of every token-head, plus each sequence's
    # state read and written once
    comp = 1280 * tokens * w.H + 2 * 65536 * len(w.lengths) * w.H
    ms = res["varlen_one_call"]["gpu_ms"]
    return {"workload": w.name, "sequences": len(w.lengths), "prefill_sequences": n_pre,
            "decode_sequences": n_dec, "tokens": tokens, "steps": steps,
            "tokens_per_s": round(tokens / (ms / 1e3), 1),
            "compulsory_bytes": comp, "achieved_GBps": round(comp / (ms / 1e3) / 1e9, 1),
            "hbm_roof_frac": round(comp / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4), **res}


def bench_layer(la, torch, workloads, hip, args, steps=5):
    """One layer on the 32K-token prompt: la_layer_forward, and its two projections
    timed alone (la_linear with the same shapes) against the bf16 MFMA peak."""
    w = workloads.LAYER_32K
    x, w_qkvg, w_o = workloads.layer_inputs(w.B, w.T, w.hidden, w.H, w.D, w.seed, "cuda")
    M, HD = w.B * w.T, w.H * w.D
    y = torch.empty_like(x)
    S_out = torch.empty((w.B, w.H, w.D, w.D), dtype=torch.float32, device="cuda")
    ws = torch.empty(la.layer_workspace_bytes(w.B, w.T, w.H), dtype=torch.uint8, device="cuda")
    proj = torch.empty((M, 4 * HD), dtype=torch.bfloat16, device="cuda")
    o = torch.randn((M, HD), device="cuda").to(torch.bfloat16)
    y2 = torch.empty((M, w.hidden), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def timed(fn):
        settle(torch, fn)
        e = hip.create(2)
        torch.cuda.synchronize()
        hip.record(e[0], stream)
        for _ in range(steps):
            fn()
        hip.record(e[1], stream)
        ms = hip.ms(e[0], e[1]) / steps
        hip.destroy(e)
        return ms

    layer_ms = timed(lambda: la.layer_forward(x, w_qkvg, w_o, out=y, S_out=S_out, workspace=ws))
    in_ms = timed(lambda: la.linear(x.view(M, w.hidden), w_qkvg, out=proj))
    out_ms = timed(lambda: la.linear(o, w_o, out=y2))
    f_in, f_out = 2 * M * 4 * HD * w.hidden, 2 * M * w.hidden * HD
    tf_in = f_in / (in_ms / 1e3) / 1e12
    return {
        "workload": w.name, "tokens": M, "steps": steps,
        "layer_ms": round(layer_ms, 4), "tokens_per_s": round(M / (layer_ms / 1e3), 1),
        "qkvg_projection": {"ms": round(in_ms, 4), "tflops": round(tf_in, 1),
                            "roofline": {"bound": "mfma", "kernel": "la_linear_ring_kernel", "achieved": round(tf_in, 1),
                                         "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                         "frac": round(tf_in / BF16_MFMA_PEAK_TFLOPS, 4)}},
        "o_projection": {"ms": round(out_ms, 4), "tflops": round(f_out / (out_ms / 1e3) / 1e12, 1),
                         "frac_of_bf16_peak": round(f_out / (out_ms / 1e3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)},
        "attention_ms": round(layer_ms - in_ms - out_ms, 4),
    }


def bench_backward(la, torch, workloads, hip, tensors, steps=3):
    """la_backward over the 256K-token prefill input (seeded output gradient)."""
    q, k, v, g = tensors
    B, T, H, D = q.shape
    gen = workloads.generator(7, "cuda")
    d_o = torch.randn(q.shape, generator=gen, device="cuda").to(torch.bfloat16)
    ws = torch.empty(la.backward_workspace_bytes(B, T, H, D), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def timed(fn):
        settle(torch, fn)
        e = hip.create(2)
        torch.cuda.synchronize()
        hip.record(e[0], stream)
        for _ in range(steps):
            fn()
        hip.record(e[1], stream)
        ms = hip.ms(e[0], e[1]) / steps
        hip.destroy(e)
        return ms

    ms = timed(lambda: la.backward(q, k, v, g, d_o, workspace=ws))
    # the backward reusing the segment states of the forward call that produced o
    fws = torch.empty(la.prefill_workspace_bytes(B, T, H, D), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    la.prefill(q, k, v, g, out=o, workspace=fws)
    saved_ms = timed(lambda: la.backward(q, k, v, g, d_o, workspace=ws, fwd_workspace=fws))
    step_ms = timed(lambda: (la.prefill(q, k, v, g, out=o, workspace=fws),
                             la.backward(q, k, v, g, d_o, workspace=ws, fwd_workspace=fws)))
    del o, fws
    # bytes every backward must move: read q, k, v, g, d_o and write dq, dk, dv, dgate
    comp = 9 * 256 * B * T * H
    roof = comp / (HBM_PEAK_GBS * 1e9)
    return {"workload": "backward_" + workloads.PREFILL_256K.name, "steps": steps, "ms": round(ms, 4),
            "tokens_per_s": round(B * T / (ms / 1e3), 1), "compulsory_bytes": comp,
            "hbm_roof_ms": round(roof * 1e3, 4), "path_frac": round(roof / (ms / 1e3), 4),
            "saved_forward_states": {
                "note": "la_backward_saved: the segment states of the la_prefill call that computed the "
                        "forward are reused (no forward state pass or scan in the backward)",
                "ms": round(saved_ms, 4), "tokens_per_s": round(B * T / (saved_ms / 1e3), 1),
                "path_frac": round(roof / (saved_ms / 1e3), 4),
                "forward_plus_backward_ms": round(step_ms, 4)}}


def sparse_prefill_keys(T: int, topk: int, block: int = 64) -> int:
    """Keys attended over all rows of one (b, h): row t of query block i sees
    min(i, topk) whole blocks and its own block up to itself."""
    total = 0
    for i in range(-(-T // block)):
        r0, r1 = i * block, min(i * block + block, T)
        n = r1 - r0
        total += n * min(i, topk) * block + n * (n + 1) // 2
    return total


def bench_sparse(la, torch, workloads, hip, steps=5):
    """The sparse layer: prefill of the 32K workload (MFMA-bound: 4 D flops per
    attended key and query, q k and p v) and one batched decode step against 128K
    caches (HBM-bound: the key means scanned and the chosen key/value rows)."""
    w = workloads.SPARSE_32K
    q, k, v, g = workloads.activations(w.B, w.T, w.H, w.D, w.seed, "cuda")
    o = torch.empty_like(q)
    ws = torch.empty(la.sparse_prefill_workspace_bytes(w.B, w.T, w.H, w.D, w.topk), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def timed(fn, n):
        settle(torch, fn)
        e = hip.create(2)
        torch.cuda.synchronize()
        hip.record(e[0], stream)
        for _ in range(n):
            fn()
        hip.record(e[1], stream)
        ms = hip.ms(e[0], e[1]) / n
        hip.destroy(e)
        return ms

    pre_ms = timed(lambda: la.sparse_prefill(q, k, v, g, topk=w.topk, out=o, workspace=ws), steps)
    flops = 4 * w.D * sparse_prefill_keys(w.T, w.topk) * w.B * w.H
    tf = flops / (pre_ms / 1e3) / 1e12
    prefill = {"workload": w.name, "ms": round(pre_ms, 4), "tokens_per_s": round(w.B * w.T / (pre_ms / 1e3), 1),
               "flops": flops, "roofline": {"bound": "mfma", "kernel": "la_sparse_prefill (means + selection + attention)",
                                            "achieved": round(tf, 1), "peak": BF16_MFMA_PEAK_TFLOPS,
                                            "unit": "TFLOP/s", "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4)}}
    del q, k, v, g, o, ws

    d = workloads.SPARSE_DECODE
    qd, kc, vc, gd = workloads.sparse_decode_inputs(d, "cuda")
    means = la.sparse_block_means(kc)
    lens = torch.full((d.B,), d.T, dtype=torch.int32, device="cuda")
    od = torch.empty_like(qd)
    dec_ms = timed(lambda: la.sparse_decode(qd, kc, vc, means, gd, lens, topk=d.topk, out=od), 20)
    nblk = d.T // 64
    own = (d.T - 1) // 64
    cand = own
    keys = min(cand, d.topk) * 64 + (d.T - 1 - own * 64 + 1)
    bytes_step = d.B * d.H * (cand * d.D * 4 + keys * 2 * d.D * 2 + 3 * d.D * 2)
    gbs = bytes_step / (dec_ms / 1e3) / 1e9
    decode = {"workload": d.name, "us_per_step": round(dec_ms * 1e3, 2), "bytes_per_step": bytes_step,
              "key_blocks": nblk, "roofline": {"bound": "hbm", "kernel": "la_sparse_decode_kernel",
                                               "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                               "frac": round(gbs / HBM_PEAK_GBS, 4)}}
    del qd, kc, vc, gd, means
    return {"prefill": prefill, "decode": decode}


def bench_stream(la, torch, workloads, hip, steps=3):
    """The 1M-token streamed prefill: 16 calls of 65536 tokens with the state carried
    in place (pos0 = 65536 s), and the same tokens in one call."""
    w = workloads.STREAM_1M
    q, k, v, g = workloads.activations(w.B, w.T, w.H, w.D, w.seed, "cuda")
    seg = w.T // w.segments
    S = torch.empty((w.B, w.H, w.D, w.D), dtype=torch.float32, device="cuda")
    o = torch.empty_like(q)
    ws = torch.empty(max(la.prefill_workspace_bytes(w.B, seg, w.H), la.prefill_workspace_bytes(w.B, w.T, w.H)),
                     dtype=torch.uint8, device="cuda")

    def streamed():
        for s in range(w.segments):
            sl = slice(s * seg, (s + 1) * seg)
            la.prefill(q[:, sl], k[:, sl], v[:, sl], g[:, sl], S_in=S if s else None, S_out=S, pos0=s * seg,
                       out=o[:, sl], workspace=ws)

    def single():
        la.prefill(q, k, v, g, S_out=S, out=o, workspace=ws)

    stream = torch.cuda.current_stream().cuda_stream
    out = {"workload": w.name, "segments": w.segments, "steps": steps}
    for name, fn in (("streamed", streamed), ("single_shot", single)):
        fn()
        e = hip.create(2)
        torch.cuda.synchronize()
        hip.record(e[0], stream)
        for _ in range(steps):
            fn()
        hip.record(e[1], stream)
        ms = hip.ms(e[0], e[1]) / steps
        hip.destroy(e)
        out[name] = {"ms": round(ms, 3), "tokens_per_s": round(w.B * w.T / (ms / 1e3), 1)}
    comp = 1280 * w.B * w.T * w.H
    out["hbm_roof_ms"] = round(comp / (HBM_PEAK_GBS * 1e9) * 1e3, 4)
    del q, k, v, g, o, ws
    return out


def settle(torch, fn, min_s=0.05, min_calls=2):
    """Untimed calls of fn until min_s seconds have passed (at least min_calls): the
    GPU clock takes tens of milliseconds to settle under a new load."""
    t0, n = time.perf_counter(), 0
    while n < min_calls or time.perf_counter() - t0 < min_s:
        fn()
        torch.cuda.synchronize()
        n += 1


def timed_calls(torch, hip, fn, n, warm=2):
    """GPU ms of each of n calls of fn (HIP events on the current stream around
    each call), after `warm` untimed calls."""
    settle(torch, fn, min_calls=warm)
    stream = torch.cuda.current_stream().cuda_stream
    evs = [hip.create(2) for _ in range(n)]
    torch.cuda.synchronize()
    for e in evs:
        hip.record(e[0], stream)
        fn()
        hip.record(e[1], stream)
    times = [hip.ms(e[0], e[1]) for e in evs]
    for e in evs:
        hip.destroy(e)
    return times


def bench_prefill_32k(la, torch, workloads, hip, n=50):
    """The 32K-token prefill (one layer's 32 heads) alone: median of n calls."""
    w = workloads.PREFILL_32K
    q, k, v, g = workloads.activations(w.B, w.T, w.H, w.D, w.seed, "cuda")
    o = torch.empty_like(q)
    S_out = torch.empty((w.B, w.H, w.D, w.D), dtype=torch.float32, device="cuda")
    ws = torch.empty(la.prefill_workspace_bytes(w.B, w.T, w.H), dtype=torch.uint8, device="cuda")
    ts = timed_calls(torch, hip, lambda: la.prefill(q, k, v, g, out=o, S_out=S_out, workspace=ws), n)
    med = statistics.median(ts)
    comp = TOKEN_HEAD_BYTES * w.B * w.T * w.H
    return {"workload": w.name, "calls": n, "median_ms": round(med, 4), "min_ms": round(min(ts), 4),
            "max_ms": round(max(ts), 4), "tokens_per_s": round(w.B * w.T / (med / 1e3), 1),
            "hbm_roof_ms": round(comp / (HBM_PEAK_GBS * 1e9) * 1e3, 4),
            "path_frac": round(comp / (HBM_PEAK_GBS * 1e9) / (med / 1e3), 4)}


def bench_batched_prefill(la, torch, workloads, hip, n=10):
    """8 prompts of 32K tokens (256 sequence-heads, as many tokens as the 256K
    prefill): one segment per (b, h), so one kernel reads k and v once."""
    w = workloads.PREFILL_B8_32K
    q, k, v, g = workloads.activations(w.B, w.T, w.H, w.D, w.seed, "cuda")
    o = torch.empty_like(q)
    S_out = torch.empty((w.B, w.H, w.D, w.D), dtype=torch.float32, device="cuda")
    ws = torch.empty(la.prefill_workspace_bytes(w.B, w.T, w.H), dtype=torch.uint8, device="cuda")
    ts = timed_calls(torch, hip, lambda: la.prefill(q, k, v, g, out=o, S_out=S_out, workspace=ws), n)
    med = statistics.median(ts)
    comp = TOKEN_HEAD_BYTES * w.B * w.T * w.H
    out = {"workload": w.name, "calls": n, "median_ms": round(med, 4),
           "tokens_per_s": round(w.B * w.T / (med / 1e3), 1), "one_segment_per_head": ws.numel() == 256,
           "hbm_roof_ms": round(comp / (HBM_PEAK_GBS * 1e9) * 1e3, 4),
           "path_frac": round(comp / (HBM_PEAK_GBS * 1e9) / (med / 1e3), 4),
           "achieved_GBps": round(comp / (med / 1e3) / 1e9, 1)}
    del q, k, v, g, o, ws
    return out


def _decode_steps_us(la, torch, hip, S0, q, k, v, g, pos):
    """µs per step of consecutive decode steps (plain launches) from S0 at pos."""
    S = S0.clone()
    out = torch.empty_like(q)
    steps = q.shape[0]
    for n in range(min(3, steps)):
        la.decode_step(q[n], k[n], v[n], g[n], S, pos + n, out=out[n])
    S.copy_(S0)
    stream = torch.cuda.current_stream().cuda_stream
    ev = hip.create(2)
    torch.cuda.synchronize()
    hip.record(ev[0], stream)
    for n in range(steps):
        la.decode_step(q[n], k[n], v[n], g[n], S, pos + n, out=out[n])
    hip.record(ev[1], stream)
    us = hip.ms(ev[0], ev[1]) * 1e3 / steps
    hip.destroy(ev)
    return us


def bench_decode_more(la, torch, workloads, hip, steps=200):
    """Decode step time at three positions (a step's cost must not depend on it),
    and at batches whose states exceed the 256 MB memory-side cache: 256 sequences
    (512 MiB; written back with non-temporal stores, which still leaves part of the
    working set to that cache) and 384 (768 MiB: every step streams its states from
    and to DRAM, at the same rate with either store kind)."""
    w = workloads.DECODE_B64
    S0, q, k, v, g = workloads.decode_inputs(w, steps=steps, device="cuda")
    pos = {str(p): round(_decode_steps_us(la, torch, hip, S0, q, k, v, g, p), 3) for p in (0, 262144, 1048575)}
    vals = list(pos.values())
    del S0, q, k, v, g
    out = {"us_per_step_by_position": pos, "position_max_over_min": round(max(vals) / min(vals), 4)}
    notes = {"b256": "the 512 MiB of states exceed the 256 MB memory-side cache; written back with non-temporal "
                     "stores, part of them is still served by that cache (compare b384)",
             "b384": "the 768 MiB of states exceed the 256 MB memory-side cache: each step reads and writes them "
                     "in DRAM (plain and non-temporal stores measured the same)"}
    for key, w2 in (("b256", workloads.DECODE_B256), ("b384", workloads.DECODE_B384)):
        S0, q, k, v, g = workloads.decode_inputs(w2, steps=w2.steps, device="cuda")
        us = _decode_steps_us(la, torch, hip, S0, q, k, v, g, w2.pos0)
        bytes_step = 2 * w2.B * w2.H * STATE_BYTES + 5 * w2.B * w2.H * w2.D * 2
        gbs = bytes_step / (us * 1e-6) / 1e9
        del S0, q, k, v, g
        torch.cuda.empty_cache()
        out[key] = {"workload": w2.name, "steps": w2.steps, "us_per_step": round(us, 3), "bytes_per_step": bytes_step,
                    "state_bytes": w2.B * w2.H * STATE_BYTES,
                    "roofline": {"bound": "hbm", "kernel": "la_decode_kernel", "achieved": round(gbs, 1),
                                 "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                                 "note": notes[key]}}
    return out


def _sclk_files():
    files = []
    for d in sorted(glob.glob("/sys/class/drm/card*/device")):
        f = os.path.join(d, "pp_dpm_sclk")
        try:
            if open(os.path.join(d, "vendor")).read().strip() == "0x1002" and os.access(f, os.R_OK):
                files.append(f)
        except OSError:
            pass
    return files


def _sclk_levels(path):
    """(current MHz, highest MHz) from a pp_dpm_sclk listing (current marked '*')."""
    cur, top = None, None
    for line in open(path):
        m = re.search(r"(\d+)\s*mhz", line, re.I)
        if not m:
            continue
        mhz = int(m.group(1))
        top = mhz if top is None else max(top, mhz)
        if "*" in line:
            cur = mhz
    return cur, top


def environment(torch, workloads, busy_fn):
    """Host and GPU facts for the record, with the GPU clock sampled while busy_fn's
    work (enqueued, not yet finished) keeps the GPU busy."""
    cpu = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    files = _sclk_files()
    busy_fn()
    samples, top = [], None
    for _ in range(10):
        for f in files:
            try:
                cur, t = _sclk_levels(f)
            except OSError:
                continue
            if cur is not None:
                samples.append(cur)
            top = t if top is None else max(top, t or 0)
        time.sleep(0.005)
    torch.cuda.synchronize()
    seeds = {w.name: w.seed for w in (*workloads.ALL, workloads.PREFILL_B8_32K, workloads.DECODE_B256, workloads.DECODE_B384,
                                      workloads.SERVING_MIX, workloads.LAYER_32K, workloads.SPARSE_32K,
                                      workloads.SPARSE_DECODE)}
    return {"gpu": torch.cuda.get_device_name(0), "torch": torch.__version__, "hip": torch.version.hip,
            "cpu_model": cpu, "nproc": os.cpu_count(),
            "cpus_usable": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
            "sclk_mhz_while_busy": samples or None, "sclk_mhz_max_level": top,
            "sclk_source": files[0] if files else None, "seeds": seeds}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--chunk", type=int, default=0)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--cpu-tokens", type=int, default=65536)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-varlen", action="store_true", help="skip the mixed prefill/decode batch")
    ap.add_argument("--no-layer", action="store_true", help="skip the layer forward with its projections")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward of the 256K prefill")
    ap.add_argument("--no-sparse", action="store_true", help="skip the sparse layer (32K prefill, 128K decode)")
    ap.add_argument("--no-stream", action="store_true",
                    help="skip the 1M-token prefill (16 carried calls of 65536, and one call)")
    ap.add_argument("--no-chunk-sweep", action="store_true",
                    help="skip timing the prefill at the other chunk sizes")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the 32K prefill alone, the batched prefill and the extra decode timings")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first run one plain device-to-device copy of this many MiB (a kernel of "
                         "known traffic, used to scale rocprofv3 FETCH_SIZE/WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this layer's path runs on a single MI355X "
              "(heads and sequences shard with no communication); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import hybrid_sparse_linear_la_amd as la
    import workloads

    la.library()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    hip = HipEvents()
    if args.calib_copy_mib:
        src = torch.ones(args.calib_copy_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    w, tps, step_s, roofline, detail, tensors = bench_prefill(la, torch, workloads, hip, args)
    q256, k256, v256, g256 = tensors
    o256 = torch.empty_like(q256)
    ws256 = torch.empty(la.prefill_workspace_bytes(*q256.shape[:3]), dtype=torch.uint8, device="cuda")
    env = environment(torch, workloads, lambda: [la.prefill(q256, k256, v256, g256, out=o256, workspace=ws256)
                                                 for _ in range(30)])
    del o256, ws256
    prefill_32k = None if args.no_extra else bench_prefill_32k(la, torch, workloads, hip)
    batched = None if args.no_extra else bench_batched_prefill(la, torch, workloads, hip)
    decode = None if args.no_decode else bench_decode(la, torch, workloads, hip, args)
    if decode is not None and not args.no_extra:
        decode.update(bench_decode_more(la, torch, workloads, hip))
    varlen = None if args.no_varlen else bench_varlen(la, torch, workloads, hip, args)
    layer = None if args.no_layer else bench_layer(la, torch, workloads, hip, args)
    backward = None if args.no_backward else bench_backward(la, torch, workloads, hip, tensors)
    sparse = None if args.no_sparse else bench_sparse(la, torch, workloads, hip)
    stream_1m = None if args.no_stream else bench_stream(la, torch, workloads, hip)
    invariants = {"description": "linear-time prefill and constant-cost decode: time ratios of the GPU "
                                 "medians (ideal 8 and 4 for the prefill, 1 for decode positions)"}
    t256 = detail["gpu_ms_per_step_median"]
    if prefill_32k is not None:
        invariants["t_256k_over_t_32k"] = round(t256 / prefill_32k["median_ms"], 4)
    if stream_1m is not None:
        invariants["t_1m_single_over_t_256k"] = round(stream_1m["single_shot"]["ms"] / t256, 4)
        invariants["t_1m_streamed_over_t_256k"] = round(stream_1m["streamed"]["ms"] / t256, 4)
    if decode is not None and "position_max_over_min" in decode:
        invariants["decode_position_max_over_min"] = decode["position_max_over_min"]
    cpu = None if args.no_cpu_baseline else cpu_baseline(tensors, args)
    if decode is not None and not args.no_cpu_baseline:
        decode["cpu_baseline"] = cpu_decode_baseline(workloads)
    line = {
        "metric": "linear-attn prefill tokens/s @256K (MFMA util %) + decode step us & GB/s",
        "value": round(tps, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 q/k/v/gate logits, S0 = 0)",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "D": w.D,
                   "chunk": detail["chunk"], "pos0": 0},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "prefill_detail": detail,
        "prefill_32k": prefill_32k,
        "batched_prefill": batched,
        "invariants": invariants,
        "environment": env,
        "decode": decode,
        "varlen": varlen,
        "layer": layer,
        "backward": backward,
        "sparse": sparse,
        "stream_1m": stream_1m,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
