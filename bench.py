#!/usr/bin/env python3
"""Benchmark of libwkv7 on one MI355X: decode-step us/layer and prefill Mtok/s.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1|2|3|4] [--no-cpu-baseline]
    python bench.py --entry NAME [--no-cpu-baseline]     (one measurement alone, e.g. for a profiler)

Prints ONE JSON line.  The headline workload (default) is the 2.9B-shaped
decode step (B=32, T=1, H=40, N=64, bf16 inputs, fp32 state), one layer per
call over 32 distinct layer buffer sets, state updated in place: a timed
"step" is one sweep over the 32 layers, replayed from a captured HIP graph.
``value`` is microseconds per layer.  The same line carries the roofline of
the dominant kernel (live HIP-event timing; HBM traffic from committed
rocprofv3 counter summaries when they were taken on the current kernel
source), the fp64 CPU oracle timed on a bounded sample of the same workload,
and (default run) every other measurement ("other_workloads": the prefill and
verify workloads, the fused tail, the variable-length prefill, the commit, and
the training pair of forward with checkpoints and backward from them), each with
its own roofline and its own oracle baseline.

Workloads (all synthetic, seeded; see synth/):
  1 decode-2.9B       B=32 T=1    H=40  step kernel, 32 layers, in place
  2 prefill-0.1B      B=8  T=4096 H=12  chunked kernel, one call
  3 prefill-7.2B      B=4  T=8192 H=64  chunked kernel, one call, state carried in
  4 mtp-verify-13.3B  B=16 T=5    H=64  step kernel + per-position states, 61 layers
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix, published
N = 64
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "rwkv_linear_attention_amd", "csrc")


def algorithmic_bytes(wl, kind: str, o_bytes: int = 4) -> int:
    """Bytes the method must move per call: inputs once, o once (fp32 unless o_bytes says
    otherwise), state read and written once, plus per-position states for the verify step."""
    e_in = 2 if wl.dtype == "bf16" else 4
    tokheads = wl.B * wl.T * wl.H
    b = tokheads * (6 * N * e_in + o_bytes * N)
    b += 2 * wl.B * wl.H * N * N * 4 if (wl.state_std > 0 or kind == "step") else wl.B * wl.H * N * N * 4
    if kind == "verify":
        b += tokheads * N * N * 4
    return b


def recurrent_flops(wl) -> int:
    return wl.B * wl.T * wl.H * 9 * N * N


def kernel_source_hash(kind: str) -> str:
    name = {"step": "wkv7_step.hip", "verify": "wkv7_step.hip", "chunk": "wkv7_chunk.hip", "chunk_tail": "wkv7_chunk.hip",
            "chunk_ckpt": "wkv7_chunk.hip", "step_tail": "wkv7_step.hip", "tail_pass": "wkv7_tail.hip",
            "bwd_ckpt": "wkv7_bwdc.hip", "bwd": "wkv7_bwd.hip", "bwd_zero": "wkv7_bwd.hip",
            "commit": "wkv7_step.hip"}[kind]
    h = hashlib.sha256()
    for f in (name, "wkv7_device.h"):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def call_kernels(kind: str, workload: int):
    """The kernels one call of `kind` runs on `workload`: the backward pass from
    per-position states with two workgroups per head (at most 128 heads) first zeroes
    the outputs they add into ("bwd_zero").  The backward from checkpoints ("bwd_ckpt")
    counts its three launches (chunk kernel, chain, chunk kernel) together."""
    if kind == "bwd":
        import synth
        wl = synth.WORKLOADS[workload]
        return (kind, "bwd_zero") if wl.B * wl.H * 2 <= 256 else (kind,)
    return (kind,)


def read_traffic(kind: str, workload: int):
    """HBM bytes per launch (per call: every kernel of call_kernels(kind, workload))
    from profiles/hbm_traffic.txt, or None when absent or stale.

    Lines: <kernel-kind> <workload> <source-hash> <fetch_bytes> <write_bytes>
    (bytes already scaled by the copy-kernel calibration factor).
    """
    path = os.path.join(PROFILES, "hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    cur = kernel_source_hash(kind)
    want = call_kernels(kind, workload)
    found = {}
    with open(path) as f:
        for line in f:
            parts = line.split("#", 1)[0].split()
            if len(parts) == 5 and parts[0] in want and parts[1] == str(workload):
                if parts[2] != cur:
                    return None
                found[parts[0]] = float(parts[3]) + float(parts[4])
    return int(sum(found.values())) if len(found) == len(want) else None


def roofline(bytes_per_launch: int, sec_per_launch: float, kind: str, workload: int):
    ach = bytes_per_launch / sec_per_launch / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": read_traffic(kind, workload)}


# ----------------------------------------------------------------------------- GPU timing

WARM_SECONDS = 0.3  # untimed warm-up: at least this long (clocks settle) and at least W steps


def warm(fn, steps: int):
    """Run fn() at least `steps` times and for at least WARM_SECONDS, then synchronize."""
    import torch
    t0, n = time.perf_counter(), 0
    while n < steps or time.perf_counter() - t0 < WARM_SECONDS:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()

def tail_params(H: int, seed: int):
    """Per-head parameters of the time-mix tail (random, fp32 [H, N]) on the GPU."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(seed)
    r_k = torch.randn((H, N), generator=g, device="cuda") * 0.1
    ln_w = 1 + 0.1 * torch.randn((H, N), generator=g, device="cuda")
    ln_b = 0.1 * torch.randn((H, N), generator=g, device="cuda")
    return r_k, ln_w, ln_b


def make_layers(K, synth, idx: int, nlayers: int, tail=False):
    """nlayers distinct buffer sets of workload idx on the GPU (inputs, state, outputs; with tail,
    also a gate and the tail's per-head parameters)."""
    import torch
    wl = synth.WORKLOADS[idx]
    sets = []
    for l in range(nlayers):
        inp = synth.workload_inputs(idx, seed_offset=1000 * l)
        d = {n: inp[n].cuda() for n in ("r", "w", "k", "v", "a", "b")}
        d["state"] = inp["state_in"].cuda()
        d["o"] = torch.empty((wl.B, wl.T, wl.H, N), dtype=torch.float32, device="cuda")
        d["pos"] = torch.empty((wl.B, wl.T, wl.H, N, N), dtype=torch.float32, device="cuda") if idx == 4 else None
        if tail == "pos_only":  # the verify step with per-position states only (no separate state_out)
            d["mode"] = tail
        elif tail:  # "fused" (the tail in the step's epilogue) or "separate" (a second launch)
            gen = torch.Generator(device="cuda").manual_seed(77 + l)
            d["g"] = torch.sigmoid(torch.randn(d["r"].shape, generator=gen, device="cuda")).to(d["r"].dtype)
            d["tail"] = tail_params(wl.H, 78 + l)
            d["mode"] = tail
            if tail == "separate":
                d["x"] = torch.empty_like(d["o"])
        sets.append(d)
    return sets


def sweep(K, sets):
    for d in sets:
        if d.get("mode") == "pos_only":
            K.wkv7_step(d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], d["state"], o=d["o"],
                        state_pos=d["pos"], write_state_out=False)
        elif d.get("mode") == "fused":
            K.wkv7_step_tail(d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], d["g"], *d["tail"], 64e-5,
                             d["state"], x=d["o"], state_out=d["state"], state_pos=d["pos"])
        elif d.get("mode") == "separate":
            K.wkv7_step(d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], d["state"], o=d["o"],
                        state_out=d["state"], state_pos=d["pos"])
            K.wkv7_tmix_tail(d["o"], d["r"], d["k"], d["v"], d["g"], *d["tail"], 64e-5, x=d["x"])
        else:
            K.wkv7_step(d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], d["state"], o=d["o"],
                        state_out=d["state"], state_pos=d["pos"])


def time_step_workload(K, synth, idx: int, steps: int, warmup: int, tail=False):
    """Graph-captured sweeps over the layer sets; returns dict of timings."""
    import torch
    wl = synth.WORKLOADS[idx]
    sets = make_layers(K, synth, idx, wl.layers, tail)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        sweep(K, sets)                      # eager warm-up (loads the code objects)
        # graph replay must reproduce the eager result bit for bit
        saved = [d["state"].clone() for d in sets]
        sweep(K, sets)
        eager = [d["state"].clone() for d in sets] + [d["o"].clone() for d in sets]
        for d, s in zip(sets, saved):
            d["state"].copy_(s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            sweep(K, sets)
        for d, s in zip(sets, saved):
            d["state"].copy_(s)
        g.replay()
        torch.cuda.synchronize()
        replay = [d["state"] for d in sets] + [d["o"] for d in sets]
        if not all(torch.equal(a, b) for a, b in zip(eager, replay)):
            raise RuntimeError("graph replay differs from the eager sweep")
        warm(g.replay, warmup)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            g.replay()
        e1.record(stream)
        e1.synchronize()
    ms = e0.elapsed_time(e1)
    per_layer_s = ms / 1e3 / (steps * wl.layers)
    return {"ms_per_step": ms / steps, "us_per_layer": per_layer_s * 1e6, "sec_per_launch": per_layer_s,
            "layers": wl.layers}


def time_prefill_workload(K, synth, idx: int, steps: int, warmup: int, o_bf16: bool = False, lengths=None):
    """One prefill call over workload idx; with lengths ([B] int32 on the GPU), row b runs its
    first lengths[b] tokens (the variable-length form), and mtok_s counts those tokens."""
    import torch
    wl = synth.WORKLOADS[idx]
    d = synth.workload_inputs(idx, device="cuda")
    o = torch.empty((wl.B, wl.T, wl.H, N), dtype=torch.bfloat16 if o_bf16 else torch.float32, device="cuda")
    s_out = torch.empty((wl.B, wl.H, N, N), dtype=torch.float32, device="cuda")
    args = [d[n] for n in ("r", "w", "k", "v", "a", "b")]
    run = lambda: K.wkv7_forward(*args, d["state_in"], o=o, state_out=s_out, lengths=lengths)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        warm(run, warmup)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            run()
        e1.record(stream)
        e1.synchronize()
    ms = e0.elapsed_time(e1) / steps
    tokens = wl.B * wl.T if lengths is None else int(lengths.sum().item())
    return {"ms_per_step": ms, "sec_per_launch": ms / 1e3, "mtok_s": tokens / (ms / 1e3) / 1e6}


def varlen_lengths(wl, seed: int = 91):
    """A right-padded batch: row lengths drawn uniformly from [T/2, T] (seeded)."""
    import torch
    gen = torch.Generator().manual_seed(seed)
    return torch.randint(wl.T // 2, wl.T + 1, (wl.B,), generator=gen, dtype=torch.int32)


def varlen_bytes(wl, lengths) -> int:
    """Algorithmic bytes of a variable-length prefill: inputs and o of the real tokens only,
    the state read and written once."""
    e_in = 2 if wl.dtype == "bf16" else 4
    b = int(lengths.sum().item()) * wl.H * (6 * N * e_in + 4 * N)
    return b + (2 if wl.state_std > 0 else 1) * wl.B * wl.H * N * N * 4


def time_commit(K, synth, idx: int, steps: int, warmup: int, nsets: int = 8):
    """wkv7_state_commit after the verify step of workload idx: the state after each row's
    accepted prefix (accepted counts drawn from [0, T], seeded), over nsets distinct buffer
    sets in one graph (more bytes than the caches hold), replayed."""
    import torch
    wl = synth.WORKLOADS[idx]
    d = synth.workload_inputs(idx, device="cuda")
    ins = [d[n] for n in ("r", "w", "k", "v", "a", "b")]
    gen = torch.Generator().manual_seed(97)
    acc = torch.randint(0, wl.T + 1, (wl.B,), generator=gen, dtype=torch.int32)
    sets = []
    for _ in range(nsets):
        _, _, s_pos = K.wkv7_step(*ins, d["state_in"], per_position=True, write_state_out=False)
        sets.append((s_pos, acc.cuda(), torch.empty((wl.B, wl.H, N, N), device="cuda")))
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for s_pos, a_, s_o in sets:
            K.wkv7_state_commit(s_pos, a_, d["state_in"], state_out=s_o)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for s_pos, a_, s_o in sets:
                K.wkv7_state_commit(s_pos, a_, d["state_in"], state_out=s_o)
        warm(g.replay, warmup)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            g.replay()
        e1.record(stream)
        e1.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / (steps * nsets)
    return {"sec_per_launch": sec, "bytes": 2 * wl.B * wl.H * N * N * 4 + wl.B * 4}


def time_tail_pass(K, synth, idx: int, steps: int, warmup: int):
    """The time-mix tail as a pass of its own over the outputs of prefill workload idx."""
    import torch
    wl = synth.WORKLOADS[idx]
    d = synth.workload_inputs(idx, device="cuda")
    o, _ = K.wkv7_forward(*[d[n] for n in ("r", "w", "k", "v", "a", "b")], d["state_in"])
    gen = torch.Generator(device="cuda").manual_seed(79)
    g = torch.sigmoid(torch.randn(d["r"].shape, generator=gen, device="cuda")).to(d["r"].dtype)
    prm = tail_params(wl.H, 80)
    x = torch.empty_like(o)
    stream = torch.cuda.Stream()
    run = lambda: K.wkv7_tmix_tail(o, d["r"], d["k"], d["v"], g, *prm, 64e-5, x=x)
    with torch.cuda.stream(stream):
        warm(run, warmup)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            run()
        e1.record(stream)
        e1.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"sec_per_launch": ms / 1e3}


def time_forward_tail(K, synth, idx: int, steps: int, warmup: int):
    """The parallel pass with the time-mix tail fused (wkv7_forward_tail) over prefill workload
    idx: x (fp32) is written instead of o."""
    import torch
    wl = synth.WORKLOADS[idx]
    d = synth.workload_inputs(idx, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(79)
    g = torch.sigmoid(torch.randn(d["r"].shape, generator=gen, device="cuda")).to(d["r"].dtype)
    prm = tail_params(wl.H, 80)
    x = torch.empty((wl.B, wl.T, wl.H, N), dtype=torch.float32, device="cuda")
    s_out = torch.empty((wl.B, wl.H, N, N), dtype=torch.float32, device="cuda")
    ins = [d[n] for n in ("r", "w", "k", "v", "a", "b")]
    stream = torch.cuda.Stream()
    run = lambda: K.wkv7_forward_tail(*ins, g, *prm, 64e-5, d["state_in"], x=x, state_out=s_out)
    with torch.cuda.stream(stream):
        warm(run, warmup)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            run()
        e1.record(stream)
        e1.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"sec_per_launch": ms / 1e3, "mtok_s": wl.B * wl.T / (ms / 1e3) / 1e6}


def forward_tail_bytes(wl) -> int:
    """Algorithmic bytes of the fused prefill + tail: the six inputs and the gate read once,
    x (fp32) written once, the state read and written once, the tail's per-head parameters."""
    e_in = 2 if wl.dtype == "bf16" else 4
    b = wl.B * wl.T * wl.H * N * (7 * e_in + 4)
    return b + (2 if wl.state_std > 0 else 1) * wl.B * wl.H * N * N * 4 + 3 * wl.H * N * 4


def checkpoint_bytes(wl) -> int:
    """The chunk checkpoints of workload wl: one fp32 state per head and 16 tokens."""
    return wl.B * ((wl.T + 15) // 16) * wl.H * N * N * 4


def forward_ckpt_bytes(wl) -> int:
    """Algorithmic bytes of the forward pass with checkpoints: the prefill's, plus the
    checkpoints written once."""
    return algorithmic_bytes(wl, "chunk") + checkpoint_bytes(wl)


def backward_ckpt_bytes(wl) -> int:
    """Algorithmic bytes of one backward call from checkpoints: the six inputs and d_o read
    once, the six fp32 gradients written once, the checkpoints read once; per head the final
    state's gradient read and the input state's gradient written."""
    e_in = 2 if wl.dtype == "bf16" else 4
    tokheads = wl.B * wl.T * wl.H
    return tokheads * (6 * N * e_in + N * 4 + 6 * N * 4) + checkpoint_bytes(wl) + wl.B * wl.H * 2 * N * N * 4


def perpos_backward_bytes(wl) -> int:
    """Algorithmic bytes of one call of the backward from per-position states (wkv7_backward):
    the states, the six inputs and d_o read once, the six gradients written once; per head the
    input state and the final state's gradient read, the input state's gradient written."""
    e_in = 2 if wl.dtype == "bf16" else 4
    tokheads = wl.B * wl.T * wl.H
    per_head = (3 if wl.state_std > 0 else 2) * N * N * 4
    return tokheads * (N * N * 4 + 6 * N * e_in + N * 4 + 6 * N * 4) + wl.B * wl.H * per_head


def time_call(run, steps: int, warmup: int) -> float:
    """Seconds per call of run() on a stream of its own (HIP events around `steps` calls)."""
    import torch
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        warm(run, warmup)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            run()
        e1.record(stream)
        e1.synchronize()
    return e0.elapsed_time(e1) / 1e3 / steps


def time_forward_ckpt(K, synth, idx: int, steps: int, warmup: int):
    """The forward pass of training over prefill workload idx: o, state_out and the chunk
    checkpoints."""
    import torch
    wl = synth.WORKLOADS[idx]
    d = synth.workload_inputs(idx, device="cuda")
    ins = [d[n] for n in ("r", "w", "k", "v", "a", "b")]
    o, s_out, ck = K.wkv7_forward_ckpt(*ins, d["state_in"])
    sec = time_call(lambda: K.wkv7_forward_ckpt(*ins, d["state_in"], o=o, state_out=s_out, ckpt=ck), steps, warmup)
    return {"sec_per_launch": sec, "mtok_s": wl.B * wl.T / sec / 1e6}


def time_backward_ckpt(K, synth, idx: int, steps: int, warmup: int):
    """The backward pass over workload idx from the checkpoints of its forward pass (written
    once, untimed), a random d_o and a random final-state gradient."""
    import torch
    wl = synth.WORKLOADS[idx]
    d = synth.workload_inputs(idx, device="cuda")
    ins = [d[n] for n in ("r", "w", "k", "v", "a", "b")]
    _, _, ck = K.wkv7_forward_ckpt(*ins, d["state_in"])
    gen = torch.Generator(device="cuda").manual_seed(83)
    d_o = torch.randn(d["r"].shape, generator=gen, device="cuda")
    d_so = torch.randn((wl.B, wl.H, N, N), generator=gen, device="cuda")
    grads = K.wkv7_backward_ckpt(*ins, ck, d_o, d_so)
    sec = time_call(lambda: K.wkv7_backward_ckpt(*ins, ck, d_o, d_so, grads=grads), steps, warmup)
    return {"sec_per_launch": sec, "mtok_s": wl.B * wl.T / sec / 1e6}


def copy_ceiling(idx: int, steps: int, warmup: int):
    """A plain device copy moving the same bytes as one call of workload idx (state in ->
    state out, per-position states included), over the same number of distinct buffer sets,
    graph-replayed like the step workloads: the HBM rate a streaming read+write reaches here."""
    import torch
    import synth
    wl = synth.WORKLOADS[idx]
    kind = "verify" if idx == 4 else "step" if idx == 1 else "chunk"
    nbytes = algorithmic_bytes(wl, kind)
    n = nbytes // 8  # floats per side: half the bytes read, half written
    layers = max(1, wl.layers)
    src = [torch.randn(n, device="cuda") for _ in range(layers)]
    dst = [torch.empty(n, device="cuda") for _ in range(layers)]
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for s_, d_ in zip(src, dst):
            d_.copy_(s_)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for s_, d_ in zip(src, dst):
                d_.copy_(s_)
        warm(g.replay, warmup)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            g.replay()
        e1.record(stream)
        e1.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / (steps * layers)
    return {"bytes_per_copy": 8 * n, "us_per_copy": round(sec * 1e6, 3), "GB/s": round(8 * n / sec / 1e9, 1)}


def fill_ceiling(idx: int, steps: int, warmup: int):
    """A write-only fill of the bytes one call of workload idx writes (o, state_out and, for
    the verify step, the per-position states), over the same number of distinct buffers,
    graph-replayed: the HBM rate a streaming write reaches here."""
    import torch
    import synth
    wl = synth.WORKLOADS[idx]
    tokheads = wl.B * wl.T * wl.H
    nbytes = tokheads * N * 4 + wl.B * wl.H * N * N * 4 + (tokheads * N * N * 4 if idx == 4 else 0)
    n = nbytes // 4
    layers = max(1, wl.layers)
    bufs = [torch.empty(n, device="cuda") for _ in range(layers)]
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for b_ in bufs:
            b_.fill_(1.0)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for b_ in bufs:
                b_.fill_(1.0)
        warm(g.replay, warmup)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            g.replay()
        e1.record(stream)
        e1.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / (steps * layers)
    return {"bytes_per_fill": 4 * n, "us_per_fill": round(sec * 1e6, 3), "GB/s": round(4 * n / sec / 1e9, 1)}


def time_backward_perpos(K, synth, idx: int, steps: int, warmup: int):
    """The training pair without checkpoints, for comparison: the recurrent pass writing every
    per-position state (wkv7_step), then the backward reading them (wkv7_backward)."""
    import torch
    wl = synth.WORKLOADS[idx]
    d = synth.workload_inputs(idx, device="cuda")
    ins = [d[n] for n in ("r", "w", "k", "v", "a", "b")]
    o, s_out, s_pos = K.wkv7_step(*ins, d["state_in"], per_position=True)
    gen = torch.Generator(device="cuda").manual_seed(83)
    d_o = torch.randn(d["r"].shape, generator=gen, device="cuda")
    d_so = torch.randn((wl.B, wl.H, N, N), generator=gen, device="cuda")
    grads = K.wkv7_backward(*ins, d["state_in"], s_pos, d_o, d_so)
    fwd = time_call(lambda: K.wkv7_step(*ins, d["state_in"], o=o, state_out=s_out, state_pos=s_pos), steps, warmup)
    bwd = time_call(lambda: K.wkv7_backward(*ins, d["state_in"], s_pos, d_o, d_so, grads=grads), steps, warmup)
    return {"sec_per_launch": bwd, "sec_forward": fwd, "state_bytes": s_pos.numel() * 4}


# ----------------------------------------------------------------------------- CPU baseline

def _threads() -> int:
    return min(16, len(os.sched_getaffinity(0)))


def _timed(fn, budget_s: float):
    """fn() once untimed, then repeatedly for at least budget_s: (calls, seconds)."""
    fn()
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            return reps, el


def cpu_baseline(synth, idx: int, budget_s: float = 12.0, tail: bool = False):
    """The fp64 oracle, as it stands, on full layers of a step workload (1 or 4): µs per layer.
    With tail, the time-mix tail follows each layer's recurrence."""
    import numpy as np
    import oracle
    wl = synth.WORKLOADS[idx]
    th = _threads()
    inp = synth.workload_inputs(idx)
    args = [inp[n] for n in ("r", "w", "k", "v", "a", "b")]
    if tail:
        rng = np.random.default_rng(5)
        g = 1 / (1 + np.exp(-rng.standard_normal(args[0].shape)))
        prm = [rng.standard_normal((wl.H, N)) * 0.1, 1 + rng.standard_normal((wl.H, N)) * 0.1,
               rng.standard_normal((wl.H, N)) * 0.1]
        fn = lambda: oracle.tmix_tail(oracle.forward(*args, inp["state_in"], nthreads=th)[0], args[0], args[2],
                                      args[3], g, *prm, 64e-5)
    else:
        fn = lambda: oracle.forward(*args, inp["state_in"], nthreads=th, per_position=(idx == 4))
    reps, el = _timed(fn, budget_s)
    return {"value": round(el / reps * 1e6, 1), "unit": "us/layer", "cores": th, "kind": "oracle",
            "sample": f"{reps} calls of one full layer of workload {idx} ({wl.B}x{wl.T}x{wl.H} token-heads)"
                      + (" with the time-mix tail" if tail else "") + f", {el:.1f} s wall"}


def cpu_baseline_prefill(synth, idx: int, budget_s: float = 8.0, what: str = "forward", Ts: int = 256):
    """The fp64 oracle on the first Ts tokens of prefill workload idx, in Mtok/s (B Ts tokens
    per call, every head).  what: "forward", "varlen" (the rows' lengths of the variable-length
    measurement, scaled to Ts), "per_position" (the states every checkpoint is taken from),
    "tail" (the time-mix tail alone), "forward_tail" (both), "backward" (the adjoint; one row
    and 32 tokens per call: its loop runs in Python)."""
    import numpy as np
    import oracle
    wl = synth.WORKLOADS[idx]
    th = _threads()
    B = 1 if what == "backward" else wl.B
    Ts = 32 if what == "backward" else Ts
    inp = synth.make_inputs(wl.B, Ts, wl.H, N, seed=wl.seed, dtype=wl.dtype, sigma_w=wl.sigma_w,
                            state_std=wl.state_std)
    args = [inp[n][:B] for n in ("r", "w", "k", "v", "a", "b")]
    s_in = None if inp["state_in"] is None else inp["state_in"][:B]
    rng = np.random.default_rng(6)
    if what in ("tail", "forward_tail"):
        g = 1 / (1 + np.exp(-rng.standard_normal(args[0].shape)))
        prm = [rng.standard_normal((wl.H, N)) * 0.1, 1 + rng.standard_normal((wl.H, N)) * 0.1,
               rng.standard_normal((wl.H, N)) * 0.1]
    if what == "forward":
        fn = lambda: oracle.forward(*args, s_in, nthreads=th)
    elif what == "per_position":
        fn = lambda: oracle.forward(*args, s_in, nthreads=th, per_position=True)
    elif what == "varlen":
        lens = (varlen_lengths(wl).numpy().astype(np.int64) * Ts) // wl.T
        fn = lambda: oracle.forward_varlen(*args, s_in, lengths=lens, nthreads=th)
    elif what == "tail":
        o = oracle.forward(*args, s_in, nthreads=th)[0]
        fn = lambda: oracle.tmix_tail(o, args[0], args[2], args[3], g, *prm, 64e-5)
    elif what == "forward_tail":
        fn = lambda: oracle.tmix_tail(oracle.forward(*args, s_in, nthreads=th)[0], args[0], args[2], args[3], g,
                                      *prm, 64e-5)
    elif what == "backward":
        d_o = rng.standard_normal((B, Ts, wl.H, N))
        d_so = rng.standard_normal((B, wl.H, N, N))
        fn = lambda: oracle.backward(*args, s_in, d_o, d_so)
    else:
        raise ValueError(what)
    reps, el = _timed(fn, budget_s)
    tokens = int(lens.sum()) if what == "varlen" else B * Ts  # (the rows' real tokens only)
    return {"value": round(tokens * reps / el / 1e6, 5), "unit": "Mtok/s",
            "cores": 1 if what in ("tail", "backward") else th, "kind": "oracle",
            "sample": f"{reps} calls of the oracle's {what.replace('_', ' ')} over {B}x{Ts}x{wl.H} token-heads "
                      f"of workload {idx}, {el:.1f} s wall"}


def cpu_baseline_commit(synth, idx: int, budget_s: float = 3.0):
    """The oracle's commit of each row's accepted prefix after the verify step: µs per call."""
    import numpy as np
    import oracle
    wl = synth.WORKLOADS[idx]
    inp = synth.workload_inputs(idx)
    _, _, s_pos = oracle.forward(*[inp[n] for n in ("r", "w", "k", "v", "a", "b")], inp["state_in"],
                                 per_position=True, nthreads=_threads())
    acc = np.random.default_rng(97).integers(0, wl.T + 1, wl.B)
    reps, el = _timed(lambda: oracle.state_commit(s_pos, acc, inp["state_in"]), budget_s)
    return {"value": round(el / reps * 1e6, 1), "unit": "us/call", "cores": 1, "kind": "oracle",
            "sample": f"{reps} commits of workload {idx}'s per-position states ({wl.B} rows), {el:.1f} s wall"}


# ----------------------------------------------------------------------------- measurements

def measurements(K, synth, args):
    """Every measurement of the default run, by name: a function returning its entry
    (timing, roofline, oracle baseline unless --no-cpu-baseline)."""
    steps, warmup = args.steps, args.warmup
    psteps = max(20, steps)
    bsteps, bwarm = max(5, steps // 4), min(warmup, 2)
    cpu = not args.no_cpu_baseline
    budget = 3.0
    W = synth.WORKLOADS

    def step_wl(j):
        t = time_step_workload(K, synth, j, steps, warmup)
        kind = "step" if j == 1 else "verify"
        e = {"workload": W[j].name, "ms_per_call": round(t["sec_per_launch"] * 1e3, 4),
             "us_per_layer": round(t["us_per_layer"], 3),
             "roofline": roofline(algorithmic_bytes(W[j], kind), t["sec_per_launch"], kind, j)}
        if cpu:
            e["cpu_baseline"] = cpu_baseline(synth, j, budget)
        return e

    def prefill_wl(j):
        t = time_prefill_workload(K, synth, j, psteps, warmup)
        e = {"workload": W[j].name, "ms_per_call": round(t["sec_per_launch"] * 1e3, 4),
             "mtok_s": round(t["mtok_s"], 2),
             "roofline": roofline(algorithmic_bytes(W[j], "chunk"), t["sec_per_launch"], "chunk", j),
             "alg_flops_frac_bf16": round(recurrent_flops(W[j]) / t["sec_per_launch"] / 1e12 / PEAK_BF16_TFLOPS, 5)}
        if cpu:
            e["cpu_baseline"] = cpu_baseline_prefill(synth, j, budget)
        return e

    def bf16o():
        # workload 3 with a bf16 o (the ABI's o_dtype option): 896 instead of 1024 algorithmic
        # bytes per token-head; its HBM counters are not taken (traffic null)
        w3 = W[3]
        t = time_prefill_workload(K, synth, 3, psteps, warmup, o_bf16=True)
        r = roofline(algorithmic_bytes(w3, "chunk", o_bytes=2), t["sec_per_launch"], "chunk", 3)
        r["traffic"] = None
        e = {"workload": w3.name + " (bf16 o)", "ms_per_call": round(t["sec_per_launch"] * 1e3, 4), "roofline": r,
             "mtok_s": round(t["mtok_s"], 2)}
        if cpu:
            e["cpu_baseline"] = cpu_baseline_prefill(synth, 3, budget)
        return e

    def tail1():
        # the time-mix tail fused into the decode step, and the step followed by the tail pass
        w1 = W[1]
        tt = time_step_workload(K, synth, 1, steps, warmup, tail="fused")
        ts = time_step_workload(K, synth, 1, steps, warmup, tail="separate")
        b = algorithmic_bytes(w1, "step") + w1.B * w1.T * w1.H * N * 2 + 3 * w1.H * N * 4
        e = {"workload": w1.name + " (fused time-mix tail)", "us_per_layer": round(tt["us_per_layer"], 3),
             "roofline": roofline(b, tt["sec_per_launch"], "step_tail", 1),
             "us_per_layer_step_then_tail_pass": round(ts["us_per_layer"], 3)}
        if cpu:
            e["cpu_baseline"] = cpu_baseline(synth, 1, budget, tail=True)
        return e

    def pos_only():
        # the verify step writing per-position states only (the final state is the last of them)
        w4 = W[4]
        t = time_step_workload(K, synth, 4, steps, warmup, tail="pos_only")
        r = roofline(algorithmic_bytes(w4, "verify") - w4.B * w4.H * N * N * 4, t["sec_per_launch"], "verify", 4)
        r["traffic"] = None
        e = {"workload": w4.name + " (per-position states only)", "us_per_layer": round(t["us_per_layer"], 3),
             "roofline": r}
        if cpu:
            e["cpu_baseline"] = cpu_baseline(synth, 4, budget)
        return e

    def tail_pass():
        w3 = W[3]
        t = time_tail_pass(K, synth, 3, psteps, warmup)
        b = w3.B * w3.T * w3.H * N * (4 + 4 * 2 + 4) + 3 * w3.H * N * 4
        e = {"workload": w3.name + " (time-mix tail pass)", "ms_per_call": round(t["sec_per_launch"] * 1e3, 4),
             "mtok_s": round(w3.B * w3.T / t["sec_per_launch"] / 1e6, 2),
             "roofline": roofline(b, t["sec_per_launch"], "tail_pass", 3)}
        if cpu:
            e["cpu_baseline"] = cpu_baseline_prefill(synth, 3, budget, what="tail")
        return e

    def fused_tail():
        # the prefill with the tail fused into the chunked kernel (x instead of o)
        w3 = W[3]
        t = time_forward_tail(K, synth, 3, psteps, warmup)
        e = {"workload": w3.name + " (prefill with the time-mix tail fused)",
             "ms_per_call": round(t["sec_per_launch"] * 1e3, 4), "mtok_s": round(t["mtok_s"], 2),
             "roofline": roofline(forward_tail_bytes(w3), t["sec_per_launch"], "chunk_tail", 3)}
        if cpu:
            e["cpu_baseline"] = cpu_baseline_prefill(synth, 3, budget, what="forward_tail")
        return e

    def fwd_ckpt(j):
        # the forward pass of training: the prefill plus the state before every 16-token chunk
        t = time_forward_ckpt(K, synth, j, psteps, warmup)
        e = {"workload": W[j].name + " (forward with chunk checkpoints)",
             "ms_per_call": round(t["sec_per_launch"] * 1e3, 4), "mtok_s": round(t["mtok_s"], 2),
             "roofline": roofline(forward_ckpt_bytes(W[j]), t["sec_per_launch"], "chunk_ckpt", j)}
        if cpu:
            e["cpu_baseline"] = cpu_baseline_prefill(synth, j, budget, what="per_position")
        return e

    def bwd_ckpt(j):
        # the backward pass from those checkpoints (every state rebuilt in the kernel)
        t = time_backward_ckpt(K, synth, j, bsteps, bwarm)
        e = {"workload": W[j].name + " (backward pass from chunk checkpoints)",
             "ms_per_call": round(t["sec_per_launch"] * 1e3, 4), "mtok_s": round(t["mtok_s"], 2),
             "roofline": roofline(backward_ckpt_bytes(W[j]), t["sec_per_launch"], "bwd_ckpt", j)}
        if cpu:
            e["cpu_baseline"] = cpu_baseline_prefill(synth, j, budget, what="backward")
        return e

    def bwd_perpos(j):
        # for comparison: the backward from per-position states, which the recurrent pass
        # must write first (16 KB per token-head)
        t = time_backward_perpos(K, synth, j, bsteps, bwarm)
        e = {"workload": W[j].name + " (backward pass from per-position states)",
             "ms_per_call": round(t["sec_per_launch"] * 1e3, 4),
             "ms_forward_writing_the_states": round(t["sec_forward"] * 1e3, 4),
             "state_bytes": t["state_bytes"],
             "roofline": roofline(perpos_backward_bytes(W[j]), t["sec_per_launch"], "bwd", j)}
        if cpu:
            e["cpu_baseline"] = cpu_baseline_prefill(synth, j, budget, what="backward")
        return e

    def varlen():
        # variable-length prefill (a right-padded batch) over workload 3
        w3 = W[3]
        lens = varlen_lengths(w3)
        t = time_prefill_workload(K, synth, 3, psteps, warmup, lengths=lens.cuda())
        r = roofline(varlen_bytes(w3, lens), t["sec_per_launch"], "chunk", 3)
        r["traffic"] = None
        e = {"workload": w3.name + " (rows of " + ",".join(str(int(x)) for x in lens) + " tokens)",
             "ms_per_call": round(t["sec_per_launch"] * 1e3, 4), "roofline": r, "mtok_s": round(t["mtok_s"], 2)}
        if cpu:
            e["cpu_baseline"] = cpu_baseline_prefill(synth, 3, budget, what="varlen")
        return e

    def commit():
        # the commit of each row's accepted prefix after the verify step of workload 4
        w4 = W[4]
        t = time_commit(K, synth, 4, steps, warmup)
        r = roofline(t["bytes"], t["sec_per_launch"], "commit", 4)
        r["traffic"] = None
        e = {"workload": w4.name + " (commit of the accepted prefixes)",
             "us_per_call": round(t["sec_per_launch"] * 1e6, 3), "roofline": r}
        if cpu:
            e["cpu_baseline"] = cpu_baseline_commit(synth, 4, budget)
        return e

    return {"1": lambda: step_wl(1), "2": lambda: prefill_wl(2), "3": lambda: prefill_wl(3),
            "4": lambda: step_wl(4), "3-bf16o": bf16o, "1-tail": tail1, "4-pos-only": pos_only,
            "3-tail-pass": tail_pass, "3-fused-tail": fused_tail, "2-fwd-ckpt": lambda: fwd_ckpt(2),
            "2-bwd": lambda: bwd_ckpt(2), "2-bwd-perpos": lambda: bwd_perpos(2), "3-fwd-ckpt": lambda: fwd_ckpt(3),
            "3-bwd": lambda: bwd_ckpt(3), "3-bwd-perpos": lambda: bwd_perpos(3),
            "3-varlen": varlen, "4-commit": commit}


# ----------------------------------------------------------------------------- main

def main():
    global WARM_SECONDS
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=1, choices=[1, 2, 3, 4])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", action="store_true", help="measure the chosen workload only")
    ap.add_argument("--entry", default=None,
                    help="run one named measurement of the default run alone (e.g. 3-bwd) and print its entry")
    ap.add_argument("--warm-seconds", type=float, default=WARM_SECONDS,
                    help="minimum untimed warm-up per measurement (0: just --warmup steps)")
    ap.add_argument("--fill-ceiling", action="store_true",
                    help="time a write-only fill of the bytes the workload writes instead (write ceiling)")
    ap.add_argument("--copy-ceiling", action="store_true",
                    help="time a plain device copy of the workload's bytes instead (HBM ceiling / counter calibration)")
    args = ap.parse_args()
    WARM_SECONDS = args.warm_seconds
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the WKV-7 kernels here are measured on one MI355X "
              f"(--gpus {args.gpus} is not supported; heads shard across GPUs with no exchange).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    if args.fill_ceiling:
        print(json.dumps({"fill_ceiling": fill_ceiling(args.workload, args.steps, args.warmup),
                          "workload": synth.WORKLOADS[args.workload].name}), flush=True)
        return
    if args.copy_ceiling:
        print(json.dumps({"copy_ceiling": copy_ceiling(args.workload, args.steps, args.warmup),
                          "workload": synth.WORKLOADS[args.workload].name}), flush=True)
        return
    import rwkv_linear_attention_amd as K
    K.lib()
    table = measurements(K, synth, args)
    if args.entry is not None:
        if args.entry not in table:
            raise SystemExit(f"unknown entry {args.entry!r}; one of {', '.join(table)}")
        print(json.dumps({"entry": args.entry, **table[args.entry]()}), flush=True)
        return

    idx = args.workload
    wl = synth.WORKLOADS[idx]
    if idx in (1, 4):
        kind = "step" if idx == 1 else "verify"
        t = time_step_workload(K, synth, idx, args.steps, args.warmup)
        rl = roofline(algorithmic_bytes(wl, kind), t["sec_per_launch"], kind, idx)
        metric_value, unit, hib = t["us_per_layer"], "us/layer", False
    else:
        t = time_prefill_workload(K, synth, idx, max(20, args.steps), args.warmup)
        rl = roofline(algorithmic_bytes(wl, "chunk"), t["sec_per_launch"], "chunk", idx)
        metric_value, unit, hib = t["mtok_s"], "Mtok/s", True

    line = {
        "metric": "WKV-7 prefill Mtok/s & decode-step µs per layer; % of HBM/MFMA roofline",
        "value": round(metric_value, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps if idx in (1, 4) else max(20, args.steps),
        "warmup": args.warmup,
        "ms_per_step": round(t["ms_per_step"], 4),
        "higher_is_better": hib,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "T": wl.T, "H": wl.H, "N": N, "inputs": wl.dtype,
                   "state": "fp32", "layers_per_step": wl.layers, "parallelism": "single-gpu"},
        "roofline": rl,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = (cpu_baseline(synth, idx) if idx in (1, 4) else cpu_baseline_prefill(synth, idx))
    if not args.only:
        others = {}
        for name, fn in table.items():
            if name != str(idx):
                others[name] = fn()
                print(f"bench: {name} measured", file=sys.stderr, flush=True)  # (progress, on stderr)
        line["other_workloads"] = others
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
