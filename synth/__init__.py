"""Seeded synthetic WKV-7 inputs, shared by the tests, the smoke check and the benchmark.

This module holds no part of the recurrence itself: it only draws the six
per-token input vectors (r, w, k, v, a, b) and the incoming state the way the
RWKV-7 time-mix block produces them, so that both the GPU path and the CPU
oracle can be fed the same numbers.

Recipe (one (b, t, h) row of N channels at a time, all drawn in fp32 on the
CPU with one ``torch.Generator`` seeded per workload):

* r, k, v ~ N(0, 1); gate_x ~ N(0, 1); w_x ~ N(0, sigma_w)   (drawn in this order)
* kk = k / max(||k||_2, 1e-12) over the N channels of the row
* a = -kk;  b = kk * sigmoid(gate_x)           (the rank-1 "in-context learning rate" pair)
* w = exp(-0.6065306597 * sigmoid(w_x))        (decay multiplier, always in (0.5453, 1))
* state_in ~ N(0, 0.1) per element, or absent (zeros)
* in bf16 workloads each of r, w, k, v, a, b is rounded to bf16 (RNE) on its
  own; the state always stays fp32.

The decay form and the a = -kk, b = kk*a_gate pair are the RWKV-7 inputs of
the Core AI note, section 1, whose rank-1 term removes the gated projection of
the state onto the normalised key.  Shapes
follow the model sizes the pages quote: 0.1B (D=768, 12 heads) in the
SwiftRWKV Inference guide; 2.9B (32 layers / 2560), 7.2B (32 / 4096) and
13.3B (61 / 4096) in the RWKV7-MTP-Exp model card; batch 32 (and 16 for
13.3B) from that card's --max-batch settings; T = K+1 = 5 from its one
speculative step (base token plus four drafts).  No public dataset stands
behind these workloads; the synthetic draws stand in for activations.
"""
from __future__ import annotations

import dataclasses
import hashlib

import torch

DECAY_SCALE = 0.6065306597  # e^{-1/2}: keeps w = exp(-DECAY_SCALE * sigmoid(x)) in (0.5453, 1)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    N: int
    dtype: str          # "f32" or "bf16": dtype of r, w, k, v, a, b
    sigma_w: float      # std of the decay logit x
    state_std: float    # 0.0 -> state_in absent (zeros)
    seed: int
    layers: int = 1     # distinct buffer sets a timed sweep rotates over


# The five workloads (index = seed).
WORKLOADS = {
    0: Workload("tiny-f32", 1, 64, 2, 64, "f32", 1.0, 0.0, 0),
    1: Workload("decode-2.9B", 32, 1, 40, 64, "bf16", 1.0, 0.1, 1, layers=32),
    2: Workload("prefill-0.1B", 8, 4096, 12, 64, "bf16", 1.0, 0.0, 2),
    3: Workload("prefill-7.2B", 4, 8192, 64, 64, "bf16", 1.5, 0.1, 3),
    4: Workload("mtp-verify-13.3B", 16, 5, 64, 64, "bf16", 1.0, 0.1, 4, layers=61),
}


def make_inputs(B: int, T: int, H: int, N: int = 64, *, seed: int = 0, dtype: str = "bf16",
                sigma_w: float = 1.0, state_std: float = 0.1, device: str = "cpu") -> dict:
    """Draw one input set.  Returns a dict of tensors on ``device``.

    Keys r, w, k, v, a, b ([B,T,H,N], bf16 or fp32) and state_in ([B,H,N,N]
    fp32, or None when state_std == 0).  The same seed gives the same numbers
    on every CPU run; a GPU generator (device="cuda", used only for inputs that
    are timed and never compared) follows the same recipe with its own stream
    of random numbers.
    """
    g = torch.Generator(device=device).manual_seed(int(seed))
    shape = (B, T, H, N)
    rn = lambda shp: torch.randn(shp, generator=g, device=device)
    r = rn(shape)
    k = rn(shape)
    v = rn(shape)
    gate_x = rn(shape)
    w_x = rn(shape) * sigma_w
    state_in = None
    if state_std > 0:
        state_in = rn((B, H, N, N)) * state_std
    kk = k / k.norm(dim=-1, keepdim=True).clamp_min(1e-12)
    a = -kk
    b = kk * torch.sigmoid(gate_x)
    w = torch.exp(-DECAY_SCALE * torch.sigmoid(w_x))
    out = dict(r=r, w=w, k=k, v=v, a=a, b=b)
    if dtype == "bf16":
        out = {n: x.to(torch.bfloat16) for n, x in out.items()}
    elif dtype != "f32":
        raise ValueError(f"unknown dtype {dtype}")
    out = {n: x.contiguous() for n, x in out.items()}
    out["state_in"] = state_in
    return out


def workload_inputs(idx: int, *, T: int | None = None, seed_offset: int = 0, device: str = "cpu") -> dict:
    """Inputs of workload ``idx`` (optionally with another T, a shifted seed, or on the GPU)."""
    wl = WORKLOADS[idx]
    return make_inputs(wl.B, wl.T if T is None else T, wl.H, wl.N, seed=wl.seed + seed_offset,
                       dtype=wl.dtype, sigma_w=wl.sigma_w, state_std=wl.state_std, device=device)


def content_hash(inputs: dict) -> str:
    """sha256 over the raw bytes of every tensor, in a fixed order (drift detector)."""
    h = hashlib.sha256()
    for n in ("r", "w", "k", "v", "a", "b", "state_in"):
        x = inputs.get(n)
        if x is None:
            h.update(b"none")
            continue
        h.update(n.encode())
        h.update(str(x.dtype).encode())
        h.update(x.contiguous().view(torch.uint8).numpy().tobytes())
    return h.hexdigest()
