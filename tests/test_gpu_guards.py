"""Guard bands: no entry point writes outside its outputs.

Every output of every call below is a view into a larger buffer filled with
NaN, with 64 elements of NaN on each side.  After the call the guard bands must
still be NaN, and the output itself fully written (no NaN left), or, where an
entry point leaves elements untouched on purpose (outputs past a row's length),
exactly those still NaN.
"""
import pytest
import torch

import synth
from test_gpu_parity import K, to_dev  # noqa: F401  (K is a fixture)

pytestmark = pytest.mark.gpu

PAD = 64
NAMES = ("r", "w", "k", "v", "a", "b")


class Guarded:
    """A tensor of `shape` between two NaN guard bands of PAD elements."""

    def __init__(self, shape, dtype=torch.float32):
        n = 1
        for s in shape:
            n *= s
        self.buf = torch.full((n + 2 * PAD,), float("nan"), dtype=dtype, device="cuda")
        self.t = self.buf[PAD:PAD + n].view(*shape)

    def bands_intact(self):
        return bool(torch.isnan(self.buf[:PAD]).all() and torch.isnan(self.buf[-PAD:]).all())

    def full(self):
        return not bool(torch.isnan(self.t).any())


def _check(what, *gs):
    torch.cuda.synchronize()
    for i, g in enumerate(gs):
        assert g.bands_intact(), f"{what}: output {i} wrote into its guard band"


@pytest.mark.parametrize("o_dtype", [torch.float32, torch.bfloat16])
def test_step_outputs_and_per_position_states(K, o_dtype):
    B, T, H = 3, 5, 4
    d = to_dev(synth.make_inputs(B, T, H, 64, seed=401, dtype="bf16", state_std=0.1))
    o, s, sp = Guarded((B, T, H, 64), o_dtype), Guarded((B, H, 64, 64)), Guarded((B, T, H, 64, 64))
    K.wkv7_step(*[d[n] for n in NAMES], d["state_in"], o=o.t, state_out=s.t, state_pos=sp.t)
    _check("step", o, s, sp)
    assert o.full() and s.full() and sp.full()
    # per-position states only
    o2, sp2 = Guarded((B, T, H, 64), o_dtype), Guarded((B, T, H, 64, 64))
    K.wkv7_step(*[d[n] for n in NAMES], d["state_in"], o=o2.t, state_pos=sp2.t, write_state_out=False)
    _check("step, per-position states only", o2, sp2)
    assert o2.full() and sp2.full()


@pytest.mark.parametrize("T", [6, 37])
def test_varlen_forward(K, T):
    # T = 6 runs the step kernel, T = 37 the chunked one; rows past their length stay NaN
    B, H = 4, 3
    d = to_dev(synth.make_inputs(B, T, H, 64, seed=402 + T, dtype="bf16", state_std=0.1))
    lengths = [0, 1, T // 2, T]
    o, s = Guarded((B, T, H, 64)), Guarded((B, H, 64, 64))
    K.wkv7_forward(*[d[n] for n in NAMES], d["state_in"], o=o.t, state_out=s.t, lengths=lengths)
    _check("varlen forward", o, s)
    assert s.full()
    for bb, L in enumerate(lengths):
        assert not torch.isnan(o.t[bb, :L]).any(), f"row {bb}: an output inside the row is missing"
        assert torch.isnan(o.t[bb, L:]).all(), f"row {bb}: an output past the row's length was written"


def test_forward_bf16_output(K):
    B, T, H = 2, 41, 5
    d = to_dev(synth.make_inputs(B, T, H, 64, seed=404, dtype="bf16", state_std=0.1))
    o, s = Guarded((B, T, H, 64), torch.bfloat16), Guarded((B, H, 64, 64))
    K.wkv7_forward(*[d[n] for n in NAMES], d["state_in"], o=o.t, state_out=s.t)
    _check("forward, bf16 o", o, s)
    assert o.full() and s.full()


def test_state_commit(K):
    B, T, H = 6, 5, 3
    d = to_dev(synth.make_inputs(B, T, H, 64, seed=405, dtype="bf16", state_std=0.1))
    _, _, sp = K.wkv7_step(*[d[n] for n in NAMES], d["state_in"], per_position=True)
    s = Guarded((B, H, 64, 64))
    accepted = [0, 1, 3, 5, -1, 9]   # the last two rows are out of range: left untouched (NaN)
    K.wkv7_state_commit(sp, accepted, d["state_in"], state_out=s.t)
    _check("commit", s)
    assert not torch.isnan(s.t[:4]).any() and torch.isnan(s.t[4:]).all()


@pytest.mark.parametrize("x_dtype", [torch.float32, torch.bfloat16])
def test_tail_outputs(K, x_dtype):
    B, T, H = 2, 5, 3
    d = to_dev(synth.make_inputs(B, T, H, 64, seed=406, dtype="bf16", state_std=0.1))
    gen = torch.Generator(device="cuda").manual_seed(407)
    gate = torch.sigmoid(torch.randn((B, T, H, 64), generator=gen, device="cuda")).to(torch.bfloat16)
    r_k = 0.1 * torch.randn((H, 64), generator=gen, device="cuda")
    ln_w = 1 + 0.1 * torch.randn((H, 64), generator=gen, device="cuda")
    ln_b = 0.1 * torch.randn((H, 64), generator=gen, device="cuda")
    x, s, sp = Guarded((B, T, H, 64), x_dtype), Guarded((B, H, 64, 64)), Guarded((B, T, H, 64, 64))
    K.wkv7_step_tail(*[d[n] for n in NAMES], gate, r_k, ln_w, ln_b, 64e-5, d["state_in"], x=x.t,
                     state_out=s.t, state_pos=sp.t)
    _check("step with the fused tail", x, s, sp)
    assert x.full() and s.full() and sp.full()
    o, _ = K.wkv7_forward(*[d[n] for n in NAMES], d["state_in"])
    x2 = Guarded((B, T, H, 64), x_dtype)
    K.wkv7_tmix_tail(o, d["r"], d["k"], d["v"], gate, r_k, ln_w, ln_b, 64e-5, x=x2.t)
    _check("tail pass", x2)
    assert x2.full()


@pytest.mark.parametrize("T", [6, 45])
def test_forward_tail_outputs(K, T):
    # the fused prefill tail: x and state_out only (T = 45: the chunked kernel's tail wave)
    B, H = 2, 3
    d = to_dev(synth.make_inputs(B, T, H, 64, seed=410 + T, dtype="bf16", state_std=0.1))
    gen = torch.Generator(device="cuda").manual_seed(411)
    gate = torch.sigmoid(torch.randn((B, T, H, 64), generator=gen, device="cuda")).to(torch.bfloat16)
    prm = [0.1 * torch.randn((H, 64), generator=gen, device="cuda") + c for c in (0.0, 1.0, 0.0)]
    x, s = Guarded((B, T, H, 64)), Guarded((B, H, 64, 64))
    K.wkv7_forward_tail(*[d[n] for n in NAMES], gate, *prm, 64e-5, d["state_in"], x=x.t, state_out=s.t)
    _check("forward with the fused tail", x, s)
    assert x.full() and s.full()


@pytest.mark.parametrize("H", [3, 129])
def test_backward_outputs(K, H):
    # H = 3: two workgroups per head (a fill kernel, then atomic adds); H = 129: one
    B, T = 1, 11
    inp = synth.make_inputs(B, T, H, 64, seed=408 + H, dtype="bf16", state_std=0.1)
    d = to_dev(inp)
    _, _, sp = K.wkv7_step(*[d[n] for n in NAMES], d["state_in"], per_position=True)
    gen = torch.Generator(device="cuda").manual_seed(409)
    d_o = torch.randn((B, T, H, 64), generator=gen, device="cuda")
    d_so = torch.randn((B, H, 64, 64), generator=gen, device="cuda")
    gs = {n: Guarded((B, T, H, 64)) for n in ("dr", "dw", "dk", "dv", "da", "db")}
    gs["d_state_in"] = Guarded((B, H, 64, 64))
    K.wkv7_backward(*[d[n] for n in NAMES], d["state_in"], sp, d_o, d_so, grads={n: g.t for n, g in gs.items()})
    _check("backward", *gs.values())
    for n, g in gs.items():
        assert g.full(), f"{n} not fully written"


@pytest.mark.parametrize("T", [7, 45])
def test_training_pair_outputs(K, T):
    # T = 7: a state copy then the step kernel; T = 45: the chunked kernel writing the
    # checkpoints; then the backward from them (H = 3: two workgroups per head)
    B, H = 2, 3
    d = to_dev(synth.make_inputs(B, T, H, 64, seed=420 + T, dtype="bf16", state_std=0.1))
    nck = (T + 15) // 16
    o, s, ck = Guarded((B, T, H, 64)), Guarded((B, H, 64, 64)), Guarded((B, nck, H, 64 * 64))
    K.wkv7_forward_ckpt(*[d[n] for n in NAMES], d["state_in"], o=o.t, state_out=s.t, ckpt=ck.t)
    _check("forward with checkpoints", o, s, ck)
    assert o.full() and s.full() and ck.full()
    gen = torch.Generator(device="cuda").manual_seed(421)
    d_o = torch.randn((B, T, H, 64), generator=gen, device="cuda")
    d_so = torch.randn((B, H, 64, 64), generator=gen, device="cuda")
    gs = {n: Guarded((B, T, H, 64)) for n in ("dr", "dw", "dk", "dv", "da", "db")}
    gs["d_state_in"] = Guarded((B, H, 64, 64))
    K.wkv7_backward_ckpt(*[d[n] for n in NAMES], ck.t, d_o, d_so, grads={n: g.t for n, g in gs.items()})
    _check("backward from checkpoints", *gs.values())
    for n, g in gs.items():
        assert g.full(), f"{n} not fully written"


def test_backward_ckpt_one_workgroup_per_head_outputs(K):
    B, T, H = 1, 21, 129
    d = to_dev(synth.make_inputs(B, T, H, 64, seed=422, dtype="f32", state_std=0.1))
    _, _, ck = K.wkv7_forward_ckpt(*[d[n] for n in NAMES], d["state_in"])
    gen = torch.Generator(device="cuda").manual_seed(423)
    d_o = torch.randn((B, T, H, 64), generator=gen, device="cuda")
    gs = {n: Guarded((B, T, H, 64)) for n in ("dr", "dw", "dk", "dv", "da", "db")}
    gs["d_state_in"] = Guarded((B, H, 64, 64))
    K.wkv7_backward_ckpt(*[d[n] for n in NAMES], ck, d_o, None, grads={n: g.t for n, g in gs.items()})
    _check("backward from checkpoints, whole heads", *gs.values())
    for n, g in gs.items():
        assert g.full(), f"{n} not fully written"
