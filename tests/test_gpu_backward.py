"""GPU parity of the backward pass (wkv7_backward, through the C ABI) against the
fp64 adjoint of the oracle.

The GPU kernel reads the per-position states that the step kernel writes (fp32);
the oracle forms its own fp64 states.  Tolerance 1e-5 on every gradient, for
bf16 and fp32 inputs alike (all gradient arithmetic is fp32): relative L2 over
the tensor and per (batch, head), and every element within 1e-5 times its
head's RMS (tests/parity.py).
"""
import numpy as np
import pytest
import torch

import synth
from parity import HEADS_SEQ, HEADS_STATE, check, rel_l2  # noqa: F401

pytestmark = pytest.mark.gpu

TOL = 1e-5
NAMES = ("dr", "dw", "dk", "dv", "da", "db")


@pytest.fixture(scope="module")
def K():
    import rwkv_linear_attention_amd as m
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: GPU tests must run on an MI355X")
    m.lib()
    return m


def run_both(K, oracle_mod, inp, d_o, d_state_out):
    d = {n: inp[n].cuda() for n in "rwkvab"}
    s_in = None if inp["state_in"] is None else inp["state_in"].cuda()
    _, _, s_pos = K.wkv7_step(*(d[n] for n in "rwkvab"), s_in, per_position=True)
    g = K.wkv7_backward(*(d[n] for n in "rwkvab"), s_in, s_pos, d_o.cuda(),
                        None if d_state_out is None else d_state_out.cuda())
    torch.cuda.synchronize()
    ref = oracle_mod.backward(*(inp[n] for n in "rwkvab"), inp["state_in"], d_o,
                              d_state_out)
    return g, ref


def check_all(g, ref, what):
    # every gradient globally, per (batch, head) and elementwise (tests/parity.py)
    for n in NAMES:
        check(g[n], ref[n], TOL, f"{what} {n}", HEADS_SEQ)
    check(g["d_state_in"], ref["d_state_in"], TOL, f"{what} d_state_in", HEADS_STATE)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 7, 33])
def test_backward_vs_oracle(K, oracle_mod, dtype, T):
    inp = synth.make_inputs(2, T, 3, 64, seed=3000 + T, dtype=dtype, state_std=0.1)
    gen = torch.Generator().manual_seed(3100 + T)
    d_o = torch.randn((2, T, 3, 64), generator=gen)
    d_so = torch.randn((2, 3, 64, 64), generator=gen)
    g, ref = run_both(K, oracle_mod, inp, d_o, d_so)
    check_all(g, ref, f"{dtype} T={T}")


def test_backward_no_state_in_no_final_gradient(K, oracle_mod):
    inp = synth.make_inputs(2, 20, 5, 64, seed=3200, dtype="bf16", state_std=0.0)
    assert inp["state_in"] is None
    d_o = torch.randn((2, 20, 5, 64), generator=torch.Generator().manual_seed(3201))
    g, ref = run_both(K, oracle_mod, inp, d_o, None)
    check_all(g, ref, "no state_in")


def test_backward_longer_sequence_sampled_heads(K, oracle_mod):
    # 0.1B-shaped heads over 300 tokens, every head against the oracle
    B, T, H = 4, 300, 12
    inp = synth.make_inputs(B, T, H, 64, seed=3300, dtype="bf16", state_std=0.1)
    gen = torch.Generator().manual_seed(3301)
    d_o = torch.randn((B, T, H, 64), generator=gen)
    d_so = torch.randn((B, H, 64, 64), generator=gen)
    d = {n: inp[n].cuda() for n in "rwkvab"}
    s_in = inp["state_in"].cuda()
    _, _, s_pos = K.wkv7_step(*(d[n] for n in "rwkvab"), s_in, per_position=True)
    g = K.wkv7_backward(*(d[n] for n in "rwkvab"), s_in, s_pos, d_o.cuda(), d_so.cuda())
    torch.cuda.synchronize()
    ref = oracle_mod.backward(*(inp[n] for n in "rwkvab"), inp["state_in"], d_o, d_so)
    check_all(g, ref, f"B={B} T={T} H={H}")


def test_backward_many_heads_one_workgroup_per_head(K, oracle_mod):
    # 150 heads: more than half the compute units, so each head runs in one
    # workgroup (up to 128 heads, in two); every head against the oracle
    B, T, H = 3, 9, 50
    inp = synth.make_inputs(B, T, H, 64, seed=3500, dtype="f32", state_std=0.1)
    gen = torch.Generator().manual_seed(3501)
    d_o = torch.randn((B, T, H, 64), generator=gen)
    d_so = torch.randn((B, H, 64, 64), generator=gen)
    d = {n: inp[n].cuda() for n in "rwkvab"}
    s_in = inp["state_in"].cuda()
    _, _, s_pos = K.wkv7_step(*(d[n] for n in "rwkvab"), s_in, per_position=True)
    g = K.wkv7_backward(*(d[n] for n in "rwkvab"), s_in, s_pos, d_o.cuda(), d_so.cuda())
    torch.cuda.synchronize()
    ref = oracle_mod.backward(*(inp[n] for n in "rwkvab"), inp["state_in"], d_o, d_so)
    check_all(g, ref, f"B={B} T={T} H={H}")


@pytest.mark.parametrize("H", [2, 129])
def test_backward_every_short_length(K, oracle_mod, H):
    # T = 1 .. 10 covers every way the token loop splits into its first step, whole
    # rounds of four and the last partial rounds; H = 2 runs two workgroups per head,
    # H = 129 one (more than 128 heads); every head against the oracle
    for T in range(1, 11):
        inp = synth.make_inputs(1, T, H, 64, seed=3600 + T, dtype="bf16", state_std=0.1)
        gen = torch.Generator().manual_seed(3700 + T)
        d_o = torch.randn((1, T, H, 64), generator=gen)
        d_so = torch.randn((1, H, 64, 64), generator=gen)
        d = {n: inp[n].cuda() for n in "rwkvab"}
        s_in = inp["state_in"].cuda()
        _, _, s_pos = K.wkv7_step(*(d[n] for n in "rwkvab"), s_in, per_position=True)
        g = K.wkv7_backward(*(d[n] for n in "rwkvab"), s_in, s_pos, d_o.cuda(), d_so.cuda())
        torch.cuda.synchronize()
        ref = oracle_mod.backward(*(inp[n] for n in "rwkvab"), inp["state_in"], d_o, d_so)
        check_all(g, ref, f"H={H} T={T}")


def test_backward_empty_sequence_and_in_place(K):
    inp = synth.make_inputs(2, 0, 3, 64, seed=3400, dtype="bf16", state_std=0.1)
    d = {n: inp[n].cuda() for n in "rwkvab"}
    s_in = inp["state_in"].cuda()
    s_pos = torch.empty((2, 0, 3, 64, 64), device="cuda")
    d_o = torch.empty((2, 0, 3, 64), device="cuda")
    d_so = torch.randn((2, 3, 64, 64), device="cuda")
    g = K.wkv7_backward(*(d[n] for n in "rwkvab"), s_in, s_pos, d_o, d_so)
    torch.cuda.synchronize()
    assert torch.equal(g["d_state_in"], d_so)
    g0 = K.wkv7_backward(*(d[n] for n in "rwkvab"), s_in, s_pos, d_o, None)
    torch.cuda.synchronize()
    assert not torch.any(g0["d_state_in"])
    # d_state_in may be d_state_out itself
    inp = synth.make_inputs(1, 9, 2, 64, seed=3401, dtype="bf16", state_std=0.1)
    d = {n: inp[n].cuda() for n in "rwkvab"}
    s_in = inp["state_in"].cuda()
    _, _, s_pos = K.wkv7_step(*(d[n] for n in "rwkvab"), s_in, per_position=True)
    d_o = torch.randn((1, 9, 2, 64), device="cuda")
    d_so = torch.randn((1, 2, 64, 64), device="cuda")
    ref = K.wkv7_backward(*(d[n] for n in "rwkvab"), s_in, s_pos, d_o, d_so.clone())
    grads = {n: torch.empty_like(ref[n]) for n in NAMES}
    grads["d_state_in"] = d_so
    K.wkv7_backward(*(d[n] for n in "rwkvab"), s_in, s_pos, d_o, d_so, grads=grads)
    torch.cuda.synchronize()
    assert torch.equal(d_so, ref["d_state_in"])
    for n in NAMES:
        assert torch.equal(grads[n], ref[n])
