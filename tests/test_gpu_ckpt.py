"""GPU parity of the training pair (wkv7_forward_ckpt, wkv7_backward_ckpt, through
the C ABI) against the fp64 oracle.

The forward's checkpoints are compared with the oracle's states at the chunk
boundaries (ckpt[:, c] = the state after token 16 c - 1, the input state for
c = 0), put in the checkpoints' tile order; o and state_out as for wkv7_forward.  The backward rebuilds every state
from those fp32 checkpoints; its gradients are compared with the oracle's fp64
adjoint (which forms its own fp64 states) at 1e-5 for bf16 and fp32 inputs alike,
globally, per (batch, head) and elementwise (tests/parity.py).
"""
import numpy as np
import pytest
import torch

import synth
from parity import HEADS_SEQ, HEADS_STATE, check

pytestmark = pytest.mark.gpu

TOL = 1e-5                                # gradients, every input dtype
TOL_FWD = {"f32": 1e-5, "bf16": 2e-3}     # o, state_out, checkpoints
NAMES = ("dr", "dw", "dk", "dv", "da", "db")
RWKVAB = ("r", "w", "k", "v", "a", "b")


@pytest.fixture(scope="module")
def K():
    import rwkv_linear_attention_amd as m
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: GPU tests must run on an MI355X")
    m.lib()
    return m


def tile_order(s):
    """States [..., N, N] (key row i, value column j) in the checkpoints' element order:
    element (i, j) of a state at offset 1024 (j // 16) + 256 (i // 16) + 64 (i // 4 % 4)
    + 4 (j % 16) + i % 4 of its [N*N] block."""
    lead = s.shape[:-2]
    x = s.reshape(*lead, 4, 4, 4, 4, 16)  # i = 16 ib + 4 iq + ie, j = 16 jb + jm
    k = len(lead)
    return x.transpose(*range(k), k + 3, k, k + 1, k + 4, k + 2).reshape(*lead, 64 * 64)


def expected_ckpt(s_pos, state_in, B, T, H):
    """[B, ceil(T/16), H, N*N]: the state before each chunk of 16 tokens, in tile order."""
    nck = (T + 15) // 16
    out = np.zeros((B, nck, H, 64, 64))
    if state_in is not None:
        out[:, 0] = state_in.double().numpy()
    for c in range(1, nck):
        out[:, c] = s_pos[:, 16 * c - 1]
    return tile_order(out)


def grads_vs_oracle(K, oracle_mod, inp, d_o, d_so, what):
    d = {n: inp[n].cuda() for n in RWKVAB}
    s_in = None if inp["state_in"] is None else inp["state_in"].cuda()
    _, _, ck = K.wkv7_forward_ckpt(*(d[n] for n in RWKVAB), s_in)
    g = K.wkv7_backward_ckpt(*(d[n] for n in RWKVAB), ck, d_o.cuda(), None if d_so is None else d_so.cuda())
    torch.cuda.synchronize()
    ref = oracle_mod.backward(*(inp[n] for n in RWKVAB), inp["state_in"], d_o, d_so)
    for n in NAMES:
        check(g[n], ref[n], TOL, f"{what} {n}", HEADS_SEQ)
    check(g["d_state_in"], ref["d_state_in"], TOL, f"{what} d_state_in", HEADS_STATE)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,H,state", [
    (2, 45, 3, True),     # few heads: four column blocks per head
    (2, 41, 40, True),    # two column blocks
    (3, 37, 50, True),    # whole heads
    (2, 5, 3, True),      # one chunk, the step kernel: the checkpoint is state_in in tile order
    (1, 8, 2, False),     # ... or zeros
    (1, 16, 2, True),     # exactly one chunk (chunked kernel)
    (1, 17, 2, False),    # a last chunk of one token
])
def test_forward_ckpt_vs_oracle(K, oracle_mod, dtype, B, T, H, state):
    inp = synth.make_inputs(B, T, H, 64, seed=4000 + T + H, dtype=dtype, state_std=0.1 if state else 0.0)
    d = {n: inp[n].cuda() for n in RWKVAB}
    s_in = None if inp["state_in"] is None else inp["state_in"].cuda()
    o, s, ck = K.wkv7_forward_ckpt(*(d[n] for n in RWKVAB), s_in)
    torch.cuda.synchronize()
    o_ref, s_ref, sp_ref = oracle_mod.forward(*(inp[n] for n in RWKVAB), inp["state_in"], per_position=True)
    tol = TOL_FWD[dtype]
    what = f"{dtype} B={B} T={T} H={H}"
    check(o, o_ref, tol, f"{what} o", HEADS_SEQ)
    check(s, s_ref, tol, f"{what} state_out", HEADS_STATE)
    check(ck, expected_ckpt(sp_ref, inp["state_in"], B, T, H), tol, f"{what} ckpt", HEADS_SEQ)
    # o and state_out are those of wkv7_forward, bit for bit
    o2, s2 = K.wkv7_forward(*(d[n] for n in RWKVAB), s_in)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(s, s2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 8, 9, 16, 17, 33, 45])
def test_backward_ckpt_vs_oracle(K, oracle_mod, dtype, T):
    # B * H = 6: two workgroups per head; every way a sequence ends inside a chunk
    inp = synth.make_inputs(2, T, 3, 64, seed=4100 + T, dtype=dtype, state_std=0.1)
    gen = torch.Generator().manual_seed(4200 + T)
    d_o = torch.randn((2, T, 3, 64), generator=gen)
    d_so = torch.randn((2, 3, 64, 64), generator=gen)
    grads_vs_oracle(K, oracle_mod, inp, d_o, d_so, f"{dtype} T={T}")


@pytest.mark.parametrize("dtype,T", [("bf16", 5), ("bf16", 16), ("bf16", 40), ("f32", 23)])
def test_backward_ckpt_one_workgroup_per_head(K, oracle_mod, dtype, T):
    # 129 heads: one workgroup per head
    inp = synth.make_inputs(1, T, 129, 64, seed=4300 + T, dtype=dtype, state_std=0.1)
    gen = torch.Generator().manual_seed(4400 + T)
    d_o = torch.randn((1, T, 129, 64), generator=gen)
    d_so = torch.randn((1, 129, 64, 64), generator=gen)
    grads_vs_oracle(K, oracle_mod, inp, d_o, d_so, f"{dtype} H=129 T={T}")


@pytest.mark.parametrize("B,H", [(2, 5), (1, 129)])
def test_backward_ckpt_no_state_in_no_final_gradient(K, oracle_mod, B, H):
    # with 129 heads the chunk-form chain starts from a zero gradient, and the chunk
    # kernel's last chunk has no G_end to read
    inp = synth.make_inputs(B, 40, H, 64, seed=4500 + H, dtype="bf16", state_std=0.0)
    assert inp["state_in"] is None
    d_o = torch.randn((B, 40, H, 64), generator=torch.Generator().manual_seed(4501))
    grads_vs_oracle(K, oracle_mod, inp, d_o, None, f"no state_in, H={H}")


def test_backward_ckpt_longer_sequence_every_head(K, oracle_mod):
    # 0.1B-shaped heads over 300 tokens (19 chunks), every head against the oracle
    B, T, H = 4, 300, 12
    inp = synth.make_inputs(B, T, H, 64, seed=4600, dtype="bf16", state_std=0.1)
    gen = torch.Generator().manual_seed(4601)
    d_o = torch.randn((B, T, H, 64), generator=gen)
    d_so = torch.randn((B, H, 64, 64), generator=gen)
    grads_vs_oracle(K, oracle_mod, inp, d_o, d_so, f"B={B} T={T} H={H}")


@pytest.mark.parametrize("dtype,B,H", [("f32", 2, 3), ("bf16", 2, 3), ("f32", 1, 129), ("bf16", 1, 129)])
def test_backward_ckpt_tiny_decays(K, oracle_mod, dtype, B, H):
    # chunks with w = 0 and w = 1e-3 (the exact paths) among ordinary ones; with few
    # heads the gradient chain runs token by token, with 129 it runs in chunk form
    T = 70
    inp = synth.make_inputs(B, T, H, 64, seed=4700 + H, dtype=dtype, state_std=0.1)
    w = inp["w"].clone()
    w[:, 16:32] = 0.0
    w[B - 1, 40:44, 2] = 1e-3
    w[0, 50:52, H - 1] = 2.0 ** -14  # just above the exact-path threshold
    inp["w"] = w.contiguous()
    gen = torch.Generator().manual_seed(4701)
    d_o = torch.randn((B, T, H, 64), generator=gen)
    d_so = torch.randn((B, H, 64, 64), generator=gen)
    grads_vs_oracle(K, oracle_mod, inp, d_o, d_so, f"{dtype} tiny decays")


@pytest.mark.parametrize("H", [3, 129])
def test_backward_ckpt_empty_sequence_and_in_place(K, H):
    inp = synth.make_inputs(2, 0, H, 64, seed=4800, dtype="bf16", state_std=0.1)
    d = {n: inp[n].cuda() for n in RWKVAB}
    s_in = inp["state_in"].cuda()
    o, s, ck = K.wkv7_forward_ckpt(*(d[n] for n in RWKVAB), s_in)
    torch.cuda.synchronize()
    assert ck.shape == (2, 0, H, 64 * 64) and torch.equal(s, s_in)
    d_o = torch.empty((2, 0, H, 64), device="cuda")
    d_so = torch.randn((2, H, 64, 64), device="cuda")
    g = K.wkv7_backward_ckpt(*(d[n] for n in RWKVAB), ck, d_o, d_so)
    torch.cuda.synchronize()
    assert torch.equal(g["d_state_in"], d_so)
    # d_state_in may be d_state_out itself
    inp = synth.make_inputs(1, 40, H, 64, seed=4801, dtype="bf16", state_std=0.1)
    d = {n: inp[n].cuda() for n in RWKVAB}
    _, _, ck = K.wkv7_forward_ckpt(*(d[n] for n in RWKVAB), inp["state_in"].cuda())
    d_o = torch.randn((1, 40, H, 64), device="cuda")
    d_so = torch.randn((1, H, 64, 64), device="cuda")
    ref = K.wkv7_backward_ckpt(*(d[n] for n in RWKVAB), ck, d_o, d_so.clone())
    grads = {n: torch.empty_like(ref[n]) for n in NAMES}
    grads["d_state_in"] = d_so
    K.wkv7_backward_ckpt(*(d[n] for n in RWKVAB), ck, d_o, d_so, grads=grads)
    torch.cuda.synchronize()
    assert torch.equal(d_so, ref["d_state_in"])
    for n in NAMES:
        assert torch.equal(grads[n], ref[n])


@pytest.mark.parametrize("T", [5, 40])
def test_forward_ckpt_in_place(K, T):
    # state_out may be state_in itself: the one-chunk path takes its checkpoint before the
    # step kernel updates the state, the chunked kernel keeps the input state in registers
    inp = synth.make_inputs(2, T, 3, 64, seed=4810 + T, dtype="bf16", state_std=0.1)
    d = {n: inp[n].cuda() for n in RWKVAB}
    s_in = inp["state_in"].cuda()
    o_ref, s_ref, ck_ref = K.wkv7_forward_ckpt(*(d[n] for n in RWKVAB), s_in)
    state = s_in.clone()
    o, s, ck = K.wkv7_forward_ckpt(*(d[n] for n in RWKVAB), state, state_out=state)
    torch.cuda.synchronize()
    assert s.data_ptr() == state.data_ptr()
    assert torch.equal(o, o_ref) and torch.equal(state, s_ref) and torch.equal(ck, ck_ref)


@pytest.mark.parametrize("idx,heads", [(2, [(0, 0), (7, 11)]), (3, [(0, 0), (2, 37), (3, 63)])])
def test_workload_training_pair_sampled_heads(K, oracle_mod, idx, heads):
    # the prefill workloads at full size, in the launch configuration the benchmark
    # times; the oracle runs the sampled heads alone (heads are independent)
    inp = synth.workload_inputs(idx)
    B, T, H, _ = inp["r"].shape
    d = {n: inp[n].cuda() for n in RWKVAB}
    s_in = None if inp["state_in"] is None else inp["state_in"].cuda()
    gen = torch.Generator(device="cuda").manual_seed(4900 + idx)
    d_o = torch.randn((B, T, H, 64), generator=gen, device="cuda")
    d_so = torch.randn((B, H, 64, 64), generator=gen, device="cuda")
    o, s, ck = K.wkv7_forward_ckpt(*(d[n] for n in RWKVAB), s_in)
    g = K.wkv7_backward_ckpt(*(d[n] for n in RWKVAB), ck, d_o, d_so)
    torch.cuda.synchronize()
    for bb, hh in heads:
        one = {n: inp[n][bb:bb + 1, :, hh:hh + 1].contiguous() for n in RWKVAB}
        one_s = None if inp["state_in"] is None else inp["state_in"][bb:bb + 1, hh:hh + 1].contiguous()
        what = f"workload {idx} head ({bb}, {hh})"
        o_ref, s_ref, sp_ref = oracle_mod.forward(*(one[n] for n in RWKVAB), one_s, per_position=True)
        tol = TOL_FWD["bf16"]
        check(o[bb:bb + 1, :, hh:hh + 1], o_ref, tol, f"{what} o", HEADS_SEQ)
        check(ck[bb:bb + 1, :, hh:hh + 1], expected_ckpt(sp_ref, one_s, 1, T, 1), tol, f"{what} ckpt", HEADS_SEQ)
        del sp_ref
        ref = oracle_mod.backward(*(one[n] for n in RWKVAB), one_s, d_o[bb:bb + 1, :, hh:hh + 1].cpu(),
                                  d_so[bb:bb + 1, hh:hh + 1].cpu())
        for n in NAMES:
            check(g[n][bb:bb + 1, :, hh:hh + 1], ref[n], TOL, f"{what} {n}", HEADS_SEQ)
        check(g["d_state_in"][bb:bb + 1, hh:hh + 1], ref["d_state_in"], TOL, f"{what} d_state_in", HEADS_STATE)


def _high_window(nbytes_each, count):
    """count fp32 views of nbytes_each bytes, all at device addresses whose low 32-bit word
    has bit 31 set (a lane read of such a word, taken as a signed int and widened, would
    turn the address into a wild one).  Returns (owner, views)."""
    need = count * (nbytes_each + 256)
    big = torch.empty(((1 << 32) + need) // 4 + 64, dtype=torch.float32, device="cuda")
    base = big.data_ptr()
    off = (0x80000000 - (base & 0xFFFFFFFF)) % (1 << 32)
    off = (off + 255) // 256 * 256
    views = []
    for j in range(count):
        o = off + j * (nbytes_each + 256)
        v = big[o // 4:o // 4 + nbytes_each // 4]
        assert (v.data_ptr() & 0xFFFFFFFF) >= 0x80000000
        views.append(v)
    return big, views


@pytest.mark.parametrize("H", [3, 129])
def test_backward_ckpt_outputs_at_high_addresses(K, H):
    # H = 3: two workgroups per head (atomic adds); H = 129: one (plain stores)
    B, T = 1, 37
    inp = synth.make_inputs(B, T, H, 64, seed=5000 + H, dtype="bf16", state_std=0.1)
    d = {n: inp[n].cuda() for n in RWKVAB}
    _, _, ck = K.wkv7_forward_ckpt(*(d[n] for n in RWKVAB), inp["state_in"].cuda())
    gen = torch.Generator(device="cuda").manual_seed(5001)
    d_o = torch.randn((B, T, H, 64), generator=gen, device="cuda")
    d_so = torch.randn((B, H, 64, 64), generator=gen, device="cuda")
    ref = K.wkv7_backward_ckpt(*(d[n] for n in RWKVAB), ck, d_o, d_so)
    n_seq = B * T * H * 64 * 4
    owner, views = _high_window(max(n_seq, B * H * 64 * 64 * 4), 7)
    grads = {n: views[j][:n_seq // 4].view(B, T, H, 64) for j, n in enumerate(NAMES)}
    grads["d_state_in"] = views[6][:B * H * 64 * 64].view(B, H, 64, 64)
    K.wkv7_backward_ckpt(*(d[n] for n in RWKVAB), ck, d_o, d_so, grads=grads)
    torch.cuda.synchronize()
    for n in NAMES + ("d_state_in",):
        assert torch.equal(grads[n], ref[n]), n
    del owner
