"""GPU parity of the serving-path entry points against the fp64 oracle:
right-padded rows of their own lengths (wkv7_forward_varlen) and the commit of
a speculative verify step (wkv7_state_commit)."""
import numpy as np
import pytest
import torch

import synth
from parity import HEADS_SEQ, HEADS_STATE, check
from test_gpu_parity import K, TOL, to_dev  # noqa: F401  (K is a fixture)

pytestmark = pytest.mark.gpu

NAMES = ("r", "w", "k", "v", "a", "b")


def _lengths(B, T):
    base = [0, 1, T // 2 + 1, T, T + 7, 3, max(T - 1, 0), T // 3]
    return [base[i % len(base)] for i in range(B)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,H", [(3, 1, 2), (5, 6, 3), (5, 40, 3), (4, 40, 64), (3, 100, 50)])
def test_forward_varlen(K, oracle_mod, dtype, B, T, H):
    # T < 9 runs the step kernel, longer T the chunked one (J = 4, 1 and 2 column blocks)
    inp = synth.make_inputs(B, T, H, 64, seed=5000 + 7 * T + H, dtype=dtype, state_std=0.1)
    lengths = _lengths(B, T)
    print(f"  varlen {dtype} B={B} T={T} H={H} lengths={lengths}", flush=True)
    d = to_dev(inp)
    sentinel = 1234.5
    o = torch.full((B, T, H, 64), sentinel, device="cuda")
    o, s = K.wkv7_forward(*[d[n] for n in NAMES], d["state_in"], o=o, lengths=lengths)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_mod.forward_varlen(*[inp[n] for n in NAMES], inp["state_in"], lengths)
    L = np.clip(np.asarray(lengths), 0, T)
    valid = np.arange(T)[None, :] < L[:, None]                       # [B, T]
    og = o.double().cpu().numpy()
    # per head over each row's own tokens (the rest set to zero on both sides)
    m = valid[:, :, None, None]
    check(np.where(m, og, 0.0), np.where(m, o_ref, 0.0), TOL[dtype], "o (valid tokens)", HEADS_SEQ)
    assert (og[~valid] == sentinel).all(), "o past a row's length must be left untouched"
    check(s, s_ref, TOL[dtype], "state_out", HEADS_STATE)
    for bb in np.nonzero(L == 0)[0]:
        assert torch.equal(s[bb], d["state_in"][bb]), "an empty row passes its state through"


def test_forward_varlen_full_lengths_equal_forward(K):
    # lengths of T on every row: the same kernels, the same results, bit for bit
    inp = synth.make_inputs(3, 50, 5, 64, seed=77, dtype="bf16", state_std=0.1)
    d = to_dev(inp)
    args = [d[n] for n in NAMES]
    o1, s1 = K.wkv7_forward(*args, d["state_in"])
    o2, s2 = K.wkv7_forward(*args, d["state_in"], lengths=[50, 50, 50])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_state_commit(K, oracle_mod):
    B, T, H = 7, 5, 3
    inp = synth.make_inputs(B, T, H, 64, seed=61, dtype="bf16", state_std=0.1)
    d = to_dev(inp)
    _, _, sp = K.wkv7_step(*[d[n] for n in NAMES], d["state_in"], per_position=True)
    accepted = [0, 1, 2, 4, 5, 6, -1]
    before = torch.full((B, H, 64, 64), 3.5, device="cuda")
    got = K.wkv7_state_commit(sp, accepted, d["state_in"], state_out=before.clone())
    torch.cuda.synchronize()
    # a copy: bit-exact against the step's own per-position states
    for bb, n in enumerate(accepted):
        if 1 <= n <= T:
            assert torch.equal(got[bb], sp[bb, n - 1])
        elif n == 0:
            assert torch.equal(got[bb], d["state_in"][bb])
        else:
            assert torch.equal(got[bb], before[bb])
    # and against the oracle's commit of its own per-position states
    _, _, sp_ref = oracle_mod.forward(*[inp[n] for n in NAMES], inp["state_in"], per_position=True)
    ref = oracle_mod.state_commit(sp_ref, accepted, inp["state_in"], before.cpu())
    check(got, ref, TOL["bf16"], "committed state", HEADS_STATE)
    # in place over the state the step started from
    st = d["state_in"].clone()
    K.wkv7_state_commit(sp, accepted, st, state_out=st)
    torch.cuda.synchronize()
    for bb, n in enumerate(accepted):
        expect = sp[bb, n - 1] if 1 <= n <= T else d["state_in"][bb]
        assert torch.equal(st[bb], expect)
    # no state_in: an accepted count of 0 gives the zero state
    z = K.wkv7_state_commit(sp, [0] * B)
    torch.cuda.synchronize()
    assert not torch.any(z)


def test_bf16_output_accuracy_workload3(K, workload3_oracle):
    # The cost of a bf16 o (the o_dtype option) on the prefill workload, every head over
    # the full sequence; it stays inside the bf16-input tolerance (each element within
    # half a bf16 ulp of its own plus the tolerance times its head's RMS).
    inp, o_ref, _ = workload3_oracle
    d = to_dev(inp)
    o16, _ = K.wkv7_forward(*[d[n] for n in NAMES], d["state_in"], o_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    o16 = o16.float().cpu()
    del d
    check(o16, o_ref, TOL["bf16"], "workload 3 o bf16", HEADS_SEQ, elem_rel=2.0 ** -8)


def _tail_params(H, seed):
    g = torch.Generator().manual_seed(seed)
    r_k = (torch.randn((H, 64), generator=g) * 0.1).contiguous()
    ln_w = (1 + 0.1 * torch.randn((H, 64), generator=g)).contiguous()
    ln_b = (0.1 * torch.randn((H, 64), generator=g)).contiguous()
    return r_k, ln_w, ln_b


def _gate(shape, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.sigmoid(torch.randn(shape, generator=g))
    return x.to(torch.bfloat16 if dtype == "bf16" else torch.float32).contiguous()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("x_dtype", [torch.float32, torch.bfloat16])
def test_tmix_tail_vs_oracle(K, oracle_mod, dtype, x_dtype):
    B, T, H = 2, 37, 5
    inp = synth.make_inputs(B, T, H, 64, seed=91, dtype=dtype, state_std=0.1)
    gate = _gate((B, T, H, 64), dtype, 92)
    r_k, ln_w, ln_b = _tail_params(H, 93)
    eps = 64e-5
    o_ref, _ = oracle_mod.forward(*[inp[n] for n in NAMES], inp["state_in"])
    o_dev = torch.from_numpy(o_ref).float().cuda()           # the tail's own input: a fixed fp32 o
    d = to_dev(inp)
    x = K.wkv7_tmix_tail(o_dev, d["r"], d["k"], d["v"], gate.cuda(), r_k.cuda(), ln_w.cuda(), ln_b.cuda(), eps,
                         x_dtype=x_dtype)
    torch.cuda.synchronize()
    x_ref = oracle_mod.tmix_tail(o_dev.cpu(), inp["r"], inp["k"], inp["v"], gate, r_k, ln_w, ln_b, eps)
    # a bf16 x carries its own rounding (about 1.7e-3 relative L2): held to 4e-3 and half an ulp
    bf = x_dtype == torch.bfloat16
    check(x, x_ref, 4e-3 if bf else 1e-5, f"tail ({dtype} inputs, {x_dtype} x)", HEADS_SEQ,
          elem_rel=2.0 ** -8 if bf else 0.0)
    # in place over o
    o2 = o_dev.clone()
    K.wkv7_tmix_tail(o2, d["r"], d["k"], d["v"], gate.cuda(), r_k.cuda(), ln_w.cuda(), ln_b.cuda(), eps, x=o2)
    torch.cuda.synchronize()
    x32 = K.wkv7_tmix_tail(o_dev, d["r"], d["k"], d["v"], gate.cuda(), r_k.cuda(), ln_w.cuda(), ln_b.cuda(), eps)
    torch.cuda.synchronize()
    assert torch.equal(o2, x32)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 5])
def test_step_tail_vs_oracle(K, oracle_mod, dtype, T):
    B, H = 4, 6
    inp = synth.make_inputs(B, T, H, 64, seed=95 + T, dtype=dtype, state_std=0.1)
    gate = _gate((B, T, H, 64), dtype, 96)
    r_k, ln_w, ln_b = _tail_params(H, 97)
    eps = 64e-5
    d = to_dev(inp)
    x, s, sp = K.wkv7_step_tail(*[d[n] for n in NAMES], gate.cuda(), r_k.cuda(), ln_w.cuda(), ln_b.cuda(), eps,
                                d["state_in"], per_position=True)
    torch.cuda.synchronize()
    o_ref, s_ref, sp_ref = oracle_mod.forward(*[inp[n] for n in NAMES], inp["state_in"], per_position=True)
    x_ref = oracle_mod.tmix_tail(o_ref, inp["r"], inp["k"], inp["v"], gate, r_k, ln_w, ln_b, eps)
    check(x, x_ref, TOL[dtype], f"fused tail T={T} x", HEADS_SEQ)
    check(s, s_ref, TOL[dtype], f"fused tail T={T} state", HEADS_STATE)
    check(sp, sp_ref, TOL[dtype], f"fused tail T={T} state_pos", HEADS_SEQ)
    # the fused epilogue and the separate pass: the same arithmetic on the same o, summed in
    # another order (64 lanes against 16 lanes of four channels)
    o, _ = K.wkv7_step(*[d[n] for n in NAMES], d["state_in"])
    x2 = K.wkv7_tmix_tail(o, d["r"], d["k"], d["v"], gate.cuda(), r_k.cuda(), ln_w.cuda(), ln_b.cuda(), eps)
    torch.cuda.synchronize()
    check(x, x2.double().cpu().numpy(), 1e-6, "fused against separate tail", HEADS_SEQ)


def test_verify_without_separate_state_out(K, oracle_mod):
    # the verify step with per-position states only, then the commit: the same states
    B, T, H = 4, 5, 8
    inp = synth.make_inputs(B, T, H, 64, seed=99, dtype="bf16", state_std=0.1)
    d = to_dev(inp)
    args = [d[n] for n in NAMES]
    o1, s1, sp1 = K.wkv7_step(*args, d["state_in"], per_position=True)
    o2, none, sp2 = K.wkv7_step(*args, d["state_in"], per_position=True, write_state_out=False)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(o1, o2) and torch.equal(sp1, sp2)
    assert torch.equal(sp2[:, T - 1], s1)
    committed = K.wkv7_state_commit(sp2, [T] * B)
    torch.cuda.synchronize()
    assert torch.equal(committed, s1)


# --- the parallel pass with the time-mix tail fused (wkv7_forward_tail) -------------

def _forward_tail_case(K, oracle_mod, B, T, H, dtype, x_dtype, state_std, seed, w_zero=False):
    inp = synth.make_inputs(B, T, H, 64, seed=seed, dtype=dtype, state_std=state_std)
    if w_zero:  # a zero decay: its chunk takes the exact path
        w = inp["w"].clone()
        w[0, T // 2, 0, 3] = 0.0
        inp["w"] = w
    gate = _gate((B, T, H, 64), dtype, seed + 1)
    r_k, ln_w, ln_b = _tail_params(H, seed + 2)
    eps = 64e-5
    d = to_dev(inp)
    x, s = K.wkv7_forward_tail(*[d[n] for n in NAMES], gate.cuda(), r_k.cuda(), ln_w.cuda(), ln_b.cuda(), eps,
                               d["state_in"], x_dtype=x_dtype)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_mod.forward(*[inp[n] for n in NAMES], inp["state_in"])
    x_ref = oracle_mod.tmix_tail(o_ref, inp["r"], inp["k"], inp["v"], gate, r_k, ln_w, ln_b, eps)
    return inp, d, gate, (r_k, ln_w, ln_b, eps), x, s, x_ref, s_ref


@pytest.mark.parametrize("x_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("B,T,H,state_std", [(2, 40, 3, 0.1), (1, 17, 2, 0.0), (2, 100, 64, 0.1), (4, 37, 64, 0.1),
                                             (3, 8, 5, 0.1), (2, 9, 4, 0.1)])
def test_forward_tail_vs_oracle(K, oracle_mod, B, T, H, state_std, x_dtype):
    # bf16 inputs: one chunked kernel with the tail wave (T >= 9, every head count), or
    # the step kernel's fused tail (T < 9)
    *_, x, s, x_ref, s_ref = _forward_tail_case(K, oracle_mod, B, T, H, "bf16", x_dtype, state_std,
                                                seed=4000 + B * T + H)
    bf = x_dtype == torch.bfloat16
    check(x, x_ref, 4e-3 if bf else TOL["bf16"], f"forward tail B={B} T={T} H={H} x", HEADS_SEQ,
          elem_rel=2.0 ** -8 if bf else 0.0)
    check(s, s_ref, TOL["bf16"], f"forward tail B={B} T={T} H={H} state", HEADS_STATE)


@pytest.mark.parametrize("x_dtype", [torch.float32, torch.bfloat16])
def test_forward_tail_f32_inputs(K, oracle_mod, x_dtype):
    # fp32 inputs: the chunked kernel into x then the tail pass in place (fp32 x), or
    # the step kernel's fused tail (bf16 x)
    *_, x, s, x_ref, s_ref = _forward_tail_case(K, oracle_mod, 2, 41, 5, "f32", x_dtype, 0.1, seed=4100)
    bf = x_dtype == torch.bfloat16
    check(x, x_ref, 4e-3 if bf else TOL["f32"], "forward tail f32 x", HEADS_SEQ, elem_rel=2.0 ** -8 if bf else 0.0)
    check(s, s_ref, TOL["f32"], "forward tail f32 state", HEADS_STATE)


def test_forward_tail_exact_path_chunk(K, oracle_mod):
    *_, x, s, x_ref, s_ref = _forward_tail_case(K, oracle_mod, 2, 70, 8, "bf16", torch.float32, 0.1, seed=4200,
                                                w_zero=True)
    check(x, x_ref, TOL["bf16"], "forward tail, zero decay x", HEADS_SEQ)
    check(s, s_ref, TOL["bf16"], "forward tail, zero decay state", HEADS_STATE)


@pytest.mark.parametrize("x_dtype", [torch.float32, torch.bfloat16])
def test_forward_tail_equals_forward_then_tail_pass(K, x_dtype):
    # The fused kernel forms each chunk's o exactly as the plain chunked kernel does and
    # applies the same row arithmetic to it: bit for bit the two-launch result.
    B, T, H = 2, 75, 64
    inp = synth.make_inputs(B, T, H, 64, seed=4300, dtype="bf16", state_std=0.1)
    d = to_dev(inp)
    gate = _gate((B, T, H, 64), "bf16", 4301).cuda()
    prm = [t.cuda() for t in _tail_params(H, 4302)]
    x1, s1 = K.wkv7_forward_tail(*[d[n] for n in NAMES], gate, *prm, 64e-5, d["state_in"], x_dtype=x_dtype)
    o, s2 = K.wkv7_forward(*[d[n] for n in NAMES], d["state_in"])
    x2 = K.wkv7_tmix_tail(o, d["r"], d["k"], d["v"], gate, *prm, 64e-5, x_dtype=x_dtype)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)
    assert torch.equal(x1, x2), f"max |diff| {(x1.float() - x2.float()).abs().max().item():.3e}"


def test_forward_tail_workload3_all_heads(K, workload3_oracle, oracle_mod):
    # the 7.2B-shaped prefill with the tail fused, every head over the full sequence
    inp, o_ref, s_ref = workload3_oracle
    B, T, H = inp["r"].shape[:3]
    gate = _gate((B, T, H, 64), "bf16", 4400)
    r_k, ln_w, ln_b = _tail_params(H, 4401)
    d = to_dev(inp)
    x, s = K.wkv7_forward_tail(*[d[n] for n in NAMES], gate.cuda(), r_k.cuda(), ln_w.cuda(), ln_b.cuda(), 64e-5,
                               d["state_in"])
    torch.cuda.synchronize()
    x, s = x.cpu(), s.cpu()
    del d
    x_ref = oracle_mod.tmix_tail(o_ref, inp["r"], inp["k"], inp["v"], gate, r_k, ln_w, ln_b, 64e-5)
    check(x, x_ref, TOL["bf16"], "workload 3 fused tail x", HEADS_SEQ)
    check(s, s_ref, TOL["bf16"], "workload 3 fused tail state", HEADS_STATE)
