"""GPU parity: the HIP kernels (through the C ABI) against the fp64 CPU oracle.

Tolerances: 1e-5 with fp32 inputs and 2e-3 with bf16 inputs and an fp32
state, each applied three ways (tests/parity.py): relative L2 over the whole
tensor, relative L2 of every (batch, head), and every element within the
tolerance times its head's RMS.  Outputs compared are o, the
final state and, for the verify step, every per-position state.  Inputs come
from the shared seeded generator; expected values only from the oracle.
"""
import math

import numpy as np
import pytest
import torch

import synth
from parity import HEADS_SEQ, HEADS_STATE, check, rel_l2  # noqa: F401

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-3}


@pytest.fixture(scope="module")
def K():
    import rwkv_linear_attention_amd as m
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: GPU tests must run on an MI355X")
    m.lib()  # raises if the library is not built
    return m


def to_dev(inp):
    d = {n: inp[n].cuda() for n in ("r", "w", "k", "v", "a", "b")}
    d["state_in"] = None if inp["state_in"] is None else inp["state_in"].cuda()
    return d


def oracle_run(oracle_mod, inp, per_position=False):
    return oracle_mod.forward(inp["r"], inp["w"], inp["k"], inp["v"], inp["a"], inp["b"], inp["state_in"],
                              per_position=per_position)


def gpu_run(K, d, kernel, per_position=False, o_dtype=torch.float32, state_out=None):
    args = (d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], d["state_in"])
    if kernel == "forward":
        res = K.wkv7_forward(*args, o_dtype=o_dtype, state_out=state_out)
    else:
        res = K.wkv7_step(*args, per_position=per_position, o_dtype=o_dtype, state_out=state_out)
    torch.cuda.synchronize()
    return res


# --- unit level: both kernels on small shapes, ragged T ---------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 2, 5, 16, 63, 64, 65])
@pytest.mark.parametrize("kernel", ["step", "forward"])
def test_small_vs_oracle(K, oracle_mod, dtype, T, kernel):
    inp = synth.make_inputs(2, T, 3, 64, seed=1000 + T, dtype=dtype, state_std=0.1)
    o_ref, s_ref = oracle_run(oracle_mod, inp)
    o, s = gpu_run(K, to_dev(inp), kernel)
    check(o, o_ref, TOL[dtype], f"{kernel} {dtype} T={T} o", HEADS_SEQ)
    check(s, s_ref, TOL[dtype], f"{kernel} {dtype} T={T} state", HEADS_STATE)


@pytest.mark.parametrize("B,H", [(1, 2), (2, 64), (4, 64), (3, 50)])
@pytest.mark.parametrize("T", [17, 100, 300])
def test_forward_column_blocks_and_tails(K, oracle_mod, B, H, T):
    # B*H = 2, 128, 256, 150 exercise 4, 2, 1 and 2 column blocks per head
    inp = synth.make_inputs(B, T, H, 64, seed=2000 + B * H + T, dtype="bf16", state_std=0.1)
    o_ref, s_ref = oracle_run(oracle_mod, inp)
    o, s = gpu_run(K, to_dev(inp), "forward")
    check(o, o_ref, TOL["bf16"], f"forward B={B} H={H} T={T} o", HEADS_SEQ)
    check(s, s_ref, TOL["bf16"], f"forward B={B} H={H} T={T} state", HEADS_STATE)


@pytest.mark.parametrize("B,H", [(2, 50), (3, 50)])
def test_forward_f32_inputs_column_blocks(K, oracle_mod, B, H):
    # fp32 inputs build the chunked kernel with three bf16 pieces per operand and a
    # shallower pipeline; B*H = 100 and 150 take 2 and 1 column blocks per head
    inp = synth.make_inputs(B, 41, H, 64, seed=2500 + B * H, dtype="f32", state_std=0.1)
    o_ref, s_ref = oracle_run(oracle_mod, inp)
    o, s = gpu_run(K, to_dev(inp), "forward")
    check(o, o_ref, TOL["f32"], f"forward f32 B={B} H={H} o", HEADS_SEQ)
    check(s, s_ref, TOL["f32"], f"forward f32 B={B} H={H} state", HEADS_STATE)


@pytest.mark.parametrize("kernel", ["step", "forward"])
def test_zero_state_in_is_null_state(K, oracle_mod, kernel):
    inp = synth.make_inputs(2, 40, 4, 64, seed=31, dtype="bf16", state_std=0.0)
    assert inp["state_in"] is None
    o_ref, s_ref = oracle_run(oracle_mod, inp)
    o, s = gpu_run(K, to_dev(inp), kernel)
    check(o, o_ref, TOL["bf16"], "o", HEADS_SEQ)
    check(s, s_ref, TOL["bf16"], "state", HEADS_STATE)


@pytest.mark.parametrize("kernel", ["step", "forward"])
def test_in_place_state(K, oracle_mod, kernel):
    inp = synth.make_inputs(2, 33, 4, 64, seed=32, dtype="bf16", state_std=0.1)
    o_ref, s_ref = oracle_run(oracle_mod, inp)
    d = to_dev(inp)
    st = d["state_in"]
    o, s = gpu_run(K, d, kernel, state_out=st)
    assert s.data_ptr() == st.data_ptr()
    check(o, o_ref, TOL["bf16"], "o", HEADS_SEQ)
    check(st, s_ref, TOL["bf16"], "state (in place)", HEADS_STATE)


@pytest.mark.parametrize("kernel", ["step", "forward"])
def test_empty_sequence(K, kernel):
    inp = synth.make_inputs(2, 0, 3, 64, seed=33, dtype="bf16", state_std=0.1)
    d = to_dev(inp)
    o, s = gpu_run(K, d, kernel)
    assert o.shape == (2, 0, 3, 64)
    assert torch.equal(s, d["state_in"])
    d["state_in"] = None
    _, s0 = gpu_run(K, d, kernel)
    assert not torch.any(s0)


@pytest.mark.parametrize("kernel", ["step", "forward"])
def test_bf16_output_rounding(K, oracle_mod, kernel):
    # o_dtype=bf16 must be the fp32 result rounded to nearest even, bit for bit
    inp = synth.make_inputs(2, 24, 3, 64, seed=34, dtype="bf16", state_std=0.1)
    d = to_dev(inp)
    o32, s32 = gpu_run(K, d, kernel)
    o16, s16 = gpu_run(K, d, kernel, o_dtype=torch.bfloat16)
    assert o16.dtype == torch.bfloat16
    assert torch.equal(s16, s32)
    expect = o32.to(torch.bfloat16)
    differ = int((o16.view(torch.int16) != expect.view(torch.int16)).sum())
    assert differ == 0, f"{differ} of {o16.numel()} bf16 outputs are not RNE of the fp32 output"
    o_ref, _ = oracle_run(oracle_mod, inp)
    # rounding o alone costs about 1.7e-3 relative L2, so bf16 outputs are held to 4e-3
    check(o16, o_ref, 4e-3, f"{kernel} bf16 o vs oracle", HEADS_SEQ, elem_rel=2.0 ** -8)


def test_per_position_states(K, oracle_mod):
    inp = synth.make_inputs(3, 6, 5, 64, seed=35, dtype="bf16", state_std=0.1)
    o_ref, s_ref, sp_ref = oracle_run(oracle_mod, inp, per_position=True)
    o, s, sp = gpu_run(K, to_dev(inp), "step", per_position=True)
    check(o, o_ref, TOL["bf16"], "o", HEADS_SEQ)
    check(s, s_ref, TOL["bf16"], "state", HEADS_STATE)
    check(sp, sp_ref, TOL["bf16"], "state_pos", HEADS_SEQ)
    assert torch.equal(sp[:, -1], s)


@pytest.mark.parametrize("wval", [0.0, 1e-3])
@pytest.mark.parametrize("kernel", ["step", "forward"])
def test_extreme_decays(K, oracle_mod, wval, kernel):
    # both kernels are exact for every decay in [0, 1]; the chunked kernel evaluates a
    # chunk that holds a decay below 2^-15 token by token
    inp = synth.make_inputs(2, 50, 3, 64, seed=36, dtype="f32", state_std=0.3)
    w = inp["w"].clone()
    w[:, ::3, :, ::2] = wval  # every third token, half the key channels
    inp["w"] = w
    o_ref, s_ref = oracle_run(oracle_mod, inp)
    o, s = gpu_run(K, to_dev(inp), kernel)
    check(o, o_ref, TOL["f32"], f"{kernel} w={wval} o", HEADS_SEQ)
    check(s, s_ref, TOL["f32"], f"{kernel} w={wval} state", HEADS_STATE)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,H", [(1, 2), (2, 64), (4, 64)])
def test_tiny_decay_chunks_among_ordinary_ones(K, oracle_mod, dtype, B, H):
    # Chunks 0, 3 and the last, partial one hold a decay below 2^-15 in a few (b, h, key)
    # entries (0, a denormal, 2^-15 just below); chunk 5 holds exactly 2^-15, which the
    # factored form still takes; the rest are ordinary.  B*H = 2, 128, 256 run 4, 2 and 1
    # column blocks per head.
    T = 16 * 7 + 5
    inp = synth.make_inputs(B, T, H, 64, seed=3900 + B * H, dtype=dtype, state_std=0.2)
    w = inp["w"].clone()
    # the largest value below 2^-15 in the input type
    below = (torch.nextafter(torch.tensor(2.0 ** -15), torch.tensor(0.0)) if dtype == "f32"
             else torch.tensor(2.0 ** -15 * (1 - 2.0 ** -8))).to(w.dtype)
    assert float(below) < 2.0 ** -15
    w[0, 3, 0, 5] = 0.0
    w[-1, 50, H - 1, 63] = 1e-40 if dtype == "f32" else 0.0
    w[:, 16 * 7 + 2, :, 9] = below
    w[0, 16 * 5 + 7, 0, :] = 2.0 ** -15
    inp["w"] = w
    o_ref, s_ref = oracle_run(oracle_mod, inp)
    o, s = gpu_run(K, to_dev(inp), "forward")
    check(o, o_ref, TOL[dtype], f"tiny decays {dtype} B={B} H={H} o", HEADS_SEQ)
    check(s, s_ref, TOL[dtype], f"tiny decays {dtype} B={B} H={H} state", HEADS_STATE)


def test_tiny_decays_variable_lengths(K, oracle_mod):
    # rows of their own lengths, with a zero decay in the last (partial) chunk of one row
    # and past the end of another (where it must not matter)
    B, T, H = 3, 60, 4
    inp = synth.make_inputs(B, T, H, 64, seed=3950, dtype="f32", state_std=0.2)
    w = inp["w"].clone()
    w[0, 40, 1, 7] = 0.0   # row 0 runs 45 tokens: inside its last chunk
    w[1, 50, 2, 3] = 0.0   # row 1 runs 33 tokens: past its end
    w[2, 1, 0, 0] = 0.0    # row 2 runs all 60
    inp["w"] = w
    lengths = [45, 33, 60]
    o_ref, s_ref = oracle_mod.forward_varlen(*[inp[n] for n in ("r", "w", "k", "v", "a", "b")], inp["state_in"],
                                             lengths)
    d = to_dev(inp)
    o, s = K.wkv7_forward(*[d[n] for n in ("r", "w", "k", "v", "a", "b")], d["state_in"], lengths=lengths)
    torch.cuda.synchronize()
    valid = (np.arange(T)[None, :] < np.asarray(lengths)[:, None])[:, :, None, None]
    og = o.double().cpu().numpy()
    check(np.where(valid, og, 0.0), np.where(valid, o_ref, 0.0), TOL["f32"], "varlen tiny decays o", HEADS_SEQ)
    check(s, s_ref, TOL["f32"], "varlen tiny decays state", HEADS_STATE)


@pytest.mark.parametrize("kernel", ["step", "forward"])
def test_deterministic(K, kernel):
    inp = synth.make_inputs(2, 70, 6, 64, seed=37, dtype="bf16", state_std=0.1)
    d = to_dev(inp)
    o1, s1 = gpu_run(K, d, kernel)
    o2, s2 = gpu_run(K, d, kernel)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


@pytest.mark.parametrize("kernel", ["step", "forward"])
def test_no_writes_outside_outputs(K, kernel):
    inp = synth.make_inputs(2, 37, 3, 64, seed=38, dtype="bf16", state_std=0.1)
    d = to_dev(inp)
    pad = 64
    n_o = 2 * 37 * 3 * 64
    n_s = 2 * 3 * 64 * 64
    obuf = torch.full((n_o + 2 * pad,), float("nan"), device="cuda")
    sbuf = torch.full((n_s + 2 * pad,), float("nan"), device="cuda")
    o = obuf[pad:pad + n_o].view(2, 37, 3, 64)
    s = sbuf[pad:pad + n_s].view(2, 3, 64, 64)
    args = (d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], d["state_in"])
    if kernel == "forward":
        K.wkv7_forward(*args, o=o, state_out=s)
    else:
        K.wkv7_step(*args, o=o, state_out=s)
    torch.cuda.synchronize()
    assert torch.isnan(obuf[:pad]).all() and torch.isnan(obuf[-pad:]).all()
    assert torch.isnan(sbuf[:pad]).all() and torch.isnan(sbuf[-pad:]).all()
    assert not torch.isnan(o).any() and not torch.isnan(s).any()


@pytest.mark.parametrize("which", ["r", "w", "k", "v", "a", "b", "state_in"])
@pytest.mark.parametrize("kernel", ["step", "forward"])
def test_every_input_matters(K, which, kernel):
    inp = synth.make_inputs(1, 20, 2, 64, seed=39, dtype="f32", state_std=0.1)
    d = to_dev(inp)
    o1, s1 = gpu_run(K, d, kernel)
    x = d[which].clone()
    x.view(-1)[123] += 0.5
    d[which] = x
    o2, s2 = gpu_run(K, d, kernel)
    assert not (torch.equal(o1, o2) and torch.equal(s1, s2))


def test_state_reset(K):
    st = torch.randn(4, 3, 64, 64, device="cuda")
    keep = st.clone()
    K.wkv7_state_reset(st, torch.tensor([1, 0, 0, 1], dtype=torch.uint8))
    torch.cuda.synchronize()
    assert not torch.any(st[0]) and not torch.any(st[3])
    assert torch.equal(st[1], keep[1]) and torch.equal(st[2], keep[2])
    K.wkv7_state_reset(st)
    torch.cuda.synchronize()
    assert not torch.any(st)


# --- the five workloads at full size --------------------------------------------

def test_workload0_tiny_f32_both_kernels(K, oracle_mod):
    inp = synth.workload_inputs(0)
    o_ref, s_ref = oracle_run(oracle_mod, inp)
    for kernel in ("forward", "step"):
        o, s = gpu_run(K, to_dev(inp), kernel)
        check(o, o_ref, TOL["f32"], f"workload 0 {kernel} o", HEADS_SEQ)
        check(s, s_ref, TOL["f32"], f"workload 0 {kernel} state", HEADS_STATE)


def test_workload1_decode(K, oracle_mod):
    inp = synth.workload_inputs(1)
    o_ref, s_ref = oracle_run(oracle_mod, inp)
    d = to_dev(inp)
    o, s = gpu_run(K, d, "step", state_out=d["state_in"])  # in place, as timed
    check(o, o_ref, TOL["bf16"], "workload 1 o", HEADS_SEQ)
    check(s, s_ref, TOL["bf16"], "workload 1 state", HEADS_STATE)


def test_workload4_verify_step(K, oracle_mod):
    inp = synth.workload_inputs(4)
    o_ref, s_ref, sp_ref = oracle_run(oracle_mod, inp, per_position=True)
    d = to_dev(inp)
    o, s, sp = gpu_run(K, d, "step", per_position=True, state_out=d["state_in"])
    check(o, o_ref, TOL["bf16"], "workload 4 o", HEADS_SEQ)
    check(s, s_ref, TOL["bf16"], "workload 4 state", HEADS_STATE)
    check(sp, sp_ref, TOL["bf16"], "workload 4 state_pos", HEADS_SEQ)


def test_workload2_prefill(K, oracle_mod):
    inp = synth.workload_inputs(2)
    d = to_dev(inp)
    # (i) first 512 tokens against the oracle
    head = {n: (x[:, :512].contiguous() if n != "state_in" else x) for n, x in inp.items()}
    o_ref, s_ref = oracle_run(oracle_mod, head)
    dh = to_dev(head)
    o, s = gpu_run(K, dh, "forward")
    check(o, o_ref, TOL["bf16"], "workload 2 first 512 o", HEADS_SEQ)
    check(s, s_ref, TOL["bf16"], "workload 2 first 512 state", HEADS_STATE)
    # (ii) full T against [0, T/2) then [T/2, T) with the state carried
    o_full, s_full = gpu_run(K, d, "forward")
    T = inp["r"].shape[1]
    h1 = {n: (x[:, :T // 2].contiguous() if n != "state_in" else x) for n, x in d.items()}
    h2 = {n: (x[:, T // 2:].contiguous() if n != "state_in" else x) for n, x in d.items()}
    o1, s1 = gpu_run(K, h1, "forward")
    h2["state_in"] = s1
    o2, s2 = gpu_run(K, h2, "forward")
    check(torch.cat([o1, o2], dim=1), o_full.double().cpu().numpy(), 1e-5, "workload 2 split-T o", HEADS_SEQ)
    check(s2, s_full.double().cpu().numpy(), 1e-5, "workload 2 split-T state", HEADS_STATE)
    # (iii) chunked kernel against the step kernel over the full sequence
    o_st, s_st = gpu_run(K, d, "step")
    check(o_full, o_st.double().cpu().numpy(), TOL["bf16"], "workload 2 chunked vs step o", HEADS_SEQ)
    check(s_full, s_st.double().cpu().numpy(), TOL["bf16"], "workload 2 chunked vs step state", HEADS_STATE)


def test_workload3_prefill_all_heads(K, workload3_oracle):
    # every one of the 256 heads over the full 8192 tokens against the oracle
    inp, o_ref, s_ref = workload3_oracle
    d = to_dev(inp)
    o, s = gpu_run(K, d, "forward")
    o, s = o.cpu(), s.cpu()
    del d
    check(o, o_ref, TOL["bf16"], "workload 3 o", HEADS_SEQ)
    check(s, s_ref, TOL["bf16"], "workload 3 state", HEADS_STATE)


@pytest.mark.parametrize("kernel", ["step", "forward"])
def test_nan_in_a_value_channel_stays_in_its_column(K, kernel):
    # Value channels evolve independently: a NaN in v[b, t, h, j] reaches o[b, t', h, j] for
    # t' >= t and nothing else -- no other column, head or batch row.  The step kernel keeps
    # every earlier token finite; the chunked kernel forms a chunk's outputs together (its
    # masked products multiply 0 by the NaN), so there only the chunks before stay finite.
    B, T, H, t_nan, j_nan = 2, 40, 3, 21, 5
    inp = synth.make_inputs(B, T, H, 64, seed=123, dtype="bf16", state_std=0.1)
    inp["v"][1, t_nan, 2, j_nan] = float("nan")
    o, s = gpu_run(K, to_dev(inp), kernel)
    o, s = o.cpu(), s.cpu()
    bad = torch.isnan(o)
    assert bad[1, t_nan:, 2, j_nan].all(), "the NaN must reach every later output of its column"
    mask = torch.zeros_like(bad)
    first = t_nan if kernel == "step" else (t_nan // 16) * 16
    mask[1, first:, 2, j_nan] = True
    assert not (bad & ~mask).any(), "the NaN leaked out of its column, head or time range"
    assert torch.isnan(s[1, 2, :, j_nan]).all() and torch.isfinite(s[1, 2, :, :j_nan]).all()
    assert torch.isfinite(s[0]).all() and torch.isfinite(s[1, :2]).all()


# --- element offsets beyond 32 bits ------------------------------------------------
# Every (b, h) row of these inputs is one seeded head, with v scaled by a power of
# two c[b, h] = 2^((b H + h) % 8 - 4).  With a zero input state the recurrence is
# linear in v, and a power-of-two scale is exact in every floating-point step, so
# each head's o and state must equal c[b, h] times those of head (0, 0) bit for
# bit; an offset that wrapped at 32 bits would read a head of another scale.
# Head (0, 0) itself is checked against the oracle.

def _tiled_inputs(base, B, H):
    T = base["r"].shape[1]
    d = {}
    for n in ("r", "w", "k", "v", "a", "b"):
        x = torch.empty((B, T, H, 64), dtype=base[n].dtype, device="cuda")
        x.copy_(base[n][0, :, 0, :].cuda()[None, :, None, :].expand(B, T, H, 64))
        d[n] = x
    idx = torch.arange(B * H, device="cuda").view(B, H)
    c = torch.pow(2.0, (idx % 8 - 4).double()).float()
    d["v"].mul_(c.view(B, 1, H, 1).to(d["v"].dtype))
    d["state_in"] = None
    return d, c


@pytest.mark.parametrize("kernel,B,T,H", [("forward", 5, 65536, 256), ("step", 4100, 128, 128)])
def test_offsets_beyond_32_bits(K, oracle_mod, kernel, B, T, H):
    assert B * T * H * 64 > 2**32
    base = synth.make_inputs(1, T, 1, seed=11, dtype="bf16", state_std=0.0)
    d, c = _tiled_inputs(base, B, H)
    o, s = gpu_run(K, d, kernel)
    del d
    c0 = c[0, 0].item()
    o_ref, s_ref = oracle_run(oracle_mod, base)
    check(o[0:1, :, 0:1].cpu() / c0, o_ref, TOL["bf16"], f"{kernel} B={B} T={T} H={H} head (0, 0) o", HEADS_SEQ)
    check(s[0:1, 0:1].cpu() / c0, s_ref, TOL["bf16"], f"{kernel} B={B} T={T} H={H} head (0, 0) state", HEADS_STATE)
    o00, s00 = o[0, :, 0] / c0, s[0, 0] / c0
    for bb, hh in [(B // 2, H // 3), (B - 2, 7), (B - 1, H - 1)]:
        first = ((bb * T) * H + hh) * 64
        cb = c[bb, hh].item()
        assert torch.equal(o[bb, :, hh] / cb, o00), f"{kernel}: o of head ({bb}, {hh}) (offset {first}) differs"
        assert torch.equal(s[bb, hh] / cb, s00), f"{kernel}: state of head ({bb}, {hh}) differs"
        print(f"  head ({bb}, {hh}), first element offset {first}: o and state = {cb} x head (0, 0)", flush=True)
    del o, s
    torch.cuda.empty_cache()
