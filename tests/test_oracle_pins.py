"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test fixes the oracle to a value or property the pages or the mathematics
determine: a hand-worked example, closed forms of special cases (linear
attention, pure decay, projection / delta-rule recall), exact rational
arithmetic, a dense matrix brute force, the chunked-parallel form, split-T state
carry, linearity and value-column separability, and the zero / empty cases.
The gradients (``backward``) are pinned by central finite differences of the
forward oracle, the closed form of linear attention, and causality.
A dropped term, a wrong sign, a transposed state or an off-by-one in time
fails at least one of them.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import independent_routes as routes

HERE = os.path.dirname(os.path.abspath(__file__))


def _one_head(oracle_mod, r, w, k, v, a, b, S0, per_position=False):
    """Run the oracle on one head given [T,N] fp64 arrays."""
    ex = lambda x: np.asarray(x, np.float64)[None, :, None, :]
    s_in = None if S0 is None else np.asarray(S0, np.float64)[None, None]
    res = oracle_mod.forward(ex(r), ex(w), ex(k), ex(v), ex(a), ex(b), s_in,
                             per_position=per_position, f64_inputs=True)
    if per_position:
        o, s, sp = res
        return o[0, :, 0, :], s[0, 0], sp[0, :, 0]
    o, s = res
    return o[0, :, 0, :], s[0, 0]


def _rand_head(rng, T, N, w_lo=0.55, w_hi=1.0, s_std=0.3):
    r, k, v = (rng.standard_normal((T, N)) for _ in range(3))
    kk = k / np.linalg.norm(k, axis=1, keepdims=True)
    gate = 1 / (1 + np.exp(-rng.standard_normal((T, N))))
    a = -kk
    b = kk * gate
    w = rng.uniform(w_lo, w_hi, (T, N))
    S0 = rng.standard_normal((N, N)) * s_std
    return r, w, k, v, a, b, S0


def _rel(x, ref):
    n = np.linalg.norm(ref)
    return np.linalg.norm(x - ref) / (n if n > 0 else 1.0)


# --- hand-worked example -----------------------------------------------------

def _read_golden(name):
    vals = {}
    with open(os.path.join(HERE, "golden", name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *nums = line.split()
            vals[key] = np.array([float(Fraction(x)) for x in nums])
    return vals


def test_golden_handworked_n2_t2(oracle_mod):
    g = _read_golden("wkv7_n2_t2_handworked.txt")
    T, N = 2, 2
    sh = lambda x: x.reshape(T, N)
    o, s = _one_head(oracle_mod, sh(g["r"]), sh(g["w"]), sh(g["k"]), sh(g["v"]), sh(g["a"]),
                     sh(g["b"]), g["state_in"].reshape(N, N))
    assert np.array_equal(o, sh(g["expect_o"]))
    assert np.array_equal(s, g["expect_state_out"].reshape(N, N))


# --- I7: exact rational arithmetic on dyadic inputs ---------------------------

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_exact_rational_dyadic(oracle_mod, seed):
    rng = np.random.default_rng(100 + seed)
    T, N = 3, 3
    dy = lambda *shape: rng.integers(-8, 9, shape) / 8.0      # multiples of 1/8: exact in fp64
    r, k, v, a, b = dy(T, N), dy(T, N), dy(T, N), dy(T, N), dy(T, N)
    w = rng.integers(1, 9, (T, N)) / 8.0
    S0 = dy(N, N)
    o, s = _one_head(oracle_mod, r, w, k, v, a, b, S0)
    F = lambda x: [[Fraction(float(e)) for e in row] for row in x]
    eo, es = routes.exact_rational(F(r), F(w), F(k), F(v), F(a), F(b), F(S0))
    # every intermediate is a short dyadic rational, so fp64 is exact here
    assert np.array_equal(o, np.array([[float(e) for e in row] for row in eo]))
    assert np.array_equal(s, np.array([[float(e) for e in row] for row in es]))


# --- orientation: S = [K, V], write k (x) v, readout r^T S -----------------------

def test_orientation_unit_vectors(oracle_mod):
    N, T = 8, 1
    for (i, j) in [(0, 5), (6, 1), (3, 3)]:
        z = np.zeros((T, N))
        k = z.copy(); k[0, i] = 1.0
        v = z.copy(); v[0, j] = 1.0
        r = np.arange(1, N + 1, dtype=np.float64)[None]
        o, s = _one_head(oracle_mod, r, np.ones((T, N)), k, v, z, z, None)
        expect = np.zeros((N, N)); expect[i, j] = 1.0
        assert np.array_equal(s, expect)               # row = key channel, column = value channel
        eo = np.zeros(N); eo[j] = r[0, i]
        assert np.array_equal(o[0], eo)                # o = S^T r


# --- I1: linear attention ---------------------------------------------------------

def test_linear_attention_closed_form(oracle_mod):
    rng = np.random.default_rng(1)
    T, N = 37, 64
    r, k, v = (rng.standard_normal((T, N)) for _ in range(3))
    S0 = rng.standard_normal((N, N))
    z = np.zeros((T, N))
    o, s = _one_head(oracle_mod, r, np.ones((T, N)), k, v, z, z, S0)
    eo, es = routes.linear_attention(r, k, v, S0)
    assert _rel(o, eo) < 1e-13 and _rel(s, es) < 1e-13


# --- I2: pure decay -----------------------------------------------------------

def test_pure_decay_closed_form(oracle_mod):
    rng = np.random.default_rng(2)
    T, N = 20, 64
    r, k, v = (rng.standard_normal((T, N)) for _ in range(3))
    w = rng.uniform(0.3, 1.0, (T, N))
    S0 = rng.standard_normal((N, N))
    z = np.zeros((T, N))
    o, s = _one_head(oracle_mod, r, w, k, v, z, z, S0)
    eo, es = routes.pure_decay(r, w, k, v, S0)
    assert _rel(o, eo) < 1e-13 and _rel(s, es) < 1e-13


def test_pure_decay_constant_w_power(oracle_mod):
    rng = np.random.default_rng(3)
    T, N = 50, 16
    wrow = rng.uniform(0.5, 1.0, N)
    w = np.tile(wrow, (T, 1))
    S0 = rng.standard_normal((N, N))
    z = np.zeros((T, N))
    _, s = _one_head(oracle_mod, z, w, z, z, z, z, S0)
    expect = (wrow ** T)[:, None] * S0           # decay acts on rows (key channels)
    assert _rel(s, expect) < 1e-13


# --- I3: projection (w = 1, gate = 1, unit kk) ------------------------------------

def _unit(rng, N):
    x = rng.standard_normal(N)
    return x / np.linalg.norm(x)


def test_projection_idempotent(oracle_mod):
    rng = np.random.default_rng(4)
    N = 64
    kk = _unit(rng, N)
    S0 = rng.standard_normal((N, N))
    one = np.ones((1, N)); z = np.zeros((1, N))
    _, s1 = _one_head(oracle_mod, z, one, z, z, -kk[None], kk[None], S0)
    z2 = np.zeros((2, N))
    _, s2 = _one_head(oracle_mod, z2, np.ones((2, N)), z2, z2, np.tile(-kk, (2, 1)),
                      np.tile(kk, (2, 1)), S0)
    P = np.eye(N) - np.outer(kk, kk)
    assert _rel(s1, P @ S0) < 1e-13
    assert _rel(s2, s1) < 1e-13                  # P^2 = P


def test_delta_rule_recall(oracle_mod):
    # S' = (I - kk kk^T) S + kk v^T  =>  kk^T S' = v^T, so reading with r = kk returns v.
    rng = np.random.default_rng(5)
    N = 64
    kk = _unit(rng, N)
    v = rng.standard_normal(N)
    S0 = rng.standard_normal((N, N))
    o, _ = _one_head(oracle_mod, kk[None], np.ones((1, N)), kk[None], v[None], -kk[None], kk[None], S0)
    assert np.max(np.abs(o[0] - v)) < 1e-12


@pytest.mark.parametrize("g", [0.0, 0.3, 0.7, 1.0])
def test_projection_contracts(oracle_mod, g):
    rng = np.random.default_rng(6)
    N = 64
    kk = _unit(rng, N)
    S0 = rng.standard_normal((N, N))
    z = np.zeros((1, N))
    _, s = _one_head(oracle_mod, z, np.ones((1, N)), z, z, -kk[None], g * kk[None], S0)
    assert np.linalg.norm(s) <= np.linalg.norm(S0) * (1 + 1e-14)
    assert _rel(s, (np.eye(N) - g * np.outer(kk, kk)) @ S0) < 1e-13


# --- I6: dense brute force -----------------------------------------------------

@pytest.mark.parametrize("N,T", [(2, 8), (4, 7), (64, 8)])
def test_dense_bruteforce(oracle_mod, N, T):
    rng = np.random.default_rng(7 + N)
    r, w, k, v, a, b, S0 = _rand_head(rng, T, N, w_lo=0.0, w_hi=1.0)
    # independent a and b (not tied to kk) so the rank-1 term is general
    a = rng.standard_normal((T, N)) * 0.3
    b = rng.standard_normal((T, N)) * 0.3
    o, s, sp = _one_head(oracle_mod, r, w, k, v, a, b, S0, per_position=True)
    eo, es, estates = routes.dense_bruteforce(r, w, k, v, a, b, S0)
    assert _rel(o, eo) < 1e-13 and _rel(s, es) < 1e-13 and _rel(sp, estates) < 1e-13


# --- I5: step form == chunked-parallel form -----------------------------------------

@pytest.mark.parametrize("C", [1, 3, 16, 64, 100])
def test_chunk_form_equals_loop(oracle_mod, C):
    rng = np.random.default_rng(8)
    T, N = 100, 64
    r, w, k, v, a, b, S0 = _rand_head(rng, T, N)
    o, s = _one_head(oracle_mod, r, w, k, v, a, b, S0)
    eo, es = routes.chunk_form(r, w, k, v, a, b, S0, C)
    assert _rel(o, eo) < 1e-12 and _rel(s, es) < 1e-12


# --- I4: split-T state carry is bit-exact ----------------------------------------

@pytest.mark.parametrize("split", [0, 1, 17, 33, 34])
def test_split_T_bit_exact(oracle_mod, split):
    rng = np.random.default_rng(9)
    B, T, H, N = 2, 34, 3, 64
    ins = [rng.standard_normal((B, T, H, N)).astype(np.float32) for _ in range(6)]
    ins[1] = rng.uniform(0.55, 1.0, (B, T, H, N)).astype(np.float32)
    S0 = rng.standard_normal((B, H, N, N)) * 0.1
    o, s = oracle_mod.forward(*ins, S0)
    o1, s1 = oracle_mod.forward(*[x[:, :split] for x in ins], S0)
    o2, s2 = oracle_mod.forward(*[x[:, split:] for x in ins], s1)
    assert np.array_equal(np.concatenate([o1, o2], axis=1), o)
    assert np.array_equal(s2, s)


def test_per_position_states_match_prefixes(oracle_mod):
    rng = np.random.default_rng(10)
    B, T, H, N = 2, 5, 3, 64
    ins = [rng.standard_normal((B, T, H, N)).astype(np.float32) for _ in range(6)]
    S0 = rng.standard_normal((B, H, N, N)) * 0.1
    o, s, sp = oracle_mod.forward(*ins, S0, per_position=True)
    assert np.array_equal(sp[:, T - 1], s)
    for t in range(T):
        _, st = oracle_mod.forward(*[x[:, :t + 1] for x in ins], S0)
        assert np.array_equal(sp[:, t], st)


# --- I8: linearity in (v, S0) and value-column separability ---------------------------

def test_linearity_in_v_and_state(oracle_mod):
    rng = np.random.default_rng(11)
    T, N = 12, 64
    r, w, k, v1, a, b, S1 = _rand_head(rng, T, N)
    v2 = rng.standard_normal((T, N))
    S2 = rng.standard_normal((N, N))
    al, be = 0.75, -1.5
    o1, s1 = _one_head(oracle_mod, r, w, k, v1, a, b, S1)
    o2, s2 = _one_head(oracle_mod, r, w, k, v2, a, b, S2)
    o3, s3 = _one_head(oracle_mod, r, w, k, al * v1 + be * v2, a, b, al * S1 + be * S2)
    assert _rel(o3, al * o1 + be * o2) < 1e-12 and _rel(s3, al * s1 + be * s2) < 1e-12


def test_value_column_permutation(oracle_mod):
    rng = np.random.default_rng(12)
    T, N = 12, 64
    r, w, k, v, a, b, S0 = _rand_head(rng, T, N)
    p = rng.permutation(N)
    o, s = _one_head(oracle_mod, r, w, k, v, a, b, S0)
    op, sp = _one_head(oracle_mod, r, w, k, v[:, p], a, b, S0[:, p])
    assert np.array_equal(op, o[:, p]) and np.array_equal(sp, s[:, p])


# --- I9: zeros, empty, and sensitivity to every input -----------------------------------

def test_zero_values_and_state_give_zero(oracle_mod):
    rng = np.random.default_rng(13)
    T, N = 9, 64
    r, w, k, _, a, b, _ = _rand_head(rng, T, N)
    o, s = _one_head(oracle_mod, r, w, k, np.zeros((T, N)), a, b, np.zeros((N, N)))
    assert not np.any(o) and not np.any(s)


def test_empty_sequence_passes_state_through(oracle_mod):
    rng = np.random.default_rng(14)
    B, H, N = 2, 3, 64
    e = np.zeros((B, 0, H, N), np.float32)
    S0 = rng.standard_normal((B, H, N, N))
    o, s = oracle_mod.forward(e, e, e, e, e, e, S0)
    assert o.shape == (B, 0, H, N) and np.array_equal(s, S0)
    _, s0 = oracle_mod.forward(e, e, e, e, e, e, None)
    assert not np.any(s0)


@pytest.mark.parametrize("which", ["r", "w", "k", "v", "a", "b", "S0"])
def test_every_input_matters(oracle_mod, which):
    rng = np.random.default_rng(15)
    T, N = 4, 64
    r, w, k, v, a, b, S0 = _rand_head(rng, T, N)
    args = dict(r=r, w=w, k=k, v=v, a=a, b=b, S0=S0)
    o, s = _one_head(oracle_mod, **args)
    x = args[which].copy()
    x.flat[rng.integers(x.size)] += 0.5
    args[which] = x
    o2, s2 = _one_head(oracle_mod, **args)
    changed = not np.array_equal(o, o2) or not np.array_equal(s, s2)
    assert changed


def test_varlen_rows_match_the_full_run(oracle_mod):
    # Each row of the variable-length pass against a different route: one run
    # over the whole padded sequence with per-position states.  By causality the
    # first L_b outputs agree and the state after L_b tokens is state_pos[b, L_b-1];
    # the same fp64 loop in the same order makes both bit-equal.
    import synth
    T = 23
    inp = synth.make_inputs(6, T, 2, seed=41, dtype="f32")
    lengths = [0, 1, 9, T, T + 5, -3]
    args = [inp[n] for n in ("r", "w", "k", "v", "a", "b")]
    o_full, _, s_pos = oracle_mod.forward(*args, inp["state_in"], per_position=True)
    o, s = oracle_mod.forward_varlen(*args, inp["state_in"], lengths)
    s_in = inp["state_in"].double().numpy()
    for bb, L in enumerate(lengths):
        L = min(max(L, 0), T)
        assert np.array_equal(o[bb, :L], o_full[bb, :L])
        assert np.isnan(o[bb, L:]).all()
        expect = s_in[bb] if L == 0 else s_pos[bb, L - 1]
        assert np.array_equal(s[bb], expect)


def test_state_commit_matches_prefix_runs(oracle_mod):
    # The commit against a different route: a separate run over the accepted
    # prefix of each row (bit-equal: the same loop in the same order).
    import synth
    T = 6
    inp = synth.make_inputs(7, T, 3, seed=43, dtype="f32")
    args = [inp[n] for n in ("r", "w", "k", "v", "a", "b")]
    _, _, s_pos = oracle_mod.forward(*args, inp["state_in"], per_position=True)
    accepted = [0, 1, 2, 5, T, T + 1, -1]
    before = np.full((7, 3, 64, 64), 7.25)
    got = oracle_mod.state_commit(s_pos, accepted, inp["state_in"], before)
    s_in = inp["state_in"].double().numpy()
    for bb, n in enumerate(accepted):
        if 1 <= n <= T:
            rows = [x[bb:bb + 1, :n] for x in args]
            _, s_ref = oracle_mod.forward(*rows, inp["state_in"][bb:bb + 1])
            assert np.array_equal(got[bb], s_ref[0])
        elif n == 0:
            assert np.array_equal(got[bb], s_in[bb])
        else:
            assert np.array_equal(got[bb], before[bb])


def _tail_inputs(seed, B=2, T=3, H=2, N=64):
    rng = np.random.default_rng(seed)
    o, r, k, v = (rng.standard_normal((B, T, H, N)) for _ in range(4))
    g = 1 / (1 + np.exp(-rng.standard_normal((B, T, H, N))))
    r_k = rng.standard_normal((H, N)) * 0.1
    ln_w = 1 + 0.1 * rng.standard_normal((H, N))
    ln_b = 0.1 * rng.standard_normal((H, N))
    return o, r, k, v, g, r_k, ln_w, ln_b


def test_tail_group_norm_moments(oracle_mod):
    # unit affine, no bonus, open gate: every (b,t,h) row has mean 0 and variance
    # var/(var+eps) (closed form of the normalisation)
    o, r, k, v, g, r_k, ln_w, ln_b = _tail_inputs(71)
    eps = 0.3
    x = oracle_mod.tmix_tail(o, r, k, v, np.ones_like(g), np.zeros_like(r_k), np.ones_like(ln_w),
                             np.zeros_like(ln_b), eps)
    var = o.var(axis=-1)
    np.testing.assert_allclose(x.mean(axis=-1), 0.0, atol=1e-12)
    np.testing.assert_allclose(x.var(axis=-1), var / (var + eps), rtol=1e-12)


def test_tail_constant_row_leaves_bias_and_bonus(oracle_mod):
    # a constant o row normalises to 0: x = (ln_b + bonus * v) * g, bonus by hand
    o, r, k, v, g, r_k, ln_w, ln_b = _tail_inputs(72)
    o[:] = 2.5
    x = oracle_mod.tmix_tail(o, r, k, v, g, r_k, ln_w, ln_b, 1e-3)
    for bb in range(o.shape[0]):
        for t in range(o.shape[1]):
            for h in range(o.shape[2]):
                bonus = sum(r[bb, t, h, i] * k[bb, t, h, i] * r_k[h, i] for i in range(o.shape[3]))
                expect = (ln_b[h] + bonus * v[bb, t, h]) * g[bb, t, h]
                np.testing.assert_allclose(x[bb, t, h], expect, rtol=1e-12, atol=1e-14)


def test_tail_gate_and_head_parameters(oracle_mod):
    # the gate scales elementwise; each head uses its own r_k / ln_w / ln_b row
    o, r, k, v, g, r_k, ln_w, ln_b = _tail_inputs(73)
    x1 = oracle_mod.tmix_tail(o, r, k, v, np.ones_like(g), r_k, ln_w, ln_b, 1e-4)
    xg = oracle_mod.tmix_tail(o, r, k, v, g, r_k, ln_w, ln_b, 1e-4)
    np.testing.assert_allclose(xg, x1 * g, rtol=1e-13)
    ln_b2 = ln_b.copy()
    ln_b2[1] += 1.0
    x2 = oracle_mod.tmix_tail(o, r, k, v, g, r_k, ln_w, ln_b2, 1e-4)
    np.testing.assert_allclose(x2[:, :, 0], xg[:, :, 0], rtol=0, atol=0)
    np.testing.assert_allclose(x2[:, :, 1], xg[:, :, 1] + g[:, :, 1], rtol=1e-12)


def test_tail_affine_scale_per_head_and_channel(oracle_mod):
    # With no shift (ln_b = 0), no bonus (r_k = 0) and an open gate, the affine
    # scale multiplies the normalised row channel by channel: x(ln_w) equals
    # ln_w[h, j] times x(ones), whose moments the first tail pin fixes.  Every
    # (head, channel) scale differs and none is 1, so a dropped scale, one taken
    # from another head or channel, or one applied before the normalisation
    # (which would cancel it) fails here.
    rng = np.random.default_rng(74)
    o, r, k, v, g, r_k, _, _ = _tail_inputs(74, B=2, T=3, H=3)
    H, N = r_k.shape
    ln_w = 0.5 + rng.permutation(H * N).reshape(H, N) / (H * N)   # all distinct, in [0.5, 1.5)
    zb, zk, one = np.zeros((H, N)), np.zeros((H, N)), np.ones_like(g)
    base = oracle_mod.tmix_tail(o, r, k, v, one, zk, np.ones((H, N)), zb, 0.2)
    x = oracle_mod.tmix_tail(o, r, k, v, one, zk, ln_w, zb, 0.2)
    np.testing.assert_allclose(x, base * ln_w[None, None], rtol=1e-13, atol=0)
    # scaling one (head, channel) entry changes that channel of that head only, by that factor
    ln_w2 = ln_w.copy()
    ln_w2[1, 5] *= 3.0
    x2 = oracle_mod.tmix_tail(o, r, k, v, one, zk, ln_w2, zb, 0.2)
    changed = x2 != x
    assert changed[:, :, 1, 5].all()
    changed[:, :, 1, 5] = False
    assert not changed.any()
    np.testing.assert_allclose(x2[:, :, 1, 5], 3.0 * x[:, :, 1, 5], rtol=1e-14)


# --- the backward pass (gradients of the recurrence) ----------------------------

def _loss_and_grads(oracle_mod, x, s0, go, gs):
    """L = sum(o * go) + sum(S_T * gs) through the forward oracle, and the adjoint."""
    def L(xx, s):
        o, st = oracle_mod.forward(*(xx[n] for n in "rwkvab"), s, f64_inputs=True)
        return float((o * go).sum() + (st * gs).sum())
    g = oracle_mod.backward(*(x[n] for n in "rwkvab"), s0, go, gs)
    return L, g


def _rand_inputs(rng, B, T, H, N):
    x = {n: rng.standard_normal((B, T, H, N)) for n in "rkv"}
    kk = x["k"] / np.linalg.norm(x["k"], axis=-1, keepdims=True)
    x["a"] = -kk
    x["b"] = kk / (1 + np.exp(-rng.standard_normal((B, T, H, N))))
    x["w"] = np.exp(-0.6065306597 / (1 + np.exp(-rng.standard_normal((B, T, H, N)))))
    return x


@pytest.mark.parametrize("B,T,H", [(1, 9, 1), (2, 5, 3)])
def test_backward_matches_finite_differences(oracle_mod, B, T, H):
    # central differences of the (separately pinned) forward oracle along random
    # directions, one per input; fp64 makes them good to ~1e-8
    rng = np.random.default_rng(40 + T)
    N = 64
    x = _rand_inputs(rng, B, T, H, N)
    s0 = 0.2 * rng.standard_normal((B, H, N, N))
    go = rng.standard_normal((B, T, H, N))
    gs = rng.standard_normal((B, H, N, N))
    L, g = _loss_and_grads(oracle_mod, x, s0, go, gs)
    eps = 1e-6
    for n in "rwkvab":
        u = rng.standard_normal((B, T, H, N))
        xp, xm = dict(x), dict(x)
        xp[n], xm[n] = x[n] + eps * u, x[n] - eps * u
        fd = (L(xp, s0) - L(xm, s0)) / (2 * eps)
        an = float((g["d" + n] * u).sum())
        assert abs(fd - an) <= 1e-6 * max(abs(an), 1.0), (n, fd, an)
    u = rng.standard_normal((B, H, N, N))
    fd = (L(x, s0 + eps * u) - L(x, s0 - eps * u)) / (2 * eps)
    an = float((g["d_state_in"] * u).sum())
    assert abs(fd - an) <= 1e-6 * max(abs(an), 1.0), ("state_in", fd, an)


def test_backward_linear_attention_closed_form(oracle_mod):
    # a = b = 0, w = 1: S_t = S_0 + sum_{s<=t} k_s v_s^T, and with
    # G_t = GS + sum_{t'>=t} r_t' do_t'^T the gradients are
    # dr_t = S_t do_t, dk_t = G_t v_t, dv_t = G_t^T k_t, dw_t = rowsum(G_t * S_{t-1}),
    # and d_state_in = G_0
    rng = np.random.default_rng(44)
    T, N = 11, 64
    r, k, v, do = (rng.standard_normal((T, N)) for _ in range(4))
    S0 = rng.standard_normal((N, N))
    GS = rng.standard_normal((N, N))
    z = np.zeros((T, N))
    ex = lambda m: m[None, :, None, :]
    g = oracle_mod.backward(ex(r), ex(np.ones((T, N))), ex(k), ex(v), ex(z), ex(z), S0[None, None],
                            ex(do), GS[None, None])
    S = [S0]
    for t in range(T):
        S.append(S[-1] + np.outer(k[t], v[t]))
    G = [GS + sum(np.outer(r[u], do[u]) for u in range(t, T)) for t in range(T)]
    get = lambda n: g[n][0, :, 0, :]
    assert _rel(get("dr"), np.array([S[t + 1] @ do[t] for t in range(T)])) < 1e-12
    assert _rel(get("dk"), np.array([G[t] @ v[t] for t in range(T)])) < 1e-12
    assert _rel(get("dv"), np.array([G[t].T @ k[t] for t in range(T)])) < 1e-12
    assert _rel(get("dw"), np.array([(G[t] * S[t]).sum(axis=1) for t in range(T)])) < 1e-12
    assert _rel(g["d_state_in"][0, 0], G[0]) < 1e-12
    # a = b = 0 still has gradients: db_t = G_t S_{t-1}^T a_t = 0 and da_t = S_{t-1} G_t^T b_t = 0
    assert not np.any(get("da")) and not np.any(get("db"))


def test_backward_is_causal(oracle_mod):
    # with no gradient after token t0 (and none on the final state), every input
    # gradient after t0 is zero, and those up to t0 do not change
    rng = np.random.default_rng(45)
    B, T, H, N, t0 = 1, 8, 2, 64, 4
    x = _rand_inputs(rng, B, T, H, N)
    s0 = 0.2 * rng.standard_normal((B, H, N, N))
    go = rng.standard_normal((B, T, H, N))
    go[:, t0 + 1:] = 0.0
    g = oracle_mod.backward(*(x[n] for n in "rwkvab"), s0, go, None)
    short = {n: x[n][:, :t0 + 1] for n in x}
    gs = oracle_mod.backward(*(short[n] for n in "rwkvab"), s0, go[:, :t0 + 1], None)
    for n in ("dr", "dw", "dk", "dv", "da", "db"):
        assert not np.any(g[n][:, t0 + 1:]), n
        assert _rel(g[n][:, :t0 + 1], gs[n]) < 1e-13, n
    assert _rel(g["d_state_in"], gs["d_state_in"]) < 1e-13


def _chunk_route(oracle_mod, r, w, k, v, a, b, S0, do, GS, dtype, C=16):
    """The gradients by another route: the state-free gradient chain gives each chunk's
    end gradient, and the chunk-form adjoint (tests/independent_routes.py) each chunk's
    gradients from the state entering it (the oracle's per-position states) and that end
    gradient.  Inputs one head, [T, N] fp64; the chunk algebra runs in ``dtype``."""
    T, N = r.shape
    _, _, sp = _one_head(oracle_mod, r, w, k, v, a, b, S0, per_position=True)
    ends, d_state_in = routes.g_chain(r, w, a, b, do, GS, C)
    out = {n: np.zeros((T, N)) for n in ("dr", "dw", "dk", "dv", "da", "db")}
    for c in range(-(-T // C)):
        t0, t1 = c * C, min(T, (c + 1) * C)
        s_enter = S0 if c == 0 else sp[t0 - 1]
        cast = lambda x: np.asarray(x, dtype)
        g = routes.chunk_adjoint(*(cast(x[t0:t1]) for x in (r, w, k, v, a, b)), cast(s_enter),
                                 cast(do[t0:t1]), cast(ends[c]))
        for n in out:
            out[n][t0:t1] = g[n]
    return out, d_state_in


@pytest.mark.parametrize("T,tiny", [(37, False), (40, True)])
def test_backward_matches_chunk_form_route(oracle_mod, T, tiny):
    # every gradient of the oracle's adjoint loop against the chunk-form route in fp64;
    # with tiny decays (2^-14 .. 2^-10 on some tokens, above the exact-path threshold)
    # the direct decay gradient keeps its accuracy where a log-decay form would not
    rng = np.random.default_rng(46 + T)
    N = 64
    x = _rand_inputs(rng, 1, T, 1, N)
    if tiny:
        x["w"][0, 18:22, 0, :7] = 2.0 ** rng.uniform(-14, -10, (4, 7))
    h = {n: x[n][0, :, 0, :] for n in "rwkvab"}
    S0 = 0.2 * rng.standard_normal((N, N))
    do = rng.standard_normal((T, N))
    GS = rng.standard_normal((N, N))
    ex = lambda m: m[None, :, None, :]
    g = oracle_mod.backward(*(ex(h[n]) for n in "rwkvab"), S0[None, None], ex(do), GS[None, None])
    route, dsi = _chunk_route(oracle_mod, *(h[n] for n in "rwkvab"), S0, do, GS, np.float64)
    for n in route:
        assert _rel(route[n], g[n][0, :, 0, :]) < 1e-11, n
        # per token and key, against the row's scale: no element hides under the norm
        scale = np.abs(g[n][0, :, 0, :]).max(axis=1, keepdims=True) + 1e-300
        assert np.max(np.abs(route[n] - g[n][0, :, 0, :]) / scale) < 1e-9, n
    assert _rel(dsi, g["d_state_in"][0, 0]) < 1e-12
    # the same algebra in fp32 stays within the kernels' fp32 bar (1e-5)
    r32, _ = _chunk_route(oracle_mod, *(h[n] for n in "rwkvab"), S0, do, GS, np.float32)
    for n in r32:
        assert _rel(r32[n], g[n][0, :, 0, :]) < 1e-5, n
