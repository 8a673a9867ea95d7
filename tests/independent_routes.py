"""Independent CPU routes to the WKV-7 result, used only to pin the oracle.

None of these shares code with the oracle (a C loop) or with the GPU library.
Each is a different way of writing down the same function:

* ``dense_bruteforce``: the step as a matrix product, with the transition
  A_t = diag(w_t) + b_t a_t^T formed explicitly and S_t = A_t S_{t-1} + k_t v_t^T
  (the Core AI RWKV-7 note, section 1: decay and rank-1 term both act on the
  state the step starts from; S = [K,V]; the write is k (x) v; o = r^T S).
* ``exact_rational``: the same matrix form in exact rational arithmetic
  (``fractions.Fraction``), for tiny dyadic inputs.
* ``chunk_form``: the chunked-parallel form of the recurrence.  Unrolling the
  step over a chunk of C tokens that starts from state S0 gives, with
  gamma_t = prod_{u<=t} w_u (per key channel),
      Z = (I - M_ab)^{-1} (A~ S0 + M_ak V)          (rows z_t = S_{t-1}^T a_t)
      O = R~ S0 + M_rb Z + M_rk V
      S_C = Gamma_C S0 + B^^T Z + K^^T V
  where A~[t] = a_t*gamma_{t-1}, R~[t] = r_t*gamma_t, B^[s] = b_s*gamma_C/gamma_s,
  K^[s] = k_s*gamma_C/gamma_s, and M_xy[t,s] = sum_i x~_t[i] y_s[i]/gamma_s[i]
  (strictly lower triangular for the a-rows, lower triangular including the
  diagonal for the r-rows).  The SwiftRWKV Inference guide states that the
  parallel pass and the recurrent pass compute the same function; this form is
  the algebra behind that statement, derived here, not printed on the pages.
* ``linear_attention`` and ``pure_decay``: closed forms of two special cases.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def dense_bruteforce(r, w, k, v, a, b, S0):
    """One head.  r..b: [T, N] fp64; S0: [N, N].  Returns (o [T,N], S_T, states [T,N,N])."""
    T, N = r.shape
    S = np.array(S0, dtype=np.float64, copy=True)
    o = np.zeros((T, N))
    states = np.zeros((T, N, N))
    for t in range(T):
        A = np.diag(w[t]) + np.outer(b[t], a[t])
        S = A @ S + np.outer(k[t], v[t])
        o[t] = S.T @ r[t]
        states[t] = S
    return o, S, states


def exact_rational(r, w, k, v, a, b, S0):
    """Same matrix form in exact rationals.  Inputs: nested lists of Fractions / ints."""
    T = len(r)
    N = len(r[0])
    S = [[Fraction(S0[i][j]) for j in range(N)] for i in range(N)]
    outs = []
    for t in range(T):
        A = [[(Fraction(w[t][i]) if i == m else Fraction(0)) + Fraction(b[t][i]) * Fraction(a[t][m])
              for m in range(N)] for i in range(N)]
        S = [[sum((A[i][m] * S[m][j] for m in range(N)), Fraction(0)) + Fraction(k[t][i]) * Fraction(v[t][j])
              for j in range(N)] for i in range(N)]
        outs.append([sum((Fraction(r[t][i]) * S[i][j] for i in range(N)), Fraction(0)) for j in range(N)])
    return outs, S


def chunk_form(r, w, k, v, a, b, S0, C):
    """One head, chunk length C (the last chunk may be shorter).  fp64 numpy."""
    T, N = r.shape
    S = np.array(S0, dtype=np.float64, copy=True)
    O = np.zeros((T, N))
    for c0 in range(0, T, C):
        sl = slice(c0, min(c0 + C, T))
        L = sl.stop - sl.start
        gam = np.cumprod(w[sl], axis=0)                      # gamma_t, t = 1..L
        gam_prev = np.vstack([np.ones((1, N)), gam[:-1]])     # gamma_{t-1}
        A_t = a[sl] * gam_prev
        R_t = r[sl] * gam
        B_inv = b[sl] / gam
        K_inv = k[sl] * (1.0 / gam)
        M_ab = np.tril(A_t @ B_inv.T, -1)
        M_ak = np.tril(A_t @ K_inv.T, -1)
        M_rb = np.tril(R_t @ B_inv.T, 0)
        M_rk = np.tril(R_t @ K_inv.T, 0)
        V = v[sl]
        Z = np.linalg.solve(np.eye(L) - M_ab, A_t @ S + M_ak @ V)
        O[sl] = R_t @ S + M_rb @ Z + M_rk @ V
        gC = gam[-1]
        S = gC[:, None] * S + (b[sl] * (gC / gam)).T @ Z + (k[sl] * (gC / gam)).T @ V
    return O, S


def linear_attention(r, k, v, S0):
    """Closed form for a = b = 0, w = 1: causal linear attention plus the carried state.

    o_t = S0^T r_t + sum_{s<=t} (k_s . r_t) v_s ;  S_T = S0 + sum_s k_s v_s^T.
    Written as a masked score matrix, as linear attention is usually stated.
    """
    T = r.shape[0]
    scores = np.tril(r @ k.T)          # scores[t, s] = r_t . k_s for s <= t
    o = r @ S0 + scores @ v
    S = S0 + k.T @ v
    return o, S


def pure_decay(r, w, k, v, S0):
    """Closed form for a = b = 0: S_t = Gamma_t S0 + sum_{s<=t} diag(gamma_t/gamma_s) k_s v_s^T."""
    T, N = r.shape
    logg = np.cumsum(np.log(w), axis=0)
    o = np.zeros((T, N))
    S_t = None
    for t in range(T):
        S_t = np.exp(logg[t])[:, None] * S0
        for s in range(t + 1):
            S_t = S_t + (np.exp(logg[t] - logg[s]) * k[s])[:, None] * v[s][None, :]
        o[t] = S_t.T @ r[t]
    return o, S_t


def g_chain(r, w, a, b, d_o, G_T, C):
    """The gradient recurrence alone (it needs no states): with G = dL/dS_t, going back
    over the tokens, G += r_t d_o_t^T, then G <- diag(w_t) G + a_t (G^T b_t)^T.
    Returns [G at the end of chunk c for every c] (c's last token not yet applied) and
    the gradient of the input state.  One head, fp arrays [T, N], G_T [N, N]."""
    T, N = r.shape
    nck = -(-T // C)
    G = np.array(G_T, copy=True)
    ends = [None] * nck
    for t in range(T - 1, -1, -1):
        if t == min(T, (t // C + 1) * C) - 1:
            ends[t // C] = G.copy()
        G = G + np.outer(r[t], d_o[t])
        c = G.T @ b[t]
        G = w[t][:, None] * G + np.outer(a[t], c)
    return ends, G


def chunk_adjoint(r, w, k, v, a, b, S0, d_o, G_end, ref=7):
    """Gradients of one chunk in chunk form, from the state entering it (S0) and the
    gradient for the state leaving it (G_end).  Tokens tau = 0..L-1 of one head.

    Forward, with P_tau the running product of w over the chunk, d_tau = P_tau/P_ref
    (a reference position keeps the factors inside the exponent range),
    A' = a d_{tau-1}, R' = r d_tau, B' = b / d_tau, K' = k / d_tau, S^ = diag(P_ref) S0,
    M_xy = tril(X'Y'^T) (strict for the a-rows), T = (I - M_ab)^{-1}:
        X = A' S^ + M_ak V,   Z = T X,   O = R' S^ + M_rb Z + M_rk V,
        S_end = diag(d_last) (S^ + B'^T Z + K'^T V).
    Reverse mode through those products, with G^ = diag(d_last) G_end:
        dZ = B' G^ + M_rb^T dO,  dX = T^T dZ,  dV = K' G^ + M_rk^T dO + M_ak^T dX,
        dM_ab = tril(dX Z^T, -1), dM_ak = tril(dX V^T, -1), dM_rb = tril(dO Z^T), dM_rk = tril(dO V^T),
        dA' = dX S^T + dM_ab B' + dM_ak K',   dR' = dO S^T + dM_rb B' + dM_rk K',
        dB' = Z G^T + dM_ab^T A' + dM_rb^T R', dK' = V G^T + dM_ak^T A' + dM_rk^T R',
    then da = dA' d_{tau-1}, dr = dR' d_tau, db = dB' / d_tau, dk = dK' / d_tau.  The decay
    gradient is taken in its direct form dw_t = rowsum(G_t * S_{t-1}), with both states in
    the chunk's terms, S_{t-1} = diag(d_{t-1}) (S^ + sum_{s<t} B'_s^T z_s + K'_s^T v_s) and
    G_t = diag(1/d_t) (G^ + sum_{s>=t} R'_s^T dO_s + sum_{s>t} A'_s^T dX_s), so that
        w_t dw_t = rowsum(G^ * S^) + sum_{s<t} (B'_s (G^ z_s) + K'_s (G^ v_s))
                 + sum_{s>=t} R'_s (S^ dO_s) + sum_{s>t} A'_s (S^ dX_s)
                 + sum_{s>=t} sum_{u<t} R'_s (B'_u (dO_s . z_u) + K'_u (dO_s . v_u))
                 + sum_{s>t} sum_{u<t} A'_s (B'_u (dX_s . z_u) + K'_u (dX_s . v_u))
    (elementwise in the key index).  Every term carries w_t among its decay factors, so
    the division by w_t cancels without loss.  (The log-decay form, a suffix sum of
    d(log P_tau) divided by w_s, loses about eps / w_s to cancellation.)
    Returns dict of [L, N] arrays."""
    L, N = r.shape
    dt = r.dtype
    rho = min(ref, L - 1)
    Pr = np.prod(w[:rho + 1], axis=0)                       # P_ref
    d = np.ones((L, N), dt)                                  # d_tau = P_tau / P_ref, formed
    for t in range(rho + 1, L):                              # from the nearer end so that
        d[t] = d[t - 1] * w[t]                               # no absolute P is needed
    for t in range(rho - 1, -1, -1):
        d[t] = d[t + 1] / w[t + 1]
    d_prev = np.vstack([d[:1] / w[:1], d[:-1]])             # d_{tau-1}; d_{-1} = 1 / P_ref
    Ap, Rp, Bp, Kp = a * d_prev, r * d, b / d, k / d
    Sh = Pr[:, None] * S0
    with np.errstate(over="ignore", invalid="ignore"):  # entries above the diagonal may
        M_ab = np.tril(Ap @ Bp.T, -1)                      # overflow; they are dropped
        M_ak = np.tril(Ap @ Kp.T, -1)
        M_rb = np.tril(Rp @ Bp.T, 0)
        M_rk = np.tril(Rp @ Kp.T, 0)
    Tm = np.linalg.inv(np.eye(L, dtype=dt) - M_ab)
    X = Ap @ Sh + M_ak @ v
    Z = Tm @ X
    Gh = d[-1][:, None] * G_end
    dZ = Bp @ Gh + M_rb.T @ d_o
    dX = Tm.T @ dZ
    dV = Kp @ Gh + M_rk.T @ d_o + M_ak.T @ dX
    dM_ab = np.tril(dX @ Z.T, -1)
    dM_ak = np.tril(dX @ v.T, -1)
    dM_rb = np.tril(d_o @ Z.T, 0)
    dM_rk = np.tril(d_o @ v.T, 0)
    dA = dX @ Sh.T + dM_ab @ Bp + dM_ak @ Kp
    dR = d_o @ Sh.T + dM_rb @ Bp + dM_rk @ Kp
    dBz, dKv = Z @ Gh.T, v @ Gh.T
    dB = dBz + dM_ab.T @ Ap + dM_rb.T @ Rp
    dK = dKv + dM_ak.T @ Ap + dM_rk.T @ Rp
    # the direct decay gradient: the quantities G^ z_s, G^ v_s, S^ dO_s, S^ dX_s per key
    # (the first terms of dB', dK', dR', dA') and the token-pair dot products
    dR0, dA0 = d_o @ Sh.T, dX @ Sh.T
    W1, W2, W3, W4 = d_o @ Z.T, d_o @ v.T, dX @ Z.T, dX @ v.T
    wdw = np.zeros((L, N), dt)
    base = (Gh * Sh).sum(axis=1)
    for t in range(L):
        acc = base.copy()
        for u in range(t):
            acc += Bp[u] * dBz[u] + Kp[u] * dKv[u]
        for s_ in range(t, L):
            acc += Rp[s_] * dR0[s_]
            for u in range(t):
                acc += Rp[s_] * (Bp[u] * W1[s_, u] + Kp[u] * W2[s_, u])
        for s_ in range(t + 1, L):
            acc += Ap[s_] * dA0[s_]
            for u in range(t):
                acc += Ap[s_] * (Bp[u] * W3[s_, u] + Kp[u] * W4[s_, u])
        wdw[t] = acc
    dw = wdw / w
    return {"dr": dR * d, "dk": dK / d, "da": dA * d_prev, "db": dB / d, "dv": dV, "dw": dw}
