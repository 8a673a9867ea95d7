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
