"""TEST INFRASTRUCTURE ONLY: the fp64 CPU oracle of the WKV-7 recurrence.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library
(``rwkv_linear_attention_amd``) never imports it, and it imports nothing from
the GPU library: the two share no code.

``forward`` wraps the plain C loop in ``wkv7_oracle.c`` (fp64, sums in
ascending key order, no fused multiply-adds).  ``backward`` is the plain
reverse-mode adjoint of that loop in numpy fp64, pinned by finite differences
of ``forward``.  Its header comment names the
passages of the pages it follows: the "WKV-7 Kernel (Generalized Delta Rule)"
section of the RWKV-X Architecture page and section 1 of the Core AI RWKV-7
note.  Every value it returns is fp64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "wkv7_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libwkv7_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no FMA contraction). Returns the .so path."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC",
               "-shared", "-pthread", _SRC, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        lib.wkv7_oracle_forward.argtypes = [vp] * 6 + [ctypes.c_int, vp, vp, vp, vp,
                                                       i64, i64, i64, i64, ctypes.c_int]
        lib.wkv7_oracle_forward.restype = ctypes.c_int
        lib.wkv7_oracle_default_threads.argtypes = []
        lib.wkv7_oracle_default_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    return int(_load().wkv7_oracle_default_threads())


def _as_input(x, dtype):
    """bf16 / fp32 / fp64 values converted to the carrier dtype, refusing any rounding."""
    if hasattr(x, "detach"):  # a torch tensor: bf16 and fp32 widen exactly
        import torch
        x = x.detach().to("cpu")
        x = x.to(torch.float64).numpy()
    src = np.asarray(x)
    out = np.ascontiguousarray(src, dtype=dtype)
    if out.dtype != src.dtype and not np.array_equal(out.astype(np.float64), src.astype(np.float64),
                                                     equal_nan=True):
        raise ValueError("inputs are not exact in the oracle's input carrier (pass f64_inputs=True)")
    return out


def forward(r, w, k, v, a, b, state_in=None, *, per_position=False, nthreads=0,
            f64_inputs=False):
    """Run the fp64 recurrence.

    r, w, k, v, a, b: arrays [B, T, H, N] (numpy or CPU torch; fp32/bf16/fp64).
    state_in: [B, H, N, N] or None (zeros).  Row i of a head's state is a key
    channel, column j a value channel.
    Returns (o [B,T,H,N], state_out [B,H,N,N]) or, with per_position=True,
    (o, state_out, state_pos [B,T,H,N,N]) where state_pos[:, t] is the state
    after token t.  All fp64.
    """
    lib = _load()
    cdt = np.float64 if f64_inputs else np.float32
    arrs = [_as_input(x, cdt) for x in (r, w, k, v, a, b)]
    shape = arrs[0].shape
    if len(shape) != 4 or any(x.shape != shape for x in arrs):
        raise ValueError(f"inputs must share one [B,T,H,N] shape, got {[x.shape for x in arrs]}")
    B, T, H, N = shape
    s_in = None
    if state_in is not None:
        s_in = _as_input(state_in, np.float64)
        if s_in.shape != (B, H, N, N):
            raise ValueError(f"state_in must be {(B, H, N, N)}, got {s_in.shape}")
    o = np.zeros((B, T, H, N), np.float64)
    s_out = np.zeros((B, H, N, N), np.float64)
    s_pos = np.zeros((B, T, H, N, N), np.float64) if per_position else None
    ptr = lambda x: None if x is None else x.ctypes.data_as(ctypes.c_void_p)
    rc = lib.wkv7_oracle_forward(*[ptr(x) for x in arrs], 1 if f64_inputs else 0,
                                 ptr(s_in), ptr(o), ptr(s_out), ptr(s_pos),
                                 B, T, H, N, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"wkv7_oracle_forward failed with code {rc}")
    if per_position:
        return o, s_out, s_pos
    return o, s_out


def forward_varlen(r, w, k, v, a, b, state_in=None, lengths=None, **kw):
    """Rows of their own lengths: row b runs only its first L_b tokens.

    The batched prefill of the SwiftRWKV Inference guide (its batched
    generation) pads prompts on the right and ends each row on its own last
    real token.  Plain definition: L_b = lengths[b] clamped to [0, T]; row b is
    ``forward`` over tokens [0, L_b) of that row from state_in[b] (zeros when
    None).  Returns (o [B,T,H,N], state_out [B,H,N,N]), fp64, with o[b, t] = NaN
    for t >= L_b (those outputs are not defined).
    """
    B, T, H, N = np.asarray(r.shape if hasattr(r, "shape") else np.shape(r))
    L = np.clip(np.asarray(lengths, dtype=np.int64).reshape(-1), 0, T)
    if L.shape != (B,):
        raise ValueError(f"lengths must have {B} entries")
    o = np.full((B, T, H, N), np.nan)
    s_out = np.zeros((B, H, N, N))
    for bb in range(B):
        s0 = None if state_in is None else state_in[bb:bb + 1]
        if L[bb] == 0:
            if s0 is not None:
                s_out[bb] = _as_input(s0, np.float64)[0]
            continue
        rows = [x[bb:bb + 1, :L[bb]] for x in (r, w, k, v, a, b)]
        o_b, s_b = forward(*rows, s0, **kw)
        o[bb, :L[bb]] = o_b[0]
        s_out[bb] = s_b[0]
    return o, s_out


def state_commit(state_pos, accepted, state_in=None, state_out=None):
    """The state after each row's accepted prefix of a speculative verify step.

    The RWKV7-MTP-Exp model card ("Inference") rolls the recurrent state back
    to the accepted prefix.  Plain definition, with n = accepted[b] and T the
    step length: row b is state_pos[b, n - 1] for 1 <= n <= T, state_in[b]
    (zeros when None) for n = 0, and state_out[b] unchanged (zeros when None)
    for n outside [0, T].  Returns [B, H, N, N] fp64.
    """
    sp = _as_input(state_pos, np.float64)
    B, T, H, N, _ = sp.shape
    acc = np.asarray(accepted, dtype=np.int64).reshape(-1)
    out = np.zeros((B, H, N, N)) if state_out is None else _as_input(state_out, np.float64).copy()
    for bb in range(B):
        n = int(acc[bb])
        if 1 <= n <= T:
            out[bb] = sp[bb, n - 1]
        elif n == 0:
            out[bb] = 0.0 if state_in is None else _as_input(state_in, np.float64)[bb]
    return out


def tmix_tail(o, r, k, v, g, r_k, ln_w, ln_b, eps):
    """The time-mix tail after WKV: group norm, bonus and gate.

    The SwiftRWKV Inference guide (its decode-path list and the fused frozen
    pass) fuses these three steps after the WKV output and names only their
    parts.  The reading taken, per (b, t, h), over the N value channels j:
        mu   = mean_j o[j],  var = mean_j (o[j] - mu)^2          (biased)
        y[j] = (o[j] - mu) / sqrt(var + eps) * ln_w[h, j] + ln_b[h, j]
        x[j] = (y[j] + (sum_i r[i] k[i] r_k[h, i]) * v[j]) * g[j]
    o, r, k, v, g: [B,T,H,N]; r_k, ln_w, ln_b: [H,N]; returns x [B,T,H,N] fp64.
    """
    f = lambda a: _as_input(a, np.float64)
    o, r, k, v, g = (f(a) for a in (o, r, k, v, g))
    r_k, ln_w, ln_b = (f(a) for a in (r_k, ln_w, ln_b))
    B, T, H, N = o.shape
    # every (b, t, h) row at once: the sums run over the last axis (the N channels)
    mu = o.sum(axis=-1, keepdims=True) / N
    var = ((o - mu) ** 2).sum(axis=-1, keepdims=True) / N
    y = (o - mu) / np.sqrt(var + eps) * ln_w[None, None] + ln_b[None, None]
    bonus = (r * k * r_k[None, None]).sum(axis=-1, keepdims=True)
    return (y + bonus * v) * g


def backward(r, w, k, v, a, b, state_in=None, d_o=None, d_state_out=None):
    """Gradients of the recurrence (fp64): the adjoint of ``forward``'s loop.

    The SwiftRWKV Inference guide (its `.rwkvq` backend section) keeps a
    trainable WKV kernel whose backward pass rebuilds the state chunk by chunk;
    the pages give no formulas.  This is the plain reverse-mode adjoint of the
    recurrence of the RWKV-X Architecture page ("WKV-7 Kernel (Generalized
    Delta Rule)"),
        S_t = diag(w_t) S_{t-1} + b_t (a_t^T S_{t-1}) + k_t v_t^T,   o_t = S_t^T r_t,
    for a loss L with dL/do_t = d_o[t] and dL/dS_T = d_state_out.  With G the
    gradient of L with respect to S_t (rows = key channels), going backward in t:
        G    += r_t d_o_t^T
        dr_t  = S_t d_o_t            dk_t = G v_t            dv_t = G^T k_t
        dw_t  = rowsum(G * S_{t-1})  db_t = G (S_{t-1}^T a_t)
        c     = G^T b_t              da_t = S_{t-1} c
        G     = diag(w_t) G + a_t c^T            (the gradient for S_{t-1})
    and finally d_state_in = G.  The states S_t come from ``forward``.
    Inputs as for ``forward`` (fp64 carriers are taken as given); d_o [B,T,H,N]
    or None (zeros), d_state_out [B,H,N,N] or None (zeros).  Returns a dict of
    fp64 arrays dr, dw, dk, dv, da, db [B,T,H,N] and d_state_in [B,H,N,N].
    """
    f = lambda x: _as_input(x, np.float64)
    r, w, k, v, a, b = (f(x) for x in (r, w, k, v, a, b))
    B, T, H, N = r.shape
    s0 = np.zeros((B, H, N, N)) if state_in is None else f(state_in)
    _, _, s_pos = forward(r, w, k, v, a, b, s0, per_position=True, f64_inputs=True)
    g_o = np.zeros((B, T, H, N)) if d_o is None else f(d_o)
    out = {n: np.zeros((B, T, H, N)) for n in ("dr", "dw", "dk", "dv", "da", "db")}
    d_s0 = np.zeros((B, H, N, N))
    for bb in range(B):
        for h in range(H):
            G = np.zeros((N, N)) if d_state_out is None else f(d_state_out)[bb, h].copy()
            for t in range(T - 1, -1, -1):
                S = s_pos[bb, t, h]
                Sp = s_pos[bb, t - 1, h] if t > 0 else s0[bb, h]
                rt, wt, kt, vt, at, bt = (x[bb, t, h] for x in (r, w, k, v, a, b))
                do = g_o[bb, t, h]
                G = G + np.outer(rt, do)
                out["dr"][bb, t, h] = S @ do
                out["dk"][bb, t, h] = G @ vt
                out["dv"][bb, t, h] = G.T @ kt
                out["dw"][bb, t, h] = (G * Sp).sum(axis=1)
                out["db"][bb, t, h] = G @ (Sp.T @ at)
                c = G.T @ bt
                out["da"][bb, t, h] = Sp @ c
                G = wt[:, None] * G + np.outer(at, c)
            d_s0[bb, h] = G
    out["d_state_in"] = d_s0
    return out
