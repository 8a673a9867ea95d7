"""TEST INFRASTRUCTURE ONLY: the fp64 CPU oracle of the WKV-7 recurrence.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library
(``rwkv_linear_attention_amd``) never imports it, and it imports nothing from
the GPU library: the two share no code.

``forward`` wraps the plain C loop in ``wkv7_oracle.c`` (fp64, sums in
ascending key order, no fused multiply-adds).  Its header comment names the
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
