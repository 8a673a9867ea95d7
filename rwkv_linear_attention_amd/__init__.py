"""libwkv7 for MI355X: the WKV-7 recurrence (RWKV-7 generalized delta rule) on gfx950.

A thin ctypes binding over the C ABI of ``libwkv7.so`` (declared in
``include/wkv7.h``).  This module only marshals arguments: it checks device,
dtype, shape and contiguity of torch tensors, passes their device pointers and
the current HIP stream, and raises on a nonzero status.  Every step of the
computation runs in the HIP kernels of the library; there is no CPU or
PyTorch fallback, and the calls fail loudly when the library is not built.

Functions (names as in the C ABI):

* ``wkv7_forward(r, w, k, v, a, b, state_in=None, o_dtype=torch.float32, lengths=None)``
  -> ``(o, state_out)``: the parallel (prefill) pass; with ``lengths`` ([B] int32),
  row b runs its first lengths[b] tokens (``wkv7_forward_varlen`` of the C ABI).
* ``wkv7_step(r, w, k, v, a, b, state_in=None, per_position=False, ...)``
  -> ``(o, state_out[, state_pos])``: the recurrent (decode / verify) pass.
* ``wkv7_step_tail(r, w, k, v, a, b, g, r_k, ln_w, ln_b, eps, state_in=None, ...)``
  -> ``(x, state_out[, state_pos])``: the recurrent pass with the time-mix tail
  (group norm, bonus, gate) fused into its epilogue.
* ``wkv7_forward_tail(r, w, k, v, a, b, g, r_k, ln_w, ln_b, eps, state_in=None, ...)``
  -> ``(x, state_out)``: the parallel pass with the time-mix tail fused (o is never
  written).
* ``wkv7_tmix_tail(o, r, k, v, g, r_k, ln_w, ln_b, eps, x_dtype=torch.float32)`` -> ``x``:
  the same tail as a pass of its own, after the parallel pass.
* ``wkv7_state_commit(state_pos, accepted, state_in=None)`` -> ``state_out``: the state
  after each row's accepted prefix of a speculative verify step.
* ``wkv7_state_reset(state, row_mask=None)``: zero the state (all rows or masked ones).
* ``wkv7_backward(r, w, k, v, a, b, state_in, state_pos, d_o, d_state_out=None)`` -> a dict of
  the gradients ``dr, dw, dk, dv, da, db`` and ``d_state_in`` (fp32), given the
  per-position states of the forward pass.

Tensors: r, w, k, v, a, b are [B, T, H, 64] bf16 or fp32 on the GPU; the
state is [B, H, 64, 64] fp32 with row i a key channel and column j a value
channel.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libwkv7.so")

WKV7_F32, WKV7_BF16 = 0, 1
HEAD_SIZE = 64
_lib = None


class Wkv7Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def build() -> str:
    """Compile libwkv7.so in-tree for gfx950 (always recompiles)."""
    from . import _build
    global _lib
    _lib = None
    return _build.build()


def lib():
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                               "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        vp, ci = ctypes.c_void_p, ctypes.c_int
        L.wkv7_forward.argtypes = [vp] * 6 + [ci, vp, vp, ci, vp, ci, ci, ci, ci, vp]
        L.wkv7_forward.restype = ci
        L.wkv7_forward_varlen.argtypes = [vp] * 6 + [ci, vp, vp, ci, vp, vp, ci, ci, ci, ci, vp]
        L.wkv7_forward_varlen.restype = ci
        L.wkv7_step.argtypes = [vp] * 6 + [ci, vp, vp, ci, vp, vp, ci, ci, ci, ci, vp]
        L.wkv7_step.restype = ci
        L.wkv7_state_commit.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, vp]
        L.wkv7_state_commit.restype = ci
        cf = ctypes.c_float
        L.wkv7_step_tail.argtypes = [vp] * 6 + [ci, vp, vp, vp, vp, vp, cf, vp, ci, vp, vp, ci, ci, ci, ci, vp]
        L.wkv7_step_tail.restype = ci
        L.wkv7_forward_tail.argtypes = [vp] * 6 + [ci, vp, vp, vp, vp, vp, cf, vp, ci, vp, ci, ci, ci, ci, vp]
        L.wkv7_forward_tail.restype = ci
        L.wkv7_tmix_tail.argtypes = [vp, ci, vp, vp, vp, vp, ci, vp, vp, vp, cf, vp, ci, ci, ci, ci, ci, vp]
        L.wkv7_tmix_tail.restype = ci
        L.wkv7_state_reset.argtypes = [vp, ci, ci, ci, vp, vp]
        L.wkv7_backward.argtypes = [vp] * 6 + [ci] + [vp] * 11 + [ci, ci, ci, ci, vp]
        L.wkv7_backward.restype = ci
        L.wkv7_forward_ckpt.argtypes = [vp] * 6 + [ci, vp, vp, vp, vp, ci, ci, ci, ci, vp]
        L.wkv7_forward_ckpt.restype = ci
        L.wkv7_backward_ckpt.argtypes = [vp] * 6 + [ci] + [vp] * 10 + [ci, ci, ci, ci, vp]
        L.wkv7_backward_ckpt.restype = ci
        L.wkv7_state_reset.restype = ci
        L.wkv7_status_string.argtypes = [ci]
        L.wkv7_status_string.restype = ctypes.c_char_p
        L.wkv7_abi_version.argtypes = []
        L.wkv7_abi_version.restype = ci
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().wkv7_status_string(int(status)).decode()


def _check(status: int):
    if status != 0:
        raise Wkv7Error(status, status_string(status))


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return WKV7_BF16
    if t.dtype == torch.float32:
        return WKV7_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32 only)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_inputs(r, w, k, v, a, b):
    ins = (r, w, k, v, a, b)
    if r.dim() != 4:
        raise ValueError(f"inputs must be [B, T, H, N], got {tuple(r.shape)}")
    for x in ins:
        if not x.is_cuda:
            raise ValueError("inputs must be on the GPU")
        if x.shape != r.shape or x.dtype != r.dtype or x.device != r.device:
            raise ValueError("r, w, k, v, a, b must share shape, dtype and device")
        if not x.is_contiguous():
            raise ValueError("inputs must be contiguous")
    return r.shape


def _state_arg(state, B, H, N, device, name):
    if state is None:
        return None
    if (state.dtype != torch.float32 or tuple(state.shape) != (B, H, N, N) or not state.is_contiguous()
            or state.device != device):
        raise ValueError(f"{name} must be a contiguous fp32 [{B}, {H}, {N}, {N}] tensor on {device}")
    return state


def _out_arg(x, shape, device, name, dtypes=(torch.float32, torch.bfloat16)):
    """A caller-supplied output: a contiguous tensor of `shape` on `device` with one of `dtypes`.

    The C ABI cannot see buffer sizes, so an undersized or strided output would be
    written past its end; every wrapper checks its outputs here first."""
    if not torch.is_tensor(x):
        raise ValueError(f"{name} must be a tensor")
    if tuple(x.shape) != tuple(shape) or not x.is_contiguous() or x.device != device or x.dtype not in dtypes:
        kinds = " or ".join(str(d).replace("torch.", "") for d in dtypes)
        raise ValueError(f"{name} must be a contiguous {kinds} {list(shape)} tensor on {device}")
    return x


def _int_rows(x, B, device, name):
    """A [B] int32 device tensor (converted from any integer tensor or sequence)."""
    x = torch.as_tensor(x, device=device).to(torch.int32).contiguous()
    if x.shape != (B,):
        raise ValueError(f"{name} must have shape [{B}]")
    return x


def wkv7_forward(r, w, k, v, a, b, state_in=None, *, o_dtype=torch.float32, o=None, state_out=None,
                 lengths=None):
    """Parallel pass over the whole sequence.  Returns (o, state_out).

    state_out may be passed as state_in itself to update the state in place.
    With lengths ([B] integers), row b runs its first lengths[b] tokens (clamped
    to [0, T]); o[b, t] for t >= lengths[b] is left as it was.
    """
    B, T, H, N = _check_inputs(r, w, k, v, a, b)
    dev = r.device
    state_in = _state_arg(state_in, B, H, N, dev, "state_in")
    if state_out is None:
        state_out = torch.empty((B, H, N, N), dtype=torch.float32, device=dev)
    _state_arg(state_out, B, H, N, dev, "state_out")
    if o is None:
        o = torch.empty((B, T, H, N), dtype=o_dtype, device=dev)
    _out_arg(o, (B, T, H, N), dev, "o")
    if lengths is None:
        _check(lib().wkv7_forward(*[_ptr(x) for x in (r, w, k, v, a, b)], _dt(r), _ptr(state_in), _ptr(o),
                                  _dt(o), _ptr(state_out), B, T, H, N, _stream(dev)))
    else:
        lengths = _int_rows(lengths, B, dev, "lengths")
        _check(lib().wkv7_forward_varlen(*[_ptr(x) for x in (r, w, k, v, a, b)], _dt(r), _ptr(state_in),
                                         _ptr(o), _dt(o), _ptr(state_out), _ptr(lengths), B, T, H, N,
                                         _stream(dev)))
    return o, state_out


def wkv7_step(r, w, k, v, a, b, state_in=None, *, per_position=False, o_dtype=torch.float32, o=None,
              state_out=None, state_pos=None, write_state_out=True):
    """Recurrent pass, token by token.  Returns (o, state_out) or (o, state_out, state_pos).

    With per_position=True, state_pos[:, t] is the state after token t; then
    write_state_out=False skips the separate final state (state_out is None).
    """
    B, T, H, N = _check_inputs(r, w, k, v, a, b)
    dev = r.device
    state_in = _state_arg(state_in, B, H, N, dev, "state_in")
    if not write_state_out:
        if not (per_position or state_pos is not None) or state_out is not None:
            raise ValueError("write_state_out=False needs per-position states and no state_out")
    elif state_out is None:
        state_out = torch.empty((B, H, N, N), dtype=torch.float32, device=dev)
    if state_out is not None:
        _state_arg(state_out, B, H, N, dev, "state_out")
    if o is None:
        o = torch.empty((B, T, H, N), dtype=o_dtype, device=dev)
    _out_arg(o, (B, T, H, N), dev, "o")
    if per_position and state_pos is None:
        state_pos = torch.empty((B, T, H, N, N), dtype=torch.float32, device=dev)
    if state_pos is not None:
        _out_arg(state_pos, (B, T, H, N, N), dev, "state_pos", (torch.float32,))
    _check(lib().wkv7_step(*[_ptr(x) for x in (r, w, k, v, a, b)], _dt(r), _ptr(state_in), _ptr(o), _dt(o),
                           _ptr(state_out), _ptr(state_pos), B, T, H, N, _stream(dev)))
    if state_pos is not None:
        return o, state_out, state_pos
    return o, state_out


def _head_params(H, N, device, **named):
    out = []
    for name, t in named.items():
        if (t.dtype != torch.float32 or tuple(t.shape) != (H, N) or not t.is_contiguous() or t.device != device):
            raise ValueError(f"{name} must be a contiguous fp32 [{H}, {N}] tensor on {device}")
        out.append(t)
    return out


def wkv7_step_tail(r, w, k, v, a, b, g, r_k, ln_w, ln_b, eps, state_in=None, *, per_position=False,
                   x_dtype=torch.float32, x=None, state_out=None, state_pos=None):
    """wkv7_step with the time-mix tail fused: returns (x, state_out) or (x, state_out, state_pos).

    g: gate [B, T, H, N] like r; r_k, ln_w, ln_b: fp32 [H, N]; eps: float.
    """
    B, T, H, N = _check_inputs(r, w, k, v, a, b)
    dev = r.device
    if g.shape != r.shape or g.dtype != r.dtype or not g.is_contiguous() or g.device != dev:
        raise ValueError("g must match r in shape, dtype and device, and be contiguous")
    r_k, ln_w, ln_b = _head_params(H, N, dev, r_k=r_k, ln_w=ln_w, ln_b=ln_b)
    state_in = _state_arg(state_in, B, H, N, dev, "state_in")
    if state_out is None:
        state_out = torch.empty((B, H, N, N), dtype=torch.float32, device=dev)
    _state_arg(state_out, B, H, N, dev, "state_out")
    if x is None:
        x = torch.empty((B, T, H, N), dtype=x_dtype, device=dev)
    _out_arg(x, (B, T, H, N), dev, "x")
    if per_position and state_pos is None:
        state_pos = torch.empty((B, T, H, N, N), dtype=torch.float32, device=dev)
    if state_pos is not None:
        _out_arg(state_pos, (B, T, H, N, N), dev, "state_pos", (torch.float32,))
    _check(lib().wkv7_step_tail(*[_ptr(t) for t in (r, w, k, v, a, b)], _dt(r), _ptr(state_in), _ptr(g),
                                _ptr(r_k), _ptr(ln_w), _ptr(ln_b), float(eps), _ptr(x), _dt(x), _ptr(state_out),
                                _ptr(state_pos), B, T, H, N, _stream(dev)))
    if state_pos is not None:
        return x, state_out, state_pos
    return x, state_out


def wkv7_forward_tail(r, w, k, v, a, b, g, r_k, ln_w, ln_b, eps, state_in=None, *, x_dtype=torch.float32,
                      x=None, state_out=None):
    """wkv7_forward with the time-mix tail fused: returns (x, state_out); o is never written.

    g: gate [B, T, H, N] like r; r_k, ln_w, ln_b: fp32 [H, N]; eps: float.
    """
    B, T, H, N = _check_inputs(r, w, k, v, a, b)
    dev = r.device
    if g.shape != r.shape or g.dtype != r.dtype or not g.is_contiguous() or g.device != dev:
        raise ValueError("g must match r in shape, dtype and device, and be contiguous")
    r_k, ln_w, ln_b = _head_params(H, N, dev, r_k=r_k, ln_w=ln_w, ln_b=ln_b)
    state_in = _state_arg(state_in, B, H, N, dev, "state_in")
    if state_out is None:
        state_out = torch.empty((B, H, N, N), dtype=torch.float32, device=dev)
    _state_arg(state_out, B, H, N, dev, "state_out")
    if x is None:
        x = torch.empty((B, T, H, N), dtype=x_dtype, device=dev)
    _out_arg(x, (B, T, H, N), dev, "x")
    _check(lib().wkv7_forward_tail(*[_ptr(t) for t in (r, w, k, v, a, b)], _dt(r), _ptr(state_in), _ptr(g),
                                   _ptr(r_k), _ptr(ln_w), _ptr(ln_b), float(eps), _ptr(x), _dt(x),
                                   _ptr(state_out), B, T, H, N, _stream(dev)))
    return x, state_out


def wkv7_tmix_tail(o, r, k, v, g, r_k, ln_w, ln_b, eps, *, x_dtype=torch.float32, x=None):
    """The time-mix tail of o (from wkv7_forward): returns x [B, T, H, N].  x may be o itself."""
    B, T, H, N = _check_inputs(r, r, k, v, g, g)
    dev = r.device
    _out_arg(o, (B, T, H, N), dev, "o")
    r_k, ln_w, ln_b = _head_params(H, N, dev, r_k=r_k, ln_w=ln_w, ln_b=ln_b)
    if x is None:
        x = torch.empty((B, T, H, N), dtype=x_dtype, device=dev)
    _out_arg(x, (B, T, H, N), dev, "x")
    _check(lib().wkv7_tmix_tail(_ptr(o), _dt(o), _ptr(r), _ptr(k), _ptr(v), _ptr(g), _dt(r), _ptr(r_k),
                                _ptr(ln_w), _ptr(ln_b), float(eps), _ptr(x), _dt(x), B, T, H, N, _stream(dev)))
    return x


def wkv7_state_commit(state_pos, accepted, state_in=None, *, state_out=None):
    """State after each row's accepted prefix of a verify step.  Returns state_out.

    state_pos: [B, T, H, N, N] from wkv7_step(per_position=True); accepted: [B]
    integers.  Row b becomes state_pos[b, accepted[b] - 1], or state_in[b] (zeros
    when None) for accepted[b] == 0; rows with accepted[b] outside [0, T] keep
    state_out (pass state_out=state_in to commit in place).
    """
    if state_pos.dim() != 5 or not state_pos.is_cuda or state_pos.dtype != torch.float32 \
            or not state_pos.is_contiguous():
        raise ValueError("state_pos must be a contiguous fp32 [B, T, H, N, N] GPU tensor")
    B, T, H, N, _ = state_pos.shape
    dev = state_pos.device
    accepted = _int_rows(accepted, B, dev, "accepted")
    state_in = _state_arg(state_in, B, H, N, dev, "state_in")
    if state_out is None:
        state_out = torch.empty((B, H, N, N), dtype=torch.float32, device=dev)
    _state_arg(state_out, B, H, N, dev, "state_out")
    _check(lib().wkv7_state_commit(_ptr(state_pos), _ptr(accepted), _ptr(state_in), _ptr(state_out),
                                   B, T, H, N, _stream(dev)))
    return state_out


def wkv7_backward(r, w, k, v, a, b, state_in, state_pos, d_o, d_state_out=None, *, grads=None):
    """Gradients of the recurrence: the backward pass of wkv7_forward.

    state_pos: [B, T, H, N, N] fp32, the state after each token (wkv7_step with
    per_position=True writes it); d_o: [B, T, H, N] fp32, the gradient of o;
    d_state_out: [B, H, N, N] fp32 gradient of the final state, or None (zeros).
    Returns a dict with dr, dw, dk, dv, da, db ([B, T, H, N] fp32) and d_state_in
    ([B, H, N, N] fp32); ``grads`` may pass that dict preallocated.
    """
    B, T, H, N = _check_inputs(r, w, k, v, a, b)
    dev = r.device
    state_in = _state_arg(state_in, B, H, N, dev, "state_in")
    d_state_out = _state_arg(d_state_out, B, H, N, dev, "d_state_out")
    f32 = (torch.float32,)
    _out_arg(state_pos, (B, T, H, N, N), dev, "state_pos", f32)
    _out_arg(d_o, (B, T, H, N), dev, "d_o", f32)
    names = ("dr", "dw", "dk", "dv", "da", "db")
    if grads is None:
        grads = {n: torch.empty((B, T, H, N), dtype=torch.float32, device=dev) for n in names}
        grads["d_state_in"] = torch.empty((B, H, N, N), dtype=torch.float32, device=dev)
    for n in names:
        _out_arg(grads[n], (B, T, H, N), dev, n, f32)
    _out_arg(grads["d_state_in"], (B, H, N, N), dev, "d_state_in", f32)
    _check(lib().wkv7_backward(*[_ptr(x) for x in (r, w, k, v, a, b)], _dt(r), _ptr(state_in),
                               _ptr(state_pos), _ptr(d_o), _ptr(d_state_out),
                               *[_ptr(grads[n]) for n in names], _ptr(grads["d_state_in"]),
                               B, T, H, N, _stream(dev)))
    return grads


def wkv7_forward_ckpt(r, w, k, v, a, b, state_in=None, *, o=None, state_out=None, ckpt=None):
    """Forward pass for training: (o, state_out, ckpt), o in fp32.

    ckpt: [B, ceil(T/16), H, N*N] fp32, the state before each chunk of 16 tokens
    (state_in, or zeros, first): what wkv7_backward_ckpt rebuilds the other states from.
    Each state is in the C ABI's tile order: element (i, j) at (j//16)*1024 + (i//16)*256
    + (i//4 % 4)*64 + (j % 16)*4 + i % 4.
    """
    B, T, H, N = _check_inputs(r, w, k, v, a, b)
    dev = r.device
    f32 = (torch.float32,)
    state_in = _state_arg(state_in, B, H, N, dev, "state_in")
    if state_out is None:
        state_out = torch.empty((B, H, N, N), dtype=torch.float32, device=dev)
    _state_arg(state_out, B, H, N, dev, "state_out")
    if o is None:
        o = torch.empty((B, T, H, N), dtype=torch.float32, device=dev)
    _out_arg(o, (B, T, H, N), dev, "o", f32)
    nck = (T + 15) // 16
    if ckpt is None:
        ckpt = torch.empty((B, nck, H, N * N), dtype=torch.float32, device=dev)
    _out_arg(ckpt, (B, nck, H, N * N), dev, "ckpt", f32)
    _check(lib().wkv7_forward_ckpt(*[_ptr(x) for x in (r, w, k, v, a, b)], _dt(r), _ptr(state_in), _ptr(o),
                                   _ptr(state_out), _ptr(ckpt) if nck else None, B, T, H, N, _stream(dev)))
    return o, state_out, ckpt


def wkv7_backward_ckpt(r, w, k, v, a, b, ckpt, d_o, d_state_out=None, *, grads=None):
    """Gradients of the recurrence from the checkpoints of wkv7_forward_ckpt.

    Returns the same dict as wkv7_backward (dr, dw, dk, dv, da, db, d_state_in).
    """
    B, T, H, N = _check_inputs(r, w, k, v, a, b)
    dev = r.device
    f32 = (torch.float32,)
    d_state_out = _state_arg(d_state_out, B, H, N, dev, "d_state_out")
    nck = (T + 15) // 16
    _out_arg(ckpt, (B, nck, H, N * N), dev, "ckpt", f32)
    _out_arg(d_o, (B, T, H, N), dev, "d_o", f32)
    names = ("dr", "dw", "dk", "dv", "da", "db")
    if grads is None:
        grads = {n: torch.empty((B, T, H, N), dtype=torch.float32, device=dev) for n in names}
        grads["d_state_in"] = torch.empty((B, H, N, N), dtype=torch.float32, device=dev)
    for n in names:
        _out_arg(grads[n], (B, T, H, N), dev, n, f32)
    _out_arg(grads["d_state_in"], (B, H, N, N), dev, "d_state_in", f32)
    _check(lib().wkv7_backward_ckpt(*[_ptr(x) for x in (r, w, k, v, a, b)], _dt(r),
                                    _ptr(ckpt) if nck else None, _ptr(d_o), _ptr(d_state_out),
                                    *[_ptr(grads[n]) for n in names], _ptr(grads["d_state_in"]),
                                    B, T, H, N, _stream(dev)))
    return grads


def wkv7_state_reset(state, row_mask=None):
    """Zero state [B, H, 64, 64] in place; with row_mask ([B] bool/uint8) only the flagged rows."""
    if state.dim() != 4 or not state.is_cuda or state.dtype != torch.float32 or not state.is_contiguous():
        raise ValueError("state must be a contiguous fp32 [B, H, N, N] GPU tensor")
    B, H, N, _ = state.shape
    if row_mask is not None:
        row_mask = row_mask.to(device=state.device, dtype=torch.uint8).contiguous()
        if row_mask.shape != (B,):
            raise ValueError(f"row_mask must have shape [{B}]")
    _check(lib().wkv7_state_reset(_ptr(state), B, H, N, _ptr(row_mask), _stream(state.device)))
    return state


def abi_version() -> int:
    return int(lib().wkv7_abi_version())
