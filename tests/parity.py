"""Comparison of a GPU result with the fp64 oracle, used by every GPU parity test.

Three bounds, each at the test's tolerance `tol`:
  * relative L2 over the whole tensor: ||x - ref|| / ||ref||;
  * relative L2 of every (batch, head) slice on its own, so a local corruption in
    one head cannot hide under the norm of the others;
  * every element within ELEM x tol x the RMS of its head's reference, so a single
    wrong element (its error is of the order of that RMS) fails even in a head of
    half a million elements.  ELEM = 10 leaves room for an element whose terms
    cancel (its rounding error is relative to its terms, not to itself): the
    backward pass's da at fp32 shows 1.04 x tol x RMS in one such element.
A head whose reference is exactly zero must be exactly zero.  The worst head and
the worst element ratio are printed with each check.

Head axes: HEADS_SEQ = (0, 2) for [B, T, H, ...] tensors (o, x, gradients,
per-position states), HEADS_STATE = (0, 1) for [B, H, N, N] states.
"""
import math

import numpy as np
import torch

HEADS_SEQ = (0, 2)
HEADS_STATE = (0, 1)
ELEM = 10.0


def as_f64(x):
    if torch.is_tensor(x):
        return x.detach().double().cpu().numpy()
    return np.asarray(x, np.float64)


def rel_l2(x, ref):
    x, ref = as_f64(x), as_f64(ref)
    n = np.linalg.norm(ref)
    d = np.linalg.norm(x - ref)
    if n == 0:
        return 0.0 if d == 0 else math.inf
    return d / n


def per_head(x, ref, heads, elem_rel=0.0):
    """(worst relative L2 of a head, its index, worst element error / allowance, its head index).

    An element's allowance is its head's RMS, plus elem_rel / tol times its own magnitude
    when elem_rel > 0 (see check)."""
    x, ref = as_f64(x), as_f64(ref)
    d = x - ref
    front = list(range(len(heads)))
    hshape = [ref.shape[a] for a in heads]
    d = np.moveaxis(d, heads, front).reshape(int(np.prod(hshape)), -1)
    r = np.moveaxis(ref, heads, front).reshape(d.shape)
    nr = np.linalg.norm(r, axis=1)
    nd = np.linalg.norm(d, axis=1)
    zero = nr == 0
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(zero, np.where(nd == 0, 0.0, np.inf), nd / nr)
        rms = nr / math.sqrt(max(d.shape[1], 1))
        allow = rms[:, None] + elem_rel * np.abs(r)
        ratio = np.where(allow > 0, np.abs(d) / allow, np.where(d == 0, 0.0, np.inf))
        elem = ratio.max(axis=1) if d.shape[1] else np.zeros(d.shape[0])
    hw, he = int(np.argmax(rel)), int(np.argmax(elem))
    return float(rel[hw]), np.unravel_index(hw, hshape), float(elem[he]), np.unravel_index(he, hshape)


def check(got, ref, tol, what, heads, elem_rel=0.0):
    """Assert the three bounds above; heads=None compares a flat selection globally only.

    elem_rel widens each element's bound to ELEM x tol x head RMS + elem_rel x |ref element|:
    outputs rounded to bf16 carry up to half an ulp (2^-8 relative) of their own."""
    e = rel_l2(got, ref)
    msg = f"  {what}: rel_l2 = {e:.3e}"
    if heads is not None:
        hr, hi, er, ei = per_head(got, ref, heads, elem_rel / (ELEM * tol))
        msg += (f"; worst head {tuple(int(v) for v in hi)} rel_l2 = {hr:.3e}; "
                f"worst element {er:.3e} x its head's RMS (head {tuple(int(v) for v in ei)})")
    print(msg + f" (tol {tol:.0e})", flush=True)
    assert e <= tol, f"{what}: rel_l2 {e:.3e} > {tol:.0e}"
    if heads is not None:
        assert hr <= tol, f"{what}: head {tuple(int(v) for v in hi)} rel_l2 {hr:.3e} > {tol:.0e}"
        assert er <= ELEM * tol, (f"{what}: an element of head {tuple(int(v) for v in ei)} is off by "
                                  f"{er:.3e} x its RMS (bound {ELEM * tol:.0e})")
