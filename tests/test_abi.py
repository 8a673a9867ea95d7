"""The C ABI of libwkv7 on the CPU: the library loads, exports every function the
header declares, and refuses bad arguments before any HIP call (so no GPU is
needed for these)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wkv7.h")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_ALIGN, ERR_ALIAS, ERR_HIP = 0, -1, -2, -3, -4, -5, -6
F32, BF16 = 0, 1


@pytest.fixture(scope="module")
def L():
    import rwkv_linear_attention_amd as m
    if not os.path.exists(m.LIB_PATH):
        m.build()
    return m.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(wkv7_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    assert names == sorted(["wkv7_forward", "wkv7_forward_varlen", "wkv7_step", "wkv7_step_tail",
                            "wkv7_forward_tail", "wkv7_tmix_tail", "wkv7_state_commit", "wkv7_state_reset",
                            "wkv7_backward", "wkv7_forward_ckpt", "wkv7_backward_ckpt", "wkv7_status_string",
                            "wkv7_abi_version"])


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_abi_version(L):
    src = open(HEADER).read()
    ver = int(re.search(r"#define WKV7_ABI_VERSION (\d+)", src).group(1))
    assert L.wkv7_abi_version() == ver


def test_status_strings(L):
    for st in (OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_ALIGN, ERR_ALIAS, ERR_HIP, 12345):
        s = L.wkv7_status_string(st)
        assert isinstance(s, bytes) and len(s) > 0


# Fake device addresses: far apart, 16-byte aligned.  Validation must reject
# every case below before touching them.
BASE = 1 << 40
SPAN = 1 << 34


def fake(i, off=0):
    return ctypes.c_void_p(BASE + i * SPAN + off)


def fwd(L, B=2, T=8, H=3, N=64, in_dt=BF16, o_dt=F32, ptrs=None, sin="fake", sout=None):
    p = [fake(i) for i in range(6)] if ptrs is None else ptrs
    s_in = fake(7) if sin == "fake" else sin
    s_out = fake(8) if sout is None else sout
    return L.wkv7_forward(*p, in_dt, s_in, fake(6), o_dt, s_out, B, T, H, N, None)


def step(L, B=2, T=5, H=3, N=64, pos="fake", **kw):
    p = [fake(i) for i in range(6)]
    sp = fake(9) if pos == "fake" else pos
    return L.wkv7_step(*p, BF16, fake(7), fake(6), F32, fake(8), sp, B, T, H, N, None)


@pytest.mark.parametrize("N", [0, 16, 32, 63, 65, 128])
def test_head_size_must_be_64(L, N):
    assert fwd(L, N=N) == ERR_UNSUPPORTED
    assert step(L, N=N) == ERR_UNSUPPORTED
    assert L.wkv7_state_reset(fake(8), 2, 3, N, None, None) == ERR_UNSUPPORTED


@pytest.mark.parametrize("in_dt,o_dt", [(2, F32), (-1, F32), (BF16, 7)])
def test_unknown_dtypes(L, in_dt, o_dt):
    assert fwd(L, in_dt=in_dt, o_dt=o_dt) == ERR_UNSUPPORTED


@pytest.mark.parametrize("B,T,H", [(0, 8, 3), (2, -1, 3), (2, 8, 0), (-3, 8, 3), (1 << 30, 1 << 30, 64)])
def test_bad_shapes(L, B, T, H):
    assert fwd(L, B=B, T=T, H=H) == ERR_SHAPE
    assert step(L, B=B, T=T, H=H) == ERR_SHAPE


@pytest.mark.parametrize("which", range(6))
def test_null_inputs(L, which):
    p = [fake(i) for i in range(6)]
    p[which] = None
    assert fwd(L, ptrs=p) == ERR_NULL


def test_null_outputs(L):
    p = [fake(i) for i in range(6)]
    assert L.wkv7_forward(*p, BF16, fake(7), None, F32, fake(8), 2, 8, 3, 64, None) == ERR_NULL
    assert L.wkv7_forward(*p, BF16, fake(7), fake(6), F32, None, 2, 8, 3, 64, None) == ERR_NULL
    assert L.wkv7_state_reset(None, 2, 3, 64, None, None) == ERR_NULL


@pytest.mark.parametrize("which", range(6))
def test_misaligned(L, which):
    p = [fake(i) for i in range(6)]
    p[which] = fake(which, 2)
    assert fwd(L, ptrs=p) == ERR_ALIGN
    assert fwd(L, sout=fake(8, 4)) == ERR_ALIGN
    assert L.wkv7_state_reset(fake(8, 8), 2, 3, 64, None, None) == ERR_ALIGN


def test_aliasing_rules(L):
    p = [fake(i) for i in range(6)]
    # o overlapping an input
    assert L.wkv7_forward(*p, BF16, fake(7), fake(0, 64), F32, fake(8), 2, 8, 3, 64, None) == ERR_ALIAS
    # state_out overlapping state_in without being equal to it
    assert L.wkv7_forward(*p, BF16, fake(7), fake(6), F32, fake(7, 256), 2, 8, 3, 64, None) == ERR_ALIAS
    # state_out overlapping o
    assert L.wkv7_forward(*p, BF16, fake(7), fake(6), F32, fake(6, 16), 2, 8, 3, 64, None) == ERR_ALIAS
    # state_pos overlapping state_out
    assert L.wkv7_step(*p, BF16, fake(7), fake(6), F32, fake(8), fake(8, 1024), 2, 5, 3, 64, None) == ERR_ALIAS
    # state_pos overlapping an input
    assert L.wkv7_step(*p, BF16, fake(7), fake(6), F32, fake(8), fake(3, 32), 2, 5, 3, 64, None) == ERR_ALIAS
    # row mask inside the state
    assert L.wkv7_state_reset(fake(8), 2, 3, 64, fake(8, 100), None) == ERR_ALIAS


def test_errors_come_before_any_launch(L):
    # A NULL required pointer with an otherwise impossible shape still reports one
    # of the argument errors, never a HIP error: nothing reached the runtime.
    p = [None] * 6
    st = L.wkv7_forward(*p, BF16, None, None, F32, None, 1, 4, 1, 64, None)
    assert st == ERR_NULL


def varlen(L, B=2, T=8, H=3, N=64, lengths="fake", o=None, sout=None):
    p = [fake(i) for i in range(6)]
    ln = fake(10) if lengths == "fake" else lengths
    return L.wkv7_forward_varlen(*p, BF16, fake(7), fake(6) if o is None else o, F32,
                                 fake(8) if sout is None else sout, ln, B, T, H, N, None)


def commit(L, B=2, T=5, H=3, N=64, pos="fake", acc="fake", sin="fake", sout="fake"):
    pick = lambda x, d: d if x == "fake" else x
    return L.wkv7_state_commit(pick(pos, fake(9)), pick(acc, fake(10)), pick(sin, fake(7)),
                               pick(sout, fake(8)), B, T, H, N, None)


def test_varlen_validation(L):
    # the checks of wkv7_forward apply unchanged
    assert varlen(L, N=32) == ERR_UNSUPPORTED
    assert varlen(L, B=0) == ERR_SHAPE
    # the lengths array: required, 4-byte aligned, not inside an output
    assert varlen(L, lengths=None) == ERR_NULL
    assert varlen(L, lengths=fake(10, 2)) == ERR_ALIGN
    assert varlen(L, lengths=fake(6, 8)) == ERR_ALIAS        # inside o
    assert varlen(L, lengths=fake(8, 64)) == ERR_ALIAS       # inside state_out


def test_commit_validation(L):
    assert commit(L, N=128) == ERR_UNSUPPORTED
    assert commit(L, B=0) == ERR_SHAPE
    assert commit(L, T=-1) == ERR_SHAPE
    assert commit(L, acc=None) == ERR_NULL
    assert commit(L, sout=None) == ERR_NULL
    assert commit(L, pos=None) == ERR_NULL                   # T > 0 needs the per-position states
    assert commit(L, acc=fake(10, 2)) == ERR_ALIGN
    assert commit(L, pos=fake(9, 8)) == ERR_ALIGN
    assert commit(L, sout=fake(8, 4)) == ERR_ALIGN
    assert commit(L, sin=fake(7, 8)) == ERR_ALIGN
    assert commit(L, sout=fake(9, 4096)) == ERR_ALIAS        # state_out inside state_pos
    assert commit(L, acc=fake(8, 16)) == ERR_ALIAS           # accepted inside state_out
    assert commit(L, sin=fake(8, 256)) == ERR_ALIAS          # partial overlap with state_in


def step_tail(L, B=2, T=5, H=3, N=64, gate="fake", rk="fake", x="fake", pos="fake"):
    p = [fake(i) for i in range(6)]
    pick = lambda v, d: d if v == "fake" else v
    return L.wkv7_step_tail(*p, BF16, fake(7), pick(gate, fake(11)), pick(rk, fake(12)), fake(13), fake(14),
                            ctypes.c_float(1e-5), pick(x, fake(6)), F32, fake(8), pick(pos, fake(9)), B, T, H, N, None)


def tmix(L, B=2, T=8, H=3, N=64, o="fake", x="fake", o_dt=F32, x_dt=F32, lnw="fake"):
    pick = lambda v, d: d if v == "fake" else v
    return L.wkv7_tmix_tail(pick(o, fake(6)), o_dt, fake(0), fake(2), fake(3), fake(11), BF16, fake(12),
                            pick(lnw, fake(13)), fake(14), ctypes.c_float(1e-5), pick(x, fake(8)), x_dt,
                            B, T, H, N, None)


def fwd_tail(L, B=2, T=40, H=3, N=64, in_dt=BF16, gate="fake", x="fake", x_dt=F32, sout="fake"):
    p = [fake(i) for i in range(6)]
    pick = lambda v, d: d if v == "fake" else v
    return L.wkv7_forward_tail(*p, in_dt, fake(7), pick(gate, fake(11)), fake(12), fake(13), fake(14),
                               ctypes.c_float(1e-5), pick(x, fake(6)), x_dt, pick(sout, fake(8)), B, T, H, N, None)


def test_forward_tail_validation(L):
    # every refusal comes before any launch (fake pointers)
    assert fwd_tail(L, N=32) == ERR_UNSUPPORTED
    assert fwd_tail(L, x_dt=9) == ERR_UNSUPPORTED
    assert fwd_tail(L, B=0) == ERR_SHAPE
    assert fwd_tail(L, gate=None) == ERR_NULL
    assert fwd_tail(L, x=None) == ERR_NULL
    assert fwd_tail(L, sout=None) == ERR_NULL
    assert fwd_tail(L, gate=fake(11, 8)) == ERR_ALIGN
    assert fwd_tail(L, gate=fake(6, 64)) == ERR_ALIAS      # the gate inside x
    assert fwd_tail(L, x=fake(0)) == ERR_ALIAS             # x on r
    assert fwd_tail(L, sout=fake(14)) == ERR_ALIAS         # state_out on ln_b
    assert fwd_tail(L, B=1, T=80, H=1048577) == ERR_SHAPE  # the chunked kernel's head limit
    # fp32 inputs with an fp32 x take the tail pass too, and its row limit
    assert fwd_tail(L, B=1, T=2 * 10**8 + 1, H=1, in_dt=F32) == ERR_SHAPE


def test_step_tail_validation(L):
    assert step_tail(L, N=32) == ERR_UNSUPPORTED
    assert step_tail(L, B=0) == ERR_SHAPE
    assert step_tail(L, gate=None) == ERR_NULL
    assert step_tail(L, rk=None) == ERR_NULL
    assert step_tail(L, gate=fake(11, 4)) == ERR_ALIGN
    assert step_tail(L, rk=fake(6, 64)) == ERR_ALIAS          # r_k inside x
    assert step_tail(L, gate=fake(9, 1024)) == ERR_ALIAS      # gate inside state_pos
    assert step_tail(L, x=fake(0, 16)) == ERR_ALIAS           # x inside an input


def test_tmix_tail_validation(L):
    assert tmix(L, N=128) == ERR_UNSUPPORTED
    assert tmix(L, o_dt=5) == ERR_UNSUPPORTED
    assert tmix(L, x_dt=-1) == ERR_UNSUPPORTED
    assert tmix(L, H=0) == ERR_SHAPE
    assert tmix(L, o=None) == ERR_NULL
    assert tmix(L, lnw=None) == ERR_NULL
    assert tmix(L, x=fake(8, 8)) == ERR_ALIGN
    assert tmix(L, x=fake(0, 32)) == ERR_ALIAS                # x inside r
    assert tmix(L, x=fake(6, 64)) == ERR_ALIAS                # x partly over o
    assert tmix(L, x=fake(6), x_dt=BF16) == ERR_ALIAS         # x == o with another type
    assert tmix(L, lnw=fake(8, 16)) == ERR_ALIAS              # a parameter inside x
    assert tmix(L, T=0, o=None, x=None) == OK                 # nothing to do


def test_state_out_needs_per_position_states(L):
    # state_out may be NULL only for the recurrent pass with per-position states and T > 0
    p = [fake(i) for i in range(6)]
    assert L.wkv7_step(*p, BF16, fake(7), fake(6), F32, None, None, 2, 5, 3, 64, None) == ERR_NULL
    assert L.wkv7_step(*p, BF16, fake(7), fake(6), F32, None, fake(9), 2, 0, 3, 64, None) == ERR_NULL
    assert L.wkv7_forward(*p, BF16, fake(7), fake(6), F32, None, 2, 8, 3, 64, None) == ERR_NULL


def test_launch_size_limits(L):
    # B * H beyond what one launch covers is refused on the host (the limits are
    # the header's WKV7_MAX_* values); at the limit itself validation goes on
    # (here to the overlap checks, which the fake addresses then fail).
    max_step, max_chunk, max_rows = 8000000, 4000000, 200000000
    assert fwd(L, B=max_chunk + 1, T=16, H=1) == ERR_SHAPE
    assert fwd(L, B=2000, T=9, H=2001) == ERR_SHAPE
    assert varlen(L, B=max_chunk + 1, T=16, H=1) == ERR_SHAPE
    assert fwd(L, B=max_chunk, T=16, H=1) == ERR_ALIAS
    # short sequences take the step kernel and its own limit
    assert fwd(L, B=max_chunk + 1, T=8, H=1) == ERR_ALIAS
    assert fwd(L, B=max_step + 1, T=8, H=1) == ERR_SHAPE
    assert step(L, B=max_step + 1, T=5, H=1) == ERR_SHAPE
    assert step(L, B=4000, T=5, H=2001) == ERR_SHAPE
    assert step_tail(L, B=max_step + 1, T=1, H=1) == ERR_SHAPE
    assert commit(L, B=max_step + 1, T=5, H=1) == ERR_SHAPE
    assert tmix(L, B=1, T=max_rows + 1, H=1) == ERR_SHAPE
    assert tmix(L, B=1, T=max_rows // 64 + 1, H=64) == ERR_SHAPE
    # the chunked kernel's 32-bit output offsets: H up to WKV7_MAX_H_CHUNK = 2^20
    max_h = 1048576
    assert fwd(L, B=1, T=16, H=max_h + 1) == ERR_SHAPE
    assert varlen(L, B=1, T=16, H=max_h + 1) == ERR_SHAPE
    # at the limit validation goes on (T = 80 makes o span the next fake buffer)
    assert fwd(L, B=1, T=80, H=max_h) == ERR_ALIAS
    # the step kernel (T < 9) has no such limit: validation goes on to the (forced) overlap
    assert fwd(L, B=1, T=8, H=2 * max_h, sout=fake(0)) == ERR_ALIAS


def bwd(L, B=2, T=6, H=3, N=64, in_dt=BF16, sin="fake", pos="fake", do="fake", dso="fake", grads=None,
        dsi="fake"):
    pick = lambda x, d: d if x == "fake" else x
    p = [fake(i) for i in range(6)]
    g = [fake(11 + i) for i in range(6)] if grads is None else grads
    return L.wkv7_backward(*p, in_dt, pick(sin, fake(7)), pick(pos, fake(9)), pick(do, fake(10)),
                           pick(dso, fake(17)), *g, pick(dsi, fake(18)), B, T, H, N, None)


def test_backward_validation(L):
    assert bwd(L, N=32) == ERR_UNSUPPORTED
    assert bwd(L, in_dt=5) == ERR_UNSUPPORTED
    assert bwd(L, B=0) == ERR_SHAPE
    assert bwd(L, T=-1) == ERR_SHAPE
    assert bwd(L, B=8000001, H=1) == ERR_SHAPE
    assert bwd(L, dsi=None) == ERR_NULL
    assert bwd(L, pos=None) == ERR_NULL
    assert bwd(L, do=None) == ERR_NULL
    for q in range(6):
        g = [fake(11 + i) for i in range(6)]
        g[q] = None
        assert bwd(L, grads=g) == ERR_NULL
    assert bwd(L, dsi=fake(18, 4)) == ERR_ALIGN
    assert bwd(L, do=fake(10, 8)) == ERR_ALIGN
    # an output on an input, on another output, or on part of d_state_out
    assert bwd(L, dsi=fake(9)) == ERR_ALIAS
    g = [fake(11 + i) for i in range(6)]
    g[3] = fake(11)
    assert bwd(L, grads=g) == ERR_ALIAS
    g = [fake(11 + i) for i in range(6)]
    g[0] = fake(2, 64)
    assert bwd(L, grads=g) == ERR_ALIAS
    assert bwd(L, dsi=fake(17, 256)) == ERR_ALIAS
    # a gradient inside d_state_out, which the pass reads
    for q in range(6):
        g = [fake(11 + i) for i in range(6)]
        g[q] = fake(17, 1024)
        assert bwd(L, grads=g) == ERR_ALIAS, q
    # T = 0 needs only d_state_in
    assert L.wkv7_backward(*([None] * 6), BF16, None, None, None, None, *([None] * 6), None, 2, 0, 3, 64,
                           None) == ERR_NULL


def fck(L, B=2, T=40, H=3, N=64, in_dt=BF16, sin="fake", o=None, ck="fake"):
    pick = lambda x, d: d if x == "fake" else x
    p = [fake(i) for i in range(6)]
    return L.wkv7_forward_ckpt(*p, in_dt, pick(sin, fake(7)), fake(6) if o is None else o, fake(8),
                               pick(ck, fake(9)), B, T, H, N, None)


def bck(L, B=2, T=30, H=3, N=64, in_dt=BF16, ck="fake", do="fake", grads=None, dsi="fake"):
    pick = lambda x, d: d if x == "fake" else x
    p = [fake(i) for i in range(6)]
    g = [fake(11 + i) for i in range(6)] if grads is None else grads
    return L.wkv7_backward_ckpt(*p, in_dt, pick(ck, fake(9)), pick(do, fake(10)), fake(17), *g,
                                pick(dsi, fake(18)), B, T, H, N, None)


def test_forward_ckpt_validation(L):
    assert fck(L, N=32) == ERR_UNSUPPORTED
    assert fck(L, in_dt=7) == ERR_UNSUPPORTED
    assert fck(L, B=0) == ERR_SHAPE
    assert fck(L, ck=None) == ERR_NULL
    assert fck(L, ck=fake(9, 8)) == ERR_ALIGN
    assert fck(L, ck=fake(6, 4096)) == ERR_ALIAS   # inside o
    assert fck(L, ck=fake(2, 256)) == ERR_ALIAS    # inside k
    assert fck(L, ck=fake(7, 16)) == ERR_ALIAS     # inside state_in
    # [2, ceil(40/16) = 3, 3, 64, 64] fp32: o just below the checkpoints' end overlaps them
    assert fck(L, o=fake(9, 2 * 3 * 3 * 64 * 64 * 4 - 16)) == ERR_ALIAS


def test_backward_ckpt_validation(L):
    assert bck(L, N=16) == ERR_UNSUPPORTED
    assert bck(L, T=-1) == ERR_SHAPE
    assert bck(L, ck=None) == ERR_NULL
    assert bck(L, do=None) == ERR_NULL
    assert bck(L, dsi=None) == ERR_NULL
    assert bck(L, ck=fake(9, 4)) == ERR_ALIGN
    assert bck(L, dsi=fake(9)) == ERR_ALIAS
    # T = 30: two chunks, [2, 2, 3, 64, 64] fp32; a gradient inside the second overlaps
    g = [fake(11 + i) for i in range(6)]
    g[2] = fake(9, 2 * 2 * 3 * 64 * 64 * 4 - 16)
    assert bck(L, grads=g) == ERR_ALIAS
    g = [fake(11 + i) for i in range(6)]
    g[4] = fake(10, 128)   # inside d_o
    assert bck(L, grads=g) == ERR_ALIAS
