"""The Python binding's argument checks, on the CPU.

The C ABI cannot see buffer sizes, so the binding refuses an output tensor of
the wrong shape, dtype, layout or device before any pointer reaches the
library.  These run the checks themselves with CPU tensors (a CPU tensor never
reaches the library: every wrapper first requires GPU inputs)."""
import pytest
import torch

import rwkv_linear_attention_amd as K

GPU = torch.device("cuda", 0)
CPU = torch.device("cpu")


def test_out_arg_accepts_a_matching_output():
    x = torch.empty((2, 5, 3, 64))
    assert K._out_arg(x, (2, 5, 3, 64), CPU, "o") is x
    xb = torch.empty((2, 5, 3, 64), dtype=torch.bfloat16)
    assert K._out_arg(xb, (2, 5, 3, 64), CPU, "o") is xb


@pytest.mark.parametrize("case", ["short", "long", "strided", "dtype", "device", "not a tensor"])
def test_out_arg_refuses(case):
    shape = (2, 5, 3, 64)
    x = {
        "short": torch.empty((2, 4, 3, 64)),
        "long": torch.empty((2, 6, 3, 64)),
        "strided": torch.empty((2, 5, 3, 128))[..., ::2],
        "dtype": torch.empty(shape, dtype=torch.float16),
        "device": torch.empty(shape),
        "not a tensor": [0.0] * 10,
    }[case]
    dev = GPU if case == "device" else CPU
    with pytest.raises(ValueError):
        K._out_arg(x, shape, dev, "o")


def test_out_arg_fp32_only_outputs():
    # per-position states and gradients are fp32 only
    sp = torch.empty((2, 5, 3, 64, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        K._out_arg(sp, (2, 5, 3, 64, 64), CPU, "state_pos", (torch.float32,))


def test_state_arg_checks_shape_dtype_layout_device():
    B, H, N = 2, 3, 64
    ok = torch.empty((B, H, N, N))
    assert K._state_arg(ok, B, H, N, CPU, "state_in") is ok
    assert K._state_arg(None, B, H, N, CPU, "state_in") is None
    bad = [torch.empty((B, H, N, N - 1)), torch.empty((B, H, N, N), dtype=torch.bfloat16),
           torch.empty((B, H, N, 2 * N))[..., ::2]]
    for x in bad:
        with pytest.raises(ValueError):
            K._state_arg(x, B, H, N, CPU, "state_in")
    with pytest.raises(ValueError):
        K._state_arg(ok, B, H, N, GPU, "state_in")


def test_wrappers_refuse_cpu_inputs():
    # the product path has no CPU fallback: CPU tensors are refused outright
    x = torch.zeros((1, 4, 2, 64))
    with pytest.raises(ValueError):
        K.wkv7_forward(x, x, x, x, x, x)
    with pytest.raises(ValueError):
        K.wkv7_step(x, x, x, x, x, x)
