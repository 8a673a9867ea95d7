import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle.build(force=False)
    return oracle


@pytest.fixture(scope="session")
def workload3_oracle(oracle_mod):
    """The fp64 oracle over the whole 7.2B-shaped prefill workload (B=4, T=8192, H=64:
    every head, the full sequence), computed once per session: (inputs, o, state_out)."""
    import synth
    inp = synth.workload_inputs(3)
    o_ref, s_ref = oracle_mod.forward(*(inp[n] for n in ("r", "w", "k", "v", "a", "b")), inp["state_in"])
    return inp, o_ref, s_ref
