import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def orc():
    """The oracle under test; ORACLE_LIB selects a variant build (used by the mutant tests)."""
    import oracle
    path = os.environ.get("ORACLE_LIB")
    if path:
        return oracle.Oracle(path)
    oracle.build()
    return oracle.get()


@pytest.fixture(scope="session")
def synth():
    import synth_inputs
    synth_inputs.build()
    return synth_inputs


@pytest.fixture(scope="session")
def q():
    """The HIP library through its binding (GPU tests only)."""
    import torch
    import weight_quantization_codec_amd as qamw
    qamw.load()
    assert torch.cuda.is_available()
    return qamw
