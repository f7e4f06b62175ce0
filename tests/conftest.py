import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads (seconds of host work)")


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded HIP library plus torch on cuda:0; fails loudly if either is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a host without a GPU")
    from transformer_ffn_block_amd import ffn
    return ffn.lib()


def pytest_sessionfinish(session, exitstatus):
    """Write the achieved parity errors of this session (tests/helpers.record)
    to the file FFN_PARITY_LOG names, one JSON object per case."""
    path = os.environ.get("FFN_PARITY_LOG")
    if not path:
        return
    helpers = sys.modules.get("helpers")
    if helpers is None or not getattr(helpers, "PARITY", None):
        return
    import json
    d = os.path.dirname(path)
    if d:
        os.makedirs(d, exist_ok=True)
    with open(path, "w") as fh:
        for row in helpers.PARITY:
            fh.write(json.dumps(row) + "\n")
