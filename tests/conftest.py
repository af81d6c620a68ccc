import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    if not os.path.exists(oracle.LIB_PATH):
        oracle.build(force=False)
    return oracle


@pytest.fixture(scope="session")
def device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """How many compared requests differed from the oracle and were accepted
    by the step-wise near-tie validator (gpu_util.assert_parity)."""
    import gpu_util
    t = gpu_util.NEAR_TIE_TOTAL
    if t["requests"]:
        terminalreporter.write_line(
            f"[near-tie] {t['accepted']} of {t['requests']} compared requests differed from the oracle "
            f"within the {gpu_util.SCORE_TOL:g} band (every other request matched exactly)")
