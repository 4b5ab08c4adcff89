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
def moe_share():
    """One GPU's MoE share at full size (65536 routed rows over 8 experts), drawn once per session."""
    from fp8_fine_grained_amax_amd import workloads as wl
    return wl.moe_inputs()


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    oracle.lib()
    return oracle


def pytest_terminal_summary(terminalreporter):
    """The GEMM parity checks' error figures: the normwise gate and the elementwise error over the entries
    at least 1% of the largest."""
    mod = sys.modules.get("tests.gpu_util")
    rows = getattr(mod, "GEMM_ERRORS", None) if mod else None
    if not rows:
        return
    tr = terminalreporter
    tr.section("GEMM errors against the oracle (normwise gate | elementwise over |ref| >= 1% max)")
    for name, what, n, nw, ew in rows:
        tr.write_line(f"{name[:70]:70s} {what:12s} n={n:<9d} normwise {nw:.2e}  elementwise {ew:.2e}")
