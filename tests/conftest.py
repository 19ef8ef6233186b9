import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU-oracle case")


@pytest.fixture(scope="session")
def orc():
    import oracle

    oracle.lib()
    return oracle


def pytest_terminal_summary(terminalreporter):
    """Reports every use of the fp64 fallback of the y verdict (tests/cases.py)."""
    try:
        from cases import FALLBACKS
    except ImportError:
        return
    terminalreporter.write_line(f"y verdict: {len(FALLBACKS)} use(s) of the fp64-oracle fallback")
    for what, r32, floor, r64 in FALLBACKS:
        terminalreporter.write_line(
            f"  {what}: vs fp32 oracle {r32[0]:.3e}/{r32[1]:.3e}, fp32 vs fp64 oracle "
            f"{floor[0]:.3e}/{floor[1]:.3e}, vs fp64 oracle {r64[0]:.3e}/{r64[1]:.3e}")
