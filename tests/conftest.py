import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")
    config.addinivalue_line("markers", "slow: large CPU work (full-size workloads)")


@pytest.fixture(scope="session")
def orc():
    import oracle

    override = os.environ.get("MOE_ORACLE_LIB_OVERRIDE")
    if override:  # a deliberately mutated oracle build, loaded by the mutation test's subprocesses
        return oracle.OracleLib(override)
    oracle.build(force=False)
    return oracle.default()
