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


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Per-case output errors of every GPU parity check that ran (relative to rms(ref); "bar" is the
    form of the max bar asserted: the raw error, or the excess over bf16 rounding where even the
    exactly rounded result misses 2e-2)."""
    gpu_helpers = sys.modules.get("_gpu")  # imported only by the GPU tests that ran
    PARITY_ROWS = getattr(gpu_helpers, "PARITY_ROWS", None)
    if not PARITY_ROWS:
        return
    tr = terminalreporter
    tr.section("output parity against the oracle (max bar 2e-2*rms, mean bar 5e-3)")
    tr.write_line(f"{'case':<58} {'max|err|/rms':>12} {'bf16 floor':>11} {'excess':>10} {'l1':>10} bar")
    for label, raw, floor, excess, l1, bar in PARITY_ROWS:
        tr.write_line(f"{label[:58]:<58} {raw:12.3e} {floor:11.3e} {excess:10.3e} {l1:10.3e} {bar}")
    n_raw = sum(1 for r in PARITY_ROWS if r[5] == "raw")
    tr.write_line(f"{len(PARITY_ROWS)} checks: {n_raw} on the raw error, {len(PARITY_ROWS) - n_raw} on the excess; "
                  f"largest raw where asserted {max([r[1] for r in PARITY_ROWS if r[5] == 'raw'] or [0]):.3e}")
