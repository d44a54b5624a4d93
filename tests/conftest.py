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
def oracle_lib():
    import oracle
    oracle.build(force=False)
    return oracle


def pytest_terminal_summary(terminalreporter):
    """Worst per-(sequence, head) relative L2 of each parity test that ran."""
    try:
        from tests.helpers import CHAIN_RECORDS
    except ImportError:
        return
    if not CHAIN_RECORDS:
        return
    per_test = {}
    for tid, _label, wo, wf in CHAIN_RECORDS:
        o, f, n = per_test.get(tid, (0.0, 0.0, 0))
        per_test[tid] = (max(o, wo), max(f, wf or 0.0), n + 1)
    tr = terminalreporter
    tr.write_sep("-", "worst per-(sequence, head) relative L2 (bar 2e-2)")
    for tid, (o, f, n) in per_test.items():
        tr.write_line("%-90s out %.3e  state %.3e  (%d checks)" % (tid[-90:], o, f, n))
    wo = max(v[0] for v in per_test.values())
    wf = max(v[1] for v in per_test.values())
    tr.write_line("overall worst chain: out %.3e  state %.3e over %d checks" % (wo, wf, len(CHAIN_RECORDS)))
