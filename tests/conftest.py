import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle

    oracle.build(force=False)
    return oracle


def pytest_terminal_summary(terminalreporter):
    import sys

    mod = sys.modules.get("gpu_util")
    recs = getattr(mod, "RECORDS", None) if mod else None
    if not recs:
        return
    total = sum(r[1] for r in recs)
    near = sum(r[2] for r in recs)
    terminalreporter.write_line(
        f"chain parity: {len(recs)} comparisons, {total} blocks compared exactly, "
        f"{near} blocks inside the 1e-6 boundary band (excluded)")
    groups = {}
    for label, n, b in recs:
        key = label.split("-s")[0].split("-u")[0]
        g = groups.setdefault(key, [0, 0])
        g[0] += n
        g[1] += b
    for key, (n, b) in sorted(groups.items()):
        terminalreporter.write_line(f"  {key}: compared {n}, in band {b}")
