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
    """Totals of every GPU-vs-oracle comparison of the run, by kind: results
    compared exactly, results inside the 1e-6 boundary band (each checked
    against the oracle's admissible outcomes), blocks outside the library's
    numeric domain (checked to be flagged), near-ties and swaps."""
    import sys

    mod = sys.modules.get("gpu_util")
    recs = getattr(mod, "RECORDS", None) if mod else None
    if not recs:
        return
    kinds = {}
    for r in recs:
        agg = kinds.setdefault(r["kind"], {"comparisons": 0})
        agg["comparisons"] += 1
        for key, val in r.items():
            if key not in ("kind", "label"):
                agg[key] = agg.get(key, 0) + val
    terminalreporter.write_line("GPU-vs-oracle parity totals (band/near-tie results are checked "
                                "against the oracle's admissible outcomes, none left unchecked):")
    for kind in sorted(kinds):
        parts = ", ".join(f"{k} {v}" for k, v in kinds[kind].items())
        terminalreporter.write_line(f"  {kind}: {parts}")
    groups = {}
    for r in recs:
        key = (r["kind"], r["label"].split("-s")[0].split("-u")[0])
        g = groups.setdefault(key, {})
        for k, v in r.items():
            if k not in ("kind", "label"):
                g[k] = g.get(k, 0) + v
    for (kind, label), g in sorted(groups.items()):
        parts = ", ".join(f"{k} {v}" for k, v in g.items())
        terminalreporter.write_line(f"    {kind} {label}: {parts}")
