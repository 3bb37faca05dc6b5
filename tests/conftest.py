import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle

    oracle.build(force=False)
    return oracle


def golden(name):
    """Parse a golden fixture: '# ...' lines are citations, others 'key = value'."""
    out = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split("=", 1)
            out[k.strip()] = v.strip()
    return out


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """One line per parity comparison of the session: worst |dO| / bound and the
    rows whose flip budget is nonzero (the evidence behind each passing case)."""
    helpers = sys.modules.get("helpers")
    rows = getattr(helpers, "PARITY", None)
    if not rows:
        return
    tr = terminalreporter
    tr.write_sep("-", f"parity against the oracle: {len(rows)} comparisons")
    for name, ratio, nf, n, med in rows:
        tr.write_line(f"parity {name}: max |dO|/bound {ratio:.3e}, flip budget on {nf}/{n} rows "
                      f"(median budget/tolerance {med:.2e})")
    worst = max(rows, key=lambda r: r[1])
    tr.write_line(f"parity worst: {worst[0]} at {worst[1]:.3e}; "
                  f"largest fragile share {max(r[2] / max(r[3], 1) for r in rows):.3f}")
