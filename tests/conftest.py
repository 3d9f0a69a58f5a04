import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the HIP library")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    # The oracle is plain C; build it once if this tree has no copy yet.
    import oracle
    if not os.path.exists(oracle.lib_path()):
        oracle.build()
    if not os.path.exists(oracle.gdn.lib_path()):
        oracle.gdn.build()
    yield


def pytest_terminal_summary(terminalreporter):
    """Per test, the worst tolerance margin (max |err| / bound; 1.0 = the
    tolerance) and normwise relative error of its GPU-vs-oracle comparisons.
    With SSM_MARGINS_OUT set, every comparison is also written there as JSON."""
    try:
        from tests.gpu_helpers import MARGINS
    except ImportError:
        return
    if not MARGINS:
        return
    worst = {}
    for test, what, margin, nrel, n in MARGINS:
        w = worst.get(test)
        if w is None or margin > w[1]:
            worst[test] = (what, margin, max(nrel, w[2] if w else 0.0))
        elif nrel > w[2]:
            worst[test] = (w[0], w[1], nrel)
    tr = terminalreporter
    tr.write_sep("-", "parity margins (max |gpu-ref| / tolerance bound per test)")
    for test, (what, margin, nrel) in sorted(worst.items()):
        tr.write_line(f"{margin:8.4f}  nrel {nrel:.2e}  {test} [{what}]")
    out = os.environ.get("SSM_MARGINS_OUT")
    if out:
        import json
        with open(out, "w") as f:
            json.dump([dict(test=t, what=w, margin=m, normwise_rel=r, elements=n)
                       for t, w, m, r, n in MARGINS], f, indent=0)
