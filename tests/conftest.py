import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "bad_pages: the test plants page-table entries outside "
                                       "the pool on purpose (poisoned parts are expected)")


@pytest.fixture(autouse=True)
def _decode_status_is_clean(request):
    """Every decode workspace a GPU test allocates is checked after the test:
    no block of any launch on it may have run out of a bounded wait (status
    word 0), and no part may have been poisoned by a page-table entry outside
    the pool (status word 1) unless the test plants such entries."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    import torch
    import bit_kv_cache_amd as kvq
    made = []
    orig = kvq.decode_workspace

    def tracked(nbytes, device="cuda"):
        ws = orig(nbytes, device)
        made.append(ws)
        return ws

    kvq.decode_workspace = tracked
    try:
        yield
    finally:
        kvq.decode_workspace = orig
    torch.cuda.synchronize()
    allow_bad = request.node.get_closest_marker("bad_pages") is not None
    for i, ws in enumerate(made):
        stalled, bad = kvq.workspace_status(ws)
        assert stalled == 0, f"workspace {i}: {stalled} decode block(s) ran out of a bounded wait"
        assert allow_bad or bad == 0, f"workspace {i}: {bad} part(s) poisoned by a bad page"



def pytest_terminal_summary(terminalreporter):
    """Largest attention error of each GPU test against the oracle (max-abs
    over all its comparisons), worst first."""
    pu = sys.modules.get("parity_util")
    if pu is None or not pu.ERRORS:
        return
    worst = {}
    for test, err in pu.ERRORS:
        worst[test] = max(worst.get(test, 0.0), err)
    rows = sorted(worst.items(), key=lambda kv: -kv[1])
    tr = terminalreporter
    tr.write_sep("-", f"max-abs attention error vs the oracle ({len(pu.ERRORS)} comparisons, "
                      f"{len(rows)} tests; bar 2e-3 unless the test scales it)")
    for test, err in rows[:25]:
        tr.write_line(f"{err:10.3e}  {test}")
