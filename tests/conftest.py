import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


GOLDEN = os.path.join(ROOT, "tests", "golden")


_WORST = []


@pytest.fixture(autouse=True)
def _record_worst_ratios(request):
    """Per test, the worst row error and element ratio of assert_rows_close."""
    import helpers

    helpers.WORST.update(row=0.0, elem=0.0, elem_free=0.0, what="")
    yield
    W = helpers.WORST
    if W["row"] or W["elem"] or W["elem_free"]:
        _WORST.append((request.node.nodeid, W["row"], W["elem"], W["elem_free"], W["what"]))


def pytest_terminal_summary(terminalreporter):
    if not _WORST:
        return
    terminalreporter.write_line("worst GPU-vs-oracle ratios per test: row rel-L2, max |d|/(|ref|+rms) in "
                                "lock-step / teacher-forced checks (where), and in free-running checks")
    for nodeid, row, elem, free, what in _WORST:
        terminalreporter.write_line(f"  {row:.3e}  {elem:.3e} ({what})  {free:.3e}  {nodeid}")
