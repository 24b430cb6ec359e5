import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload parity (GPU box only)")


@pytest.fixture(autouse=True)
def _no_unread_device_flags(request):
    """GPU tests: every library workspace a test creates must end the test with no device-error flag
    (SSD_FLAG_*) left in it. A test that expects a flag reads it, which clears it; any other flag,
    such as a wait that ran out, fails the test here."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    import draft_verification_ssd_amd._lib as L
    made = []
    orig = L.Workspace.__init__

    def init(self, *a, **k):
        orig(self, *a, **k)
        made.append(self)

    L.Workspace.__init__ = init
    try:
        yield
    finally:
        L.Workspace.__init__ = orig
    for ws in made:
        f = L.ssd_read_flags(ws)
        assert f == 0, f"a workspace of this test was left with device flags {f:#x}"
