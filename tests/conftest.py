import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


import pytest  # noqa: E402


@pytest.fixture
def plan_override():
    """Set the library's plan overrides for one test (fp_plan_override_set);
    the previous values are restored afterwards."""
    import fusion_residual_add_amd as fra
    prev = fra.get_plan_override()

    def set_(**values):
        fra.set_plan_override(values)

    yield set_
    fra.set_plan_override(prev)
