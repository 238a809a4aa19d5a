import pytest
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture
def no_stream_k():
    """Rules Stream-K plans out for the test (tests of the split-K and one-tile
    plans, whose shapes the cost model may otherwise give to Stream-K)."""
    import dense_gemm_matrix_amd as dg
    dg.dgemm_set_plan_override(dg.DGEMM_PLAN_NO_STREAM_K)
    yield
    dg.dgemm_set_plan_override(dg.DGEMM_PLAN_AUTO)
