import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


import pytest  # noqa: E402


def _ensure_built():
    lib = os.path.join(ROOT, "gemm_decode_amd", "libwq.so")
    if not os.path.exists(lib):
        from gemm_decode_amd import build as _b
        _b.build()


@pytest.fixture(scope="session")
def wqlib():
    """The Python binding of the built library (built first if nothing is built)."""
    _ensure_built()
    import gemm_decode_amd.wq as wq
    return wq


@pytest.fixture(autouse=True)
def _name_the_gpu_case(request):
    """Before each GPU test, print its id to stderr (flushed), so that a run which
    ends abruptly still names the case it was in."""
    if request.node.get_closest_marker("gpu") is not None:
        sys.stderr.write(f"[gpu case] {request.node.nodeid}\n")
        sys.stderr.flush()
    yield
