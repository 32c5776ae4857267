import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: large workload, minutes of host time")


_hip = None


def _hip_runtime():
    """The HIP runtime already loaded in this process (None if none is)."""
    global _hip
    if _hip is None:
        import ctypes
        try:
            _hip = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD | os.RTLD_GLOBAL)
            _hip.hipPeekAtLastError.restype = ctypes.c_int
            _hip.hipGetLastError.restype = ctypes.c_int
            _hip.hipGetErrorString.restype = ctypes.c_char_p
            _hip.hipGetErrorString.argtypes = [ctypes.c_int]
        except OSError:
            _hip = False
    return _hip or None


import pytest  # noqa: E402


@pytest.fixture(autouse=True)
def _no_pending_hip_error(request):
    """A GPU test must not leave a HIP error pending on its thread: the next
    unrelated HIP call would report it."""
    yield
    if request.node.get_closest_marker("gpu") is None:
        return
    hip = _hip_runtime()
    if hip is None:
        return
    e = hip.hipPeekAtLastError()
    if e != 0:
        hip.hipGetLastError()  # clear it so that the next test starts clean
        pytest.fail("HIP error %d (%s) left pending by this test" % (e, hip.hipGetErrorString(e).decode()))
