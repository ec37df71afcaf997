import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _keep_large_temporaries_on_the_heap():
    """The oracle's numpy temporaries at the full workload sizes are tens to
    hundreds of MB.  By default glibc maps each one afresh and returns it on
    free, so every call pays the page faults of its temporaries again (10x the
    arithmetic, measured).  Raising the mmap and trim thresholds lets freed
    blocks be reused.  Allocation policy only: no value changes."""
    import ctypes
    try:
        libc = ctypes.CDLL("libc.so.6")
        libc.mallopt(-3, 1 << 30)    # M_MMAP_THRESHOLD
        libc.mallopt(-1, 1 << 32)    # M_TRIM_THRESHOLD
    except OSError:   # pragma: no cover (not glibc)
        pass


_keep_large_temporaries_on_the_heap()


@pytest.fixture(scope="session")
def linear3b_inputs():
    """The 3B-shape projection's seeded inputs (X, W split into U, V, R; dY),
    drawn once per test session: the randomized low-rank split takes ~20 s."""
    import synth
    return synth.linear3b(), synth.linear3b_dy()
