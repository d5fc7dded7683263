import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    # MD_SANITIZE=1: the CPU tests against the sanitizer builds of the oracle
    # and of the library's host code (oracle.build(sanitize=True),
    # python -m moe_decode_amd.build --sanitize; the clang ASan runtime preloaded)
    if os.environ.get("MD_SANITIZE") == "1":
        import moe_decode_amd as md
        md.LIBPATH = os.path.join(ROOT, "moe_decode_amd", "libmoe_decode_san.so")
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU work (full-size oracle runs)")


@pytest.fixture(scope="session")
def orc():
    import oracle
    if not os.path.exists(oracle.LIB):
        oracle.build()
    return oracle.Oracle(threads=1)


@pytest.fixture(scope="session")
def orc_mt():
    import oracle
    if not os.path.exists(oracle.LIB):
        oracle.build()
    o = oracle.Oracle(threads=min(16, os.cpu_count() or 1))
    return o
