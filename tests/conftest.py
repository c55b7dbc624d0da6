import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_sessionstart(session):
    # The C-ABI library is a build product (git-ignored).  Cross-compile it
    # once if this tree does not have it yet; hipcc needs no GPU for that.
    lib = os.path.join(ROOT, "heterogeneous_rank_gemm_amd", "libhrglora.so")
    if not os.path.exists(lib):
        import runpy
        runpy.run_path(os.path.join(ROOT, "heterogeneous_rank_gemm_amd", "build.py"),
                       run_name="hrg_build")["build"]()
