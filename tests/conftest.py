import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
for p in (ROOT, os.path.dirname(os.path.abspath(__file__))):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long CPU test")


def _ensure_built():
    """Build only what is missing (the C oracle / generator are seconds to build)."""
    import __graft_entry__ as ge
    need_c = not (os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so"))
                  and os.path.exists(os.path.join(ROOT, "synth", "libsynth.so")))
    if need_c:
        ge.build_c()
    have_src = any(f.endswith((".cpp", ".hip"))
                   for f in os.listdir(os.path.join(ROOT, "allreduce_reduction_amd", "csrc")))
    if have_src and not os.path.exists(os.path.join(ROOT, "allreduce_reduction_amd", "libhbmcoll.so")):
        ge.build_hip()


_ensure_built()
