import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _ensure_built():
    """A fresh checkout has no libmoe.so: build it (hipcc cross-compiles here)."""
    lib = os.path.join(ROOT, "expert_token_dispatch_amd", "libmoe.so")
    if not os.path.exists(lib) and os.path.exists("/opt/rocm/bin/hipcc"):
        from expert_token_dispatch_amd.build import build
        build()


_ensure_built()
