import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def _ensure_built():
    """Build the library, the oracle and the C driver once if a fresh checkout
    has none of them yet (an existing build is used as it is)."""
    needed = [os.path.join(ROOT, "moe_expert_output_finalize_amd", "libmoe_finalize.so"),
              os.path.join(ROOT, "oracle", "liboracle.so"),
              os.path.join(TESTS, "capi_c_driver")]
    if not all(os.path.exists(p) for p in needed):
        import __graft_entry__
        __graft_entry__.build()


_ensure_built()


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
