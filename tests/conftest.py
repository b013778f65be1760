import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def _library_is_current() -> bool:
    """Whether libmoe_finalize.so exists and its recorded source digest
    matches the sources in this tree."""
    import importlib.util
    pkg = os.path.join(ROOT, "moe_expert_output_finalize_amd")
    spec = importlib.util.spec_from_file_location("_mf_build", os.path.join(pkg, "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    try:
        with open(b.digest_path(b.LIB)) as f:
            return f.read().strip() == b.source_digest(ROOT)
    except OSError:
        return False


def _ensure_built():
    """Build the library, the oracle, the C driver and the host-check library
    when one is missing or the library is older than its sources.  Only where
    no GPU is present (the build container): on a GPU machine the tests use
    what was built beforehand, and the binding refuses a stale library."""
    needed = [os.path.join(ROOT, "oracle", "liboracle.so"),
              os.path.join(TESTS, "capi_c_driver"),
              os.path.join(TESTS, "libmf_hostcheck.so")]
    if all(os.path.exists(p) for p in needed) and _library_is_current():
        return
    if os.path.exists("/dev/kfd"):
        return
    import __graft_entry__
    __graft_entry__.build()


_ensure_built()


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
