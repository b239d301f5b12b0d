import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "fullsize: a workload-sized GPU parity test")


def pytest_sessionstart(session):
    """Build the HIP library once if it is missing (tests only ever load a built one)."""
    import compressed_sparse_kv_csa_amd as ck
    if not os.path.exists(ck.lib_path()):
        from compressed_sparse_kv_csa_amd import build
        build.build()
