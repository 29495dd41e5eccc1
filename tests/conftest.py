"""Shared test setup: repository root on sys.path, the `gpu` marker, and the built libraries."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def oracle_lib():
    """Path of the oracle library, built once per session if it is missing."""
    import oracle

    if not os.path.exists(oracle.lib_path()):
        oracle.build()
    return oracle.lib_path()


@pytest.fixture
def decode_kernel():
    """Force a decode kernel for one test ("valu" or "mfma"; pa_set_decode_kernel), restoring
    the automatic choice afterwards."""
    import paged_kv_cache_82_amd as pa

    yield pa.pa_set_decode_kernel
    pa.pa_set_decode_kernel("auto")


def pytest_terminal_summary(terminalreporter):
    """Observed errors of the full-size parity runs (and their ratios to the pass rule and to
    the tight regression bound), so the run's record shows how far below the bounds they sit."""
    try:
        from gpu_harness import PARITY_LOG
    except Exception:  # no torch / not a GPU session
        return
    if PARITY_LOG:
        terminalreporter.write_line("full-size parity (observed max errors):")
        for line in PARITY_LOG:
            terminalreporter.write_line("  " + line)
        # the same lines as JSON, when PA_PARITY_JSON names a file to write them to
        path = os.environ.get("PA_PARITY_JSON")
        if path:
            import json

            try:
                os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
                with open(path, "w") as f:
                    json.dump({"full_size_parity": list(PARITY_LOG)}, f, indent=1)
            except OSError:
                pass
