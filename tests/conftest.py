import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


def pytest_sessionstart(session):
    """A GPU session starts the host pool for the oracle before any test touches the GPU."""
    expr = session.config.getoption("markexpr", "") or ""
    if "gpu" in expr and "not gpu" not in expr:
        from tests import oracle_pool
        try:
            oracle_pool.start()
        except OSError as e:                 # the checks then run in the test process
            print(f"[conftest] no oracle pool ({e}); oracle checks run in-process", flush=True)


def pytest_sessionfinish(session, exitstatus):
    from tests import oracle_pool
    oracle_pool.stop()
