import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Oracle worker processes for the full-size GPU parity tests.  They are
# started when the collected tests include GPU tests, at the end of
# collection -- before any test runs, so before this process touches the
# GPU -- with the "spawn" start method; they import numpy and the oracle only
# and never touch the GPU.
_POOL = None


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _worker_init():
    import oracle
    oracle.build(force=False)


def pytest_collection_finish(session):
    global _POOL
    if _POOL is None and any(it.get_closest_marker("gpu") for it in session.items):
        import multiprocessing as mp
        _POOL = mp.get_context("spawn").Pool(_workers(), initializer=_worker_init)


def pytest_sessionfinish(session, exitstatus):
    global _POOL
    if _POOL is not None:
        _POOL.terminate()
        _POOL.join()
        _POOL = None


@pytest.fixture(scope="session")
def oracle_pool():
    """The oracle worker pool (None when no GPU test was collected)."""
    return _POOL


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    from tests import _parity as P
    if not P.LOG:
        return
    tr = terminalreporter
    tr.write_sep("-", "parity against the oracle: near-tie rows and exact boundary ties")
    tr.write_line(f"{'comparison':52s} {'(head,row) pairs':>16s} {'near-tie rows':>13s} "
                  f"{'bound':>6s} {'exact ties':>10s}")
    for label, pairs, near, ties in P.LOG:
        tr.write_line(f"{label[:52]:52s} {pairs:16d} {near:13d} {P.near_tie_bound(pairs):6d} "
                      f"{ties:10d}")
    tot = [sum(x[i] for x in P.LOG) for i in (1, 2, 3)]
    tr.write_line(f"{'total':52s} {tot[0]:16d} {tot[1]:13d} {'':6s} {tot[2]:10d}")
