"""A process pool that runs the CPU oracle over independent units (test infrastructure).

The full-size parity tests compare every unit (batch row x KV head) of a
workload, and the oracle is plain single-threaded NumPy, so the per-unit jobs
are spread over the host's cores.  Workers are forked from a forkserver, a fresh
interpreter that never touches the GPU; each job regenerates its unit's inputs
from the seeded generator (so no large arrays cross process boundaries) and
returns the oracle's results.  BLAS runs single-threaded inside a worker.
"""
import concurrent.futures as cf
import multiprocessing as mp
import multiprocessing.forkserver as mpfs
import os

_POOL = None
MAX_WORKERS = 16     # the host share of one GPU on the machines these tests run on


def n_workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(MAX_WORKERS, n))


def _init_worker():
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)


def start():
    """Start the forkserver now (call before the GPU is initialised, so that the
    server is a clean interpreter from the start)."""
    ctx = mp.get_context("forkserver")
    ctx.set_forkserver_preload(["numpy", "oracle", "workloads"])
    mpfs.ensure_running()


def pool():
    global _POOL
    if _POOL is None:
        start()
        _POOL = cf.ProcessPoolExecutor(n_workers(), mp_context=mp.get_context("forkserver"),
                                       initializer=_init_worker)
    return _POOL


def pmap(fn, items):
    """[fn(x) for x in items], computed in the pool, in order."""
    items = list(items)
    if not items:
        return []
    return list(pool().map(fn, items))


def shutdown():
    global _POOL
    if _POOL is not None:
        _POOL.shutdown(wait=True, cancel_futures=True)
        _POOL = None
