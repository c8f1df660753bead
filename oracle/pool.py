"""Process pool for the oracle's row samples (test infrastructure only).

Query rows are independent: a row's output, log-sum-exp and dQ depend only
on that row and the keys it sees.  Large row samples of the full-size
workloads are therefore split into chunks and evaluated in worker processes,
one BLAS thread each, by the very same row functions the serial path uses
(``attention._rows_forward`` and ``backward._rows_dq``); the pool adds no
arithmetic of its own.

K, V and the segment metadata are written once to ``.npy`` files in a
memory-backed temporary directory and memory-mapped read-only by every
worker, so the workers share one copy.  Workers are started with the
``spawn`` method: the parent may hold a GPU context, which a forked child
must not inherit.
"""

from __future__ import annotations

import contextlib
import os
import shutil
import sys
import tempfile
import types
from concurrent.futures import ProcessPoolExecutor
from multiprocessing import get_context

import numpy as np

_ARRAYS: dict = {}


def pool_workers() -> int:
    """Worker processes for a pool: the host cores this process may run on
    (its CPU affinity), capped by ``OMP_NUM_THREADS`` when that is set (the
    share of a machine's cores a job is given)."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo ("unknown" if absent)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


@contextlib.contextmanager
def _bare_main():
    """Hide the parent's ``__main__`` while workers start: a spawned worker
    would otherwise re-run the parent's main script (a benchmark, a test
    runner, or a script read from stdin that it cannot find)."""
    main = sys.modules.get("__main__")
    sys.modules["__main__"] = types.ModuleType("__main__")
    try:
        yield
    finally:
        if main is not None:
            sys.modules["__main__"] = main


def _init_worker(files):
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:  # pragma: no cover
        pass
    for key, path in files.items():
        _ARRAYS[key] = np.load(path, mmap_mode="r", allow_pickle=False)


def _run(job):
    fn, qrows, rows, extra, kw = job
    a = _ARRAYS
    if fn == "forward":
        from .attention import _rows_forward
        return _rows_forward(qrows, a["k"], a["v"], a["qid"], a["qpos"], a["kid"], a["kpos"],
                             rows, **kw)
    from .backward import _rows_dq
    return _rows_dq(qrows, extra, a["k"], a["v"], a["qid"], a["qpos"], a["kid"], a["kpos"],
                    rows, **kw)


def _host(x, dtype):
    if hasattr(x, "detach"):
        import torch
        tdt = {np.float32: torch.float32, np.int64: torch.int64}[dtype]
        return x.detach().to("cpu", tdt).numpy()
    return np.asarray(x, dtype=dtype)


class RowPool:
    """Worker processes sharing one memory-mapped copy of K, V and the
    metadata.  ``forward(qrows, rows, ...)`` and ``dq(qrows, dorows, rows, ...)``
    return what the serial row functions return, with the rows spread over
    the workers in chunks.  K and V are stored as float32, which holds bf16 and
    fp32 values exactly; the row functions widen to fp64."""

    def __init__(self, k, v, qid, qpos, kid, kpos, workers=None):
        self.workers = workers or pool_workers()
        self.dv = int(v.shape[3])
        self.timeout_s = 3600.0
        base = "/dev/shm" if os.path.isdir("/dev/shm") and os.access("/dev/shm", os.W_OK) else None
        self._dir = tempfile.mkdtemp(prefix="oracle_rows_", dir=base)
        files = {}
        try:
            for key, x, dt in (("k", k, np.float32), ("v", v, np.float32), ("qid", qid, np.int64),
                               ("qpos", qpos, np.int64), ("kid", kid, np.int64),
                               ("kpos", kpos, np.int64)):
                path = os.path.join(self._dir, key + ".npy")
                np.save(path, _host(x, dt), allow_pickle=False)
                files[key] = path
            self._ex = ProcessPoolExecutor(self.workers, mp_context=get_context("spawn"),
                                           initializer=_init_worker, initargs=(files,))
        except BaseException:
            shutil.rmtree(self._dir, ignore_errors=True)
            raise

    def _map(self, fn, qrows, extra, rows, kw):
        n = len(rows)
        if n == 0:
            return []
        chunk = max(1, -(-n // (4 * self.workers)))
        jobs = [(fn, qrows[i:i + chunk], list(rows[i:i + chunk]),
                 None if extra is None else extra[i:i + chunk], kw) for i in range(0, n, chunk)]
        with _bare_main():   # workers are started by these submissions
            futures = [self._ex.submit(_run, j) for j in jobs]
        return [f.result(timeout=self.timeout_s) for f in futures]

    def forward(self, qrows, rows, **kw):
        parts = self._map("forward", qrows, None, rows, kw)
        if not parts:
            return np.zeros((0, qrows.shape[1], self.dv)), np.zeros((0, qrows.shape[1]))
        return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])

    def dq(self, qrows, dorows, rows, **kw):
        parts = self._map("dq", qrows, dorows, rows, kw)
        if not parts:
            return np.zeros((0,) + tuple(qrows.shape[1:]))
        return np.concatenate(parts)

    def close(self):
        ex, self._ex = getattr(self, "_ex", None), None
        if ex is not None:
            ex.shutdown(wait=True, cancel_futures=True)
        shutil.rmtree(self._dir, ignore_errors=True)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):  # pragma: no cover
        try:
            self.close()
        except Exception:
            pass
