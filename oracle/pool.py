"""Process pool over BF ranges for the float64 oracle.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: only the test suite, the
smoke check and the CPU-baseline leg of the benchmark use it.  It shares no code
with the GPU library.

The oracle's per-BF definition (``ssb_oracle``) is unchanged: the BF list is cut
into contiguous ranges, each range is evaluated by ``bf_moments`` (or
``corrected_sum`` for the object) in a worker process, and the range results are
added in range order in float64.  The only difference from one serial call is the
association of those float64 sums (relative effects near 1e-15).

Counts reach the workers through a read-only memory-mapped file (uint32
[n_bf][N][N]), written once per pool.  Workers are fresh interpreters (spawn start
method: nothing is forked from a process that may have initialized a GPU) with
NumPy's threading pinned to one thread each.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import shutil
import sys
import tempfile

import numpy as np

from . import ssb_oracle as O

_THREAD_VARS = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "NUMEXPR_NUM_THREADS")


def default_workers() -> int:
    """Host cores this process may use, at most 16 (one GPU's share of a shared host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _counts(path, shape):
    return np.memmap(path, dtype=np.uint32, mode="r", shape=shape)


def _task(args):
    kind, path, shape, geom, params, dc, b0, b1 = args
    counts = _counts(path, shape)
    sub = np.asarray(counts[b0:b1])
    bl = list(range(b0, b1))
    if kind == "moments":
        return O.bf_moments(geom, sub, params, dc, bl)
    if kind == "moments_full_plane":
        return O.bf_moments_full_plane(geom, sub, params, dc, bl)
    if kind == "sum":
        return O.corrected_sum(geom, sub, params, dc, bl)
    raise ValueError(kind)


class OraclePool:
    """Pooled oracle over one workload's counts.

    counts: a NumPy uint32 array [n_bf][N][N], or a callable fill(b0, b1) returning the
    rows [b0, b1) as such an array (used to stream device-resident counts to the file
    in pieces).  shape must then be given.
    """

    def __init__(self, counts, shape=None, workers: int | None = None, chunk_bf: int = 1024,
                 dirpath: str | None = None):
        # spawned workers re-import the main program by its path: a program read from stdin
        # has none, and its workers would fail at start-up while the pool respawns them
        main_file = getattr(sys.modules.get("__main__"), "__file__", None)
        if main_file is not None and not os.path.exists(main_file):
            raise RuntimeError(f"OraclePool: the main program ({main_file}) must be a file the "
                               "worker processes can import")
        if shape is None:
            shape = counts.shape
        self.shape = tuple(int(v) for v in shape)
        nbytes = int(np.prod(self.shape)) * 4
        if dirpath is None:
            shm = "/dev/shm"
            use_shm = os.path.isdir(shm) and shutil.disk_usage(shm).free > 2 * nbytes + (1 << 30)
            dirpath = shm if use_shm else None
        self.dir = tempfile.mkdtemp(prefix="ssb_oracle_", dir=dirpath)
        self.path = os.path.join(self.dir, "counts.u32")
        mm = np.memmap(self.path, dtype=np.uint32, mode="w+", shape=self.shape)
        for b0 in range(0, self.shape[0], chunk_bf):
            b1 = min(self.shape[0], b0 + chunk_bf)
            mm[b0:b1] = counts(b0, b1) if callable(counts) else counts[b0:b1]
        mm.flush()
        del mm
        self.workers = workers or default_workers()
        saved = {k: os.environ.get(k) for k in _THREAD_VARS}
        try:
            for k in _THREAD_VARS:
                os.environ[k] = "1"
            self.pool = mp.get_context("spawn").Pool(self.workers)
        finally:
            for k, v in saved.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v

    # ranges of about n_bf / (4 workers) BF pixels, so that slow ranges even out
    def _ranges(self, b0, b1):
        n = b1 - b0
        step = max(1, -(-n // (4 * self.workers)))
        return [(a, min(b1, a + step)) for a in range(b0, b1, step)]

    def _map(self, kind, geom, params, dc, b0, b1):
        geom = O.OGeom.from_any(geom)
        params = np.asarray(params, dtype=np.float32)
        jobs = [(kind, self.path, self.shape, geom, params, float(dc), a, b) for a, b in self._ranges(b0, b1)]
        return self.pool.map(_task, jobs, chunksize=1)

    def moments(self, geom, params, dc, b0: int = 0, b1: int | None = None, full_plane: bool = False):
        """S1 (N, N) and S2 over BF [b0, b1), range results added in range order."""
        b1 = self.shape[0] if b1 is None else b1
        parts = self._map("moments_full_plane" if full_plane else "moments", geom, params, dc, b0, b1)
        s1 = np.zeros(self.shape[1:], dtype=np.float64)
        s2 = 0.0
        for p1, p2 in parts:
            s1 += p1
            s2 += p2
        return s1, s2

    def loss(self, geom, params, dc, full_plane: bool = False) -> float:
        s1, s2 = self.moments(geom, params, dc, full_plane=full_plane)
        return O.loss_from_moments(s1, s2, self.shape[0])

    def object_wave(self, geom, params, dc):
        """(phase, psi) of the phase-of-mean object over every BF pixel."""
        acc = None
        for part in self._map("sum", geom, params, dc, 0, self.shape[0]):
            acc = part if acc is None else acc + part
        return O.object_from_sum(acc, self.shape[0])

    def close(self):
        if self.pool is not None:
            self.pool.terminate()
            self.pool.join()
            self.pool = None
        shutil.rmtree(self.dir, ignore_errors=True)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
