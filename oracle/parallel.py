"""Process-pool driver for the fp64 attention oracle (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it, like the rest of ``oracle/``.  It adds no arithmetic
of its own: it cuts an attention problem into units that the definition
already keeps apart and runs ``oracle.attention`` on each unit in a worker
process.

Why the units are independent.  In the definition (``oracle.attention``) the
output row of query i and head h depends only on q[i, h] and on the keys and
values of KV head h // (Hq // Hkv) up to position q_pos[i].  So rows can be
computed in any grouping, and each GQA group (one KV head with its query
heads) can be computed on its own.  A unit here is (problem, KV head, block of
query rows); a problem is one request's query rows over its pages.

Data movement.  The inputs stay as bf16 bit patterns (``uint16``) in files
that every worker maps read-only (a pool shared by several problems is written
once); a worker walks the pages of the KV head it needs with
``oracle.gather_logical`` and keeps the last head it converted.  Workers are
started fresh (``spawn``), so they never inherit a GPU context from the
parent, and each runs with one BLAS thread, so the pool's size is the number
of cores used.
"""

from __future__ import annotations

import os
import shutil
import tempfile
from concurrent.futures import ProcessPoolExecutor
from multiprocessing import get_context

import numpy as np

from .attention import attention as _attention, bf16_to_f64 as _bf16_to_f64, gather_logical as _gather_logical

BLAS_ENV = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS")


def usable_cores(cap: int = 16) -> int:
    """Cores this process may run on (its affinity mask), at most ``cap``."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - not Linux
        n = os.cpu_count() or 1
    return max(1, min(cap, n))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _scratch_dir():
    """Memory-backed /dev/shm when it has room for a few GB, else the temporary directory."""
    try:
        if shutil.disk_usage("/dev/shm").free > (16 << 30):
            return "/dev/shm"
    except OSError:
        pass
    return None


# ---- worker side ------------------------------------------------------------------------------

_W = {"maps": {}, "cache": None}


def _worker_init():
    try:  # one BLAS thread per worker, also where the environment was not honoured
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _view(desc):
    path, shape, dtype = desc
    arr = _W["maps"].get(path)
    if arr is None:
        if len(_W["maps"]) > 64:  # files of earlier calls
            _W["maps"].clear()
            _W["cache"] = None
        arr = np.memmap(path, dtype=dtype, mode="r", shape=shape)
        _W["maps"][path] = arr
    return arr


def _kv_head(prob, g):
    """Keys and values of KV head g of one problem, [n_keys][1][D] float64 (cached per worker)."""
    key = (prob["uid"], g)
    cached = _W["cache"]
    if cached is not None and cached[0] == key:
        return cached[1], cached[2]
    k_pages, v_pages = _view(prob["k"]), _view(prob["v"])
    n = prob["n_keys"]
    k = _gather_logical(k_pages[:, g:g + 1], prob["table"], n)
    v = _gather_logical(v_pages[:, g:g + 1], prob["table"], n)
    _W["cache"] = (key, k, v)
    return k, v


def _unit(args):
    pi, prob, g, lo, hi, scale = args
    q_bits = _view(prob["q"])
    k, v = _kv_head(prob, g)
    group = q_bits.shape[1] // k_heads(prob)
    q = _bf16_to_f64(q_bits[lo:hi, group * g:group * (g + 1)])
    o, lse = _attention(q, k, v, prob["q_pos"][lo:hi], scale)
    return pi, g, lo, hi, o, lse


def k_heads(prob) -> int:
    return prob["k"][1][1]


def _warm(_):
    return os.getpid()


# ---- parent side ------------------------------------------------------------------------------

class OraclePool:
    """A pool of oracle workers.  ``attention(problems, scale)`` returns, per problem, the same
    (O, LSE) as ``oracle.attention`` over that problem's logical keys.

    A problem is a dict with
      q:        bf16 bits [Nq][Hq][D]
      k_pages:  bf16 bits [n_pages][Hkv][page_size][D]   (K pool, or the request's pages)
      v_pages:  same layout
      table:    page ids in logical order (into k_pages / v_pages)
      n_keys:   keys the request holds (every q_pos is below it)
      q_pos:    absolute position of each query row [Nq]
    """

    def __init__(self, workers: int | None = None, rows_per_unit: int = 256):
        self.workers = workers or usable_cores()
        self.rows_per_unit = rows_per_unit
        saved = {k: os.environ.get(k) for k in BLAS_ENV}
        try:
            for k in BLAS_ENV:
                os.environ[k] = "1"
            self.ex = ProcessPoolExecutor(self.workers, mp_context=get_context("spawn"), initializer=_worker_init)
            # start every worker now, so that timing a call measures the oracle, not process start-up
            list(self.ex.map(_warm, range(self.workers)))
        finally:
            for k, v in saved.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v
        self._dir = None
        self._shared = {}
        self._uid = 0

    def close(self):
        self.ex.shutdown(wait=True)
        self._free()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def _share(self, arr):
        """Write an array to a file the workers map; the same array object is written once."""
        if id(arr) in self._shared:
            return self._shared[id(arr)][1]
        a = np.ascontiguousarray(arr)
        if self._dir is None:
            self._dir = tempfile.mkdtemp(prefix="oracle_pool_", dir=_scratch_dir())
        path = os.path.join(self._dir, f"seg{len(self._shared)}.bin")
        if a.nbytes:
            mm = np.memmap(path, dtype=a.dtype, mode="w+", shape=a.shape)
            mm[...] = a
            mm.flush()
            del mm
        else:
            open(path, "wb").close()
        desc = (path, a.shape, a.dtype.str)
        self._shared[id(arr)] = (arr, desc)  # keeps the object alive, so its id stays unique
        return desc

    def _free(self):
        self._shared = {}
        if self._dir is not None:
            shutil.rmtree(self._dir, ignore_errors=True)
            self._dir = None

    def stage(self, problems):
        """Write the problems' inputs where the workers map them (not part of the oracle's compute)."""
        staged = []
        for p in problems:
            self._uid += 1
            q = np.asarray(p["q"])
            if q.dtype != np.uint16 or q.ndim != 3:
                raise ValueError("q must be bf16 bits [Nq][Hq][D]")
            q_pos = np.asarray(p["q_pos"], dtype=np.int64)
            if len(q_pos) != q.shape[0]:
                raise ValueError("one position per query row")
            staged.append({"q": self._share(q), "k": self._share(p["k_pages"]), "v": self._share(p["v_pages"]),
                           "table": np.asarray(p["table"], dtype=np.int64), "n_keys": int(p["n_keys"]),
                           "q_pos": q_pos, "uid": self._uid})
        return staged

    def run(self, staged, scale: float):
        """Run the oracle over staged problems; returns [(O, LSE)] in float64, one per problem."""
        units = []
        for pi, p in enumerate(staged):
            n_q, n_qh = p["q"][1][0], p["q"][1][1]
            n_kvh = p["k"][1][1]
            if n_qh % n_kvh != 0:
                raise ValueError("query heads must be a multiple of KV heads")
            for g in range(n_kvh):  # KV-head-major, so a worker's cached head is reused
                for lo in range(0, n_q, self.rows_per_unit):
                    units.append((pi, p, g, lo, min(lo + self.rows_per_unit, n_q), scale))
        out = [(np.zeros((p["q"][1][0], p["q"][1][1], p["q"][1][2])), np.zeros((p["q"][1][0], p["q"][1][1])))
               for p in staged]
        chunk = max(1, len(units) // (4 * self.workers))
        for pi, g, lo, hi, o, lse in self.ex.map(_unit, units, chunksize=chunk):
            n_qh, n_kvh = staged[pi]["q"][1][1], staged[pi]["k"][1][1]
            group = n_qh // n_kvh
            out[pi][0][lo:hi, group * g:group * (g + 1)] = o
            out[pi][1][lo:hi, group * g:group * (g + 1)] = lse
        return out

    def attention(self, problems, scale: float):
        try:
            return self.run(self.stage(problems), scale)
        finally:
            self._free()


def prefill_problem(q_bits, k_pages, v_pages, table, prefix_len: int):
    """One prefill chunk as a problem: query i at position prefix_len + i over prefix_len + C keys."""
    c = np.asarray(q_bits).shape[0]
    return {"q": q_bits, "k_pages": k_pages, "v_pages": v_pages, "table": table,
            "n_keys": prefix_len + c, "q_pos": prefix_len + np.arange(c)}


def decode_problem(q_bits, k_pages, v_pages, table, kv_len: int):
    """One decode query (bits [1][Hq][D]) at position kv_len - 1 over kv_len keys."""
    return {"q": q_bits, "k_pages": k_pages, "v_pages": v_pages, "table": table,
            "n_keys": int(kv_len), "q_pos": np.array([int(kv_len) - 1])}
