"""Run the CPU oracle over many pair rows in worker processes.

TEST INFRASTRUCTURE ONLY, like the oracles it drives: only the tests,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. It adds no arithmetic of its own: every row is computed by
``tri_attn_oracle.forward_rows`` or ``tri_attn_train_oracle.forward_train_rows``
exactly as in one process; the rows are only split over processes.

Pair rows (b, i) are independent once their batch's LayerNorm output and pair
bias are known, so the rows of a request are cut into contiguous chunks of
one batch each and handed to a pool of worker processes. Inputs (and, for a
comparison, the result to check) go to the workers as ``.npy`` files in a
temporary directory that each worker memory-maps, so nothing large passes
through pipes; a worker reads only the batches its rows touch. Each worker
runs its BLAS on one thread. Workers are started with the ``spawn`` method:
they are fresh interpreters that import numpy and the oracle only, never the
GPU runtime of the parent.

The worker count defaults to the host's usable cores, capped at 16.
"""
from __future__ import annotations

import math
import multiprocessing as mp
import os
import shutil
import tempfile
import time
from concurrent.futures import ProcessPoolExecutor
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

MAX_WORKERS = 16

# ------------------------------------------------------------------ helpers


def default_workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # not Linux
        n = os.cpu_count() or 1
    return max(1, min(MAX_WORKERS, n))


def _tmp_root() -> str:
    shm = "/dev/shm"
    if os.path.isdir(shm) and os.access(shm, os.W_OK):
        return shm
    return tempfile.gettempdir()


class _Spill:
    """A temporary directory of .npy files: the inputs and extra arrays."""

    def __init__(self, inp: dict, extra: Optional[Dict[str, np.ndarray]] = None):
        self.path = tempfile.mkdtemp(prefix="tri_attn_oracle_", dir=_tmp_root())
        self.meta = {}
        try:
            for k, v in inp.items():
                if isinstance(v, np.ndarray):
                    np.save(os.path.join(self.path, k + ".npy"), v)
                else:
                    self.meta[k] = v
            for k, v in (extra or {}).items():
                np.save(os.path.join(self.path, "_" + k + ".npy"), np.ascontiguousarray(v))
        except BaseException:
            self.close()
            raise

    def close(self):
        shutil.rmtree(self.path, ignore_errors=True)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


_CACHE: dict = {}


def _load(path: str, meta: dict):
    """(inputs, extra arrays) of a spill directory, memory-mapped, cached per process."""
    if _CACHE.get("path") != path:
        inp, extra = dict(meta), {}
        for name in os.listdir(path):
            if not name.endswith(".npy"):
                continue
            arr = np.load(os.path.join(path, name), mmap_mode="r")
            if name.startswith("_"):
                extra[name[1:-4]] = arr
            else:
                inp[name[:-4]] = arr
        _CACHE.clear()
        _CACHE.update(path=path, inp=inp, extra=extra)
    return _CACHE["inp"], _CACHE["extra"]


def _one_thread():
    try:
        from threadpoolctl import threadpool_limits

        return threadpool_limits(limits=1)
    except Exception:  # threadpoolctl missing: environment variables were set before numpy loaded
        import contextlib

        return contextlib.nullcontext()


def _chunks(rows: Sequence[Tuple[int, int]], workers: int, per_chunk: Optional[int]) -> List[List[Tuple[int, int]]]:
    """Contiguous chunks of rows, each within one batch, about `per_chunk` rows
    (default: enough chunks for every worker to get a few)."""
    rows = [(int(b), int(i)) for b, i in rows]
    if not rows:
        return []
    if per_chunk is None:
        per_chunk = max(1, math.ceil(len(rows) / (3 * workers)))
    out: List[List[Tuple[int, int]]] = []
    cur: List[Tuple[int, int]] = []
    for r in rows:
        if cur and (r[0] != cur[-1][0] or len(cur) >= per_chunk):
            out.append(cur)
            cur = []
        cur.append(r)
    out.append(cur)
    return out


# ------------------------------------------------------------------ worker tasks (run in the workers)


def _task_compare(args):
    """Oracle rows of one chunk against the same rows of the array `y`:
    max abs error over finite reference entries, its location, whether the
    finite patterns agree, and max |reference|."""
    path, meta, chunk, kind, kw = args
    inp, extra = _load(path, meta)
    with _one_thread():
        if kind == "train":
            from oracle.tri_attn_train_oracle import forward_train_rows

            ref, lse = forward_train_rows(inp, chunk, kw["rate"], kw["seed"], kw.get("offset", 0),
                                          kw.get("fill", -1e9))
        else:
            from oracle.tri_attn_oracle import forward_rows

            ref, lse = forward_rows(inp, chunk, fill=kw.get("fill", -1e9)), None
    res = []
    for name, want, got_all in (("y", ref, extra["y"]), ("lse", lse, extra.get("lse"))):
        if want is None or got_all is None:
            continue
        got = np.stack([np.asarray(got_all[b, i], dtype=np.float64) for b, i in chunk])
        fin = np.isfinite(want)
        same_pattern = bool((np.isfinite(got) == fin).all())
        d = np.abs(np.where(fin, got, 0.0) - np.where(fin, want, 0.0))
        if name == "lse":
            # lse[t, j] of a query column whose keys are all masked is fill + ln N
            # (about -1e9 for the default fill): compared relatively, apart from
            # the columns with a valid key, whose absolute error is the measure
            mask = inp["pair_mask"]
            live = np.stack([np.asarray(mask[b]).any(-1) for b, _ in chunk])[:, None, :]  # (rows, 1, j)
            live = np.broadcast_to(live, d.shape)
            dead_fin = ~live & fin
            rel = float((d[dead_fin] / np.abs(want[dead_fin])).max()) if dead_fin.any() else 0.0
            res.append(("lse_dead_rel", rel, None, True, 0.0))
            d = np.where(live, d, 0.0)
        k = int(np.argmax(d))
        idx = np.unravel_index(k, d.shape)
        where = (chunk[idx[0]][0], chunk[idx[0]][1]) + tuple(int(x) for x in idx[1:])
        res.append((name, float(d.flat[k]), where, same_pattern,
                    float(np.abs(want[fin]).max()) if fin.any() else 0.0))
    return res


def _task_forward(args):
    path, meta, chunk, kind, kw = args
    inp, _ = _load(path, meta)
    with _one_thread():
        if kind == "ending":
            from oracle.tri_attn_oracle import forward_ending_cols

            return forward_ending_cols(inp, chunk, fill=kw.get("fill", -1e9))
        from oracle.tri_attn_oracle import forward_rows

        return forward_rows(inp, chunk, fill=kw.get("fill", -1e9))


def _task_time(args):
    """Compute the chunk and return (rows done, seconds), discarding the result."""
    t0 = time.perf_counter()
    _task_forward(args)
    return len(args[2]), time.perf_counter() - t0


def _pool(workers: int):
    # a worker that dies raises BrokenProcessPool here instead of hanging the caller
    return ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn"))


# ------------------------------------------------------------------ public entry points


def compare_rows(inp: dict, y: np.ndarray, rows: Sequence[Tuple[int, int]], fill: float = -1e9,
                 workers: Optional[int] = None, train: Optional[dict] = None,
                 lse: Optional[np.ndarray] = None) -> dict:
    """Compare y[b, i] (and lse[b, i] for training) of the listed rows with
    the oracle, in parallel. `y` is indexed [b][i][j][c] like the output;
    `train` = {"rate", "seed", "offset"} selects the training-mode oracle.
    Returns {name: {"max_abs_err", "where", "same_nan_pattern", "max_abs_ref"}}
    for "y" (and, with `lse`, "lse" over query columns that have a valid key,
    and "lse_dead_rel", whose "max_abs_err" is the largest relative error on
    the columns whose keys are all masked)."""
    workers = workers or default_workers()
    extra = {"y": y}
    if lse is not None:
        extra["lse"] = lse
    kw = dict(train or {}, fill=fill)
    kind = "train" if train else "infer"
    out: dict = {}
    with _Spill(inp, extra) as sp:
        tasks = [(sp.path, sp.meta, c, kind, kw) for c in _chunks(rows, workers, None)]
        with _pool(workers) as pool:
            for res in pool.map(_task_compare, tasks):
                for name, err, where, same, mref in res:
                    cur = out.setdefault(name, {"max_abs_err": -1.0, "where": None, "same_nan_pattern": True,
                                                "max_abs_ref": 0.0})
                    if err > cur["max_abs_err"]:
                        cur["max_abs_err"], cur["where"] = err, where
                    cur["same_nan_pattern"] &= same
                    cur["max_abs_ref"] = max(cur["max_abs_ref"], mref)
    return out


def forward_rows(inp: dict, rows: Sequence[Tuple[int, int]], fill: float = -1e9,
                 workers: Optional[int] = None, ending: bool = False) -> np.ndarray:
    """tri_attn_oracle.forward_rows (or forward_ending_cols) over processes:
    (len(rows), N, D) float64 in the order of `rows`."""
    workers = workers or default_workers()
    with _Spill(inp) as sp:
        chunks = _chunks(rows, workers, None)
        tasks = [(sp.path, sp.meta, c, "ending" if ending else "infer", {"fill": fill}) for c in chunks]
        with _pool(workers) as pool:
            parts = list(pool.map(_task_forward, tasks))
    return np.concatenate(parts) if parts else np.empty((0,))


def time_rows(inp: dict, rows: Sequence[Tuple[int, int]], seconds: float, workers: Optional[int] = None,
              ending: bool = False) -> dict:
    """Wall time of the oracle over the listed rows (all of one batch, say),
    split into one contiguous chunk per worker, the whole list computed again
    and again until `seconds` have passed. Each chunk is one oracle call, so
    each worker computes its batch's LayerNorm and pair bias once per pass,
    as one process does once per call. Pool start-up and imports are
    excluded (a one-row warm-up per worker). Returns {"rows", "seconds",
    "workers", "passes"}."""
    workers = workers or default_workers()
    rows = [(int(b), int(i)) for b, i in rows]
    workers = max(1, min(workers, len(rows)))
    with _Spill(inp) as sp:
        kind = "ending" if ending else "infer"
        per = math.ceil(len(rows) / workers)
        tasks = [(sp.path, sp.meta, rows[k:k + per], kind, {}) for k in range(0, len(rows), per)]
        warm = [(sp.path, sp.meta, [rows[0]], kind, {}) for _ in range(workers)]
        with _pool(workers) as pool:
            list(pool.map(_task_time, warm))
            done, passes = 0, 0
            t0 = time.perf_counter()
            while True:
                done += sum(n for n, _ in pool.map(_task_time, tasks))
                passes += 1
                el = time.perf_counter() - t0
                if el >= seconds:
                    break
    return {"rows": done, "seconds": el, "workers": workers, "passes": passes}
