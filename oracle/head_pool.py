"""Run the float64 oracle over groups of (batch, head) sequences in a pool of host processes.

TEST INFRASTRUCTURE, like the rest of this package: used by the full-size parity tests and
the benchmark's CPU-baseline leg, never by the library's product path.

Every (batch, head) sequence carries its own state (liuzhao09.github.io CARVE notes,
section 2.1: one d_v x d_k state per head), so splitting the flattened head axis into
groups changes nothing in what is computed: each group runs the same token-serial
functions of carve_oracle on its own heads, and the results are put back in place.
Parameters shared by the heads of one index h across the batch (the content projection
U1, U2) are given to each group for the heads it holds, and their gradients, which the
oracle sums over the batch, are summed over the groups.
"""
import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

_THREAD_VARS = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")
PER_HEAD = ("U1", "U2")            # [H, ...] parameters, shared over the batch
PER_HEAD_GRADS = ("dU1", "dU2")    # their gradients, [H, ...], summed over the batch


def host_workers(limit=16):
    """Processes to use: the cores this process may run on, at most `limit`."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, limit))


def cpu_model():
    """The host CPU's model name as the kernel reports it."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def _slice(x, idx, B, H, per_head):
    """The heads `idx` (flattened b * H + h) of x, as a batch of one with len(idx) heads."""
    if x is None or np.ndim(x) == 0:
        return x
    x = np.asarray(x)
    if per_head:
        return x[idx % H]
    return x.reshape((B * H,) + x.shape[2:])[idx][None]


def _slice_args(kwargs, idx, B, H):
    out = {}
    for key, val in kwargs.items():
        if isinstance(val, dict):
            out[key] = {k2: _slice(v2, idx, B, H, k2 in PER_HEAD) for k2, v2 in val.items()}
        else:
            out[key] = _slice(val, idx, B, H, key in PER_HEAD)
    return out


def _call(job):
    name, kwargs = job
    from oracle import carve_oracle
    return getattr(carve_oracle, name)(**kwargs)


class _Merge:
    """Puts each group's results ([1, n, ...] per output) back into [B, H, ...] arrays."""

    def __init__(self, B, H):
        self.B, self.H = B, H
        self.is_dict = False
        self.store = {}
        self.present = {}

    def add(self, res, idx):
        self.is_dict = isinstance(res, dict)
        for key, val in (res.items() if self.is_dict else enumerate(res)):
            self.present[key] = val is not None
            if val is None:
                continue
            val = np.asarray(val)
            if key in PER_HEAD_GRADS:
                dst = self.store.setdefault(key, np.zeros((self.H,) + val.shape[1:]))
                np.add.at(dst, idx % self.H, val)
            else:
                dst = self.store.setdefault(key, np.zeros((self.B * self.H,) + val.shape[2:]))
                dst[idx] = val[0]

    def _full(self, key):
        if not self.present[key]:
            return None
        x = self.store[key]
        return x if key in PER_HEAD_GRADS else x.reshape((self.B, self.H) + x.shape[1:])

    def result(self):
        if self.is_dict:
            return {key: self._full(key) for key in self.present}
        return tuple(self._full(i) for i in sorted(self.present))


class HeadPool:
    """A pool of spawned host processes, each running numpy with one thread.  A worker that
    dies (or cannot start) raises BrokenProcessPool in the caller instead of being replaced.

    with HeadPool() as pool:
        o, S_T, m = pool.run("forward", B, H, q=q, k=k, ..., L=64)
    """

    def __init__(self, workers=None):
        self.workers = workers or host_workers()
        saved = {k: os.environ.get(k) for k in _THREAD_VARS}
        for k in _THREAD_VARS:
            os.environ[k] = "1"
        try:
            self._ex = ProcessPoolExecutor(self.workers, mp_context=mp.get_context("spawn"))
            self._ex.submit(int, 0).result()      # the workers start here, with one thread each
        except BaseException:
            self._ex.shutdown(wait=True, cancel_futures=True)
            raise
        finally:
            for k, v in saved.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v

    def __enter__(self):
        return self

    def __exit__(self, exc_type, exc, tb):
        self._ex.shutdown(wait=True, cancel_futures=exc_type is not None)

    def run(self, name, B, H, groups=None, progress=None, **kwargs):
        """carve_oracle.<name>(**kwargs) over all B*H heads, split into `groups` groups of
        consecutive flattened heads (default: two per worker).  Arrays with leading [B, H]
        axes are split by head; U1 / U2 ([H, ...]) are given per head; scalars are passed
        as they are.  progress(done, total) is called as groups finish, in order."""
        n = B * H
        groups = max(1, min(n, groups or 2 * self.workers))
        parts = [p for p in np.array_split(np.arange(n), groups) if len(p)]
        futs = [self._ex.submit(_call, (name, _slice_args(kwargs, idx, B, H))) for idx in parts]
        merge = _Merge(B, H)
        for i, fut in enumerate(futs):
            merge.add(fut.result(), parts[i])
            if progress is not None:
                progress(i + 1, len(parts))
        return merge.result()
