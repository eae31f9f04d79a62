"""The oracle's decode outputs of long workloads, evaluated in parallel.

Each task replays a workload through the unchanged oracle in a process of its
own (started fresh, never touching the GPU), with K/V written only for the
layers and writing sequences its rows need, and returns the float64 outputs
of its (decode index, layer, rows) items.  Used by the GPU parity tests of the
12 x 131072 and fork workloads, whose oracle evaluation would otherwise take
many minutes on one core.
"""

from __future__ import annotations

import multiprocessing as mp
import os

MAX_WORKERS = 16  # one GPU's share of host cores on its box


def _task(task):
    factory, kwargs, layers, writers, items = task
    from threadpoolctl import threadpool_limits

    from oracle.runner import OracleReplay
    from synth import workloads

    wl = getattr(workloads, factory)(**kwargs)
    with threadpool_limits(limits=1):
        ref = OracleReplay(wl, layers=list(layers), writers=set(writers)).run()
        return [ref.attention(i, layer, rows=list(rows)) for i, layer, rows in items]


def evaluate(tasks):
    """tasks: [(workloads factory name, kwargs, layers, writers, [(decode index, layer, rows)])];
    returns, per task, the list of [len(rows), Hq, d] float64 outputs of its items."""
    workers = max(1, min(len(tasks), MAX_WORKERS, len(os.sched_getaffinity(0))))
    print(f"  oracle: {len(tasks)} replays on {workers} processes", flush=True)
    with mp.get_context("spawn").Pool(workers) as pool:
        return pool.map(_task, tasks, chunksize=1)
