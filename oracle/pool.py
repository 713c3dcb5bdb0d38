"""The oracle over many heads at once, on a pool of host processes.

TEST INFRASTRUCTURE ONLY, like the rest of this package.

Attention is independent across (batch, head) and, within a head, across
query rows: each output row depends only on its query row and the head's keys
and values (the definition in definition.py). This module only distributes
that independent work: every task calls definition.attention_head,
unchanged, on one block of query rows of one head, and the results are put
back in place. No arithmetic is added, reordered or shared between tasks.

Workers are started with the "spawn" method (never forked from a process
that may hold a GPU context), each limits its BLAS library to one thread, and
there is one worker per host core this process may run on
(os.sched_getaffinity), capped at MAX_WORKERS (the host share of one GPU on
a shared machine) and by `workers`.
"""
from __future__ import annotations

import math
import os
import platform
from concurrent.futures import ProcessPoolExecutor
from typing import Iterable, Optional, Sequence, Tuple

import multiprocessing as mp
import numpy as np

from .definition import attention_head

MAX_WORKERS = 16


def host_cores() -> int:
    """Cores this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - not Linux
        return os.cpu_count() or 1


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or the platform's."""
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def _init_worker():
    try:
        from threadpoolctl import threadpool_limits

        threadpool_limits(1)
    except Exception:  # pragma: no cover - BLAS threads stay at their default
        pass


def _run(task):
    key, q_rows, k_h, v_h, scale, causal, row_ids = task
    O, L = attention_head(q_rows, k_h, v_h, scale, causal, row_ids=row_ids)
    return key, O, L


def _as_array(t) -> np.ndarray:
    """The exact values of a CPU tensor or array, as a numpy array that pickles
    (bf16 and fp16 are widened to float32, which holds them exactly)."""
    try:
        import torch

        if isinstance(t, torch.Tensor):
            t = t.detach().cpu()
            if t.dtype in (torch.float16, torch.bfloat16):
                t = t.to(torch.float32)
            return t.numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(t)


def make_executor(workers: Optional[int] = None) -> ProcessPoolExecutor:
    """A pool of spawned workers, one per host core up to MAX_WORKERS (or
    `workers`), each with its BLAS library at one thread."""
    n = min(workers or MAX_WORKERS, host_cores(), MAX_WORKERS)
    return ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn"),
                               initializer=_init_worker)


def warm(executor: ProcessPoolExecutor) -> None:
    """Start every worker of `executor` (spawning and importing happen here)."""
    n = executor._max_workers  # noqa: SLF001 - the size the pool was made with
    list(executor.map(_noop, range(4 * n), chunksize=1))


def _noop(_):
    return 0


def attention_heads(q, k, v, heads: Sequence[Tuple[int, int]], scale: Optional[float] = None,
                    causal: bool = False, rows: Optional[Iterable[int]] = None,
                    row_block: int = 1024, workers: Optional[int] = None,
                    executor: Optional[ProcessPoolExecutor] = None):
    """Oracle O and LSE of the listed heads (b, h) of [B, H, N, d] inputs.

    rows: the query rows to compute (all rows by default), taken row_block
    at a time. executor: a pool from make_executor to run on (else one is
    made for this call). Returns (O, L): O [len(heads), len(rows), d] and
    L [len(heads), len(rows)] in float64, in the order given.
    """
    d = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    Nq = q.shape[2]
    rows = np.arange(Nq) if rows is None else np.asarray(list(rows), dtype=np.int64)
    n = min(workers or MAX_WORKERS, host_cores(), MAX_WORKERS)
    tasks = []
    for hi, (b, h) in enumerate(heads):
        qh = _as_array(q[b, h])
        kh = _as_array(k[b, h])
        vh = _as_array(v[b, h])
        for r0 in range(0, len(rows), row_block):
            rr = rows[r0:r0 + row_block]
            tasks.append(((hi, r0), qh[rr], kh, vh, scale, causal, rr))
    O = np.empty((len(heads), len(rows), d))
    L = np.empty((len(heads), len(rows)))
    if executor is not None:
        for (hi, r0), o, l in executor.map(_run, tasks, chunksize=1):
            O[hi, r0:r0 + o.shape[0]], L[hi, r0:r0 + o.shape[0]] = o, l
        return O, L
    if n <= 1 or len(tasks) == 1:
        results = map(_run, tasks)
        for (hi, r0), o, l in results:
            O[hi, r0:r0 + o.shape[0]], L[hi, r0:r0 + o.shape[0]] = o, l
        return O, L
    with make_executor(min(n, len(tasks))) as ex:
        for (hi, r0), o, l in ex.map(_run, tasks, chunksize=1):
            O[hi, r0:r0 + o.shape[0]], L[hi, r0:r0 + o.shape[0]] = o, l
    return O, L


def attention(q, k, v, scale: Optional[float] = None, causal: bool = False,
              row_block: int = 1024, workers: Optional[int] = None):
    """definition.attention (every head, every row) on the process pool:
    O [B, H, Nq, d] and LSE [B, H, Nq] in float64."""
    B, H, Nq, d = q.shape
    heads = [(b, h) for b in range(B) for h in range(H)]
    O, L = attention_heads(q, k, v, heads, scale=scale, causal=causal, row_block=row_block,
                           workers=workers)
    return O.reshape(B, H, Nq, d), L.reshape(B, H, Nq)
