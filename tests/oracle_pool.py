"""The oracle over many (batch, head) sequences at once, in parallel CPU worker processes.

The oracle is sequential per sequence and single-threaded, and the sequences are
independent, so the full-size parity cases split them into groups and run the groups in
worker processes.  The workers are started fresh (spawn) and import only numpy, the oracle
and (for the vector-Jacobian products) torch on the CPU; they run no GPU work.  At most 8
of them run at once: a GPU machine allows few processes per GPU, and a process that imports
torch may count as one.
"""
from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os

import numpy as np


def n_workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(8, n))


def _run(task):
    fn, args, kw = task
    if fn.endswith("_vjp"):  # autograd on the CPU, one thread per worker
        import torch
        torch.set_num_threads(1)
    from oracle import ttt_oracle as O
    return getattr(O, fn)(*args, **kw)


def _take(x, bs, hs, shared_ndim):
    """Sequences (bs[i], hs[i]) of x as a [1, n, ...] array: x is per sequence [B, H, ...],
    per head [H, ...] (ndim == shared_ndim), or None / a scalar (passed through)."""
    if isinstance(x, tuple):
        return tuple(_take(e, bs, hs, shared_ndim) for e in x)
    if x is None or np.ndim(x) == 0:
        return x
    x = np.asarray(x)
    if x.ndim == shared_ndim:
        return np.ascontiguousarray(x[hs][None])
    return np.ascontiguousarray(x[bs, hs][None])


def run_chains(fn, B, H, args, kw, shared_ndim, groups=None):
    """Call oracle function `fn` on every (b, h) sequence, in groups, and reassemble.

    args / kw hold the call's arguments; every array among them is either per sequence
    ([B, H, ...]), per head (ndim == shared_ndim[name or position], e.g. a shared initial
    state [H, r, c]) or not an array.  Returns the function's outputs with leading dims
    [B, H], in sequence order.
    """
    chains = [(b, h) for b in range(B) for h in range(H)]
    ng = groups or min(len(chains), 4 * n_workers())
    parts = [chains[i::ng] for i in range(ng)]
    parts = [p for p in parts if p]
    tasks = []
    for p in parts:
        bs = np.array([c[0] for c in p])
        hs = np.array([c[1] for c in p])
        a2 = tuple(_take(x, bs, hs, shared_ndim.get(i, -1)) for i, x in enumerate(args))
        k2 = {name: _take(x, bs, hs, shared_ndim.get(name, -1)) for name, x in kw.items()}
        tasks.append((fn, a2, k2))
    ctx = mp.get_context("spawn")
    with cf.ProcessPoolExecutor(max_workers=min(n_workers(), len(tasks)), mp_context=ctx) as ex:
        results = list(ex.map(_run, tasks))
    outs = []
    for j in range(len(results[0])):
        first = results[0][j]
        if first is None:
            outs.append(None)
            continue
        full = np.zeros((B, H) + first.shape[2:], dtype=first.dtype)
        for p, r in zip(parts, results):
            for i, (b, h) in enumerate(p):
                full[b, h] = r[j][0, i]
        outs.append(full)
    return tuple(outs)
