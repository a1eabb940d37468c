"""Worker processes for the oracle's per-query-block sub-problems (test
infrastructure).

A query row's output depends only on the keys its query block lists, and a
key's gradient is the sum of what the query rows that read it contribute, so
a whole head splits exactly into one sub-problem per query block.  The GPU
tests use that to check every row of large heads: the parent slices the rows
and keys of a chunk of query blocks and a worker runs the oracle on each
block's sub-problem.

Workers are started with the 'spawn' method and this module imports only
numpy and the oracle -- never torch or the HIP library -- so no worker
touches the GPU.  Each worker runs its BLAS on one thread.
"""

from __future__ import annotations

import math
import os

import numpy as np

from oracle import attention_backward, attention_forward, pattern_lists_for_head, pattern_token_mask

BLOCK = 64
_lists_cache = {}


def _init_worker():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass


def _lists(pattern, head, nb):
    key = (repr(pattern), head, nb)
    if key not in _lists_cache:
        _lists_cache.clear()
        _lists_cache[key] = pattern_lists_for_head(pattern, nb, head)
    return _lists_cache[key]


def _tokens(blocks):
    return np.concatenate([np.arange(j * BLOCK, (j + 1) * BLOCK) for j in blocks])


def _key_rows(key_blocks, wanted):
    """Row positions, inside arrays holding the tokens of ``key_blocks``, of
    the tokens of blocks ``wanted``."""
    at = {j: n for n, j in enumerate(key_blocks)}
    return np.concatenate([np.arange(at[j] * BLOCK, at[j] * BLOCK + BLOCK) for j in wanted])


def forward_chunk(task):
    """O, LSE of the rows of query blocks ``qblocks`` (float64).

    task: (pattern dict, head, L, scale, qblocks, q rows [n_q*64, d] of those
    blocks, key_blocks (sorted), k, v rows [n_k*64, d] of those blocks)."""
    pattern, head, L, scale, qblocks, q, key_blocks, k, v = task
    lists = _lists(pattern, head, -(-L // BLOCK))
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    o = np.zeros((len(qblocks) * BLOCK, q.shape[1]))
    lse = np.zeros(len(qblocks) * BLOCK)
    for n, i in enumerate(qblocks):
        rows = np.arange(i * BLOCK, (i + 1) * BLOCK)
        kr = _key_rows(key_blocks, lists[i])
        mask = pattern_token_mask(pattern, head, L, rows=rows, lists=lists)[:, _tokens(lists[i])]
        o[n * BLOCK:(n + 1) * BLOCK], lse[n * BLOCK:(n + 1) * BLOCK] = attention_forward(
            q[n * BLOCK:(n + 1) * BLOCK], k[kr], v[kr], mask, scale)
    return o, lse


def backward_chunk(task):
    """dQ of the rows of query blocks ``qblocks`` and those blocks' part of
    dK, dV on the rows of ``key_blocks`` (float64).

    task: (pattern dict, head, L, scale, qblocks, q, do rows of those blocks,
    key_blocks (sorted), k, v rows of those blocks)."""
    pattern, head, L, scale, qblocks, q, do, key_blocks, k, v = task
    lists = _lists(pattern, head, -(-L // BLOCK))
    q, do, k, v = (np.asarray(x, dtype=np.float64) for x in (q, do, k, v))
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for n, i in enumerate(qblocks):
        sl = slice(n * BLOCK, (n + 1) * BLOCK)
        rows = np.arange(i * BLOCK, (i + 1) * BLOCK)
        kr = _key_rows(key_blocks, lists[i])
        mask = pattern_token_mask(pattern, head, L, rows=rows, lists=lists)[:, _tokens(lists[i])]
        dqi, dki, dvi, _, _ = attention_backward(q[sl], k[kr], v[kr], do[sl], mask, scale)
        dq[sl] = dqi
        dk[kr] += dki
        dv[kr] += dvi
    return dq, dk, dv


def n_workers():
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, n))


def default_scale(d):
    return 1.0 / math.sqrt(d)
