"""Shared helpers of the GPU parity tests: tolerances, error metrics, and the
sub-problem extraction that lets the oracle check sampled outputs of large
inputs exactly (a query row depends only on its own key list; a key block's
dK/dV only on the query blocks that list it)."""

import math
import multiprocessing
from concurrent.futures import FIRST_COMPLETED, ProcessPoolExecutor, wait

import numpy as np
import torch

import long_context_sparse_static_amd as lcs
from oracle import (attention_backward, attention_forward, pattern_column_for_head,
                    pattern_lists_for_head, pattern_rows_for_head, pattern_token_mask)
from synth_inputs import as_f64

# bf16 path: max-abs 2e-2 and mean-abs 2e-3; fp32 path: max-abs 1e-5.
BF16_MAX, BF16_MEAN = 2e-2, 2e-3
F32_MAX = 1e-5

ORACLE_KIND = {lcs.ATTN_FULL: "full", lcs.ATTN_ATTNSINK: "attnsink", lcs.ATTN_BLOCKSPARSE: "blocksparse",
               lcs.ATTN_SLIDING: "sliding"}


def oracle_pattern(p: "lcs.Pattern") -> dict:
    return dict(kind=ORACLE_KIND[p.kind], block=p.block, sink_blocks=p.sink_blocks,
                local_blocks=p.local_blocks, stride=p.stride, causal=p.causal,
                window_tokens=p.window_tokens)


def errors(got, want):
    g = np.asarray(got, dtype=np.float64)
    w = np.asarray(want, dtype=np.float64)
    fin = np.isfinite(w)
    assert np.array_equal(np.isfinite(g), fin), "non-finite pattern differs"
    same_inf = (g[~fin] == w[~fin]).all() if (~fin).any() else True
    assert same_inf, "infinite entries differ"
    d = np.abs(g[fin] - w[fin])
    return (float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0)


def assert_bf16_close(got, want, what=""):
    mx, mean = errors(got, want)
    assert mx <= BF16_MAX and mean <= BF16_MEAN, f"{what}: max {mx:.3e} mean {mean:.3e}"
    return mx, mean


def assert_f32_close(got, want, what=""):
    mx, mean = errors(got, want)
    assert mx <= F32_MAX, f"{what}: max {mx:.3e} mean {mean:.3e}"
    return mx, mean


def need_gpu():
    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    lcs.lib()  # raises if the HIP library is not built


def sample_rows_forward(q, k, v, pattern, head, b, rows, scale=None):
    """Oracle O, LSE of sampled query rows of one (b, head), computed on the
    sub-problem of the keys those rows may see."""
    L, d = q.shape[2], q.shape[3]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    nb = -(-L // pattern.block)
    rows = np.asarray(sorted(rows))
    # only the sampled query blocks' rows ({block: list})
    lists = pattern_rows_for_head(oracle_pattern(pattern), sorted({int(r) // pattern.block for r in rows}),
                                  nb, head)
    kblocks = sorted({j for r in rows for j in lists[r // pattern.block]})
    keys = np.concatenate([np.arange(j * pattern.block, (j + 1) * pattern.block) for j in kblocks])
    mask = pattern_token_mask(oracle_pattern(pattern), head, L, rows=rows, lists=lists, keys=keys)
    qh = as_f64(q[b, head, torch.as_tensor(rows, device=q.device)])
    kh = as_f64(k[b, head, torch.as_tensor(keys, device=k.device)])
    vh = as_f64(v[b, head, torch.as_tensor(keys, device=v.device)])
    return attention_forward(qh, kh, vh, mask, scale)


def sample_backward(q, k, v, do, pattern, head, b, qblocks, kblocks, scale=None):
    """Oracle dQ rows of query blocks ``qblocks`` and dK/dV rows of key blocks
    ``kblocks`` for one (b, head).  A query block's gradients depend only on
    the keys it lists, so each query block is an exact sub-problem; a key
    block's dK/dV is the sum of the sub-problems of the query blocks that
    list it (its column).  Only the rows and columns involved are built and
    only their tokens are copied, so this scales to the longest sequences."""
    L, d = q.shape[2], q.shape[3]
    B_ = pattern.block
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    nb = -(-L // B_)
    opat = oracle_pattern(pattern)
    cols = {j: pattern_column_for_head(opat, j, nb, head) for j in kblocks}
    need = sorted(set(qblocks) | {i for j in kblocks for i in cols[j]})
    lists = pattern_rows_for_head(opat, need, nb, head)
    # token copies: the rows of the needed query blocks, the keys of their lists
    blocks = sorted(set(need) | {j for i in need for j in lists[i]})
    at = {j: n * B_ for n, j in enumerate(blocks)}
    tok = lambda bl: np.concatenate([np.arange(j * B_, (j + 1) * B_) for j in bl])
    idx = torch.as_tensor(tok(blocks), device=q.device)
    qh, kh, vh, doh = (as_f64(t[b, head].index_select(0, idx)) for t in (q, k, v, do))
    loc = lambda bl: np.concatenate([np.arange(at[j], at[j] + B_) for j in bl])
    cache = {}

    def sub(i):
        if i not in cache:
            rows, keys = loc([i]), loc(lists[i])
            mask = pattern_token_mask(opat, head, L, rows=tok([i]), lists=lists, keys=tok(lists[i]))
            cache[i] = attention_backward(qh[rows], kh[keys], vh[keys], doh[rows], mask, scale)[:3]
        return cache[i]

    out = {}
    for i in qblocks:
        out[("dq", i)] = sub(i)[0]
    for j in kblocks:
        dk = np.zeros((B_, d))
        dv = np.zeros((B_, d))
        for i in cols[j]:
            _, dki, dvi = sub(i)
            o = lists[i].index(j) * B_
            dk += dki[o:o + B_]
            dv += dvi[o:o + B_]
            if len(cache) > 256:
                cache.clear()
        out[("dk", j)] = dk
        out[("dv", j)] = dv
    return out


# ----------------------------------------------------------------------------
# Every row of whole heads: one oracle sub-problem per query block, run over a
# pool of spawned worker processes (tests/_oracle_pool.py: numpy and the
# oracle only, no GPU).
# ----------------------------------------------------------------------------
def _run_pool(fn, tasks, on_result):
    """fn(task) for each task of the iterable, at most two per worker in
    flight (tasks are built lazily: their input slices can be large);
    on_result(meta, result) in completion order."""
    import _oracle_pool as pool
    n = pool.n_workers()
    ctx = multiprocessing.get_context("spawn")
    with ProcessPoolExecutor(n, mp_context=ctx, initializer=pool._init_worker) as ex:
        pending = {}
        it = iter(tasks)
        done_all = False
        while True:
            while not done_all and len(pending) < 2 * n:
                try:
                    meta, task = next(it)
                except StopIteration:
                    done_all = True
                    break
                pending[ex.submit(fn, task)] = meta
            if not pending:
                break
            done, _ = wait(pending, return_when=FIRST_COMPLETED)
            for f in done:
                on_result(pending.pop(f), f.result())


def _blocks_tokens(blocks, block=64):
    return np.concatenate([np.arange(j * block, (j + 1) * block) for j in blocks])


def _head_rows(t, b, h):
    """One (b, h) of a device tensor as float32 host rows (bf16 values exactly)."""
    return t[b, h].to("cpu", torch.float32).numpy()


def oracle_forward_heads(q, k, v, pattern, heads, b=0, scale=None, chunk=32):
    """Oracle O [L,d] and LSE [L] (float64) of every row of each head in
    ``heads``, as {head: (o, lse)}, from exact per-query-block sub-problems."""
    import _oracle_pool as pool
    L, d = q.shape[2], q.shape[3]
    scale = pool.default_scale(d) if scale is None else scale
    nb = -(-L // pattern.block)
    opat = oracle_pattern(pattern)
    out = {h: (np.full((L, d), np.nan), np.full(L, np.nan)) for h in heads}

    def tasks():
        for h in heads:
            lists = pattern_lists_for_head(opat, nb, h)
            qh, kh, vh = (_head_rows(t, b, h) for t in (q, k, v))
            for c0 in range(0, nb, chunk):
                qblocks = list(range(c0, min(nb, c0 + chunk)))
                kb = sorted({j for i in qblocks for j in lists[i]})
                kt = _blocks_tokens(kb)
                yield (h, qblocks), (opat, h, L, scale, qblocks, qh[_blocks_tokens(qblocks)], kb,
                                     kh[kt], vh[kt])

    def put(meta, res):
        h, qblocks = meta
        rows = _blocks_tokens(qblocks)
        out[h][0][rows], out[h][1][rows] = res

    _run_pool(pool.forward_chunk, tasks(), put)
    return out


def oracle_backward_heads(q, k, v, do, pattern, heads, b=0, scale=None, chunk=32):
    """Oracle dQ, dK, dV [L,d] (float64) of each head in ``heads``, as
    {head: (dq, dk, dv)}: every query block's sub-problem, its dK/dV parts
    summed over the query blocks that read each key."""
    import _oracle_pool as pool
    L, d = q.shape[2], q.shape[3]
    scale = pool.default_scale(d) if scale is None else scale
    nb = -(-L // pattern.block)
    opat = oracle_pattern(pattern)
    out = {h: (np.full((L, d), np.nan), np.zeros((L, d)), np.zeros((L, d))) for h in heads}

    def tasks():
        for h in heads:
            lists = pattern_lists_for_head(opat, nb, h)
            qh, kh, vh, doh = (_head_rows(t, b, h) for t in (q, k, v, do))
            for c0 in range(0, nb, chunk):
                qblocks = list(range(c0, min(nb, c0 + chunk)))
                kb = sorted({j for i in qblocks for j in lists[i]})
                qt, kt = _blocks_tokens(qblocks), _blocks_tokens(kb)
                yield (h, qt, kt), (opat, h, L, scale, qblocks, qh[qt], doh[qt], kb, kh[kt], vh[kt])

    def put(meta, res):
        h, qt, kt = meta
        dq, dk, dv = res
        out[h][0][qt] = dq
        out[h][1][kt] += dk
        out[h][2][kt] += dv

    _run_pool(pool.backward_chunk, tasks(), put)
    return out
