"""Shared helpers of the GPU parity tests: tolerances, error metrics, and the
sub-problem extraction that lets the oracle check sampled outputs of large
inputs exactly (a query row depends only on its own key list; a key block's
dK/dV only on the query blocks that list it)."""

import math

import numpy as np
import torch

import long_context_sparse_static_amd as lcs
from oracle import (attention_backward, attention_forward, pattern_lists_for_head,
                    pattern_token_mask, transpose_lists)
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
    nb = L // pattern.block
    lists = pattern_lists_for_head(oracle_pattern(pattern), nb, head)
    rows = np.asarray(sorted(rows))
    kblocks = sorted({j for r in rows for j in lists[r // pattern.block]})
    keys = np.concatenate([np.arange(j * pattern.block, (j + 1) * pattern.block) for j in kblocks])
    mask = pattern_token_mask(oracle_pattern(pattern), head, L, rows=rows, lists=lists)[:, keys]
    qh = as_f64(q[b, head, torch.as_tensor(rows, device=q.device)])
    kh = as_f64(k[b, head, torch.as_tensor(keys, device=k.device)])
    vh = as_f64(v[b, head, torch.as_tensor(keys, device=v.device)])
    return attention_forward(qh, kh, vh, mask, scale)


def sample_backward(q, k, v, do, pattern, head, b, qblocks, kblocks, scale=None):
    """Oracle dQ rows of query blocks ``qblocks`` and dK/dV rows of key blocks
    ``kblocks`` for one (b, head).  A query block's gradients depend only on
    the keys it lists, so each query block is an exact sub-problem; a key
    block's dK/dV is the sum of the sub-problems of the query blocks that
    list it."""
    L, d = q.shape[2], q.shape[3]
    B_ = pattern.block
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    nb = L // B_
    opat = oracle_pattern(pattern)
    lists = pattern_lists_for_head(opat, nb, head)
    cols = transpose_lists(lists, nb)
    tok = lambda blocks: np.concatenate([np.arange(j * B_, (j + 1) * B_) for j in blocks])
    qh, kh, vh, doh = (as_f64(t[b, head]) for t in (q, k, v, do))
    cache = {}

    def sub(i):
        if i not in cache:
            rows, keys = tok([i]), tok(lists[i])
            mask = pattern_token_mask(opat, head, L, rows=rows, lists=lists)[:, keys]
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
            at = lists[i].index(j) * B_
            dk += dki[at:at + B_]
            dv += dvi[at:at + B_]
            if len(cache) > 256:
                cache.clear()
        out[("dk", j)] = dk
        out[("dv", j)] = dv
    return out
