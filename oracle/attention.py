"""Oracle for static block-sparse causal attention — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import anything in this package.  The product path (the HIP library
and its Python binding) never imports it, and this package imports nothing
from the product.

What is computed, and where it is stated
----------------------------------------
LongGen ("A Little Goes a Long Way: Efficient Long Context Training and
Inference with Partial Contexts") keeps 2/3 of the layers sparse with fixed
patterns -- attention sink (the first tokens), window attention (the most
recent tokens) and blockwise sparse attention (strided token blocks)
[mlsanity index page, section "Abstract (arXiv)"].  The sparsity is static and
block-wise and the training kernel is FlashAttention-2 based [atlas.scime.ai
summary, section "Approach"].  A static mask does not change what attention
computes; it only restricts the keys each query sees.  So this oracle is the
plain definition: build the block lists by brute-force scan, expand them to a
dense token mask, materialise the dense masked score matrix, and take an
ordinary softmax -- no tiling, no online softmax, no fusion.

Precision: every floating-point step runs in float64 on the CPU.  Inputs that
the GPU sees as bf16 are handed in as their exact values (bf16 -> float64 is
exact).

Readings taken where the pages are silent (each is listed in the design notes):
  * block size, sink / window / stride sizes come from the workload
    definitions (block 64, sink 1 block, window 4/16/64 blocks, stride 8);
  * the prefill window is block-granular and contains the diagonal block;
    causality masks keys later than the query inside any block;
  * a sequence of L tokens has ceil(L / block) blocks; when L is not a
    multiple of the block the last block is partial (its missing tokens do
    not exist: no query reads them and no row is computed for them);
  * BlockSparse head h takes blocks j < i with (j + h) mod stride == 0;
  * the softmax scale is 1/sqrt(d); LSE is the natural log of the sum of
    exp(scaled scores) over allowed keys; an empty row gives O = 0, LSE = -inf;
  * decode is token-granular: the new token t sees tokens 0..sink-1 and
    t-window+1..t (itself included);
  * the token-granular sliding window (kind "sliding", with or without sink
    blocks) applies that same token rule in prefill, so prefill row t and the
    decode of token t read the same keys.

Parity pins (tests/test_oracle_pins.py): every function here is pinned by a
check that does not re-type its formula -- closed-form counts, textbook /
library attention (torch scaled_dot_product_attention in float64 on the CPU),
Q = 0 and constant-V closed forms, and central finite differences for the
backward pass.  ``kv_cache_bytes`` is pinned to the pages' KV-memory figure
only up to the pages' unstated layer / window split (consistency only).
"""

from __future__ import annotations

import math

import numpy as np

FULL = "full"
ATTNSINK = "attnsink"
BLOCKSPARSE = "blocksparse"
SLIDING = "sliding"        # token-granular window (+ optional sink blocks)


# ----------------------------------------------------------------------------
# Block lists  [index page, Abstract: window / sink / strided-block patterns;
#               summary page, Approach: static, block-wise access]
# ----------------------------------------------------------------------------
def block_allowed(kind, i, j, *, sink_blocks=1, local_blocks=1, stride=0, head=0,
                  window_tokens=0, block=64):
    """Whether query block ``i`` reads key block ``j``:
      * full:        j <= i
      * attnsink:    j < sink_blocks (and j <= i), or i-local_blocks < j <= i
      * blocksparse: the attnsink rule, or j < i with (j + head) % stride == 0
      * sliding:     j <= i, and j < sink_blocks or the last key of block j is
                     within window_tokens of the first query of block i (the
                     blocks holding any key the token rule of
                     ``sliding_token_mask`` allows for some query of block i)
    """
    if kind == FULL:
        return j <= i
    if kind == SLIDING:
        return j <= i and (j < sink_blocks or block * i - (block * j + block - 1) < window_tokens)
    if kind in (ATTNSINK, BLOCKSPARSE):
        keep = (j < sink_blocks and j <= i) or (i - local_blocks) < j <= i
        if kind == BLOCKSPARSE and not keep and stride > 0:
            keep = j < i and (j + head) % stride == 0
        return keep
    raise ValueError(f"unknown pattern kind {kind!r}")


def block_list_row(kind, i, n_kblocks, **rule):
    """Ascending KV-block list of query block ``i``, by brute-force scan:
    every key block ``j`` in ``0..n_kblocks-1`` is tested on its own with
    ``block_allowed``."""
    return [j for j in range(n_kblocks) if block_allowed(kind, i, j, **rule)]


def block_column(kind, j, n_qblocks, **rule):
    """Ascending list of the query blocks that read key block ``j`` (column
    ``j`` of the lists), by the same scan over ``0..n_qblocks-1``."""
    return [i for i in range(n_qblocks) if block_allowed(kind, i, j, **rule)]


def block_lists(kind, n_qblocks, *, sink_blocks=1, local_blocks=1, stride=0,
                head=0, n_kblocks=None, window_tokens=0, block=64):
    """Ascending KV-block list of every query block (``block_list_row`` for
    each of ``0..n_qblocks-1``).  Returns a list of Python int lists."""
    if n_kblocks is None:
        n_kblocks = n_qblocks
    return [block_list_row(kind, i, n_kblocks, sink_blocks=sink_blocks, local_blocks=local_blocks,
                           stride=stride, head=head, window_tokens=window_tokens, block=block)
            for i in range(n_qblocks)]


def transpose_lists(lists, n_kblocks):
    """Column lists (query blocks that read key block j), ascending."""
    cols = [[] for _ in range(n_kblocks)]
    for i, row in enumerate(lists):
        for j in row:
            cols[j].append(i)
    return cols


def sliding_token_mask(n_q_tokens, n_k_tokens, sink_tokens, window_tokens, rows=None, keys=None):
    """Boolean [n_rows, n_keys] of the token-granular sliding window: query
    position q reads key position k when k <= q and either k is one of the
    first ``sink_tokens`` tokens or q - k < ``window_tokens`` (the window
    holds the query itself and the window_tokens - 1 tokens before it).
    With sink_tokens = 0 this is plain sliding-window attention.  ``rows`` /
    ``keys``: the query / key positions to evaluate (default: all)."""
    if rows is None:
        rows = np.arange(n_q_tokens)
    if keys is None:
        keys = np.arange(n_k_tokens)
    rows = np.asarray(rows)[:, None]
    k = np.asarray(keys)[None, :]
    return (k <= rows) & ((k < sink_tokens) | (rows - k < window_tokens))


def dense_token_mask(lists, block, n_q_tokens, n_k_tokens, causal, rows=None, keys=None):
    """Boolean [n_rows, n_keys]: key token allowed for a query token.

    ``rows`` lists the query-token positions (default 0..n_q_tokens-1),
    ``keys`` the key-token positions (default 0..n_k_tokens-1).  A key is
    allowed when its block is in the query block's list and, if ``causal``,
    its position does not exceed the query's position.  ``lists`` may be a
    dict holding only the query blocks of ``rows``.
    """
    if rows is None:
        rows = np.arange(n_q_tokens)
    if keys is None:
        m = np.zeros((len(rows), n_k_tokens), dtype=bool)
        for n, qi in enumerate(rows):
            for j in lists[qi // block]:
                lo = j * block
                hi = min(lo + block, n_k_tokens)
                m[n, lo:hi] = True
            if causal:
                m[n, qi + 1:] = False
        return m
    keys = np.asarray(keys)
    kb = keys // block
    m = np.zeros((len(rows), len(keys)), dtype=bool)
    for n, qi in enumerate(rows):
        m[n] = np.isin(kb, lists[qi // block]) & (keys < n_k_tokens)
        if causal:
            m[n] &= keys <= qi
    return m


# ----------------------------------------------------------------------------
# Prefill forward / backward on one head  (the plain softmax-attention
# definition under a fixed mask; FlashAttention-2 computes the same values)
# ----------------------------------------------------------------------------
def attention_forward(q, k, v, mask, scale, row_chunk=1024):
    """O, LSE for one head.  q [Lq,d], k/v [Lk,d], mask [Lq,Lk] bool.

    S = scale * q k^T; S = -inf where masked; P = softmax(S) row-wise;
    O = P v; LSE = log(sum(exp(S))).  Rows with no allowed key: O = 0,
    LSE = -inf.  Processed in query-row chunks; each chunk holds its full
    dense masked score rows.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Lq = q.shape[0]
    o = np.zeros((Lq, v.shape[1]), dtype=np.float64)
    lse = np.full((Lq,), -np.inf, dtype=np.float64)
    for r0 in range(0, Lq, row_chunk):
        r1 = min(r0 + row_chunk, Lq)
        s = (q[r0:r1] @ k.T) * scale
        mk = mask[r0:r1]
        s = np.where(mk, s, -np.inf)
        m = s.max(axis=1)
        live = np.isfinite(m)
        m_safe = np.where(live, m, 0.0)
        p = np.exp(s - m_safe[:, None])          # exp(-inf) = 0 on masked keys
        l = p.sum(axis=1)
        o_chunk = p @ v
        o[r0:r1][live] = o_chunk[live] / l[live][:, None]
        lse[r0:r1][live] = m[live] + np.log(l[live])
    return o, lse


def attention_backward(q, k, v, do, mask, scale, row_chunk=1024):
    """dQ, dK, dV of loss = sum(O * dO) for one head, plus (O, LSE).

    With P the masked softmax of the forward pass:
      D  = rowsum(dO * O)
      dV = P^T dO
      dP = dO V^T
      dS = P * (dP - D)
      dQ = scale * dS K
      dK = scale * dS^T Q
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    o, lse = attention_forward(q, k, v, mask, scale, row_chunk)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    Lq = q.shape[0]
    for r0 in range(0, Lq, row_chunk):
        r1 = min(r0 + row_chunk, Lq)
        s = (q[r0:r1] @ k.T) * scale
        mk = mask[r0:r1]
        live = np.isfinite(lse[r0:r1])
        lse_safe = np.where(live, lse[r0:r1], 0.0)
        p = np.where(mk, np.exp(s - lse_safe[:, None]), 0.0)
        p[~live] = 0.0
        d_row = (do[r0:r1] * o[r0:r1]).sum(axis=1)
        dv += p.T @ do[r0:r1]
        dp = do[r0:r1] @ v.T
        ds = p * (dp - d_row[:, None])
        dq[r0:r1] = scale * (ds @ k)
        dk += scale * (ds.T @ q[r0:r1])
    return dq, dk, dv, o, lse


# ----------------------------------------------------------------------------
# Batched prefill wrappers over [B,H,L,d]
# ----------------------------------------------------------------------------
def head_pattern(pattern, head):
    """The pattern dict head ``head`` follows: ``pattern`` itself, or its
    entry ``head`` when it is a per-head list (a mix such as retrieval heads
    with full attention beside sink + window streaming heads: DuoAttention,
    Hugging Face paper-search page "long-context decoding latency")."""
    return pattern[head] if isinstance(pattern, (list, tuple)) else pattern


def pattern_lists_for_head(pattern, n_qblocks, head):
    pattern = head_pattern(pattern, head)
    return block_lists(pattern["kind"], n_qblocks,
                       sink_blocks=pattern.get("sink_blocks", 0),
                       local_blocks=pattern.get("local_blocks", 0),
                       stride=pattern.get("stride", 0), head=head,
                       window_tokens=pattern.get("window_tokens", 0),
                       block=pattern.get("block", 64))


def _rule(p, head):
    return dict(sink_blocks=p.get("sink_blocks", 0), local_blocks=p.get("local_blocks", 0),
                stride=p.get("stride", 0), head=head, window_tokens=p.get("window_tokens", 0),
                block=p.get("block", 64))


def pattern_rows_for_head(pattern, qblocks, n_kblocks, head):
    """{i: list of query block i} for the listed query blocks only (the same
    rows ``pattern_lists_for_head`` gives, without building every row)."""
    p = head_pattern(pattern, head)
    return {i: block_list_row(p["kind"], i, n_kblocks, **_rule(p, head)) for i in qblocks}


def pattern_column_for_head(pattern, j, n_qblocks, head):
    """Ascending query blocks of head ``head`` that read key block ``j`` (the
    column ``transpose_lists`` gives, without building every row)."""
    p = head_pattern(pattern, head)
    return block_column(p["kind"], j, n_qblocks, **_rule(p, head))


def pattern_token_mask(pattern, head, L, rows=None, lists=None, keys=None):
    """Dense [n_rows, n_keys] mask of head ``head``: the token rule for a
    sliding pattern, else the block lists expanded to tokens (causal inside
    blocks).  ``lists``: this head's block lists if the caller already holds
    them (pattern_lists_for_head's result, or a dict of the rows' blocks), to
    skip building them again.  ``rows`` / ``keys``: the positions to evaluate
    (default: all)."""
    p = head_pattern(pattern, head)
    if p["kind"] == SLIDING:
        return sliding_token_mask(L, L, p["block"] * p.get("sink_blocks", 0),
                                  p["window_tokens"], rows=rows, keys=keys)
    if lists is None:
        lists = pattern_lists_for_head(pattern, -(-L // p["block"]), head)   # last block may be partial
    return dense_token_mask(lists, p["block"], L, L, p.get("causal", True), rows=rows, keys=keys)


def sparse_forward(q, k, v, pattern, scale=None, heads=None, rows=None):
    """Forward over [B,H,L,d] arrays for the given pattern dict (or list of
    dicts, one per head).

    ``heads``: optional list of head indices to compute (others left NaN).
    ``rows``:  optional array of query-token indices to compute (others NaN).
    Returns (o [B,H,L,d], lse [B,H,L]) in float64.
    """
    B, H, L, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = np.full((B, H, L, d), np.nan)
    lse = np.full((B, H, L), np.nan)
    heads = range(H) if heads is None else heads
    for h in heads:
        if rows is None:
            mask = pattern_token_mask(pattern, h, L)
            for b in range(B):
                o[b, h], lse[b, h] = attention_forward(q[b, h], k[b, h], v[b, h], mask, scale)
        else:
            rows = np.asarray(rows)
            mask = pattern_token_mask(pattern, h, L, rows=rows)
            for b in range(B):
                ob, lb = attention_forward(q[b, h][rows], k[b, h], v[b, h], mask, scale)
                o[b, h][rows] = ob
                lse[b, h][rows] = lb
    return o, lse


def sparse_backward(q, k, v, do, pattern, scale=None, heads=None):
    """Backward over [B,H,L,d]; returns dq, dk, dv, o, lse (float64)."""
    B, H, L, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    shp = (B, H, L, d)
    dq, dk, dv, o = (np.full(shp, np.nan) for _ in range(4))
    lse = np.full((B, H, L), np.nan)
    heads = range(H) if heads is None else heads
    for h in heads:
        mask = pattern_token_mask(pattern, h, L)
        for b in range(B):
            dq[b, h], dk[b, h], dv[b, h], o[b, h], lse[b, h] = attention_backward(
                q[b, h], k[b, h], v[b, h], do[b, h], mask, scale)
    return dq, dk, dv, o, lse


# ----------------------------------------------------------------------------
# Decode  [index page, Abstract: reduced KV cache; summary page, Key results:
#          KV memory cut from keeping only part of the context in sparse layers]
# ----------------------------------------------------------------------------
def decode_positions(t, sink_tokens=None, window_tokens=None):
    """Token positions the new token at absolute position t attends to.

    Full layers (sink_tokens is None): 0..t.  Sparse layers: the first
    ``sink_tokens`` tokens and the last ``window_tokens`` tokens up to and
    including t, as a sorted set.
    """
    if sink_tokens is None:
        return np.arange(t + 1)
    keep = set(range(min(sink_tokens, t + 1)))
    keep.update(range(max(0, t - window_tokens + 1), t + 1))
    return np.array(sorted(keep), dtype=np.int64)


def blocksparse_decode_positions(t, pattern, head):
    """Token positions the token at absolute position t reads in a layer with
    a block pattern (BlockSparse, or any pattern dict): the key blocks its
    query block lists, keys later than t masked -- exactly its row of the
    prefill mask.  Used for BlockSparse decode against a compacted cache."""
    block = head_pattern(pattern, head)["block"]
    i = t // block
    row = pattern_lists_for_head(pattern, i + 1, head)[i]
    keep = [p for j in row for p in range(j * block, (j + 1) * block) if p <= t]
    return np.array(keep, dtype=np.int64)


def decode_one(q, k_hist, v_hist, positions, scale):
    """o, lse of one query over the listed token rows of its history."""
    q = np.asarray(q, dtype=np.float64)
    kk = np.asarray(k_hist, dtype=np.float64)[positions]
    vv = np.asarray(v_hist, dtype=np.float64)[positions]
    s = (kk @ q) * scale
    m = s.max()
    p = np.exp(s - m)
    l = p.sum()
    return (p @ vv) / l, m + math.log(l)


# ----------------------------------------------------------------------------
# KV-cache size (closed form)  [summary page, Key results and "Measured
# effects" table: KV memory of the 1/3-full hybrid vs full attention]
# ----------------------------------------------------------------------------
def kv_cache_bytes(n_layers_full, n_layers_sparse, heads, head_dim, tokens,
                   sparse_tokens, bytes_per_elem=2, batch=1):
    """Bytes of K and V kept by a hybrid model: full layers keep every token,
    sparse layers keep only their sink+window tokens."""
    per_token_layer = 2 * heads * head_dim * bytes_per_elem * batch
    return per_token_layer * (n_layers_full * tokens + n_layers_sparse * sparse_tokens)
