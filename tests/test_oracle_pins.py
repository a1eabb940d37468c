"""Pins of the oracle against things other than itself (CPU only).

Each check is chosen so that a plausible slip in the oracle -- a dropped
term, a wrong sign, an off-by-one in a window, a transposed operand -- fails
at least one of them:
  * block lists: a hand-written golden list, and closed-form row lengths;
  * forward: torch's scaled_dot_product_attention (float64, CPU) on the
    special cases that reduce to it; Q = 0 and constant-V closed forms;
  * backward: central finite differences in float64, and torch autograd on
    the full-causal special case and on head-dependent masks built by a
    separate rule (the batched wrapper's per-head dispatch and output order);
  * per-head pattern lists: each head runs its own pattern (the same head of
    a single-pattern run, and per-head Q = 0 closed-form counts);
  * decode: library attention on its reducible cases and a Q = 0 count;
  * KV memory: the pages' own figures (consistency only).
"""

import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import (ATTNSINK, BLOCKSPARSE, FULL, SLIDING, attention_backward,
                    attention_forward, block_lists, blocksparse_decode_positions,
                    decode_one, decode_positions, dense_token_mask, kv_cache_bytes,
                    pattern_column_for_head, pattern_lists_for_head, pattern_rows_for_head,
                    pattern_token_mask, sliding_token_mask, sparse_backward,
                    sparse_forward, transpose_lists)


# --------------------------------------------------------------------------
# helpers that are NOT the oracle
# --------------------------------------------------------------------------
def sdpa(q, k, v, attn_mask=None, is_causal=False, scale=None):
    """torch's library attention in float64 on the CPU, one head, 2-D arrays."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))[None, None]
    m = None if attn_mask is None else torch.from_numpy(attn_mask)[None, None]
    out = F.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m,
                                         is_causal=is_causal, scale=scale)
    return out[0, 0].numpy()


def attnsink_row_len(i, s, w):
    """Closed form: |{0..min(s,i+1)-1} U {max(0,i-w+1)..i}|."""
    a = max(0, i - w + 1)
    return (i - a + 1) + min(s, a)


def blocksparse_row_len(i, s, w, stride, h):
    """Closed form for the sink + local + strided rule (stride offset h)."""
    a = max(0, i - w + 1)                      # first local block
    local = i - a + 1
    r = (-h) % stride                          # j = r (mod stride) are strided
    strided_below = 0 if a <= r else (a - 1 - r) // stride + 1
    sink_extra = sum(1 for j in range(min(s, a)) if (j % stride) != r)
    return local + strided_below + sink_extra


def read_golden_lists(path):
    rows = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, vals = line.split(":")
            rows[int(key)] = [int(x) for x in vals.split()]
    return [rows[i] for i in range(len(rows))]


# --------------------------------------------------------------------------
# block lists
# --------------------------------------------------------------------------
def test_attnsink_lists_match_hand_written_golden(golden_dir):
    want = read_golden_lists(os.path.join(golden_dir, "attnsink_nb16_sink1_local4_lists.txt"))
    got = block_lists(ATTNSINK, 16, sink_blocks=1, local_blocks=4)
    assert got == want
    assert sum(len(r) for r in got) == 70


@pytest.mark.parametrize("nb,s,w", [(16, 1, 4), (40, 2, 7), (33, 0, 1), (12, 3, 20), (9, 1, 1)])
def test_attnsink_row_lengths_closed_form(nb, s, w):
    lists = block_lists(ATTNSINK, nb, sink_blocks=s, local_blocks=w)
    for i, row in enumerate(lists):
        assert row == sorted(set(row))
        assert len(row) == attnsink_row_len(i, s, w)
        assert i in row if w >= 1 else True           # diagonal block always present


@pytest.mark.parametrize("h", range(8))
def test_blocksparse_row_lengths_closed_form(h):
    nb = 150
    lists = block_lists(BLOCKSPARSE, nb, sink_blocks=1, local_blocks=16, stride=8, head=h)
    for i, row in enumerate(lists):
        assert row == sorted(set(row))
        assert len(row) == blocksparse_row_len(i, 1, 16, 8, h), (i, row)
        # every strided block below the local window has (j + h) % 8 == 0
        for j in row:
            if j > 0 and j <= i - 16:
                assert (j + h) % 8 == 0


def test_workload_nnz_closed_forms():
    # AttnSink, sink 1 block: sum_{i<w}(i+1) + (nb-w)(w+1)
    for nb, w in [(16, 4), (128, 64), (1024, 64), (2048, 64)]:
        closed = w * (w + 1) // 2 + (nb - w) * (w + 1)
        got = sum(len(r) for r in block_lists(ATTNSINK, nb, sink_blocks=1, local_blocks=w))
        assert got == closed
    assert [w * (w + 1) // 2 + (nb - w) * (w + 1) for nb, w in
            [(16, 4), (128, 64), (1024, 64), (2048, 64)]] == [70, 6240, 64480, 131040]
    # full pattern: nb (nb+1) / 2
    assert sum(len(r) for r in block_lists(FULL, 100)) == 100 * 101 // 2
    # BlockSparse at 32768 tokens (512 blocks), 32 heads: closed form per head
    per_head = [sum(blocksparse_row_len(i, 1, 16, 8, h) for i in range(512)) for h in range(32)]
    assert min(per_head) == 23696 and max(per_head) == 24130 and sum(per_head) == 765216
    for h in (0, 3, 7, 12):
        got = block_lists(BLOCKSPARSE, 512, sink_blocks=1, local_blocks=16, stride=8, head=h)
        assert sum(len(r) for r in got) == per_head[h]


@pytest.mark.parametrize("kind,extra", [(ATTNSINK, dict(sink_blocks=2, local_blocks=3)),
                                        (BLOCKSPARSE, dict(sink_blocks=1, local_blocks=2, stride=3)),
                                        (FULL, dict()), (SLIDING, dict(sink_blocks=1, window_tokens=150))])
def test_row_subset_equals_whole_lists(kind, extra):
    """Building only some query blocks' rows gives the same rows."""
    pat = dict(kind=kind, block=64, causal=True, **extra)
    for h in (0, 1, 2):
        whole = pattern_lists_for_head(pat, 23, h)
        some = pattern_rows_for_head(pat, [0, 5, 17, 22], 23, h)
        assert all(some[i] == whole[i] for i in some)


@pytest.mark.parametrize("kind,extra", [(ATTNSINK, dict(sink_blocks=2, local_blocks=3)),
                                        (BLOCKSPARSE, dict(sink_blocks=1, local_blocks=2, stride=3)),
                                        (FULL, dict()), (SLIDING, dict(sink_blocks=1, window_tokens=150))])
def test_single_columns_equal_transposed_rows(kind, extra):
    """A key block's column built on its own (the same membership rule
    scanned over query blocks) is that column of the transposed rows."""
    pat = dict(kind=kind, block=64, causal=True, **extra)
    for h in (0, 1, 2):
        cols = transpose_lists(pattern_lists_for_head(pat, 23, h), 23)
        assert all(pattern_column_for_head(pat, j, 23, h) == cols[j] for j in range(23))


@pytest.mark.parametrize("kind,extra", [(BLOCKSPARSE, dict(sink_blocks=1, local_blocks=2, stride=3)),
                                        (SLIDING, dict(sink_blocks=1, window_tokens=150)),
                                        (FULL, dict())])
def test_masks_at_key_subsets(kind, extra):
    """Masks evaluated at chosen key positions equal those columns of the
    whole mask (rows as well), with the rows' lists given whole or as a dict
    of just their query blocks."""
    pat = dict(kind=kind, block=64, causal=True, **extra)
    L, h = 64 * 9, 1
    rng = np.random.default_rng(3)
    rows = np.sort(rng.choice(L, 40, replace=False))
    keys = np.concatenate([np.arange(64, 192), rng.choice(L, 50, replace=False)])
    whole = pattern_token_mask(pat, h, L, rows=rows)
    assert np.array_equal(pattern_token_mask(pat, h, L, rows=rows, keys=keys), whole[:, keys])
    some = pattern_rows_for_head(pat, sorted({int(r) // 64 for r in rows}), L // 64, h)
    assert np.array_equal(pattern_token_mask(pat, h, L, rows=rows, lists=some, keys=keys), whole[:, keys])
    lists = pattern_lists_for_head(pat, L // 64, h)
    assert np.array_equal(dense_token_mask(lists, 64, L, L, True, rows=rows, keys=keys),
                          dense_token_mask(lists, 64, L, L, True, rows=rows)[:, keys])
    assert np.array_equal(sliding_token_mask(L, L, 64, 100, rows=rows, keys=keys),
                          sliding_token_mask(L, L, 64, 100, rows=rows)[:, keys])


def test_transpose_lists_roundtrip():
    lists = block_lists(BLOCKSPARSE, 40, sink_blocks=1, local_blocks=5, stride=8, head=3)
    cols = transpose_lists(lists, 40)
    pairs_r = sorted((i, j) for i, r in enumerate(lists) for j in r)
    pairs_c = sorted((i, j) for j, c in enumerate(cols) for i in c)
    assert pairs_r == pairs_c
    for c in cols:
        assert c == sorted(c)
    assert len(cols[0]) == 40                          # the sink column is read by every row


# --------------------------------------------------------------------------
# forward
# --------------------------------------------------------------------------
rng = np.random.default_rng(20241002)


def rand(*shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("L,block,d", [(96, 16, 8), (64, 64, 16), (130, 13, 5), (100, 16, 8), (37, 64, 4)])
def test_full_pattern_is_causal_attention(L, block, d):
    q, k, v = rand(L, d), rand(L, d), rand(L, d)
    nb = -(-L // block)
    lists = block_lists(FULL, nb)
    mask = dense_token_mask(lists, block, L, L, causal=True)
    scale = 1 / math.sqrt(d)
    o, lse = attention_forward(q, k, v, mask, scale)
    np.testing.assert_allclose(o, sdpa(q, k, v, is_causal=True, scale=scale), rtol=0, atol=1e-12)
    # LSE against its definition via torch.logsumexp over the causal rows
    s = torch.from_numpy(q @ k.T * scale)
    s = s.masked_fill(torch.ones(L, L, dtype=torch.bool).triu(1), -math.inf)
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=1).numpy(), rtol=0, atol=1e-12)


def test_window_covering_sequence_is_full():
    L, block, d = 128, 16, 8
    q, k, v = rand(L, d), rand(L, d), rand(L, d)
    m_sink = dense_token_mask(block_lists(ATTNSINK, 8, sink_blocks=1, local_blocks=8), block, L, L, True)
    m_bs = dense_token_mask(block_lists(BLOCKSPARSE, 8, sink_blocks=1, local_blocks=8, stride=2, head=1),
                            block, L, L, True)
    ref = sdpa(q, k, v, is_causal=True, scale=0.3)
    for m in (m_sink, m_bs):
        o, _ = attention_forward(q, k, v, m, 0.3)
        np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_local_one_block_no_sink_is_block_diagonal():
    L, block, d = 80, 16, 6
    q, k, v = rand(L, d), rand(L, d), rand(L, d)
    mask = dense_token_mask(block_lists(ATTNSINK, 5, sink_blocks=0, local_blocks=1), block, L, L, True)
    o, _ = attention_forward(q, k, v, mask, 0.5)
    for b0 in range(0, L, block):
        sl = slice(b0, b0 + block)
        np.testing.assert_allclose(o[sl], sdpa(q[sl], k[sl], v[sl], is_causal=True, scale=0.5),
                                   rtol=0, atol=1e-12)


def test_general_pattern_matches_library_with_mask():
    # sink + window + stride pattern: compare against SDPA with the same boolean mask
    L, block, d = 160, 16, 8
    q, k, v = rand(L, d), rand(L, d), rand(L, d)
    lists = block_lists(BLOCKSPARSE, 10, sink_blocks=1, local_blocks=2, stride=3, head=2)
    mask = dense_token_mask(lists, block, L, L, True)
    o, _ = attention_forward(q, k, v, mask, 0.25)
    np.testing.assert_allclose(o, sdpa(q, k, v, attn_mask=mask, scale=0.25), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# token-granular sliding window
# --------------------------------------------------------------------------
def test_sliding_mask_examples():
    """Hand-checked rows: window 3, sink 2 tokens, 8 tokens."""
    m = sliding_token_mask(8, 8, 2, 3)
    assert [list(np.nonzero(m[q])[0]) for q in (0, 1, 2, 4, 7)] == [
        [0], [0, 1], [0, 1, 2], [0, 1, 2, 3, 4], [0, 1, 5, 6, 7]]
    m0 = sliding_token_mask(8, 8, 0, 3)
    assert list(np.nonzero(m0[7])[0]) == [5, 6, 7] and list(np.nonzero(m0[1])[0]) == [0, 1]


@pytest.mark.parametrize("L,block,s,W", [(96, 8, 0, 5), (96, 8, 1, 8), (100, 10, 2, 17),
                                         (128, 16, 0, 1), (64, 8, 3, 200)])
def test_sliding_block_lists_are_the_blocks_the_token_rule_touches(L, block, s, W):
    """Block lists of the sliding kind == the block pairs holding any allowed
    token pair, found by scanning the token mask."""
    nb = L // block
    m = sliding_token_mask(L, L, block * s, W)
    want = [[j for j in range(nb) if m[i * block:(i + 1) * block, j * block:(j + 1) * block].any()]
            for i in range(nb)]
    assert block_lists(SLIDING, nb, sink_blocks=s, window_tokens=W, block=block) == want


def test_sliding_window_reduces_to_library_attention():
    """No sink and a window covering the sequence: causal attention.  Window
    of 1: every token reads only itself (O = V).  A general band against SDPA
    with the band built from torch's triangular masks."""
    L, d = 48, 6
    q, k, v = rand(1, 1, L, d), rand(1, 1, L, d), rand(1, 1, L, d)
    pat = lambda s, W: dict(kind=SLIDING, block=8, sink_blocks=s, window_tokens=W)
    o, _ = sparse_forward(q, k, v, pat(0, L), scale=0.4)
    np.testing.assert_allclose(o[0, 0], sdpa(q[0, 0], k[0, 0], v[0, 0], is_causal=True, scale=0.4),
                               atol=1e-12)
    o, lse = sparse_forward(q, k, v, pat(0, 1), scale=0.4)
    np.testing.assert_allclose(o[0, 0], v[0, 0], atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], 0.4 * np.einsum("id,id->i", q[0, 0], k[0, 0]), atol=1e-12)
    ones = torch.ones(L, L, dtype=torch.bool)
    band = (ones.tril(0) & ~ones.tril(-7)).numpy()          # q - 6 <= k <= q
    band[:, :8] |= ones.tril(0).numpy()[:, :8]               # plus sink block 0
    o, _ = sparse_forward(q, k, v, pat(1, 7), scale=0.4)
    np.testing.assert_allclose(o[0, 0], sdpa(q[0, 0], k[0, 0], v[0, 0], attn_mask=band, scale=0.4),
                               atol=1e-12)


def test_sliding_zero_query_counts():
    """Q = 0: LSE = ln(number of keys read) = ln(min(q + 1, W + sink keys
    outside the window))."""
    L, d, block, s, W = 120, 4, 8, 1, 13
    q, k, v = np.zeros((1, 1, L, d)), rand(1, 1, L, d), rand(1, 1, L, d)
    _, lse = sparse_forward(q, k, v, dict(kind=SLIDING, block=block, sink_blocks=s, window_tokens=W),
                            scale=1.0)
    for t in range(L):
        n = min(t + 1, W) + max(0, min(block * s, t + 1 - W))
        assert lse[0, 0, t] == pytest.approx(math.log(n), abs=1e-12)


def test_sliding_prefill_row_equals_decode():
    """With the token-granular window, prefill row t reads exactly the keys
    decode of token t reads (sink tokens and the last W positions)."""
    B, H, L, d = 1, 1, 160, 4
    q, k, v = rand(B, H, L, d), rand(B, H, L, d), rand(B, H, L, d)
    pat = dict(kind=SLIDING, block=16, sink_blocks=1, window_tokens=37)
    rows = [0, 15, 16, 36, 37, 52, 53, 100, 159]
    o, lse = sparse_forward(q, k, v, pat, scale=0.3, rows=rows)
    for t in rows:
        od, ld = decode_one(q[0, 0, t], k[0, 0], v[0, 0], decode_positions(t, 16, 37), 0.3)
        np.testing.assert_allclose(od, o[0, 0, t], atol=1e-12)
        assert ld == pytest.approx(lse[0, 0, t], abs=1e-12)


@pytest.mark.parametrize("short", [0, 3], ids=["whole_blocks", "partial_last_block"])
@pytest.mark.parametrize("kind,s,w,stride,h", [(ATTNSINK, 1, 4, 0, 0), (ATTNSINK, 2, 3, 0, 0),
                                               (BLOCKSPARSE, 1, 3, 4, 1), (FULL, 0, 0, 0, 0)])
def test_zero_query_closed_form(kind, s, w, stride, h, short):
    """Q = 0: every allowed score is 0, so LSE = ln(count) and O = mean(V)
    (also with the last block 3 tokens short)."""
    block, nb, d = 8, 13, 4
    L = block * nb - short
    q, k, v = np.zeros((L, d)), rand(L, d), rand(L, d)
    lists = block_lists(kind, nb, sink_blocks=s, local_blocks=w, stride=stride, head=h)
    o, lse = attention_forward(q, k, v, dense_token_mask(lists, block, L, L, True), 0.7)
    for p in range(L):
        bi, r = divmod(p, block)
        if kind == FULL:
            n_blocks = bi + 1
        elif kind == ATTNSINK:
            n_blocks = attnsink_row_len(bi, s, w)
        else:
            n_blocks = blocksparse_row_len(bi, s, w, stride, h)
        count = block * (n_blocks - 1) + r + 1        # every list holds its diagonal block
        assert lse[p] == pytest.approx(math.log(count), abs=1e-12)
        if kind == ATTNSINK:
            keys = set(range(0, block * min(s, bi))) | set(range(max(0, bi - w + 1) * block, p + 1))
            np.testing.assert_allclose(o[p], v[sorted(keys)].mean(axis=0), atol=1e-12)


@pytest.mark.parametrize("kind,extra", [(ATTNSINK, dict(sink_blocks=1, local_blocks=2)),
                                        (BLOCKSPARSE, dict(sink_blocks=1, local_blocks=2, stride=3)),
                                        (FULL, dict()), (SLIDING, dict(sink_blocks=1, window_tokens=100))])
def test_partial_last_block_is_the_truncated_problem(kind, extra):
    """L = 64 nb - 27 tokens: the mask is the top-left L x L corner of the
    mask for 64 nb tokens, and with causality the outputs and gradients of
    the L rows equal those of the longer sequence restricted to them (its
    extra tokens come later than every one of the L queries)."""
    pat = dict(kind=kind, block=64, causal=True, **extra)
    nb, h, d = 5, 2, 8
    Lp = 64 * nb
    L = Lp - 27
    for hh in (0, h):
        np.testing.assert_array_equal(pattern_token_mask(pat, hh, L), pattern_token_mask(pat, hh, Lp)[:L, :L])
    q, k, v, do = (rand(1, 3, Lp, d) for _ in range(4))
    o_p, lse_p = sparse_forward(q, k, v, pat)
    o, lse = sparse_forward(q[:, :, :L], k[:, :, :L], v[:, :, :L], pat)
    np.testing.assert_allclose(o, o_p[:, :, :L], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_p[:, :, :L], rtol=0, atol=1e-12)
    do[:, :, L:] = 0.0   # the extra queries add nothing to dK, dV of the first L keys
    g_p = sparse_backward(q, k, v, do, pat)
    g = sparse_backward(q[:, :, :L], k[:, :, :L], v[:, :, :L], do[:, :, :L], pat)
    for a_, b_ in zip(g[:3], g_p[:3]):
        np.testing.assert_allclose(a_, b_[:, :, :L], rtol=0, atol=1e-12)


def test_constant_values_give_constant_output():
    L, block, d = 96, 16, 5
    q, k = 3 * rand(L, d), rand(L, d)
    c = rand(d)
    v = np.tile(c, (L, 1))
    lists = block_lists(BLOCKSPARSE, 6, sink_blocks=1, local_blocks=2, stride=2, head=1)
    o, _ = attention_forward(q, k, v, dense_token_mask(lists, block, L, L, True), 0.4)
    np.testing.assert_allclose(o, np.tile(c, (L, 1)), atol=1e-12)


def test_softmax_rows_sum_to_one():
    L, block, d = 64, 16, 8
    q, k, v = rand(L, d), rand(L, d), rand(L, d)
    mask = dense_token_mask(block_lists(ATTNSINK, 4, sink_blocks=1, local_blocks=2), block, L, L, True)
    _, lse = attention_forward(q, k, v, mask, 0.35)
    p = np.exp(q @ k.T * 0.35 - lse[:, None]) * mask
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12)


def test_empty_row_gives_zero_and_minus_inf():
    L, block, d = 32, 16, 4
    q, k, v = rand(L, d), rand(L, d), rand(L, d)
    lists = [[], [0, 1]]                                # query block 0 reads nothing
    o, lse = attention_forward(q, k, v, dense_token_mask(lists, block, L, L, True), 0.5)
    assert np.all(o[:16] == 0) and np.all(np.isneginf(lse[:16]))
    assert np.all(np.isfinite(lse[16:]))


def test_batched_wrapper_and_row_sampling_agree():
    B, H, L, d = 1, 3, 64, 8
    q, k, v = rand(B, H, L, d), rand(B, H, L, d), rand(B, H, L, d)
    pat = dict(kind=BLOCKSPARSE, block=16, sink_blocks=1, local_blocks=1, stride=2, causal=True)
    o, lse = sparse_forward(q, k, v, pat)
    rows = np.array([0, 5, 17, 40, 63])
    o2, lse2 = sparse_forward(q, k, v, pat, heads=[1, 2], rows=rows)
    np.testing.assert_array_equal(o2[:, 1:, rows], o[:, 1:, rows])
    np.testing.assert_array_equal(lse2[:, 1:, rows], lse[:, 1:, rows])
    assert np.isnan(o2[:, 0]).all()
    # head-dependent stride offset: heads 1 and 2 read different strided blocks
    assert (pattern_token_mask(pat, 1, L) != pattern_token_mask(pat, 2, L)).any()


@pytest.mark.parametrize("kind,extra", [(BLOCKSPARSE, dict(sink_blocks=1, local_blocks=2, stride=3)),
                                        (ATTNSINK, dict(sink_blocks=1, local_blocks=2)),
                                        (SLIDING, dict(sink_blocks=1, window_tokens=23))])
def test_token_mask_with_given_lists_is_the_same(kind, extra):
    """Handing pattern_token_mask the head's lists only skips rebuilding them."""
    pat = dict(kind=kind, block=16, causal=True, **extra)
    L, rows = 16 * 9, np.array([0, 15, 16, 40, 100, 143])
    for h in range(3):
        lists = block_lists(kind, 9, head=h, block=16, **extra)
        np.testing.assert_array_equal(pattern_token_mask(pat, h, L, rows=rows, lists=lists),
                                      pattern_token_mask(pat, h, L, rows=rows))


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------
def _loss(q, k, v, do, mask, scale):
    o, _ = attention_forward(q, k, v, mask, scale)
    return float((o * do).sum())


@pytest.mark.parametrize("kind,stride,h", [(ATTNSINK, 0, 0), (BLOCKSPARSE, 2, 1)])
def test_backward_matches_finite_differences(kind, stride, h):
    L, block, d = 40, 8, 3
    q, k, v, do = rand(L, d), rand(L, d), rand(L, d), rand(L, d)
    lists = block_lists(kind, 5, sink_blocks=1, local_blocks=2, stride=stride, head=h)
    mask = dense_token_mask(lists, block, L, L, True)
    scale = 0.6
    dq, dk, dv, _, _ = attention_backward(q, k, v, do, mask, scale)
    eps = 1e-5
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + eps
            fp = _loss(q, k, v, do, mask, scale)
            x[idx] = old - eps
            fm = _loss(q, k, v, do, mask, scale)
            x[idx] = old
            num[idx] = (fp - fm) / (2 * eps)
        err = np.abs(num - g).max() / max(1.0, np.abs(g).max())
        assert err < 1e-6, (name, err)


def test_backward_full_pattern_matches_autograd():
    L, block, d = 48, 16, 8
    q, k, v, do = rand(L, d), rand(L, d), rand(L, d), rand(L, d)
    mask = dense_token_mask(block_lists(FULL, 3), block, L, L, True)
    dq, dk, dv, o, _ = attention_backward(q, k, v, do, mask, 1 / math.sqrt(d))
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    out = F.scaled_dot_product_attention(tq[None, None], tk[None, None], tv[None, None], is_causal=True)
    out.backward(torch.from_numpy(do)[None, None])
    np.testing.assert_allclose(o, out[0, 0].detach().numpy(), atol=1e-12)
    for mine, ref in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(mine, ref.grad.numpy(), atol=1e-11)


def test_batched_backward_wrapper():
    B, H, L, d = 1, 2, 32, 4
    q, k, v, do = rand(B, H, L, d), rand(B, H, L, d), rand(B, H, L, d), rand(B, H, L, d)
    pat = dict(kind=ATTNSINK, block=16, sink_blocks=1, local_blocks=1, causal=True)
    dq, dk, dv, o, lse = sparse_backward(q, k, v, do, pat)
    o2, lse2 = sparse_forward(q, k, v, pat)
    np.testing.assert_allclose(o, o2, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, atol=1e-14)
    assert np.isfinite(dq).all() and np.isfinite(dk).all() and np.isfinite(dv).all()


def block_rule_mask(kind, h, L, block, s=0, w=0, stride=0):
    """Token mask of a block pattern written as one vectorised rule (NOT the
    oracle's brute-force scan): key block kj is read by query block qi when
    kj <= qi and (kj < s, or qi - w < kj, or -- BlockSparse -- kj < qi with
    (kj + h) % stride == 0); keys after the query are masked."""
    qt = np.arange(L)[:, None]
    kt = np.arange(L)[None, :]
    qi, kj = qt // block, kt // block
    if kind == FULL:
        blk = kj <= qi
    else:
        blk = (kj <= qi) & ((kj < s) | (kj > qi - w))
        if kind == BLOCKSPARSE:
            blk |= (kj < qi) & ((kj + h) % stride == 0)
    return blk & (kt <= qt)


def autograd_head(q, k, v, do, mask, scale):
    """O, LSE, dQ, dK, dV of one head by torch autograd (float64, CPU) on the
    dense masked softmax: an independent route to the textbook gradients."""
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    s = (tq @ tk.T) * scale
    s = s.masked_fill(~torch.from_numpy(mask), float("-inf"))
    lse = torch.logsumexp(s, dim=1)
    o = torch.softmax(s, dim=1) @ tv
    o.backward(torch.from_numpy(do))
    return (o.detach().numpy(), lse.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(),
            tv.grad.numpy())


# (kind, sink, local, stride) per head: every head differs from head 0, and
# heads 2 and 3 share a BlockSparse rule whose phase still differs by head
MIXED = [(FULL, 0, 0, 0), (ATTNSINK, 1, 2, 0), (BLOCKSPARSE, 1, 1, 3), (BLOCKSPARSE, 1, 1, 3),
         (ATTNSINK, 0, 1, 0)]


def _pattern_dict(kind, s, w, stride, block):
    return dict(kind=kind, block=block, sink_blocks=s, local_blocks=w, stride=stride, causal=True)


def test_per_head_pattern_list_runs_each_heads_own_pattern():
    """A list of per-head patterns: head h of the list run equals head h of
    a run with pattern h alone (same H-head tensors, so the BlockSparse
    phase is h in both), and Q = 0 gives each head its own closed-form key
    count (which picking pattern 0, or any other head's, would break)."""
    B, H, block, nb, d = 2, len(MIXED), 8, 7, 4
    L = block * nb
    pats = [_pattern_dict(*m, block) for m in MIXED]
    q, k, v = rand(B, H, L, d), rand(B, H, L, d), rand(B, H, L, d)
    o, lse = sparse_forward(q, k, v, pats)
    for h in range(H):
        o1, l1 = sparse_forward(q, k, v, pats[h], heads=[h])
        np.testing.assert_array_equal(o[:, h], o1[:, h])
        np.testing.assert_array_equal(lse[:, h], l1[:, h])
    _, lse0 = sparse_forward(np.zeros_like(q), k, v, pats)
    for h, (kind, s, w, stride) in enumerate(MIXED):
        for p in range(L):
            bi, r = divmod(p, block)
            n_blocks = (bi + 1 if kind == FULL else attnsink_row_len(bi, s, w) if kind == ATTNSINK
                        else blocksparse_row_len(bi, s, w, stride, h))
            assert lse0[0, h, p] == pytest.approx(math.log(block * (n_blocks - 1) + r + 1), abs=1e-12)


@pytest.mark.parametrize("per_head_list", [False, True])
def test_sparse_backward_per_head_matches_autograd(per_head_list):
    """The batched backward on head-dependent masks (BlockSparse with stride
    3, so heads 0, 1, 2 read different strided blocks; or the per-head mix
    above) against torch autograd on each head's own mask, built by a
    separate rule: pins the per-head dispatch and the (dq, dk, dv, o, lse)
    order -- dO is random, so dk and dv differ and a swap fails."""
    B, block, nb, d, scale = 2, 8, 8, 4, 0.45
    L = block * nb
    if per_head_list:
        heads = MIXED
        pat = [_pattern_dict(*m, block) for m in MIXED]
    else:
        heads = [(BLOCKSPARSE, 1, 1, 3)] * 4
        pat = _pattern_dict(BLOCKSPARSE, 1, 1, 3, block)
    H = len(heads)
    q, k, v, do = (rand(B, H, L, d) for _ in range(4))
    dq, dk, dv, o, lse = sparse_backward(q, k, v, do, pat, scale=scale)
    masks = [block_rule_mask(kind, h, L, block, s, w, stride) for h, (kind, s, w, stride) in enumerate(heads)]
    assert not np.array_equal(masks[1], masks[2]) and not np.array_equal(masks[0], masks[1])
    for b in range(B):
        for h in range(H):
            ro, rl, rq, rk, rv = autograd_head(q[b, h], k[b, h], v[b, h], do[b, h], masks[h], scale)
            for name, mine, ref in (("o", o, ro), ("lse", lse, rl), ("dq", dq, rq), ("dk", dk, rk),
                                    ("dv", dv, rv)):
                np.testing.assert_allclose(mine[b, h], ref, atol=1e-11, err_msg=f"{name} b{b} h{h}")


# --------------------------------------------------------------------------
# decode
# --------------------------------------------------------------------------
def test_decode_positions_examples():
    p = decode_positions(5000, 64, 4096)
    assert list(p[:64]) == list(range(64)) and list(p[64:]) == list(range(905, 5001))
    assert list(decode_positions(10, 64, 4096)) == list(range(11))
    assert list(decode_positions(7, None, None)) == list(range(8))
    for t in (0, 63, 64, 4159, 4160, 4161, 9000):
        assert len(decode_positions(t, 64, 4096)) == min(t + 1, 64 + 4096)


def test_decode_reduces_to_library_attention():
    d = 8
    hist_k, hist_v = rand(300, d), rand(300, d)
    q = rand(d)
    t = 250
    # window covering everything: plain attention over tokens 0..t
    o, lse = decode_one(q, hist_k, hist_v, decode_positions(t, 4, 1000), 0.3)
    ref = sdpa(q[None], hist_k[:t + 1], hist_v[:t + 1], scale=0.3)[0]
    np.testing.assert_allclose(o, ref, atol=1e-12)
    s = torch.from_numpy(hist_k[:t + 1] @ q * 0.3)
    assert lse == pytest.approx(float(torch.logsumexp(s, 0)), abs=1e-12)
    # no sink: plain attention over the last `window` tokens
    o, _ = decode_one(q, hist_k, hist_v, decode_positions(t, 0, 37), 0.3)
    ref = sdpa(q[None], hist_k[t - 36:t + 1], hist_v[t - 36:t + 1], scale=0.3)[0]
    np.testing.assert_allclose(o, ref, atol=1e-12)


def test_decode_zero_query_counts():
    d = 4
    hist_k, hist_v = rand(600, d), rand(600, d)
    for t in (0, 5, 20, 21, 22, 599):
        o, lse = decode_one(np.zeros(d), hist_k, hist_v, decode_positions(t, 6, 16), 1.0)
        assert lse == pytest.approx(math.log(min(t + 1, 22)), abs=1e-12)
        keys = sorted(set(range(min(6, t + 1))) | set(range(max(0, t - 15), t + 1)))
        np.testing.assert_allclose(o, hist_v[keys].mean(axis=0), atol=1e-12)


def test_blocksparse_decode_positions_worked_example():
    """Token 5000 of head 3 with sink 1, local 16, stride 8 (64-token blocks):
    its block 78 reads block 0, blocks 63..78 and the strided blocks
    5, 13, ..., 61 (69 and 77 are already local); keys after 5000 masked."""
    pat = dict(kind=BLOCKSPARSE, block=64, sink_blocks=1, local_blocks=16, stride=8)
    want = list(range(64))
    for j in (5, 13, 21, 29, 37, 45, 53, 61):
        want += list(range(64 * j, 64 * j + 64))
    want += list(range(63 * 64, 5001))
    assert list(blocksparse_decode_positions(5000, pat, 3)) == want
    # sink + window only (stride beyond every block): the ring rule of attnsink
    pat1 = dict(kind=BLOCKSPARSE, block=64, sink_blocks=1, local_blocks=4, stride=10 ** 6)
    for t in (0, 63, 64, 255, 256, 300, 1000):
        got = blocksparse_decode_positions(t, pat1, 1)
        keep = sorted(set(range(min(64, t + 1))) | set(range(64 * max(0, t // 64 - 3), t + 1)))
        assert list(got) == keep


def test_blocksparse_decode_equals_prefill_row():
    """Decoding token t against its positions gives row t of the prefill
    forward (whose mask is built by a separate routine, itself pinned to
    library attention above), for every head phase and rows at and around
    block edges."""
    B, H, L, d = 1, 3, 96, 4
    pat = dict(kind=BLOCKSPARSE, block=8, sink_blocks=1, local_blocks=2, stride=3, causal=True)
    q, k, v = rand(B, H, L, d), rand(B, H, L, d), rand(B, H, L, d)
    rows = [0, 7, 8, 23, 24, 25, 47, 64, 95]
    o, lse = sparse_forward(q, k, v, pat, scale=0.5, rows=rows)
    for h in range(H):
        for t in rows:
            od, ld = decode_one(q[0, h, t], k[0, h], v[0, h],
                                blocksparse_decode_positions(t, pat, h), 0.5)
            np.testing.assert_allclose(od, o[0, h, t], atol=1e-12)
            assert ld == pytest.approx(lse[0, h, t], abs=1e-12)


# --------------------------------------------------------------------------
# KV memory (the pages' figure; consistency only)
# --------------------------------------------------------------------------
def test_kv_cache_memory_consistent_with_pages(golden_dir):
    vals = {}
    with open(os.path.join(golden_dir, "kv_cache_memory_pages.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k_, v_ = line.split(":")
                vals[k_.strip()] = float(v_)
    full = kv_cache_bytes(32, 0, 32, 128, 131072, 0)
    hybrid = kv_cache_bytes(11, 21, 32, 128, 131072, 64 + 4096)
    assert full == 2 * 32 * 32 * 128 * 2 * 131072
    assert abs(full / 1e9 - vals["full_gb"]) / vals["full_gb"] < 0.01
    assert abs(hybrid / 1e9 - vals["hybrid_gb"]) / vals["hybrid_gb"] < 0.06
    assert abs(100 * (1 - hybrid / full) - vals["reduction_percent"]) < 2.0
