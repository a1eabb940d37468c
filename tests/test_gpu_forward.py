"""GPU parity of the prefill forward (attn_sparse_fwd) against the oracle."""

import math

import numpy as np
import pytest
import torch

import long_context_sparse_static_amd as lcs
from _parity import (assert_bf16_close, assert_f32_close, errors, need_gpu, oracle_forward_heads,
                     oracle_pattern, sample_rows_forward)
from oracle import sparse_forward
from synth_inputs import as_f64, randn, seed_for

pytestmark = pytest.mark.gpu


def _inputs(shape, workload, dtype, device="cuda", big=False):
    gen_dev = "cuda" if big else "cpu"
    return [randn(shape, seed_for(workload, 0, t), dtype, gen_dev).to(device) for t in ("q", "k", "v")]


def _run(q, k, v, pattern):
    B, H, L, d = q.shape
    ix = lcs.build_device_index(pattern, H, L, q.device, with_csc=False)
    o, lse = lcs.attn_sparse_fwd(q, k, v, ix, pattern)
    torch.cuda.synchronize()
    return o, lse


def test_fp32_attnsink_1k_exact_workload():
    """1024 tokens, d 64, fp32, sink 1 block + 4 most recent blocks: full oracle."""
    need_gpu()
    pat = lcs.attnsink_pattern(1, 4)
    q, k, v = _inputs((1, 1, 1024, 64), 1, torch.float32)
    o, lse = _run(q, k, v, pat)
    wo, wl = sparse_forward(as_f64(q), as_f64(k), as_f64(v), oracle_pattern(pat))
    print("fp32 1k O", assert_f32_close(as_f64(o), wo, "O"))
    print("fp32 1k LSE", assert_f32_close(as_f64(lse), wl, "LSE"))


@pytest.mark.parametrize("pat,d,H,nb", [
    (lcs.blocksparse_pattern(1, 3, 4), 128, 4, 13),
    (lcs.full_pattern(), 64, 2, 9),
    # 2 x 4 x 40 = 320 query blocks: the launch with one key group per row
    (lcs.blocksparse_pattern(1, 3, 4), 128, 4, 40),
    (lcs.sliding_pattern(1, 100), 64, 4, 40),
])
def test_fp32_other_patterns(pat, d, H, nb):
    need_gpu()
    q, k, v = _inputs((2, H, 64 * nb, d), 90, torch.float32)
    o, lse = _run(q, k, v, pat)
    wo, wl = sparse_forward(as_f64(q), as_f64(k), as_f64(v), oracle_pattern(pat))
    assert_f32_close(as_f64(o), wo, "O")
    assert_f32_close(as_f64(lse), wl, "LSE")


SMALL_BF16 = [
    # (pattern, d, B, H, n_blocks): odd block counts leave a half-filled last tile
    (lcs.attnsink_pattern(1, 4), 128, 2, 3, 11),
    (lcs.attnsink_pattern(1, 4), 64, 1, 2, 12),
    (lcs.attnsink_pattern(2, 3), 128, 1, 2, 9),
    (lcs.blocksparse_pattern(1, 5, 4), 128, 1, 8, 37),
    (lcs.blocksparse_pattern(1, 3, 8), 64, 1, 9, 21),
    (lcs.full_pattern(), 128, 1, 2, 13),
    (lcs.attnsink_pattern(1, 1), 128, 1, 1, 1),          # a single block
    (lcs.attnsink_pattern(1, 64), 128, 1, 2, 70),
]


@pytest.mark.parametrize("case", range(len(SMALL_BF16)))
def test_bf16_small_full_oracle(case):
    need_gpu()
    pat, d, B, H, nb = SMALL_BF16[case]
    q, k, v = _inputs((B, H, 64 * nb, d), 100 + case, torch.bfloat16)
    o, lse = _run(q, k, v, pat)
    wo, wl = sparse_forward(as_f64(q), as_f64(k), as_f64(v), oracle_pattern(pat))
    print(case, "O", assert_bf16_close(as_f64(o), wo, "O"))
    print(case, "LSE", assert_bf16_close(as_f64(lse), wl, "LSE"))


@pytest.mark.parametrize("pat,d", [(lcs.attnsink_pattern(1, 4), 128), (lcs.blocksparse_pattern(1, 2, 3), 128),
                                   (lcs.full_pattern(), 64), (lcs.attnsink_pattern(1, 4), 64)])
def test_zero_query_lse_counts(pat, d):
    """Q = 0: every allowed score is 0, so LSE = ln(#allowed keys) exactly and O
    is the mean of the allowed V rows -- pins the mask on the GPU."""
    need_gpu()
    B, H, nb = 1, 8, 10
    L = 64 * nb
    q = torch.zeros((B, H, L, d), dtype=torch.bfloat16, device="cuda")
    _, k, v = _inputs((B, H, L, d), 7, torch.bfloat16)
    o, lse = _run(q, k, v, pat)
    ix = lcs.attn_index_build(pat, H if pat.head_dependent else 1, L, with_csc=False)
    lse_h = lse.cpu().numpy()
    for h in range(H):
        hh = h if pat.head_dependent else 0
        for i in range(nb):
            n_blocks = len(ix.row(hh, i))
            counts = 64 * (n_blocks - 1) + np.arange(1, 65)
            np.testing.assert_allclose(lse_h[0, h, 64 * i:64 * (i + 1)], np.log(counts), rtol=0, atol=2e-6)
    wo, _ = sparse_forward(np.zeros((B, H, L, d)), as_f64(k), as_f64(v), oracle_pattern(pat))
    assert_bf16_close(as_f64(o), wo, "O")


def test_empty_rows_give_zero_and_minus_inf():
    need_gpu()
    L, d = 256, 128
    q, k, v = _inputs((1, 2, L, d), 8, torch.bfloat16)
    # query block 1 lists nothing; block 3 lists only block 0
    row_ptr = np.array([0, 1, 1, 3, 4], dtype=np.int32)
    col_idx = np.array([0, 0, 2, 0], dtype=np.int32)
    host = lcs.HostIndex(1, 4, 4, row_ptr, col_idx, None, None)
    lcs.attn_index_validate(host)
    ix = lcs.DeviceIndex(host, q.device)
    o, lse = lcs.attn_sparse_fwd(q, k, v, ix, lcs.attnsink_pattern(1, 1))
    torch.cuda.synchronize()
    assert torch.all(o[:, :, 64:128] == 0)
    assert torch.all(torch.isneginf(lse[:, :, 64:128]))
    assert torch.all(torch.isfinite(lse[:, :, :64])) and torch.all(torch.isfinite(lse[:, :, 128:]))


def test_out_of_range_index_entries_are_skipped():
    """A malformed device index must not cause out-of-bounds reads: bad ids are
    skipped and row pointers clamped."""
    need_gpu()
    L, d = 256, 128
    q, k, v = _inputs((1, 1, L, d), 9, torch.bfloat16)
    good = lcs.attn_index_build(lcs.attnsink_pattern(1, 1), 1, L, with_csc=False)
    o_ref, l_ref = lcs.attn_sparse_fwd(q, k, v, lcs.DeviceIndex(good, q.device), lcs.attnsink_pattern(1, 1))
    # same lists with junk ids (-5, 4, 1000) interleaved, and a final pointer past nnz
    rows = [good.row(0, i) for i in range(4)]
    junk = [[-5] + r + [1000] for r in rows]
    row_ptr = np.cumsum([0] + [len(r) for r in junk]).astype(np.int32)
    row_ptr[-1] += 50                                   # clamped to nnz by the kernel
    col_idx = np.array([x for r in junk for x in r], dtype=np.int32)
    ix = lcs.attn_index_t(1, 4, 4, len(col_idx), None, None, None, None)
    rp = torch.from_numpy(row_ptr).cuda()
    ci = torch.from_numpy(col_idx).cuda()
    ix.row_ptr, ix.col_idx = rp.data_ptr(), ci.data_ptr()

    class Raw:
        def c_struct(self):
            return ix
    o, lse = lcs.attn_sparse_fwd(q, k, v, Raw(), lcs.attnsink_pattern(1, 1))
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)


def _junk_index(good, nb, with_csc):
    """The lists of ``good`` (one index head) with out-of-range ids (-5, and
    1000) around every row and column, and final pointers past nnz."""
    class Raw:
        def __init__(self, device):
            rows = [[-5] + good.row(0, i) + [1000] for i in range(nb)]
            rp = np.cumsum([0] + [len(r) for r in rows]).astype(np.int32)
            rp[-1] += 50
            ci = np.array([x for r in rows for x in r], dtype=np.int32)
            self.t = [torch.from_numpy(rp).to(device), torch.from_numpy(ci).to(device)]
            self.ix = lcs.attn_index_t(1, nb, nb, len(ci), self.t[0].data_ptr(), self.t[1].data_ptr(), None, None)
            if with_csc:
                cols = [[-5] + good.col(0, j) + [1000] for j in range(nb)]
                cp = np.cumsum([0] + [len(c) for c in cols]).astype(np.int32)
                cp[-1] += 50
                ri = np.array([x for c in cols for x in c], dtype=np.int32)
                assert len(ri) == len(ci)
                self.t += [torch.from_numpy(cp).to(device), torch.from_numpy(ri).to(device)]
                self.ix.col_ptr, self.ix.row_idx = self.t[2].data_ptr(), self.t[3].data_ptr()

        def c_struct(self):
            return self.ix
    return Raw


def test_out_of_range_entries_skipped_fp32_and_backward():
    """The fp32 forward and the backward (CSR and CSC walks) skip the same
    junk entries and give the results of the clean index, bit for bit."""
    need_gpu()
    pat = lcs.attnsink_pattern(1, 2)
    L, nb = 64 * 5, 5
    good = lcs.attn_index_build(pat, 1, L, with_csc=True)
    gix = lcs.DeviceIndex(good, torch.device("cuda"))
    junk = _junk_index(good, nb, True)(torch.device("cuda"))
    q, k, v = _inputs((1, 2, L, 64), 91, torch.float32)
    o_ref, l_ref = lcs.attn_sparse_fwd(q, k, v, gix, pat)
    o, lse = lcs.attn_sparse_fwd(q, k, v, junk, pat)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
    q, k, v, do = (x.to(torch.bfloat16) for x in (q, k, v, torch.randn_like(q)))
    o, lse = lcs.attn_sparse_fwd(q, k, v, gix, pat)
    ref = lcs.attn_sparse_bwd(q, k, v, o, lse, do, gix, pat)
    got = lcs.attn_sparse_bwd(q, k, v, o, lse, do, junk, pat)
    torch.cuda.synchronize()
    for a_, b_ in zip(got, ref):
        assert torch.equal(a_, b_)


def test_deterministic_repeat():
    need_gpu()
    pat = lcs.blocksparse_pattern(1, 4, 8)
    q, k, v = _inputs((1, 4, 64 * 20, 128), 11, torch.bfloat16)
    o1, l1 = _run(q, k, v, pat)
    o2, l2 = _run(q, k, v, pat)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ----------------------------------------------------------------------------
# Full-size workloads, in the launch configuration the benchmark times.  The
# oracle runs one exact sub-problem per query block (a row depends only on the
# keys its block lists), so whole heads are checked row by row: every row of
# all 32 heads at 8K AttnSink and 32K BlockSparse, every row of two heads at
# 128K AttnSink and BlockSparse, and sampled rows of 128K full attention (a
# full head is 4.4 TFLOP of float64 work).
# ----------------------------------------------------------------------------
FULL_SIZE = {
    # name: (pattern, L, workload seed, heads checked on every row)
    "attnsink_8k": (lcs.attnsink_pattern(1, 64), 8192, 2, list(range(32))),
    "blocksparse_32k": (lcs.blocksparse_pattern(1, 16, 8), 32768, 3, list(range(32))),
    "attnsink_128k": (lcs.attnsink_pattern(1, 64), 131072, 5, [0, 29]),
    "blocksparse_128k": (lcs.blocksparse_pattern(1, 16, 8), 131072, 33, [5, 18]),
}


@pytest.mark.parametrize("name", list(FULL_SIZE))
def test_bf16_full_size_every_row(name):
    need_gpu()
    pat, L, wl, heads = FULL_SIZE[name]
    H, d = 32, 128
    q, k, v = _inputs((1, H, L, d), wl, torch.bfloat16, big=True)
    o, lse = _run(q, k, v, pat)
    want = oracle_forward_heads(q, k, v, pat, heads)
    err_max = err_sum = 0.0
    for h in heads:
        wo, wlse = want[h]
        mx, mean = assert_bf16_close(as_f64(o[0, h]), wo, f"{name} O head {h}")
        assert_bf16_close(as_f64(lse[0, h]), wlse, f"{name} LSE head {h}")
        err_max, err_sum = max(err_max, mx), err_sum + mean
    print(name, f"{len(heads)} heads x {L} rows: O max {err_max:.3e} mean {err_sum / len(heads):.3e}")


def test_bf16_full_causal_128k_sampled():
    """128K full causal attention (the hybrid's middle layers): sampled rows
    of three heads on their exact sub-problems."""
    need_gpu()
    pat, L = lcs.full_pattern(), 131072
    q, k, v = _inputs((1, 32, L, 128), 5, torch.bfloat16, big=True)
    o, lse = _run(q, k, v, pat)
    rng = np.random.default_rng(L)
    for h in [0, 7, 31]:
        rows = np.unique(np.concatenate([[0, 63, 64, L - 1, L - 64], rng.integers(0, L, 40)]))
        wo, wlse = sample_rows_forward(q, k, v, pat, h, 0, rows)
        idx = torch.as_tensor(rows, device=q.device)
        mx, mean = assert_bf16_close(as_f64(o[0, h, idx]), wo, f"full O head {h}")
        assert_bf16_close(as_f64(lse[0, h, idx]), wlse, f"full LSE head {h}")
        print("full_128k", h, mx, mean)


def test_bf16_maximum_length_sampled():
    """The longest sequence the bf16 forward takes at d = 128: 4,161,536
    tokens (65,024 key blocks, whose union bitmap plus the output staging
    fill a workgroup's LDS; one block more is rejected).  AttnSink, two
    heads; sampled rows on their exact sub-problems, among them the first and
    last blocks and blocks on either side of bitmap word boundaries."""
    need_gpu()
    pat, L, H, d = lcs.attnsink_pattern(1, 64), 4161536, 2, 128
    q, k, v = _inputs((1, H, L, d), 77, torch.bfloat16, big=True)
    o, lse = _run(q, k, v, pat)
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    rng = np.random.default_rng(5)
    edge_blocks = [0, 1, 63, 64, 1023, 1024, 32767, 32768, 65022, 65023]
    for h in range(H):
        rows = np.unique(np.concatenate([[b * 64 + r for b in edge_blocks for r in (0, 31, 63)],
                                         rng.integers(0, L, 24)]))
        wo, wlse = sample_rows_forward(q, k, v, pat, h, 0, rows)
        idx = torch.as_tensor(rows, device=q.device)
        mx, mean = assert_bf16_close(as_f64(o[0, h, idx]), wo, f"max-length O head {h}")
        assert_bf16_close(as_f64(lse[0, h, idx]), wlse, f"max-length LSE head {h}")
        print("max length", h, mx, mean)


# ----------------------------------------------------------------------------
# Per-head pattern mix (retrieval heads with full attention beside sink +
# window streaming heads) through one index and one launch.
# ----------------------------------------------------------------------------
MIXED_HEADS = [lcs.full_pattern(), lcs.attnsink_pattern(1, 4), lcs.blocksparse_pattern(1, 3, 4),
               lcs.attnsink_pattern(2, 3), lcs.full_pattern(), lcs.blocksparse_pattern(2, 5, 3)]


def test_bf16_mixed_heads_full_oracle():
    need_gpu()
    H, L, d = len(MIXED_HEADS), 64 * 19, 128
    q, k, v = _inputs((1, H, L, d), 130, torch.bfloat16)
    ix = lcs.build_device_index_mixed(MIXED_HEADS, L, q.device, with_csc=False)
    o, lse = lcs.attn_sparse_fwd(q, k, v, ix, MIXED_HEADS[0])
    torch.cuda.synchronize()
    pats = [oracle_pattern(p) for p in MIXED_HEADS]
    wo, wl = sparse_forward(as_f64(q), as_f64(k), as_f64(v), pats)
    print("mixed O", assert_bf16_close(as_f64(o), wo, "O"))
    print("mixed LSE", assert_bf16_close(as_f64(lse), wl, "LSE"))


def test_bf16_mixed_heads_32k_sampled():
    """32 heads at 32K tokens, every fourth head full attention and the rest
    AttnSink (sink 64, window 4096), as one launch; sampled rows per head."""
    need_gpu()
    H, L, d = 32, 32768, 128
    pats = [lcs.full_pattern() if h % 4 == 0 else lcs.attnsink_pattern(1, 64) for h in range(H)]
    q, k, v = _inputs((1, H, L, d), 131, torch.bfloat16, big=True)
    ix = lcs.build_device_index_mixed(pats, L, q.device, with_csc=False)
    o, lse = lcs.attn_sparse_fwd(q, k, v, ix, pats[1])
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    for h in (0, 1, 4, 30):
        rows = np.unique(np.concatenate([[0, 63, 64, L - 1], rng.integers(0, L, 24)]))
        wo, wlse = sample_rows_forward(q, k, v, pats[h], h, 0, rows)
        idx = torch.as_tensor(rows, device=q.device)
        assert_bf16_close(as_f64(o[0, h, idx]), wo, f"mixed O head {h}")
        assert_bf16_close(as_f64(lse[0, h, idx]), wlse, f"mixed LSE head {h}")


@pytest.mark.parametrize("kind", ["rising", "spikes", "thresholds"])
def test_running_max_paths(kind):
    """Inputs that drive the forward's running-max paths hard: scores that
    rise block after block along the key axis (the max moves again and
    again), and a few keys whose scores are hundreds above the rest (P would
    overflow against a stale max).  Both must match the oracle."""
    need_gpu()
    pat = lcs.full_pattern()
    B, H, L, d = 1, 2, 64 * 12, 128
    g = torch.Generator().manual_seed(4242)
    q = torch.randn((B, H, L, d), generator=g)
    k = torch.randn((B, H, L, d), generator=g) * 0.3
    v = torch.randn((B, H, L, d), generator=g)
    if kind == "rising":
        # key j leans along a shared direction with weight growing in j
        u = torch.randn(d, generator=g)
        q += 2.0 * u
        k += (torch.arange(L, dtype=torch.float32) / 64.0 * 0.35)[:, None] * u
    elif kind == "thresholds":
        # one query meets keys whose scores (base 2, scale folded in) sit about
        # 50, 70 and 330 above the rest, in that walk order: 50 stays under
        # the forward's 2^64 rescale threshold (P up to 2^50 against a stale
        # max), 70 crosses it, and 330 would overflow fp32 without the rescale
        qi = L - 5
        for blk, alpha in ((2, 3.07), (5, 4.3), (8, 20.2)):
            k[:, :, blk * 64 + 11] = q[:, :, qi] * alpha
    else:
        k[:, :, 5 * 64 + 7] = q[:, :, -1] * 10.0     # scores ~160 (base 2) above the rest
        k[:, :, 9 * 64 + 40] = -q[:, :, -1] * 10.0
        k[:, :, 11 * 64 + 3] = q[:, :, 700] * 12.0
    q, k, v = (x.to(torch.bfloat16).cuda() for x in (q, k, v))
    o, lse = _run(q, k, v, pat)
    wo, wl = sparse_forward(as_f64(q), as_f64(k), as_f64(v), oracle_pattern(pat))
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    print(kind, "O", assert_bf16_close(as_f64(o), wo, "O"))
    print(kind, "LSE", assert_bf16_close(as_f64(lse), wl, "LSE"))
