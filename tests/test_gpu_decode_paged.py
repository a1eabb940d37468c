"""GPU parity of paged full-layer decode (attn_paged_decode) and of the paged
fill (attn_paged_cache_fill): the oracle attends over token positions; the
page pool and block table only decide where the kernels find them."""

import math

import numpy as np
import pytest
import torch

import long_context_sparse_static_amd as lcs
from _parity import assert_bf16_close, need_gpu
from oracle import decode_one, decode_positions
from synth_inputs import as_f64, randn, seed_for

pytestmark = pytest.mark.gpu


def history(B, H, T, d, workload):
    k = randn((B, H, T, d), seed_for(workload, 0, "cache"), torch.bfloat16).cuda()
    v = randn((B, H, T, d), seed_for(workload, 0, "cache_v"), torch.bfloat16).cuda()
    q = randn((B, H, 1, d), seed_for(workload, 0, "q_dec"), torch.bfloat16).cuda()
    return q, k, v


def shuffled_table(B, max_pages, n_pages, seed):
    """Each sequence's blocks in distinct pages, scattered over the pool."""
    perm = np.random.default_rng(seed).permutation(n_pages)[:B * max_pages]
    return torch.from_numpy(perm.reshape(B, max_pages).astype(np.int32)).cuda()


def new_kv(kh, vh, pos):
    k_new = torch.stack([kh[b, :, t] for b, t in enumerate(pos)])[:, :, None].contiguous()
    v_new = torch.stack([vh[b, :, t] for b, t in enumerate(pos)])[:, :, None].contiguous()
    return k_new, v_new


def oracle(q, kh, vh, pos):
    B, H, _, d = q.shape
    o = np.full((B, H, d), np.nan)
    lse = np.full((B, H), np.nan)
    for b, t in enumerate(pos):
        for h in range(H):
            o[b, h], lse[b, h] = decode_one(as_f64(q[b, h, 0]), as_f64(kh[b, h]), as_f64(vh[b, h]),
                                            decode_positions(int(t)), 1 / math.sqrt(d))
    return o, lse


@pytest.mark.parametrize("d", [128, 64])
def test_paged_fill_then_decode(d):
    """Prefix -> scattered pages via the fill, then decode the next token;
    positions at a page start, a page end and mid-page; every page row the
    fill wrote holds its token."""
    need_gpu()
    B, H = 4, 3
    pos = [0, 63, 64, 700]
    max_pages = 12
    n_pages = 64
    T = max(pos) + 1
    q, kh, vh = history(B, H, T, d, 801 + d)
    table = shuffled_table(B, max_pages, n_pages, 5)
    kp = torch.full((n_pages, H, 64, d), 55.0, dtype=torch.bfloat16, device="cuda")
    vp = torch.full_like(kp, -55.0)
    lengths = torch.tensor(pos, dtype=torch.int64, device="cuda")
    lcs.attn_paged_cache_fill(kh, vh, lengths, kp, vp, table)
    torch.cuda.synchronize()
    tab = table.cpu().numpy()
    for b, n in enumerate(pos):
        for p in range(n):
            assert torch.equal(kp[tab[b, p // 64], :, p % 64], kh[b, :, p])
            assert torch.equal(vp[tab[b, p // 64], :, p % 64], vh[b, :, p])
    k_new, v_new = new_kv(kh, vh, pos)
    o, lse = lcs.attn_paged_decode(q, k_new, v_new, kp, vp, table, lengths, max_pos=64 * max_pages - 1)
    torch.cuda.synchronize()
    wo, wl = oracle(q, kh, vh, pos)
    print("o", assert_bf16_close(as_f64(o[:, :, 0]), wo, "o"))
    print("lse", assert_bf16_close(as_f64(lse), wl, "lse"))
    for b, t in enumerate(pos):          # the new token was appended in its page
        assert torch.equal(kp[tab[b, t // 64], :, t % 64], kh[b, :, t])


def test_paged_equals_contiguous_full_decode():
    """The same caches laid out contiguously and paged give bit-identical
    outputs (same split plan, same arithmetic order)."""
    need_gpu()
    B, H, d = 3, 4, 128
    pos = [5000, 131, 4095]
    max_pos = 5100
    cap = max_pos + 1
    max_pages = (cap + 63) // 64
    q, kc, vc = history(B, H, cap, d, 802)
    k_new = randn((B, H, 1, d), seed_for(802, 0, "k_new"), torch.bfloat16).cuda()
    v_new = randn((B, H, 1, d), seed_for(802, 0, "v_new"), torch.bfloat16).cuda()
    n_pages = B * max_pages + 7
    table = shuffled_table(B, max_pages, n_pages, 9)
    kp = torch.zeros((n_pages, H, 64, d), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    full = torch.full((B,), cap, dtype=torch.int64, device="cuda")
    lcs.attn_paged_cache_fill(kc, vc, full, kp, vp, table)
    p = torch.tensor(pos, dtype=torch.int64, device="cuda")
    o1, l1 = lcs.attn_full_decode(q, k_new, v_new, kc, vc, p, max_pos=max_pos)
    o2, l2 = lcs.attn_paged_decode(q, k_new, v_new, kp, vp, table, p, max_pos=max_pos)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(l1, l2)


def test_paged_consecutive_steps():
    """Decode steps in a row cross page boundaries, appending into pages the
    table names; checked against the oracle along the way."""
    need_gpu()
    B, H, d = 2, 2, 128
    start = [60, 1]
    steps = 140
    max_pages = 4
    n_pages = 16
    T = max(start) + steps
    _, kh, vh = history(B, H, T, d, 803)
    table = shuffled_table(B, max_pages, n_pages, 3)
    kp = torch.zeros((n_pages, H, 64, d), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    lcs.attn_paged_cache_fill(kh, vh, torch.tensor(start, device="cuda"), kp, vp, table)
    for s in range(steps):
        pos = [t + s for t in start]
        q = randn((B, H, 1, d), seed_for(803, s, "q_dec"), torch.bfloat16).cuda()
        k_new, v_new = new_kv(kh, vh, pos)
        o, lse = lcs.attn_paged_decode(q, k_new, v_new, kp, vp, table,
                                       torch.tensor(pos, device="cuda"), max_pos=64 * max_pages - 1)
        if s % 29 == 0 or any(t % 64 in (0, 63) for t in pos):
            torch.cuda.synchronize()
            wo, wl = oracle(q, kh, vh, pos)
            assert_bf16_close(as_f64(o[:, :, 0]), wo, f"step {s}")
            assert_bf16_close(as_f64(lse), wl, f"lse step {s}")


def test_paged_invalid_pages_and_positions():
    """A page id outside the pool in a block the position reads, and a
    position past max_pos, give o = 0 and lse = NaN for that sequence and
    write nothing; the other sequence is unaffected."""
    need_gpu()
    B, H, d = 3, 2, 128
    max_pages, n_pages = 4, 12
    q, kh, vh = history(B, H, 256, d, 804)
    table = shuffled_table(B, max_pages, n_pages, 4)
    table[0, 1] = n_pages          # block 1 of sequence 0: out of range
    table[2, 3] = -1               # block 3 of sequence 2 (not read at t = 100)
    kp = torch.zeros((n_pages, H, 64, d), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    pos = [100, 300, 100]          # sequence 1: beyond max_pos = 255
    lengths = torch.tensor(pos, device="cuda").clamp(max=255)
    lcs.attn_paged_cache_fill(kh, vh, lengths, kp, vp, table)
    k0, v0 = kp.clone(), vp.clone()
    k_new, v_new = new_kv(kh, vh, [100, 0, 100])
    o, lse = lcs.attn_paged_decode(q, k_new, v_new, kp, vp, table, torch.tensor(pos, device="cuda"),
                                   max_pos=255)
    torch.cuda.synchronize()
    for b in (0, 1):
        assert torch.all(o[b] == 0) and torch.all(torch.isnan(lse[b]))
    tab = table.cpu().numpy()
    # sequence 0's page of block 1 (where token 100 would go) is out of range: nothing written
    changed = (kp != k0).any(dim=(1, 2, 3)).nonzero().flatten().tolist()
    assert changed == [int(tab[2, 1])]
    wo, wl = oracle(q[2:], kh[2:], vh[2:], [100])
    assert_bf16_close(as_f64(o[2:, :, 0]), wo, "o")
    assert_bf16_close(as_f64(lse[2:]), wl, "lse")


def test_paged_decode_full_size_sampled():
    """16 sequences x 32 heads (d 128) at t = 131072 against a pool of
    16 x 2049 scattered pages (35 GB per K and V), in the launch
    configuration the benchmark times; the oracle checks 2 sequences x 4
    heads."""
    need_gpu()
    B, H, d, t = 16, 32, 128, 131072
    max_pages = t // 64 + 1
    n_pages = B * max_pages
    table = shuffled_table(B, max_pages, n_pages, 11)
    kp = randn((n_pages, H, 64, d), seed_for(8, 0, "cache"), torch.bfloat16, "cuda")
    vp = randn((n_pages, H, 64, d), seed_for(8, 0, "cache_v"), torch.bfloat16, "cuda")
    q = randn((B, H, 1, d), seed_for(8, 0, "q_dec"), torch.bfloat16, "cuda")
    k_new = randn((B, H, 1, d), seed_for(8, 0, "k_new"), torch.bfloat16, "cuda")
    v_new = randn((B, H, 1, d), seed_for(8, 0, "v_new"), torch.bfloat16, "cuda")
    tab = table.cpu().numpy()
    picks = [(b, h) for b in (2, 13) for h in (0, 7, 19, 31)]
    before = {}
    for b, h in picks:
        pages = torch.from_numpy(tab[b].astype(np.int64)).cuda()
        before[(b, h)] = (as_f64(kp[pages, h].reshape(-1, d)), as_f64(vp[pages, h].reshape(-1, d)))
    pos = torch.full((B,), t, dtype=torch.int64, device="cuda")
    o, lse = lcs.attn_paged_decode(q, k_new, v_new, kp, vp, table, pos, max_pos=t)
    torch.cuda.synchronize()
    for b, h in picks:
        kk, vv = before[(b, h)]
        kk = kk[:t + 1].copy()
        vv = vv[:t + 1].copy()
        kk[t] = as_f64(k_new[b, h, 0])
        vv[t] = as_f64(v_new[b, h, 0])
        wo, wl = decode_one(as_f64(q[b, h, 0]), kk, vv, np.arange(t + 1), 1 / math.sqrt(d))
        assert_bf16_close(as_f64(o[b, h, 0]), wo, f"b{b} h{h}")
        assert abs(float(lse[b, h]) - wl) < 2e-3
