"""GPU parity of decode (attn_sparse_decode, attn_full_decode) and of the ring
fill (attn_ring_fill) against the oracle, which works on token positions and
never on cache slots."""

import math

import numpy as np
import pytest
import torch

import long_context_sparse_static_amd as lcs
from _parity import assert_bf16_close, errors, need_gpu
from oracle import decode_one, decode_positions
from synth_inputs import as_f64, randn, seed_for

pytestmark = pytest.mark.gpu


def history(B, H, T, d, workload, dev="cpu"):
    """Token K/V history [B,H,T,d] (positions 0..T-1) and queries [B,H,1,d]."""
    k = randn((B, H, T, d), seed_for(workload, 0, "cache"), torch.bfloat16, dev).cuda()
    v = randn((B, H, T, d), seed_for(workload, 0, "cache_v"), torch.bfloat16, dev).cuda()
    q = randn((B, H, 1, d), seed_for(workload, 0, "q_dec"), torch.bfloat16, dev).cuda()
    return q, k, v


def oracle_decode(q, k_hist, v_hist, pos, sink, window, bs=None, heads=None):
    """o [B,H,d], lse [B,H] from the token history, for sequences ``bs``."""
    B, H, _, d = q.shape
    bs = range(B) if bs is None else bs
    heads = range(H) if heads is None else heads
    o = np.full((B, H, d), np.nan)
    lse = np.full((B, H), np.nan)
    scale = 1 / math.sqrt(d)
    for b in bs:
        t = int(pos[b])
        keep = decode_positions(t, sink, window)
        for h in heads:
            kk = as_f64(k_hist[b, h, keep])
            vv = as_f64(v_hist[b, h, keep])
            o[b, h], lse[b, h] = decode_one(as_f64(q[b, h, 0]), kk, vv, np.arange(len(keep)), scale)
    return o, lse


def test_sparse_decode_after_ring_fill():
    """Prefix of each sequence -> ring via attn_ring_fill, then decode the next
    token (append + attend); positions cover an unfilled ring, exactly full,
    and wrapped several times."""
    need_gpu()
    B, H, d, sink, window = 5, 3, 128, 64, 256
    pos = [5, 319, 320, 1000, 4097]
    T = max(pos) + 1
    q, kh, vh = history(B, H, T, d, 501)
    ring_k = torch.zeros((B, H, sink + window, d), dtype=torch.bfloat16, device="cuda")
    ring_v = torch.zeros_like(ring_k)
    lengths = torch.tensor(pos, dtype=torch.int64, device="cuda")      # tokens 0..t-1 exist
    lcs.attn_ring_fill(kh, vh, lengths, ring_k, ring_v, sink, window)
    k_new = torch.stack([kh[b, :, pos[b]] for b in range(B)])[:, :, None].contiguous()
    v_new = torch.stack([vh[b, :, pos[b]] for b in range(B)])[:, :, None].contiguous()
    o, lse = lcs.attn_sparse_decode(q, k_new, v_new, ring_k, ring_v, lengths, sink, window)
    torch.cuda.synchronize()
    wo, wl = oracle_decode(q, kh, vh, pos, sink, window)
    print("o", assert_bf16_close(as_f64(o[:, :, 0]), wo, "o"))
    print("lse", assert_bf16_close(as_f64(lse), wl, "lse"))
    # the new token was appended in its ring slot
    for b, t in enumerate(pos):
        slot = t if t < sink else sink + (t - sink) % window
        assert torch.equal(ring_k[b, :, slot], kh[b, :, t])
        assert torch.equal(ring_v[b, :, slot], vh[b, :, t])


def test_sparse_decode_host_placed_ring_and_slot_permutation():
    """Ring filled on the host by the documented slot rule (independently of
    attn_ring_fill).  A ring whose slots are permuted consistently with a
    relabelled position gives the same answer."""
    need_gpu()
    B, H, d, sink, window = 2, 4, 64, 4, 60
    pos = [200, 61]
    T = max(pos) + 1
    q, kh, vh = history(B, H, T, d, 502)
    ring_k = torch.zeros((B, H, sink + window, d), dtype=torch.bfloat16, device="cuda")
    ring_v = torch.zeros_like(ring_k)
    for b, t in enumerate(pos):
        for p in decode_positions(t, sink, window):
            if p == t:
                continue
            s = p if p < sink else sink + (p - sink) % window
            ring_k[b, :, s] = kh[b, :, p]
            ring_v[b, :, s] = vh[b, :, p]
    k_new = torch.stack([kh[b, :, pos[b]] for b in range(B)])[:, :, None].contiguous()
    v_new = torch.stack([vh[b, :, pos[b]] for b in range(B)])[:, :, None].contiguous()
    p_dev = torch.tensor(pos, dtype=torch.int64, device="cuda")
    o, lse = lcs.attn_sparse_decode(q, k_new, v_new, ring_k.clone(), ring_v.clone(), p_dev, sink, window)
    torch.cuda.synchronize()
    wo, wl = oracle_decode(q, kh, vh, pos, sink, window)
    assert_bf16_close(as_f64(o[:, :, 0]), wo, "o")
    assert_bf16_close(as_f64(lse), wl, "lse")
    # Rotate the window part of sequence 0's ring by 7 slots and move the new
    # token's position by 7: the attended set is the same multiset of rows.
    rk, rv = ring_k.clone(), ring_v.clone()
    rk[0, :, sink:] = torch.roll(ring_k[0, :, sink:], 7, dims=1)
    rv[0, :, sink:] = torch.roll(ring_v[0, :, sink:], 7, dims=1)
    p2 = torch.tensor([pos[0] + 7, pos[1]], dtype=torch.int64, device="cuda")
    o2, l2 = lcs.attn_sparse_decode(q, k_new, v_new, rk, rv, p2, sink, window)
    torch.cuda.synchronize()
    mx, _ = errors(as_f64(o2[0]), as_f64(o[0]))
    assert mx < 1e-2
    assert abs(float(l2[0, 0]) - float(lse[0, 0])) < 1e-4


def test_sparse_decode_consecutive_steps_wrap():
    """Several decode steps in a row append into the ring and wrap it."""
    need_gpu()
    B, H, d, sink, window = 2, 2, 128, 64, 128
    start = [150, 3]
    steps = 150
    T = max(start) + steps + 1
    q_all = randn((steps, B, H, 1, d), 777, torch.bfloat16).cuda()
    _, kh, vh = history(B, H, T, d, 503)
    ring_k = torch.zeros((B, H, sink + window, d), dtype=torch.bfloat16, device="cuda")
    ring_v = torch.zeros_like(ring_k)
    lcs.attn_ring_fill(kh, vh, torch.tensor(start, device="cuda"), ring_k, ring_v, sink, window)
    worst = 0.0
    for s in range(steps):
        pos = [t + s for t in start]
        p = torch.tensor(pos, dtype=torch.int64, device="cuda")
        k_new = torch.stack([kh[b, :, pos[b]] for b in range(B)])[:, :, None].contiguous()
        v_new = torch.stack([vh[b, :, pos[b]] for b in range(B)])[:, :, None].contiguous()
        o, lse = lcs.attn_sparse_decode(q_all[s], k_new, v_new, ring_k, ring_v, p, sink, window)
        if s % 37 == 0 or s == steps - 1:
            torch.cuda.synchronize()
            wo, wl = oracle_decode(q_all[s], kh, vh, pos, sink, window)
            worst = max(worst, assert_bf16_close(as_f64(o[:, :, 0]), wo, f"step {s}")[0])
            assert_bf16_close(as_f64(lse), wl, f"lse step {s}")
    print("worst", worst)


def test_full_decode_small():
    need_gpu()
    B, H, d, cap = 3, 2, 128, 3000
    pos = [0, 2047, 2999]
    q, kh, vh = history(B, H, cap, d, 504)
    kc, vc = kh.clone(), vh.clone()
    # slots at and beyond each position hold junk that must be overwritten / ignored
    for b, t in enumerate(pos):
        kc[b, :, t:] = 100.0
        vc[b, :, t:] = -100.0
    k_new = torch.stack([kh[b, :, pos[b]] for b in range(B)])[:, :, None].contiguous()
    v_new = torch.stack([vh[b, :, pos[b]] for b in range(B)])[:, :, None].contiguous()
    p = torch.tensor(pos, dtype=torch.int64, device="cuda")
    o, lse = lcs.attn_full_decode(q, k_new, v_new, kc, vc, p, max_pos=cap - 1)
    torch.cuda.synchronize()
    wo, wl = oracle_decode(q, kh, vh, pos, None, None)
    assert_bf16_close(as_f64(o[:, :, 0]), wo, "o")
    assert_bf16_close(as_f64(lse), wl, "lse")
    for b, t in enumerate(pos):
        assert torch.equal(kc[b, :, t], kh[b, :, t])


def test_decode_invalid_positions():
    need_gpu()
    B, H, d = 2, 2, 128
    q, kh, vh = history(B, H, 100, d, 505)
    k_new, v_new = kh[:, :, :1].contiguous(), vh[:, :, :1].contiguous()
    kc, vc = kh.clone(), vh.clone()
    p = torch.tensor([-1, 100], dtype=torch.int64, device="cuda")   # both out of range
    o, lse = lcs.attn_full_decode(q, k_new, v_new, kc, vc, p, max_pos=50)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isnan(lse))
    assert torch.equal(kc, kh)                                          # nothing appended
    ring = torch.zeros((B, H, 8, d), dtype=torch.bfloat16, device="cuda")
    o, lse = lcs.attn_sparse_decode(q, k_new, v_new, ring, ring.clone(),
                                    torch.tensor([-3, 5], device="cuda"), 4, 4)
    torch.cuda.synchronize()
    assert torch.all(o[0] == 0) and torch.all(torch.isnan(lse[0])) and torch.all(torch.isfinite(lse[1]))


def test_decode_full_size_all_heads():
    """The 128K-context decode of 16 sequences (32 heads, d 128): a sparse
    layer's 64+4096-slot ring and a full layer's 131073-slot cache, in the
    launch configuration the benchmark times; the oracle checks all 32 heads
    of 2 sequences per layer kind, on token positions (never ring slots)."""
    need_gpu()
    B, H, d, sink, window = 16, 32, 128, 64, 4096
    t = 131072
    pos = torch.full((B,), t, dtype=torch.int64, device="cuda")
    q = randn((B, H, 1, d), seed_for(5, 0, "q_dec"), torch.bfloat16, "cuda")
    k_new = randn((B, H, 1, d), seed_for(5, 0, "k_new"), torch.bfloat16, "cuda")
    v_new = randn((B, H, 1, d), seed_for(5, 0, "v_new"), torch.bfloat16, "cuda")
    ring_k = randn((B, H, sink + window, d), seed_for(5, 0, "cache"), torch.bfloat16, "cuda")
    ring_v = randn((B, H, sink + window, d), seed_for(5, 0, "cache_v"), torch.bfloat16, "cuda")
    rk0, rv0 = ring_k.clone(), ring_v.clone()
    o, lse = lcs.attn_sparse_decode(q, k_new, v_new, ring_k, ring_v, pos, sink, window)
    torch.cuda.synchronize()
    slot_new = sink + (t - sink) % window
    keep = decode_positions(t, sink, window)
    # token position p lives in slot p (sink) or sink + (p - sink) % window
    slots = [p if p < sink else sink + (p - sink) % window for p in keep]
    j_new = keep.tolist().index(t)
    worst = [0.0, 0.0]
    for b in (0, 9):
        for h in range(H):
            kk = as_f64(rk0[b, h])[slots]
            vv = as_f64(rv0[b, h])[slots]
            kk[j_new] = as_f64(k_new[b, h, 0])
            vv[j_new] = as_f64(v_new[b, h, 0])
            wo, wl = decode_one(as_f64(q[b, h, 0]), kk, vv, np.arange(len(keep)), 1 / math.sqrt(d))
            mx, mean = assert_bf16_close(as_f64(o[b, h, 0]), wo, f"sparse b{b} h{h}")
            worst = [max(worst[0], mx), max(worst[1], mean)]
            assert abs(float(lse[b, h]) - wl) < 2e-3
    print("sparse decode 2 seqs x 32 heads: O max", worst[0], "largest per-head mean", worst[1])
    assert torch.equal(ring_k[:, :, slot_new], k_new[:, :, 0])
    del ring_k, ring_v, rk0, rv0

    cap = t + 1
    kc = randn((B, H, cap, d), seed_for(5, 1, "cache"), torch.bfloat16, "cuda")
    vc = randn((B, H, cap, d), seed_for(5, 1, "cache_v"), torch.bfloat16, "cuda")
    seqs = (3, 15)
    before = {b: (kc[b].clone(), vc[b].clone()) for b in seqs}    # the oracle's inputs (device copies)
    o, lse = lcs.attn_full_decode(q, k_new, v_new, kc, vc, pos, max_pos=t)
    torch.cuda.synchronize()
    worst = [0.0, 0.0]
    for b in seqs:
        for h in range(H):
            kk, vv = (as_f64(x[h]) for x in before[b])
            kk[t] = as_f64(k_new[b, h, 0])
            vv[t] = as_f64(v_new[b, h, 0])
            wo, wl = decode_one(as_f64(q[b, h, 0]), kk, vv, np.arange(cap), 1 / math.sqrt(d))
            mx, mean = assert_bf16_close(as_f64(o[b, h, 0]), wo, f"full b{b} h{h}")
            worst = [max(worst[0], mx), max(worst[1], mean)]
            assert abs(float(lse[b, h]) - wl) < 2e-3
        assert torch.equal(kc[b, :, t], k_new[b, :, 0])
    print("full decode 2 seqs x 32 heads: O max", worst[0], "largest per-head mean", worst[1])
