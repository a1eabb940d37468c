"""GPU parity of BlockSparse decode (attn_blocksparse_decode) and of its
compacted-cache fill (attn_blocksparse_cache_fill) against the oracle, which
works on token positions: the token at position t reads its row of the
prefill mask (blocksparse_decode_positions)."""

import math

import numpy as np
import pytest
import torch

import long_context_sparse_static_amd as lcs
from _parity import assert_bf16_close, need_gpu
from oracle import BLOCKSPARSE, blocksparse_decode_positions, decode_one
from synth_inputs import as_f64, randn, seed_for

pytestmark = pytest.mark.gpu


def opattern(p):
    return dict(kind=BLOCKSPARSE, block=64, sink_blocks=p.sink_blocks,
                local_blocks=p.local_blocks, stride=p.stride)


def slot_positions(n, p, h, cap):
    """Token position each slot of head h's compacted cache holds once
    tokens 0..n-1 are in (-1: none), from the documented layout: sink blocks,
    then a ring of the local_blocks most recent blocks (block j at ring block
    j mod local_blocks), then the strided blocks j >= sink_blocks,
    (j + h) % stride == 0, that left the window, ascending."""
    s, w, st = p.sink_blocks, p.local_blocks, p.stride
    out = np.full(64 * (s + w + cap), -1, dtype=np.int64)
    if n <= 0:
        return out
    last = (n - 1) // 64
    for j in range(last + 1):
        if j < s:
            base = 64 * j
        elif j > last - w:
            base = 64 * (s + j % w)
        elif (j + h) % st == 0:
            m = sum(1 for x in range(s, j) if (x + h) % st == 0)
            if m >= cap:
                continue
            base = 64 * (s + w + m)
        else:
            continue
        for r in range(64):
            if 64 * j + r < n:
                out[base + r] = 64 * j + r
    return out


def history(B, H, T, d, workload):
    k = randn((B, H, T, d), seed_for(workload, 0, "cache"), torch.bfloat16).cuda()
    v = randn((B, H, T, d), seed_for(workload, 0, "cache_v"), torch.bfloat16).cuda()
    return k, v


def queries(B, H, d, workload, step=0):
    return randn((B, H, 1, d), seed_for(workload, step, "q_dec"), torch.bfloat16).cuda()


def new_kv(kh, vh, pos):
    k_new = torch.stack([kh[b, :, t] for b, t in enumerate(pos)])[:, :, None].contiguous()
    v_new = torch.stack([vh[b, :, t] for b, t in enumerate(pos)])[:, :, None].contiguous()
    return k_new, v_new


def oracle(q, kh, vh, pos, p, heads=None):
    B, H, _, d = q.shape
    o = np.full((B, H, d), np.nan)
    lse = np.full((B, H), np.nan)
    for b, t in enumerate(pos):
        for h in (range(H) if heads is None else heads):
            keep = blocksparse_decode_positions(int(t), opattern(p), h)
            o[b, h], lse[b, h] = decode_one(as_f64(q[b, h, 0]), as_f64(kh[b, h]),
                                            as_f64(vh[b, h]), keep, 1 / math.sqrt(d))
    return o, lse


def empty_cache(B, H, S, d):
    kc = torch.full((B, H, S, d), 77.0, dtype=torch.bfloat16, device="cuda")
    return kc, torch.full_like(kc, -77.0)


def check_layout(kc, vc, kh, vh, lengths, p, cap, sentinel=True):
    """Every slot that holds a token holds exactly that token's K and V;
    slots that hold none are untouched (still the sentinel)."""
    for b, n in enumerate(lengths):
        for h in range(kc.shape[1]):
            sp = torch.from_numpy(slot_positions(n, p, h, cap)).cuda()
            held = sp >= 0
            assert torch.equal(kc[b, h][held], kh[b, h][sp[held]]), (b, h, n)
            assert torch.equal(vc[b, h][held], vh[b, h][sp[held]]), (b, h, n)
            if sentinel:
                assert torch.all(kc[b, h][~held] == 77.0) and torch.all(vc[b, h][~held] == -77.0)


@pytest.mark.parametrize("d", [128, 64])
def test_blocksparse_fill_then_decode(d):
    """Prefix -> compacted cache via the fill, then decode the next token.
    Lengths cover an empty cache, a partial first block, an exact block
    edge (a strided block moves out of the ring), and ring wraps."""
    need_gpu()
    p = lcs.blocksparse_pattern(1, 3, 4)
    B, H = 6, 4
    pos = [0, 5, 64, 256, 1000, 1409]
    T = max(pos) + 1
    cap = lcs.blocksparse_strided_capacity(p, T)
    S = lcs.blocksparse_cache_slots(p, cap)
    kh, vh = history(B, H, T, d, 601 + d)
    q = queries(B, H, d, 601 + d)
    kc, vc = empty_cache(B, H, S, d)
    lengths = torch.tensor(pos, dtype=torch.int64, device="cuda")
    lcs.attn_blocksparse_cache_fill(kh, vh, lengths, kc, vc, p, cap)
    torch.cuda.synchronize()
    check_layout(kc, vc, kh, vh, pos, p, cap)
    k_new, v_new = new_kv(kh, vh, pos)
    o, lse = lcs.attn_blocksparse_decode(q, k_new, v_new, kc, vc, lengths, p, cap)
    torch.cuda.synchronize()
    wo, wl = oracle(q, kh, vh, pos, p)
    print("o", assert_bf16_close(as_f64(o[:, :, 0]), wo, "o"))
    print("lse", assert_bf16_close(as_f64(lse), wl, "lse"))
    # after the step the cache is what a fill of t + 1 tokens gives
    check_layout(kc, vc, kh, vh, [t + 1 for t in pos], p, cap, sentinel=False)


def test_blocksparse_decode_host_placed_cache():
    """Cache placed on the host by the documented layout, independently of
    the fill kernel; sink 2, stride 3 (every head phase), odd lengths."""
    need_gpu()
    p = lcs.blocksparse_pattern(2, 2, 3)
    B, H, d = 3, 3, 128
    pos = [130, 577, 1023]
    T = max(pos) + 1
    cap = lcs.blocksparse_strided_capacity(p, T)
    S = lcs.blocksparse_cache_slots(p, cap)
    kh, vh = history(B, H, T, d, 602)
    q = queries(B, H, d, 602)
    kc, vc = empty_cache(B, H, S, d)
    for b, n in enumerate(pos):
        for h in range(H):
            sp = torch.from_numpy(slot_positions(n, p, h, cap)).cuda()
            held = sp >= 0
            kc[b, h][held] = kh[b, h][sp[held]]
            vc[b, h][held] = vh[b, h][sp[held]]
    k_new, v_new = new_kv(kh, vh, pos)
    o, lse = lcs.attn_blocksparse_decode(q, k_new, v_new, kc, vc,
                                         torch.tensor(pos, device="cuda"), p, cap)
    torch.cuda.synchronize()
    wo, wl = oracle(q, kh, vh, pos, p)
    assert_bf16_close(as_f64(o[:, :, 0]), wo, "o")
    assert_bf16_close(as_f64(lse), wl, "lse")


def test_blocksparse_decode_consecutive_steps():
    """Decode steps in a row append into the ring, wrap it and move strided
    blocks out of it at every block edge; the cache then matches a fresh fill."""
    need_gpu()
    p = lcs.blocksparse_pattern(1, 2, 3)
    B, H, d = 3, 3, 128
    start = [0, 60, 250]
    steps = 330
    T = max(start) + steps
    cap = lcs.blocksparse_strided_capacity(p, T)
    S = lcs.blocksparse_cache_slots(p, cap)
    kh, vh = history(B, H, T, d, 603)
    kc, vc = empty_cache(B, H, S, d)
    lcs.attn_blocksparse_cache_fill(kh, vh, torch.tensor(start, device="cuda"), kc, vc, p, cap)
    worst = 0.0
    for s in range(steps):
        pos = [t + s for t in start]
        q = queries(B, H, d, 603, s)
        k_new, v_new = new_kv(kh, vh, pos)
        o, lse = lcs.attn_blocksparse_decode(q, k_new, v_new, kc, vc,
                                             torch.tensor(pos, device="cuda"), p, cap)
        if s % 41 == 0 or any(t % 64 in (0, 63) for t in pos) or s == steps - 1:
            torch.cuda.synchronize()
            wo, wl = oracle(q, kh, vh, pos, p)
            worst = max(worst, assert_bf16_close(as_f64(o[:, :, 0]), wo, f"step {s}")[0])
            assert_bf16_close(as_f64(lse), wl, f"lse step {s}")
    torch.cuda.synchronize()
    check_layout(kc, vc, kh, vh, [t + steps for t in start], p, cap, sentinel=False)
    print("worst", worst)


def test_blocksparse_decode_invalid_and_capacity():
    """A position whose strided blocks exceed the cache's capacity, and a
    negative position, give o = 0 and lse = NaN and append nothing; the
    other sequences are unaffected."""
    need_gpu()
    p = lcs.blocksparse_pattern(1, 2, 2)
    B, H, d = 3, 2, 128
    pos = [400, -1, 200]
    T = 401
    cap = lcs.blocksparse_strided_capacity(p, 201)      # enough for 200, not for 400
    assert cap < lcs.blocksparse_strided_capacity(p, 401)
    S = lcs.blocksparse_cache_slots(p, cap)
    kh, vh = history(B, H, T, d, 604)
    q = queries(B, H, d, 604)
    kc, vc = empty_cache(B, H, S, d)
    lengths = torch.tensor([0, 0, 200], device="cuda")
    lcs.attn_blocksparse_cache_fill(kh, vh, lengths, kc, vc, p, cap)
    k0, v0 = kc.clone(), vc.clone()
    k_new, v_new = new_kv(kh, vh, [0, 0, 200])
    o, lse = lcs.attn_blocksparse_decode(q, k_new, v_new, kc, vc,
                                         torch.tensor(pos, device="cuda"), p, cap)
    torch.cuda.synchronize()
    for b in (0, 1):
        assert torch.all(o[b] == 0) and torch.all(torch.isnan(lse[b]))
        assert torch.equal(kc[b], k0[b]) and torch.equal(vc[b], v0[b])
    wo, wl = oracle(q[2:], kh[2:], vh[2:], [200], p)
    assert_bf16_close(as_f64(o[2:, :, 0]), wo, "o")
    assert_bf16_close(as_f64(lse[2:]), wl, "lse")


def test_blocksparse_decode_full_size_sampled():
    """Token 131072 of 16 sequences x 32 heads (d 128) in a BlockSparse layer
    with sink 1, local 16, stride 8: the compacted cache holds 17 + 254
    blocks.  Position 131072 starts block 2048, so head phases with
    (2032 + h) % 8 == 0 move block 2032 out of the ring first.  The oracle
    checks 2 sequences x 4 heads."""
    need_gpu()
    p = lcs.blocksparse_pattern(1, 16, 8)
    B, H, d, t = 16, 32, 128, 131072
    cap = lcs.blocksparse_strided_capacity(p, t + 1)
    S = lcs.blocksparse_cache_slots(p, cap)
    kc = randn((B, H, S, d), seed_for(6, 0, "cache"), torch.bfloat16, "cuda")
    vc = randn((B, H, S, d), seed_for(6, 0, "cache_v"), torch.bfloat16, "cuda")
    q = randn((B, H, 1, d), seed_for(6, 0, "q_dec"), torch.bfloat16, "cuda")
    k_new = randn((B, H, 1, d), seed_for(6, 0, "k_new"), torch.bfloat16, "cuda")
    v_new = randn((B, H, 1, d), seed_for(6, 0, "v_new"), torch.bfloat16, "cuda")
    picks = [(b, h) for b in (0, 11) for h in (0, 3, 8, 29)]
    before = {bh: (as_f64(kc[bh]), as_f64(vc[bh])) for bh in picks}
    pos = torch.full((B,), t, dtype=torch.int64, device="cuda")
    o, lse = lcs.attn_blocksparse_decode(q, k_new, v_new, kc, vc, pos, p, cap)
    torch.cuda.synchronize()
    for b, h in picks:
        kk0, vv0 = before[(b, h)]
        sp = slot_positions(t, p, h, cap)          # what slot holds which token
        kk = np.zeros((t + 1, d))
        vv = np.zeros((t + 1, d))
        held = sp >= 0
        kk[sp[held]] = kk0[held]
        vv[sp[held]] = vv0[held]
        kk[t] = as_f64(k_new[b, h, 0])
        vv[t] = as_f64(v_new[b, h, 0])
        keep = blocksparse_decode_positions(t, opattern(p), h)
        assert (sp[held] >= 0).all() and np.isin(keep[:-1], sp[held]).all()
        wo, wl = decode_one(as_f64(q[b, h, 0]), kk, vv, keep, 1 / math.sqrt(d))
        assert_bf16_close(as_f64(o[b, h, 0]), wo, f"b{b} h{h}")
        assert abs(float(lse[b, h]) - wl) < 2e-3
