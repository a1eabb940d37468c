"""Entry points enqueue on the caller's current stream: forward, backward and
decode issued on two side streams at once, with no synchronisation between
them, give bit for bit what the same calls give one after another on the
default stream (every kernel is deterministic)."""

import pytest
import torch

import long_context_sparse_static_amd as lcs
from _parity import need_gpu
from synth_inputs import randn, seed_for

pytestmark = pytest.mark.gpu


def _prefill_case(pat, H, L, wl):
    q, k, v, do = (randn((1, H, L, 128), seed_for(wl, 0, t), torch.bfloat16).cuda() for t in ("q", "k", "v", "do"))
    ix = lcs.build_device_index(pat, H, L, q.device, with_csc=True)
    return pat, ix, q, k, v, do


def _train(case):
    pat, ix, q, k, v, do = case
    o, lse = lcs.attn_sparse_fwd(q, k, v, ix, pat)
    dq, dk, dv = lcs.attn_sparse_bwd(q, k, v, o, lse, do, ix, pat)
    return o, lse, dq, dk, dv


def test_two_side_streams_match_default_stream():
    need_gpu()
    a = _prefill_case(lcs.attnsink_pattern(1, 8), 4, 64 * 40, 960)
    b = _prefill_case(lcs.blocksparse_pattern(1, 4, 4), 4, 64 * 33 + 17, 961)
    # decode: 4 sequences, sink 64 + window 256, position 700
    B, H, d, S, W, t = 4, 4, 128, 64, 256, 700
    q1, kn, vn = (randn((B, H, 1, d), seed_for(962, 0, n), torch.bfloat16).cuda() for n in ("q_dec", "k_new", "v_new"))
    kc0, vc0 = (randn((B, H, S + W, d), seed_for(962, 0, n), torch.bfloat16).cuda() for n in ("cache", "cache_v"))
    pos = torch.full((B,), t, dtype=torch.int64, device="cuda")
    torch.cuda.synchronize()

    ref_a, ref_b = _train(a), _train(b)
    kc, vc = kc0.clone(), vc0.clone()
    ref_dec = lcs.attn_sparse_decode(q1, kn, vn, kc, vc, pos, S, W)
    torch.cuda.synchronize()

    kc2, vc2 = kc0.clone(), vc0.clone()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()   # default priority
    main = torch.cuda.current_stream()
    s1.wait_stream(main)
    s2.wait_stream(main)
    with torch.cuda.stream(s1):
        got_a = _train(a)
    with torch.cuda.stream(s2):
        got_b = _train(b)
        got_dec = lcs.attn_sparse_decode(q1, kn, vn, kc2, vc2, pos, S, W)
    main.wait_stream(s1)
    main.wait_stream(s2)
    torch.cuda.synchronize()
    for got, ref in ((got_a, ref_a), (got_b, ref_b), (got_dec, ref_dec)):
        for g, r in zip(got, ref):
            assert torch.equal(g, r)
    assert torch.equal(kc2, kc) and torch.equal(vc2, vc)
