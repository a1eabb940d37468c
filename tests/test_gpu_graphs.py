"""Entry points captured in a HIP graph (torch.cuda.CUDAGraph) replay
correctly: a decode step (full decode through the allocation-free entry
point plus a sink+window ring decode) and a prefill forward + backward are
captured once with preallocated outputs and workspaces, then replayed
several times with new inputs written in place between replays, with eager
work and synchronisations in between; every replay equals the eager calls on
the same inputs bit for bit (the library records no memset nodes)."""

import pytest
import torch

import long_context_sparse_static_amd as lcs
from _parity import need_gpu
from synth_inputs import randn, seed_for

pytestmark = pytest.mark.gpu


def _capture(step):
    side = torch.cuda.Stream()          # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                          # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return g


def test_decode_step_graph_replays():
    need_gpu()
    B, H, d, cap, S, W = 4, 8, 128, 5000, 64, 512
    dev = "cuda"
    q, kn, vn = (torch.empty((B, H, 1, d), dtype=torch.bfloat16, device=dev) for _ in range(3))
    kc, vc = (randn((B, H, cap, d), seed_for(970, 0, n), torch.bfloat16, dev) for n in ("cache", "cache_v"))
    rk, rv = (randn((B, H, S + W, d), seed_for(971, 0, n), torch.bfloat16, dev) for n in ("cache", "cache_v"))
    pos = torch.zeros(B, dtype=torch.int64, device=dev)
    o, o2 = torch.empty_like(q), torch.empty_like(q)
    lse, lse2 = (torch.empty((B, H), dtype=torch.float32, device=dev) for _ in range(2))
    ws2 = torch.empty(max(lcs.attn_workspace_bytes(lcs.ATTN_OP_SPARSE_DECODE, lcs.ATTN_BF16, B, H, S + W, d), 1),
                      dtype=torch.uint8, device=dev)

    def fill(r):
        for t, n in ((q, "q_dec"), (kn, "k_new"), (vn, "v_new")):
            t.copy_(randn(t.shape, seed_for(972 + r, 0, n), torch.bfloat16, dev))
        pos.copy_(torch.tensor([100 + r, 2000 + 3 * r, 4000 + r, cap - 4 + r], dtype=torch.int64))

    def step():
        lcs.attn_full_decode_noalloc(q, kn, vn, kc, vc, pos, max_pos=cap - 1, o=o, lse=lse)
        lcs.attn_sparse_decode(q, kn, vn, rk, rv, pos, S, W, o=o2, lse=lse2, workspace=ws2)

    fill(0)
    g = _capture(step)
    kr, vr, rkr, rvr = kc.clone(), vc.clone(), rk.clone(), rv.clone()
    for r in range(4):
        fill(r)
        torch.cuda.synchronize()
        g.replay()
        o_ref, l_ref = lcs.attn_full_decode(q, kn, vn, kr, vr, pos, max_pos=cap - 1)
        o2_ref, l2_ref = lcs.attn_sparse_decode(q, kn, vn, rkr, rvr, pos, S, W)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), r
        assert torch.equal(o2, o2_ref) and torch.equal(lse2, l2_ref), r
        assert torch.equal(kc, kr) and torch.equal(vc, vr) and torch.equal(rk, rkr) and torch.equal(rv, rvr), r
        assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(o2).all())


@pytest.mark.parametrize("pat", [lcs.attnsink_pattern(1, 8), lcs.blocksparse_pattern(1, 4, 4)])
def test_prefill_forward_backward_graph_replays(pat):
    need_gpu()
    H, L, d = 4, 64 * 30 + 9, 128
    dev = "cuda"
    q, k, v, do = (torch.empty((1, H, L, d), dtype=torch.bfloat16, device=dev) for _ in range(4))
    ix = lcs.build_device_index(pat, H, L, q.device, with_csc=True)
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty((1, H, L), dtype=torch.float32, device=dev)
    ws = torch.empty(max(lcs.attn_workspace_bytes(lcs.ATTN_OP_BWD, lcs.ATTN_BF16, 1, H, L, d), 1),
                     dtype=torch.uint8, device=dev)

    def fill(r):
        for t, n in ((q, "q"), (k, "k"), (v, "v"), (do, "do")):
            t.copy_(randn(t.shape, seed_for(980 + r, 0, n), torch.bfloat16, dev))

    def step():
        lcs.attn_sparse_fwd(q, k, v, ix, pat, o=o, lse=lse)
        lcs.attn_sparse_bwd(q, k, v, o, lse, do, ix, pat, dq=dq, dk=dk, dv=dv, workspace=ws)

    fill(0)
    g = _capture(step)
    for r in range(3):
        fill(r)
        torch.cuda.synchronize()
        g.replay()
        o_ref, l_ref = lcs.attn_sparse_fwd(q, k, v, ix, pat)
        dq_ref, dk_ref, dv_ref = lcs.attn_sparse_bwd(q, k, v, o_ref, l_ref, do, ix, pat)
        torch.cuda.synchronize()
        for got, ref in ((o, o_ref), (lse, l_ref), (dq, dq_ref), (dk, dk_ref), (dv, dv_ref)):
            assert torch.equal(got, ref), r
