"""attn_full_decode_noalloc -- attn_full_decode with its split-KV partials in
the library's fixed per-GPU scratch array -- against attn_full_decode itself
through the C ABI: two calls in a row (the second smaller, so stale partials
of the first would show), each equal to the workspace entry point's output
bit for bit on the same inputs and caches; and a size beyond the scratch is
rejected before anything runs."""

import pytest
import torch

import long_context_sparse_static_amd as lcs
from _parity import need_gpu
from synth_inputs import randn

pytestmark = pytest.mark.gpu


def _inputs(B, H, d, cap, seed):
    dev = "cuda"
    q, k_new, v_new = (randn((B, H, 1, d), seed + i, torch.bfloat16, dev) for i in range(3))
    kc, vc = (randn((B, H, cap, d), seed + 3 + i, torch.bfloat16, dev) for i in range(2))
    g = torch.Generator().manual_seed(seed)
    pos = torch.randint(0, cap, (B,), generator=g)
    pos[0] = cap - 1                                   # the longest history
    return q, k_new, v_new, kc, vc, pos.to(dev)


@pytest.mark.parametrize("cases", [[(16, 32, 128, 20000, 11), (3, 5, 64, 700, 12)]])
def test_noalloc_decode_equals_workspace_decode(cases):
    need_gpu()
    for B, H, d, cap, seed in cases:
        q, k_new, v_new, kc, vc, pos = _inputs(B, H, d, cap, seed)
        kc_ref, vc_ref = kc.clone(), vc.clone()
        o_ref, l_ref = lcs.attn_full_decode(q, k_new, v_new, kc_ref, vc_ref, pos, max_pos=cap - 1)
        o = torch.full_like(q, float("nan"))
        lse = torch.full((B, H), float("nan"), device=q.device)
        lcs.attn_full_decode_noalloc(q, k_new, v_new, kc, vc, pos, max_pos=cap - 1, o=o, lse=lse)
        torch.cuda.synchronize()
        assert torch.isfinite(o).all() and torch.isfinite(lse).all()
        assert torch.equal(o, o_ref), (B, H, d, cap)
        assert torch.equal(lse, l_ref), (B, H, d, cap)
        assert torch.equal(kc, kc_ref) and torch.equal(vc, vc_ref)   # the same append


def test_noalloc_decode_rejects_partials_beyond_scratch():
    """B*H = 16384 at d = 128 needs 16384 x 130 x 4 bytes of partials, more
    than the fixed 8 MiB: ATTN_ERR_WORKSPACE, outputs and cache untouched."""
    need_gpu()
    B, H, d, cap = 64, 256, 128, 2
    q, k_new, v_new, kc, vc, pos = _inputs(B, H, d, cap, 13)
    kc0 = kc.clone()
    o = torch.full_like(q, 7.0)
    lse = torch.full((B, H), 7.0, device=q.device)
    with pytest.raises(lcs.AttnError) as err:
        lcs.attn_full_decode_noalloc(q, k_new, v_new, kc, vc, pos, max_pos=cap - 1, o=o, lse=lse)
    assert err.value.status == lcs.ATTN_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(o == 7.0) and torch.all(lse == 7.0) and torch.equal(kc, kc0)
