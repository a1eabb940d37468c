"""GPU parity of the strided entry points (attn_sparse_fwd_strided,
attn_sparse_bwd_strided): [B,L,H,d] activations and Q/K/V read in place from
a fused [B,L,3,H,d] projection.  The kernels do the same arithmetic in the
same order whatever the addresses, so the strided results must equal the
contiguous ones bit for bit; the oracle checks them as well."""

import pytest
import torch

import long_context_sparse_static_amd as lcs
from _parity import assert_bf16_close, assert_f32_close, need_gpu, oracle_pattern
from oracle import sparse_backward, sparse_forward
from synth_inputs import as_f64, randn, seed_for

pytestmark = pytest.mark.gpu

PATTERNS = [lcs.attnsink_pattern(1, 3), lcs.blocksparse_pattern(1, 2, 3), lcs.sliding_pattern(1, 100),
            lcs.full_pattern()]


def blhd(B, L, H, d, workload, name, dtype=torch.bfloat16):
    """A [B,L,H,d] tensor and its [B,H,L,d]-indexed view."""
    x = randn((B, L, H, d), seed_for(workload, 0, name), dtype).cuda()
    return x, x.transpose(1, 2)


@pytest.mark.parametrize("case", range(len(PATTERNS)))
def test_forward_blhd_equals_contiguous(case):
    need_gpu()
    pat = PATTERNS[case]
    B, L, H, d = 2, 64 * 9, 3, 128
    (_, q), (_, k), (_, v) = (blhd(B, L, H, d, 900 + case, n) for n in ("q", "k", "v"))
    ix = lcs.build_device_index(pat, H, L, q.device, with_csc=False)
    o_buf = torch.empty((B, L, H, d), dtype=torch.bfloat16, device="cuda")
    o, lse = lcs.attn_sparse_fwd_strided(q, k, v, ix, pat, o=o_buf.transpose(1, 2))
    o2, lse2 = lcs.attn_sparse_fwd(q.contiguous(), k.contiguous(), v.contiguous(), ix, pat)
    torch.cuda.synchronize()
    assert torch.equal(o_buf.transpose(1, 2), o2) and torch.equal(lse, lse2)
    wo, wl = sparse_forward(as_f64(q), as_f64(k), as_f64(v), oracle_pattern(pat))
    assert_bf16_close(as_f64(o), wo, "O")
    assert_bf16_close(as_f64(lse), wl, "LSE")


def test_forward_fp32_blhd():
    need_gpu()
    pat = lcs.attnsink_pattern(1, 4)
    B, L, H, d = 1, 64 * 6, 2, 64
    (_, q), (_, k), (_, v) = (blhd(B, L, H, d, 910, n, torch.float32) for n in ("q", "k", "v"))
    ix = lcs.build_device_index(pat, H, L, q.device, with_csc=False)
    o, lse = lcs.attn_sparse_fwd_strided(q, k, v, ix, pat)
    torch.cuda.synchronize()
    wo, wl = sparse_forward(as_f64(q), as_f64(k), as_f64(v), oracle_pattern(pat))
    assert_f32_close(as_f64(o), wo, "O")
    assert_f32_close(as_f64(lse), wl, "LSE")


@pytest.mark.parametrize("d", [128, 64])
def test_fused_qkv_forward_backward(d):
    """Q, K, V as slices of one [B,L,3,H,d] projection; O and dO in
    [B,L,H,d]; dQ, dK, dV written into one fused [B,L,3,H,d] gradient."""
    need_gpu()
    pat = lcs.blocksparse_pattern(1, 3, 4)
    B, L, H = 2, 64 * 11, 4
    qkv = randn((B, L, 3, H, d), seed_for(920 + d, 0, "q"), torch.bfloat16).cuda()
    q, k, v = (qkv[:, :, i].transpose(1, 2) for i in range(3))
    _, do = blhd(B, L, H, d, 920 + d, "do")
    ix = lcs.build_device_index(pat, H, L, q.device, with_csc=True)
    o_buf = torch.empty((B, L, H, d), dtype=torch.bfloat16, device="cuda")
    o, lse = lcs.attn_sparse_fwd_strided(q, k, v, ix, pat, o=o_buf.transpose(1, 2))
    g = torch.full((B, L, 3, H, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    dq, dk, dv = (g[:, :, i].transpose(1, 2) for i in range(3))
    lcs.attn_sparse_bwd_strided(q, k, v, o, lse, do, ix, pat, dq=dq, dk=dk, dv=dv)
    # the same through the contiguous entry points
    qc, kc, vc, doc = (t.contiguous() for t in (q, k, v, do))
    o2, lse2 = lcs.attn_sparse_fwd(qc, kc, vc, ix, pat)
    dq2, dk2, dv2 = lcs.attn_sparse_bwd(qc, kc, vc, o2, lse2, doc, ix, pat)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.equal(a, b)
    assert bool(torch.isfinite(g).all())
    wq, wk, wv, wo, _ = sparse_backward(as_f64(q), as_f64(k), as_f64(v), as_f64(do), oracle_pattern(pat))
    assert_bf16_close(as_f64(o), wo, "O")
    for name, t, w in (("dq", dq, wq), ("dk", dk, wk), ("dv", dv, wv)):
        print(d, name, assert_bf16_close(as_f64(t), w, name))


@pytest.mark.parametrize("stride", [0, 8, 72])
def test_inputs_with_token_stride_below_d(stride):
    """Q, K, V and dO whose token rows overlap (row stride below d; 0 repeats
    one row), at a length with a partial last block: every tile and operand
    load stays in range, and forward and backward equal those of contiguous
    copies bit for bit."""
    need_gpu()
    pat = lcs.attnsink_pattern(1, 3)
    B, H, L, d = 1, 2, 64 * 5 + 17, 128

    def overlapping(name):
        n = (L - 1) * stride + d
        buf = randn((B, H, n), seed_for(930 + stride, 0, name), torch.bfloat16).cuda()
        return buf.as_strided((B, H, L, d), (H * n, n, stride, 1))

    q, k, v, do = (overlapping(n) for n in ("q", "k", "v", "do"))
    ix = lcs.build_device_index(pat, H, L, q.device, with_csc=True)
    o, lse = lcs.attn_sparse_fwd_strided(q, k, v, ix, pat)
    dq, dk, dv = lcs.attn_sparse_bwd_strided(q, k, v, o, lse, do, ix, pat)
    qc, kc, vc, doc = (t.contiguous() for t in (q, k, v, do))
    o2, lse2 = lcs.attn_sparse_fwd(qc, kc, vc, ix, pat)
    dq2, dk2, dv2 = lcs.attn_sparse_bwd(qc, kc, vc, o2, lse2, doc, ix, pat)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.equal(a, b)
    wo, wl = sparse_forward(as_f64(q), as_f64(k), as_f64(v), oracle_pattern(pat))
    assert_bf16_close(as_f64(o), wo, "O")
    assert_bf16_close(as_f64(lse), wl, "LSE")


@pytest.mark.parametrize("stride", [0, 32])
def test_fp32_inputs_with_token_stride_below_d(stride):
    """The fp32 forward on Q, K, V whose token rows overlap (row stride below
    d), at a length with a partial last block: equal to contiguous copies bit
    for bit, and to the oracle."""
    need_gpu()
    pat = lcs.attnsink_pattern(1, 2)
    B, H, L, d = 1, 2, 64 * 4 + 9, 64

    def overlapping(name):
        n = (L - 1) * stride + d
        buf = randn((B, H, n), seed_for(940 + stride, 0, name), torch.float32).cuda()
        return buf.as_strided((B, H, L, d), (H * n, n, stride, 1))

    q, k, v = (overlapping(n) for n in ("q", "k", "v"))
    ix = lcs.build_device_index(pat, H, L, q.device, with_csc=False)
    o, lse = lcs.attn_sparse_fwd_strided(q, k, v, ix, pat)
    o2, lse2 = lcs.attn_sparse_fwd(q.contiguous(), k.contiguous(), v.contiguous(), ix, pat)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    wo, wl = sparse_forward(as_f64(q), as_f64(k), as_f64(v), oracle_pattern(pat))
    assert_f32_close(as_f64(o), wo, "O")
    assert_f32_close(as_f64(lse), wl, "LSE")
