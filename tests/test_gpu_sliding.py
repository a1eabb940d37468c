"""GPU parity of the token-granular sliding window (kind ATTN_SLIDING: the
window masks keys inside its edge blocks) in the forward, the backward and
against decode, whose sink + window ring reads the same keys."""

import math

import numpy as np
import pytest
import torch

import long_context_sparse_static_amd as lcs
from _parity import (assert_bf16_close, assert_f32_close, need_gpu, oracle_pattern,
                     sample_backward, sample_rows_forward)
from oracle import decode_one, decode_positions, sparse_backward, sparse_forward
from synth_inputs import as_f64, randn, seed_for

pytestmark = pytest.mark.gpu


def _inputs(shape, workload, dtype=torch.bfloat16, big=False, names=("q", "k", "v")):
    gen_dev = "cuda" if big else "cpu"
    return [randn(shape, seed_for(workload, 0, t), dtype, gen_dev).cuda() for t in names]


def _fwd(q, k, v, pat, with_csc=False):
    B, H, L, d = q.shape
    ix = lcs.build_device_index(pat, H, L, q.device, with_csc=with_csc)
    o, lse = lcs.attn_sparse_fwd(q, k, v, ix, pat)
    torch.cuda.synchronize()
    return ix, o, lse


FWD_CASES = [
    # (sink blocks, window tokens, d, B, H, n_blocks)
    (0, 1, 128, 1, 2, 5),        # each token reads only itself
    (0, 37, 128, 1, 2, 11),      # window shorter than a block
    (0, 64, 64, 2, 2, 9),        # window of exactly one block
    (1, 100, 128, 1, 3, 13),     # window across two partial blocks, sink block
    (2, 65, 64, 1, 2, 12),       # two sink blocks, window one block + 1
    (1, 4096, 128, 1, 1, 70),    # the 64-block window, token-granular
    (0, 10 ** 6, 128, 1, 1, 7),  # window beyond the sequence: causal attention
]


@pytest.mark.parametrize("case", range(len(FWD_CASES)))
def test_sliding_forward_full_oracle(case):
    need_gpu()
    s, W, d, B, H, nb = FWD_CASES[case]
    pat = lcs.sliding_pattern(s, W)
    q, k, v = _inputs((B, H, 64 * nb, d), 700 + case)
    _, o, lse = _fwd(q, k, v, pat)
    wo, wl = sparse_forward(as_f64(q), as_f64(k), as_f64(v), oracle_pattern(pat))
    print(case, "O", assert_bf16_close(as_f64(o), wo, "O"))
    print(case, "LSE", assert_bf16_close(as_f64(lse), wl, "LSE"))


def test_sliding_forward_fp32():
    need_gpu()
    pat = lcs.sliding_pattern(1, 100)
    q, k, v = _inputs((1, 2, 64 * 9, 64), 720, torch.float32)
    _, o, lse = _fwd(q, k, v, pat)
    wo, wl = sparse_forward(as_f64(q), as_f64(k), as_f64(v), oracle_pattern(pat))
    assert_f32_close(as_f64(o), wo, "O")
    assert_f32_close(as_f64(lse), wl, "LSE")


BWD_CASES = [(1, 100, 128, 2, 13), (0, 37, 128, 1, 9), (2, 65, 64, 2, 11), (0, 1, 128, 1, 4)]


@pytest.mark.parametrize("case", range(len(BWD_CASES)))
def test_sliding_backward_full_oracle(case):
    need_gpu()
    s, W, d, H, nb = BWD_CASES[case]
    pat = lcs.sliding_pattern(s, W)
    q, k, v, do = _inputs((1, H, 64 * nb, d), 730 + case, names=("q", "k", "v", "do"))
    ix, o, lse = _fwd(q, k, v, pat, with_csc=True)
    dq, dk, dv = lcs.attn_sparse_bwd(q, k, v, o, lse, do, ix, pat)
    torch.cuda.synchronize()
    wq, wk, wv, _, _ = sparse_backward(as_f64(q), as_f64(k), as_f64(v), as_f64(do), oracle_pattern(pat))
    for name, g, w in (("dq", dq, wq), ("dk", dk, wk), ("dv", dv, wv)):
        print(case, name, assert_bf16_close(as_f64(g), w, name))


def test_sliding_32k_sampled():
    """32K tokens, 8 heads, sink 1 block + 4000-token window (not a multiple
    of 64): sampled forward rows at and around the window edges, and sampled
    dQ / dK / dV blocks, each on its exact sub-problem."""
    need_gpu()
    pat = lcs.sliding_pattern(1, 4000)
    L, H = 32768, 8
    q, k, v, do = _inputs((1, H, L, 128), 740, big=True, names=("q", "k", "v", "do"))
    ix, o, lse = _fwd(q, k, v, pat, with_csc=True)
    dq, dk, dv = lcs.attn_sparse_bwd(q, k, v, o, lse, do, ix, pat)
    torch.cuda.synchronize()
    rows = [0, 63, 64, 3999, 4000, 4063, 4064, 4100, 20000, L - 1]
    for h in (0, 5):
        wo, wl = sample_rows_forward(q, k, v, pat, h, 0, rows)
        assert_bf16_close(as_f64(o[0, h, rows]), wo, f"O head {h}")
        assert_bf16_close(as_f64(lse[0, h, rows]), wl, f"LSE head {h}")
    nb = L // 64
    want = sample_backward(q, k, v, do, pat, 3, 0, [0, 62, 63, 64, 300, nb - 1], [0, 1, 200, nb - 63, nb - 1])
    for (name, blk), w in want.items():
        g = {"dq": dq, "dk": dk, "dv": dv}[name][0, 3, 64 * blk:64 * (blk + 1)]
        print(name, blk, assert_bf16_close(as_f64(g), w, f"{name} block {blk}"))


def test_sliding_prefill_last_row_equals_decode():
    """Prefill of L tokens with the token-granular window, then the same
    sequence's last token decoded against a sink + window ring filled from
    tokens 0..L-2: both read the same keys, so their outputs agree with each
    other and with the oracle."""
    need_gpu()
    s, W, d, H = 1, 300, 128, 4
    L = 64 * 14
    pat = lcs.sliding_pattern(s, W)
    q, k, v = _inputs((1, H, L, d), 750)
    _, o, lse = _fwd(q, k, v, pat)
    sink_tok = 64 * s
    ring_k = torch.zeros((1, H, sink_tok + W, d), dtype=torch.bfloat16, device="cuda")
    ring_v = torch.zeros_like(ring_k)
    t = L - 1
    lcs.attn_ring_fill(k, v, torch.tensor([t], device="cuda"), ring_k, ring_v, sink_tok, W)
    od, ld = lcs.attn_sparse_decode(q[:, :, t:t + 1].contiguous(), k[:, :, t:t + 1].contiguous(),
                                    v[:, :, t:t + 1].contiguous(), ring_k, ring_v,
                                    torch.tensor([t], device="cuda"), sink_tok, W)
    torch.cuda.synchronize()
    keep = decode_positions(t, sink_tok, W)
    for h in range(H):
        wo, wl = decode_one(as_f64(q[0, h, t]), as_f64(k[0, h]), as_f64(v[0, h]), keep, 1 / math.sqrt(d))
        assert_bf16_close(as_f64(o[0, h, t]), wo, f"prefill head {h}")
        assert_bf16_close(as_f64(od[0, h, 0]), wo, f"decode head {h}")
        assert abs(float(lse[0, h, t]) - wl) < 2e-3 and abs(float(ld[0, h]) - wl) < 2e-3
    assert float((o[0, :, t] - od[0, :, 0]).abs().max()) < 2e-2


@pytest.mark.parametrize("s,W,d", [(1, 100, 128), (0, 37, 64), (2, 64, 128)])
def test_sliding_zero_query_lse_counts(s, W, d):
    """Q = 0: LSE = ln(number of keys read) exactly -- min(q + 1, W) window
    keys plus the sink keys left of the window -- which pins the token
    window's edges on the GPU."""
    need_gpu()
    H, nb = 4, 9
    L = 64 * nb
    pat = lcs.sliding_pattern(s, W)
    q = torch.zeros((1, H, L, d), dtype=torch.bfloat16, device="cuda")
    _, k, v = _inputs((1, H, L, d), 760)
    _, o, lse = _fwd(q, k, v, pat)
    t = np.arange(L)
    counts = np.minimum(t + 1, W) + np.maximum(0, np.minimum(64 * s, t + 1 - W))
    for h in range(H):
        np.testing.assert_allclose(lse[0, h].cpu().numpy(), np.log(counts), rtol=0, atol=2e-6)
    wo, _ = sparse_forward(np.zeros((1, H, L, d)), as_f64(k), as_f64(v), oracle_pattern(pat))
    assert_bf16_close(as_f64(o), wo, "O")
