"""GPU parity over seeded random pattern parameters: kind, sink and local
block counts, BlockSparse stride, token window, batch, heads, head dim and a
length that is often ragged.  bf16 forward and backward, and the fp32
forward, against the float64 oracle on every output.

Short lists (one local block and no sink) give dV entries of magnitude 6,
where consecutive bf16 values lie 2^-5 apart.  There the arithmetic of a
bf16 matrix-core product dV = P^T dO (P rounded to bf16 as an operand, the
sum exact, the result rounded to bf16) already misses 2e-2 on the same input
(0.0245 on the case with one local block).  So dV is held to the
larger of 2e-2 and 1.25 times that arithmetic's own worst error on the same
input; every other output, and every mean, to the usual bounds."""

import math

import numpy as np
import pytest
import torch

import long_context_sparse_static_amd as lcs
from _parity import BF16_MAX, BF16_MEAN, assert_bf16_close, assert_f32_close, errors, need_gpu, oracle_pattern
from oracle import pattern_token_mask, sparse_backward, sparse_forward
from synth_inputs import as_f64, randn, seed_for

pytestmark = pytest.mark.gpu


def _random_case(rng):
    kind = int(rng.integers(0, 4))
    if kind == 0:
        pat = lcs.full_pattern()
    elif kind == 1:
        pat = lcs.attnsink_pattern(int(rng.integers(0, 4)), int(rng.integers(1, 9)))
    elif kind == 2:
        pat = lcs.blocksparse_pattern(int(rng.integers(0, 4)), int(rng.integers(1, 9)), int(rng.integers(1, 8)))
    else:
        pat = lcs.sliding_pattern(int(rng.integers(0, 3)), int(rng.integers(1, 700)))
    d = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 3))
    H = int(rng.integers(1, 5))
    L = int(rng.integers(1, 64 * (14 if rng.random() < 0.5 else 40)))
    return pat, d, B, H, L


def bf16_rounded(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def dv_bound(q, k, do, lse, pattern):
    """max(2e-2, 1.25 x the worst error of bf16(bf16(P)^T dO) against the
    exact dV, with P = exp(S - LSE) from the oracle's LSE)."""
    B, H, L, d = q.shape
    worst = 0.0
    for b in range(B):
        for h in range(H):
            mask = pattern_token_mask(pattern, h, L)
            s = np.where(mask, q[b, h] @ k[b, h].T / math.sqrt(d), -np.inf)
            p = np.exp(s - lse[b, h][:, None])
            p[~np.isfinite(p)] = 0.0
            exact = p.T @ do[b, h]
            worst = max(worst, float(np.abs(bf16_rounded(bf16_rounded(p).T @ do[b, h]) - exact).max()))
    return max(BF16_MAX, 1.25 * worst)


CASES = [_random_case(np.random.default_rng(8200 + i)) for i in range(10)]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_random_pattern_forward_backward(case):
    need_gpu()
    pat, d, B, H, L = CASES[case]
    print("case", case, pat, "d", d, "B", B, "H", H, "L", L, flush=True)
    q, k, v, do = (randn((B, H, L, d), seed_for(8200 + case, 0, t), torch.bfloat16).cuda()
                   for t in ("q", "k", "v", "do"))
    ix = lcs.build_device_index(pat, H, L, q.device, with_csc=True)
    o, lse = lcs.attn_sparse_fwd(q, k, v, ix, pat)
    dq, dk, dv = lcs.attn_sparse_bwd(q, k, v, o, lse, do, ix, pat)
    torch.cuda.synchronize()
    wq, wk, wv, wo, wl = sparse_backward(as_f64(q), as_f64(k), as_f64(v), as_f64(do), oracle_pattern(pat))
    assert_bf16_close(as_f64(o), wo, "O")
    assert_bf16_close(as_f64(lse), wl, "LSE")
    for name, g, w in (("dq", dq, wq), ("dk", dk, wk)):
        assert_bf16_close(as_f64(g), w, name)
    bound = dv_bound(as_f64(q), as_f64(k), as_f64(do), wl, oracle_pattern(pat))
    mx, mean = errors(as_f64(dv), wv)
    print("dv", mx, mean, "bound", bound)
    assert mx <= bound and mean <= BF16_MEAN, f"dv: max {mx:.3e} (bound {bound:.3e}) mean {mean:.3e}"


@pytest.mark.parametrize("case", range(0, len(CASES), 2))
def test_random_pattern_fp32_forward(case):
    need_gpu()
    pat, d, B, H, L = CASES[case]
    print("case", case, pat, "d", d, "B", B, "H", H, "L", L, flush=True)
    q, k, v = (randn((B, H, L, d), seed_for(8300 + case, 0, t), torch.float32).cuda() for t in ("q", "k", "v"))
    ix = lcs.build_device_index(pat, H, L, q.device, with_csc=False)
    o, lse = lcs.attn_sparse_fwd(q, k, v, ix, pat)
    torch.cuda.synchronize()
    wo, wl = sparse_forward(as_f64(q), as_f64(k), as_f64(v), oracle_pattern(pat))
    assert_f32_close(as_f64(o), wo, "O")
    assert_f32_close(as_f64(lse), wl, "LSE")
