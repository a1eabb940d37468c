"""GPU parity where element offsets pass 2^31: 64 heads of 268,800 tokens at
d = 128 put the last head's rows at elements 2,167,603,200 and beyond of
every [B,H,L,d] tensor.  Forward and backward, AttnSink and BlockSparse (its
dK/dV in the two-key-block form), checked on the first and the last head
against the oracle's exact sub-problems."""

import numpy as np
import pytest
import torch

import long_context_sparse_static_amd as lcs
from _parity import assert_bf16_close, need_gpu, sample_backward, sample_rows_forward
from synth_inputs import as_f64, randn, seed_for

pytestmark = pytest.mark.gpu

H, L, D = 64, 64 * 4200, 128


@pytest.mark.parametrize("kind", ["attnsink", "blocksparse"])
def test_offsets_beyond_2_31_elements(kind):
    need_gpu()
    assert (H - 1) * L * D > 2 ** 31
    pat = lcs.attnsink_pattern(1, 64) if kind == "attnsink" else lcs.blocksparse_pattern(1, 16, 8)
    print("case", kind, "H", H, "L", L, flush=True)
    q, k, v, do = (randn((1, H, L, D), seed_for(9100 + (kind == "blocksparse"), 0, t), torch.bfloat16, "cuda")
                   for t in ("q", "k", "v", "do"))
    ix = lcs.build_device_index(pat, H, L, q.device, with_csc=True)
    o, lse = lcs.attn_sparse_fwd(q, k, v, ix, pat)
    dq, dk, dv = lcs.attn_sparse_bwd(q, k, v, o, lse, do, ix, pat)
    torch.cuda.synchronize()
    for t in (o, lse, dq, dk, dv):
        assert bool(torch.isfinite(t).all())
    nb = L // 64
    rng = np.random.default_rng(91)
    for h in (0, H - 1):
        rows = np.unique(np.concatenate([[0, 63, 64, L - 65, L - 1], rng.integers(0, L, 20)]))
        wo, wl = sample_rows_forward(q, k, v, pat, h, 0, rows)
        idx = torch.as_tensor(rows, device=q.device)
        assert_bf16_close(as_f64(o[0, h, idx]), wo, f"O head {h}")
        assert_bf16_close(as_f64(lse[0, h, idx]), wl, f"LSE head {h}")
        qbs = [0, 1, nb // 2, nb - 1]
        # key blocks whose columns are short: not the sink, not in head h's strided class
        kbs = [j for j in (5, nb // 2 + 3, nb - 2) if kind == "attnsink" or (j + h) % 8 != 0]
        want = sample_backward(q, k, v, do, pat, h, 0, qbs, kbs)
        for i in qbs:
            assert_bf16_close(as_f64(dq[0, h, i * 64:(i + 1) * 64]), want[("dq", i)], f"dq block {i} head {h}")
        for j in kbs:
            for n, g in (("dk", dk), ("dv", dv)):
                assert_bf16_close(as_f64(g[0, h, j * 64:(j + 1) * 64]), want[(n, j)], f"{n} block {j} head {h}")
        print(kind, "head", h, "rows", len(rows), "dq blocks", len(qbs), "dk/dv blocks", len(kbs), flush=True)
