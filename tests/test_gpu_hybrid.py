"""GPU parity of the hybrid driver path end to end on a small model: the
layer map picks full middle layers and AttnSink outer layers; every layer is
prefilled through its own index; each sparse layer's ring is filled from its
prefill K/V and each full layer's cache holds its prefill K/V; then the next
token is decoded through every layer.  The oracle checks every layer's
prefill and decode from token positions alone."""

import math

import numpy as np
import pytest
import torch

import long_context_sparse_static_amd as lcs
from _parity import assert_bf16_close, need_gpu, oracle_pattern
from oracle import decode_one, decode_positions, sparse_forward
from synth_inputs import as_f64, randn, seed_for

pytestmark = pytest.mark.gpu


def test_hybrid_prefill_then_decode_every_layer():
    need_gpu()
    n_layers, full_first, full_last = 6, 2, 3
    H, d, L = 4, 128, 64 * 10
    sink, window = 64, 192                       # decode ring of the sparse layers
    sparse_pat, full_pat = lcs.attnsink_pattern(1, 3), lcs.full_pattern()
    is_full = lcs.attn_layer_map(n_layers, full_first, full_last)
    assert list(is_full) == [0, 0, 1, 1, 0, 0]
    dev = torch.device("cuda")
    ix = {0: lcs.build_device_index(sparse_pat, H, L, dev, with_csc=False),
          1: lcs.build_device_index(full_pat, H, L, dev, with_csc=False)}
    t = L                                         # the decoded token's position
    q_dec = randn((1, H, 1, d), seed_for(30, 0, "q_dec"), torch.bfloat16).cuda()
    for layer in range(n_layers):
        full = bool(is_full[layer])
        pat = full_pat if full else sparse_pat
        q, k, v = (randn((1, H, L + 1, d), seed_for(30, layer, n), torch.bfloat16).cuda()
                   for n in ("q", "k", "v"))     # token L is the decoded one
        qp, kp, vp = (x[:, :, :L].contiguous() for x in (q, k, v))
        o, lse = lcs.attn_sparse_fwd(qp, kp, vp, ix[int(full)], pat)
        k_new, v_new = k[:, :, L:].contiguous(), v[:, :, L:].contiguous()
        if full:
            kc = torch.zeros((1, H, L + 1, d), dtype=torch.bfloat16, device=dev)
            vc = torch.zeros_like(kc)
            kc[:, :, :L], vc[:, :, :L] = kp, vp
            od, ld = lcs.attn_full_decode(q_dec, k_new, v_new, kc, vc,
                                          torch.tensor([t], device=dev), max_pos=t)
        else:
            rk = torch.zeros((1, H, sink + window, d), dtype=torch.bfloat16, device=dev)
            rv = torch.zeros_like(rk)
            lcs.attn_ring_fill(kp, vp, torch.tensor([L], device=dev), rk, rv, sink, window)
            od, ld = lcs.attn_sparse_decode(q_dec, k_new, v_new, rk, rv,
                                            torch.tensor([t], device=dev), sink, window)
        torch.cuda.synchronize()
        wo, wl = sparse_forward(as_f64(qp), as_f64(kp), as_f64(vp), oracle_pattern(pat))
        assert_bf16_close(as_f64(o), wo, f"layer {layer} prefill O")
        assert_bf16_close(as_f64(lse), wl, f"layer {layer} prefill LSE")
        keep = decode_positions(t) if full else decode_positions(t, sink, window)
        for h in range(H):
            wod, wld = decode_one(as_f64(q_dec[0, h, 0]), as_f64(k[0, h]), as_f64(v[0, h]), keep,
                                  1 / math.sqrt(d))
            assert_bf16_close(as_f64(od[0, h, 0]), wod, f"layer {layer} decode head {h}")
            assert abs(float(ld[0, h]) - wld) < 2e-3
