"""Benchmark of the static block-sparse attention hot path on one MI355X.

Default workload ("hybrid128k"): Llama-2-7B-shaped attention (32 layers,
32 heads, d 128, bf16) at 131072 tokens, LongGen's hybrid layer map -- layers
11..21 full causal attention, the other 21 layers AttnSink (sink 64 tokens,
window 4096 tokens = 64 blocks).  One step =
  prefill forward of all 32 layers (batch 1),
  ring fill of every sparse layer's sink+window cache from its prefill K/V,
  decode of 16 sequences (one new token each at position 131072) through all
  32 layers: sparse layers read their 64+4096-slot ring caches, full layers
  their 131073-slot caches.
Inputs are synthetic (seeded N(0,1), bf16) and resident in HBM before timing.

Printed: one JSON line.  ``value`` is the effective TFLOP/s of the sparse
(AttnSink) prefill layers -- algorithmic FLOPs of the computed 64x64 blocks
(4*64*64*d per block pair) divided by their kernel time.  Decode tokens/s,
the full-layer and whole-hybrid prefill rates, the roofline of the dominant
kernel and the CPU oracle baseline are reported alongside.  After the timed
hybrid steps the same run times every other configuration of the workload
definitions ("configs": the fp32 1K AttnSink forward, 8K AttnSink and 32K
BlockSparse forwards, the 64K AttnSink forward + backward, and the 128K
BlockSparse forward + backward), each with its median launch time, rate and
fraction of the bf16 matrix-core peak.

Other workloads (--workload): attnsink8k, blocksparse32k, blocksparse128k,
attnsink128k, train64k (AttnSink forward + backward), blocksparse32k_train and
blocksparse128k_train (BlockSparse forward + backward), sliding128k and
sliding64k_train (token-granular window of 4096 tokens + 1 sink block),
bsdecode128k
(BlockSparse decode against its compacted cache), pageddecode128k (full-layer
decode against 64-token pages named by a block table), and copy1g (a plain 1 GiB
device copy, the calibration kernel for the HBM byte counters).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import long_context_sparse_static_amd as lcs  # noqa: E402
from synth_inputs import randn, seed_for  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
H, D, BLK = 32, 128, 64
SINK_BLOCKS, WINDOW_BLOCKS = 1, 64
SINK_TOK, WINDOW_TOK = 64, 4096
N_LAYERS, FULL_FIRST, FULL_LAST = 32, 11, 21
DEC_BATCH = 16

# HBM bytes per launch of the dominant kernel, from two rocprofv3 --pmc runs of
# the same workload (FETCH_SIZE, then WRITE_SIZE), each scaled by what the
# counter reads for copy1g (1 GiB read + 1 GiB written).  Keyed by workload and
# a hash of the kernel's sources: a changed kernel reports null until its
# counters are taken again.
KERNEL_SOURCES = ("fwd_bf16.hip", "tiles.h", "device_common.h", "kernels.h")
TRAFFIC = {
    # fwd_bf16_kernel<128>, average over the 32 launches of one hybrid128k step
    ("hybrid128k", "304fdd23221b6386"): 10.836e9,
}


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "long_context_sparse_static_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(workload):
    return TRAFFIC.get((workload, kernel_source_hash()))


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def pair_flops(d=D):
    return 4.0 * BLK * BLK * d


class Timer:
    """hipEvent pairs on the current stream, summed per label."""

    def __init__(self):
        self.pending = []

    def span(self, label):
        t = self
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)

        class _Ctx:
            def __enter__(self_):
                s.record()

            def __exit__(self_, *a):
                e.record()
                t.pending.append((label, s, e))
        return _Ctx()

    def collect(self):
        torch.cuda.synchronize()
        out = {}
        for label, s, e in self.pending:
            out.setdefault(label, []).append(s.elapsed_time(e))
        self.pending = []
        return out


def fill_randn(shape, seed):
    """Large bf16 tensor of seeded N(0,1) values, generated on the device."""
    return randn(shape, seed, torch.bfloat16, "cuda")


# ----------------------------------------------------------------------------
# hybrid 128K workload
# ----------------------------------------------------------------------------
class Hybrid128k:
    name = "hybrid128k"
    L = 131072

    def __init__(self, n_sets=4, n_full_caches=2):
        dev = torch.device("cuda")
        L = self.L
        self.layer_full = lcs.attn_layer_map(N_LAYERS, FULL_FIRST, FULL_LAST)
        self.sparse_pat = lcs.attnsink_pattern(SINK_BLOCKS, WINDOW_BLOCKS)
        self.full_pat = lcs.full_pattern()
        t0 = time.time()
        self.ix_sparse = lcs.build_device_index(self.sparse_pat, H, L, dev, with_csc=False)
        self.ix_full = lcs.build_device_index(self.full_pat, H, L, dev, with_csc=False)
        self.index_build_s = time.time() - t0
        # distinct input sets, cycled over layers (each set 3.2 GB >> 256 MB MALL)
        self.sets = []
        for s in range(n_sets):
            self.sets.append([fill_randn((1, H, L, D), seed_for(5, s, t)) for t in ("q", "k", "v")])
        self.outs = [(torch.empty((1, H, L, D), dtype=torch.bfloat16, device=dev),
                      torch.empty((1, H, L), dtype=torch.float32, device=dev)) for _ in range(2)]
        # decode state
        B = DEC_BATCH
        self.t = L
        self.pos = torch.full((B,), self.t, dtype=torch.int64, device=dev)
        self.len0 = torch.full((1,), L, dtype=torch.int64, device=dev)
        self.q_dec = fill_randn((B, H, 1, D), seed_for(5, 0, "q_dec"))
        self.k_new = fill_randn((B, H, 1, D), seed_for(5, 0, "k_new"))
        self.v_new = fill_randn((B, H, 1, D), seed_for(5, 0, "v_new"))
        S = SINK_TOK + WINDOW_TOK
        self.rings = {}
        for layer in range(N_LAYERS):
            if not self.layer_full[layer]:
                self.rings[layer] = (fill_randn((B, H, S, D), seed_for(5, layer, "cache")),
                                     fill_randn((B, H, S, D), seed_for(5, layer, "cache_v")))
        self.cap = self.t + 1
        self.full_caches = [(fill_randn((B, H, self.cap, D), seed_for(5, 40 + c, "cache")),
                             fill_randn((B, H, self.cap, D), seed_for(5, 40 + c, "cache_v")))
                            for c in range(n_full_caches)]
        self.dec_o = torch.empty((B, H, 1, D), dtype=torch.bfloat16, device=dev)
        self.dec_lse = torch.empty((B, H), dtype=torch.float32, device=dev)
        self.ws_sparse = torch.empty(lcs.attn_workspace_bytes(lcs.ATTN_OP_SPARSE_DECODE, lcs.ATTN_BF16,
                                                              B, H, S, D), dtype=torch.uint8, device=dev)
        self.ws_full = torch.empty(lcs.attn_workspace_bytes(lcs.ATTN_OP_FULL_DECODE, lcs.ATTN_BF16,
                                                            B, H, self.cap, D), dtype=torch.uint8,
                                   device=dev)
        torch.cuda.synchronize()
        self.nnz_sparse = self.ix_sparse.host.nnz * H      # block pairs per layer
        self.nnz_full = self.ix_full.host.nnz * H

    def step(self, timer: Timer):
        L = self.L
        B = DEC_BATCH
        for layer in range(N_LAYERS):
            q, k, v = self.sets[layer % len(self.sets)]
            o, lse = self.outs[layer % 2]
            full = bool(self.layer_full[layer])
            with timer.span("prefill_full" if full else "prefill_sparse"):
                lcs.attn_sparse_fwd(q, k, v, self.ix_full if full else self.ix_sparse,
                                    self.full_pat if full else self.sparse_pat, o=o, lse=lse)
            if not full:
                # sequence 0 of this layer's decode batch continues the prefill
                rk, rv = self.rings[layer]
                with timer.span("ring_fill"):
                    lcs.attn_ring_fill(k, v, self.len0, rk[:1], rv[:1], SINK_TOK, WINDOW_TOK)
        for layer in range(N_LAYERS):
            if self.layer_full[layer]:
                kc, vc = self.full_caches[layer % len(self.full_caches)]
                with timer.span("decode_full"):
                    lcs.attn_full_decode(self.q_dec, self.k_new, self.v_new, kc, vc, self.pos,
                                         max_pos=self.t, o=self.dec_o, lse=self.dec_lse,
                                         workspace=self.ws_full)
            else:
                rk, rv = self.rings[layer]
                with timer.span("decode_sparse"):
                    lcs.attn_sparse_decode(self.q_dec, self.k_new, self.v_new, rk, rv, self.pos,
                                           SINK_TOK, WINDOW_TOK, o=self.dec_o, lse=self.dec_lse,
                                           workspace=self.ws_sparse)

    def report(self, times, steps):
        n_sparse = int((self.layer_full == 0).sum())
        n_full = int(self.layer_full.sum())
        per = lambda k: sum(times.get(k, [])) / steps            # ms per step
        fl_sparse = n_sparse * self.nnz_sparse * pair_flops()
        fl_full = n_full * self.nnz_full * pair_flops()
        t_sp, t_fu = per("prefill_sparse"), per("prefill_full")
        t_ds, t_df = per("decode_sparse"), per("decode_full")
        S = SINK_TOK + WINDOW_TOK
        # algorithmic decode bytes: every attended K and V row read once, plus q, o
        bytes_sparse = n_sparse * DEC_BATCH * H * (S * 2 * D * 2)
        bytes_full = n_full * DEC_BATCH * H * ((self.t + 1) * 2 * D * 2)
        dec_ms = t_ds + t_df
        launches_fwd = len(times.get("prefill_sparse", [])) + len(times.get("prefill_full", []))
        fwd_ms_total = sum(times.get("prefill_sparse", [])) + sum(times.get("prefill_full", []))
        flops_per_launch = (fl_sparse + fl_full) * steps / launches_fwd
        avg_ms = fwd_ms_total / launches_fwd
        achieved = flops_per_launch / (avg_ms * 1e-3) / 1e12
        return dict(
            value=fl_sparse / (t_sp * 1e-3) / 1e12,
            extra=dict(
                sparse_prefill_tflops=fl_sparse / (t_sp * 1e-3) / 1e12,
                full_prefill_tflops=fl_full / (t_fu * 1e-3) / 1e12,
                hybrid_prefill_tflops=(fl_sparse + fl_full) / ((t_sp + t_fu) * 1e-3) / 1e12,
                decode_tok_s=DEC_BATCH / (dec_ms * 1e-3),
                decode_sparse_gbps=bytes_sparse / (t_ds * 1e-3) / 1e9,
                decode_full_gbps=bytes_full / (t_df * 1e-3) / 1e9,
                decode_hbm_frac=(bytes_sparse + bytes_full) / (dec_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                ms=dict(prefill_sparse=t_sp, prefill_full=t_fu, ring_fill=per("ring_fill"),
                        decode_sparse=t_ds, decode_full=t_df),
                sparse_prefill_frac_of_peak=fl_sparse / (t_sp * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                tflop_per_step=dict(sparse=fl_sparse / 1e12, full=fl_full / 1e12),
                index_build_s=self.index_build_s,
            ),
            roofline=dict(bound="mfma", kernel="fwd_bf16_kernel<128>", achieved=achieved,
                          peak=PEAK_BF16_TFLOPS, unit="TFLOP/s", frac=achieved / PEAK_BF16_TFLOPS,
                          traffic=traffic_for(self.name), flop_per_launch=flops_per_launch,
                          avg_launch_ms=avg_ms, kernel_source_hash=kernel_source_hash()),
            config=dict(workload="hybrid128k: 32 layers (11..21 full, 21 AttnSink sink 64 + window 4096), "
                        "prefill B=1 L=131072 H=32 d=128 + decode 16 seqs at t=131072",
                        global_batch=DEC_BATCH, seq_len=self.L, layers=N_LAYERS,
                        full_layers=f"{FULL_FIRST}-{FULL_LAST}", heads=H, head_dim=D,
                        block=BLK, parallelism="single GPU",
                        input_sets=len(self.sets), full_decode_cache_buffers=len(self.full_caches)),
        )


# ----------------------------------------------------------------------------
# single-kernel workloads
# ----------------------------------------------------------------------------
class Prefill:
    def __init__(self, name, pattern, L, wl, backward=False, heads=H, d=D, dtype=torch.bfloat16):
        self.name, self.pattern, self.L, self.backward = name, pattern, L, backward
        self.H, self.d, self.dtype = heads, d, dtype
        dev = torch.device("cuda")
        self.ix = lcs.build_device_index(pattern, heads, L, dev, with_csc=backward)
        shape = (1, heads, L, d)
        self.q, self.k, self.v = (randn(shape, seed_for(wl, 0, t), dtype, "cuda") for t in ("q", "k", "v"))
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((1, heads, L), dtype=torch.float32, device=dev)
        if backward:
            self.do = randn(shape, seed_for(wl, 0, "do"), dtype, "cuda")
            self.dq, self.dk, self.dv = (torch.empty_like(self.q) for _ in range(3))
            self.ws = torch.empty(lcs.attn_workspace_bytes(lcs.ATTN_OP_BWD, lcs.ATTN_BF16, 1, heads, L, d),
                                  dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        self.pairs = self.ix.host.nnz * (heads if not pattern.head_dependent else 1)

    def fwd(self):
        lcs.attn_sparse_fwd(self.q, self.k, self.v, self.ix, self.pattern, o=self.o, lse=self.lse)

    def bwd(self):
        lcs.attn_sparse_bwd(self.q, self.k, self.v, self.o, self.lse, self.do, self.ix,
                            self.pattern, dq=self.dq, dk=self.dk, dv=self.dv, workspace=self.ws)

    def step(self, timer):
        with timer.span("fwd"):
            self.fwd()
        if self.backward:
            with timer.span("bwd"):
                self.bwd()

    def summary(self, times):
        """Per-launch medians / minima and rates from lists of per-call times
        (ms) under "fwd" and "bwd"."""
        fl = self.pairs * pair_flops(self.d)
        f = times["fwd"]
        out = dict(block_pairs=self.pairs, fwd_tflop=fl / 1e12, fwd_ms=float(np.median(f)),
                   fwd_ms_min=float(min(f)))
        out["fwd_tflops"] = fl / (out["fwd_ms"] * 1e-3) / 1e12
        out["fwd_frac_of_peak"] = out["fwd_tflops"] / PEAK_BF16_TFLOPS
        if self.backward:
            b = times["bwd"]
            out.update(bwd_tflop=2.5 * fl / 1e12, bwd_ms=float(np.median(b)), bwd_ms_min=float(min(b)))
            out["bwd_tflops"] = 2.5 * fl / (out["bwd_ms"] * 1e-3) / 1e12
            out["bwd_frac_of_peak"] = out["bwd_tflops"] / PEAK_BF16_TFLOPS
            out["step_tflops"] = 3.5 * fl / ((out["fwd_ms"] + out["bwd_ms"]) * 1e-3) / 1e12
        return out

    def describe(self):
        dt = "fp32" if self.dtype == torch.float32 else "bf16"
        return f"{self.name}: B=1 H={self.H} L={self.L} d={self.d} {dt}"

    def report(self, times, steps):
        fl = self.pairs * pair_flops(self.d)
        t_f = sum(times["fwd"]) / steps
        extra = dict(fwd_tflops=fl / (t_f * 1e-3) / 1e12, fwd_ms=t_f, block_pairs=self.pairs)
        value = extra["fwd_tflops"]
        kernel, per_launch, avg = f"fwd_bf16_kernel<{self.d}>", fl, t_f
        traffic = traffic_for(self.name)
        if self.backward:
            t_b = sum(times["bwd"]) / steps
            extra.update(bwd_tflops=2.5 * fl / (t_b * 1e-3) / 1e12, bwd_ms=t_b)
            value = 3.5 * fl / ((t_f + t_b) * 1e-3) / 1e12
            kernel, per_launch, avg = "attn_sparse_bwd (dq, then dkdv)", 2.5 * fl, t_b
            traffic = None
        ach = per_launch / (avg * 1e-3) / 1e12
        return dict(value=value, extra=extra,
                    roofline=dict(bound="mfma", kernel=kernel, achieved=ach, peak=PEAK_BF16_TFLOPS,
                                  unit="TFLOP/s", frac=ach / PEAK_BF16_TFLOPS, traffic=traffic,
                                  kernel_source_hash=kernel_source_hash()),
                    config=dict(workload=self.describe(), global_batch=1, seq_len=self.L,
                                parallelism="single GPU"))


# The five configurations of the workload definitions plus the 128K
# BlockSparse layer that the prefill target names, timed in the default run
# after the hybrid step.  Each figure is the time per call of a batch of
# back-to-back calls between one pair of hipEvents on the stream (median over
# batches): an event pair around every call adds up to about 60 us to a
# 0.4 ms launch (8K AttnSink: 0.449 ms per-call spans against 0.387 ms per
# call back to back and 0.386 ms of kernel time under rocprofv3), and nothing
# at 128K.
CONFIGS = (
    ("C1_attnsink1k_fp32", lambda: Prefill("attnsink1k_fp32", lcs.attnsink_pattern(1, 4), 1024, 1,
                                           heads=1, d=64, dtype=torch.float32)),
    ("C2_attnsink8k", lambda: Prefill("attnsink8k", lcs.attnsink_pattern(1, 64), 8192, 2)),
    ("C3_blocksparse32k", lambda: Prefill("blocksparse32k", lcs.blocksparse_pattern(1, 16, 8), 32768, 3)),
    ("C4_train64k", lambda: Prefill("train64k", lcs.attnsink_pattern(1, 64), 65536, 4, backward=True)),
    ("blocksparse128k_train", lambda: Prefill("blocksparse128k_train", lcs.blocksparse_pattern(1, 16, 8),
                                              131072, 3, backward=True)),
)


def batch_ms(call, iters, batches):
    """Per-call time (ms) of iters back-to-back calls between one event pair,
    once per batch."""
    out = []
    for _ in range(batches):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(iters):
            call()
        e.record()
        torch.cuda.synchronize()
        out.append(s.elapsed_time(e) / iters)
    return out


def config_sweep(warmup=3, iters=10, batches=5, names=None):
    """Times every configuration in CONFIGS (warmup untimed steps, then
    batches of iters back-to-back forward calls, and of backward calls where
    the configuration trains); returns {name: summary}."""
    out = {}
    for name, make in CONFIGS:
        if names and name not in names:
            continue
        log(f"[bench] config {name}")
        wl = make()
        for _ in range(warmup):
            wl.fwd()
            if wl.backward:
                wl.bwd()
        torch.cuda.synchronize()
        times = {"fwd": batch_ms(wl.fwd, iters, batches)}
        if wl.backward:
            times["bwd"] = batch_ms(wl.bwd, iters, batches)
        rep = wl.summary(times)
        rep["workload"] = wl.describe()
        rep["iters"] = iters
        rep["batches"] = batches
        if wl.dtype == torch.float32:
            # 73 MFLOP in 64 small workgroups: bound by launch latency, not by a roofline
            rep["bound"] = "launch"
            rep.pop("fwd_frac_of_peak")
        out[name] = rep
        del wl
        torch.cuda.empty_cache()
    return out


class Copy1G:
    """Calibration: one elementwise kernel that reads 1 GiB and writes 1 GiB."""
    name = "copy1g"
    BYTES = 1 << 30

    def __init__(self):
        self.src = torch.ones(self.BYTES // 2, dtype=torch.bfloat16, device="cuda")
        self.dst = torch.empty_like(self.src)
        torch.cuda.synchronize()

    def step(self, timer):
        with timer.span("copy"):
            torch.neg(self.src, out=self.dst)

    def report(self, times, steps):
        t = sum(times["copy"]) / steps
        gbps = 2 * self.BYTES / (t * 1e-3) / 1e9
        return dict(value=gbps, extra=dict(copy_ms=t, bytes_read=self.BYTES, bytes_written=self.BYTES),
                    roofline=dict(bound="hbm", kernel="torch neg (elementwise copy)", achieved=gbps,
                                  peak=PEAK_HBM_GBPS, unit="GB/s", frac=gbps / PEAK_HBM_GBPS,
                                  traffic=None),
                    config=dict(workload="copy1g: read 1 GiB, write 1 GiB", global_batch=1,
                                parallelism="single GPU"))


class BsDecode128k:
    """Decode of 16 sequences at t = 131072 in a BlockSparse layer (sink 1,
    local 16, stride 8 blocks) against its compacted cache, cycling over
    distinct layer caches so that no read hits the 256 MB MALL."""
    name = "bsdecode128k"

    def __init__(self, n_layers=4):
        dev = torch.device("cuda")
        self.pat = lcs.blocksparse_pattern(1, 16, 8)
        self.t = 131072
        B = DEC_BATCH
        self.cap_blocks = lcs.blocksparse_strided_capacity(self.pat, self.t + 1)
        S = lcs.blocksparse_cache_slots(self.pat, self.cap_blocks)
        self.S = S
        self.pos = torch.full((B,), self.t, dtype=torch.int64, device=dev)
        self.q = fill_randn((B, H, 1, D), seed_for(6, 0, "q_dec"))
        self.k_new = fill_randn((B, H, 1, D), seed_for(6, 0, "k_new"))
        self.v_new = fill_randn((B, H, 1, D), seed_for(6, 0, "v_new"))
        self.caches = [(fill_randn((B, H, S, D), seed_for(6, layer, "cache")),
                        fill_randn((B, H, S, D), seed_for(6, layer, "cache_v")))
                       for layer in range(n_layers)]
        self.o = torch.empty((B, H, 1, D), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((B, H), dtype=torch.float32, device=dev)
        self.ws = torch.empty(lcs.attn_workspace_bytes(lcs.ATTN_OP_BLOCKSPARSE_DECODE, lcs.ATTN_BF16,
                                                       B, H, S, D), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        # keys each (b, h) attends: sink block, the 16 window blocks up to t
        # (the newest holding t % 64 + 1 tokens) and the strided blocks of
        # head h that left the window
        i = self.t // BLK
        s, w, st = self.pat.sink_blocks, self.pat.local_blocks, self.pat.stride
        first = i - w + 1
        keys = 0
        for h in range(H):
            strided = sum(1 for j in range(s, first) if (j + h) % st == 0)
            keys += BLK * (s + w - 1 + strided) + self.t % BLK + 1
        self.keys_per_seq = keys                     # summed over heads

    def step(self, timer):
        for kc, vc in self.caches:
            with timer.span("decode_bs"):
                lcs.attn_blocksparse_decode(self.q, self.k_new, self.v_new, kc, vc, self.pos, self.pat,
                                            self.cap_blocks, o=self.o, lse=self.lse, workspace=self.ws)

    def report(self, times, steps):
        t = sum(times["decode_bs"]) / len(times["decode_bs"])        # ms per layer
        nbytes = DEC_BATCH * self.keys_per_seq * 2 * D * 2
        gbps = nbytes / (t * 1e-3) / 1e9
        return dict(value=DEC_BATCH / (t * 1e-3), unit="tok/s (one layer)",
                    extra=dict(layer_ms=t, layer_gbps=gbps, attended_bytes=nbytes,
                               cache_slots=self.S, strided_capacity_blocks=self.cap_blocks),
                    roofline=dict(bound="hbm", kernel="bs_move_kernel + decode_split_kernel + "
                                  "decode_combine_kernel", achieved=gbps, peak=PEAK_HBM_GBPS,
                                  unit="GB/s", frac=gbps / PEAK_HBM_GBPS, traffic=None),
                    config=dict(workload="bsdecode128k: BlockSparse (sink 1, local 16, stride 8 "
                                "blocks) decode of 16 seqs at t=131072, H=32 d=128 bf16, compacted "
                                f"cache {self.S} slots", global_batch=DEC_BATCH, seq_len=self.t,
                                parallelism="single GPU", layer_caches=len(self.caches)))


class PagedDecode128k:
    """Full-layer decode of 16 sequences at t = 131072 against paged caches:
    pools of 16 x 2049 64-token pages in shuffled order, cycled over two
    distinct pools so that no read hits the 256 MB MALL."""
    name = "pageddecode128k"

    def __init__(self, n_pools=2):
        dev = torch.device("cuda")
        B = DEC_BATCH
        self.t = 131072
        self.max_pages = self.t // BLK + 1
        n_pages = B * self.max_pages
        g = torch.Generator().manual_seed(seed_for(8, 0, "cache"))
        self.table = torch.randperm(n_pages, generator=g).to(torch.int32).reshape(B, self.max_pages).to(dev)
        self.pos = torch.full((B,), self.t, dtype=torch.int64, device=dev)
        self.q = fill_randn((B, H, 1, D), seed_for(8, 0, "q_dec"))
        self.k_new = fill_randn((B, H, 1, D), seed_for(8, 0, "k_new"))
        self.v_new = fill_randn((B, H, 1, D), seed_for(8, 0, "v_new"))
        self.pools = [(fill_randn((n_pages, H, BLK, D), seed_for(8, 10 + i, "cache")),
                       fill_randn((n_pages, H, BLK, D), seed_for(8, 10 + i, "cache_v")))
                      for i in range(n_pools)]
        self.o = torch.empty((B, H, 1, D), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((B, H), dtype=torch.float32, device=dev)
        self.ws = torch.empty(lcs.attn_workspace_bytes(lcs.ATTN_OP_FULL_DECODE, lcs.ATTN_BF16, B, H,
                                                       self.t + 1, D), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

    def step(self, timer):
        for kp, vp in self.pools:
            with timer.span("decode_paged"):
                lcs.attn_paged_decode(self.q, self.k_new, self.v_new, kp, vp, self.table, self.pos,
                                      max_pos=self.t, o=self.o, lse=self.lse, workspace=self.ws)

    def report(self, times, steps):
        t = sum(times["decode_paged"]) / len(times["decode_paged"])
        nbytes = DEC_BATCH * H * (self.t + 1) * 2 * D * 2
        gbps = nbytes / (t * 1e-3) / 1e9
        return dict(value=DEC_BATCH / (t * 1e-3), unit="tok/s (one layer)",
                    extra=dict(layer_ms=t, layer_gbps=gbps, attended_bytes=nbytes),
                    roofline=dict(bound="hbm", kernel="decode_split_kernel (paged) + decode_combine_kernel",
                                  achieved=gbps, peak=PEAK_HBM_GBPS, unit="GB/s", frac=gbps / PEAK_HBM_GBPS,
                                  traffic=None),
                    config=dict(workload="pageddecode128k: full-layer decode of 16 seqs at t=131072, "
                                "H=32 d=128 bf16, 64-token pages in shuffled order",
                                global_batch=DEC_BATCH, seq_len=self.t, parallelism="single GPU",
                                pools=len(self.pools)))


def make_workload(name):
    if name == "hybrid128k":
        return Hybrid128k()
    if name == "attnsink8k":
        return Prefill(name, lcs.attnsink_pattern(1, 64), 8192, 2)
    if name == "blocksparse32k":
        return Prefill(name, lcs.blocksparse_pattern(1, 16, 8), 32768, 3)
    if name == "blocksparse128k":
        return Prefill(name, lcs.blocksparse_pattern(1, 16, 8), 131072, 3)
    if name == "attnsink128k":
        return Prefill(name, lcs.attnsink_pattern(1, 64), 131072, 5)
    if name == "full128k":
        return Prefill(name, lcs.full_pattern(), 131072, 5)
    if name == "train64k":
        return Prefill(name, lcs.attnsink_pattern(1, 64), 65536, 4, backward=True)
    if name == "blocksparse32k_train":
        return Prefill(name, lcs.blocksparse_pattern(1, 16, 8), 32768, 3, backward=True)
    if name == "blocksparse128k_train":
        return Prefill(name, lcs.blocksparse_pattern(1, 16, 8), 131072, 3, backward=True)
    if name == "sliding128k":
        return Prefill(name, lcs.sliding_pattern(1, 4096), 131072, 7)
    if name == "sliding64k_train":
        return Prefill(name, lcs.sliding_pattern(1, 4096), 65536, 4, backward=True)
    if name == "bsdecode128k":
        return BsDecode128k()
    if name == "pageddecode128k":
        return PagedDecode128k()
    if name == "copy1g":
        return Copy1G()
    raise SystemExit(f"unknown workload {name}")


# ----------------------------------------------------------------------------
# CPU oracle baseline (bounded sample of the same workload)
# ----------------------------------------------------------------------------
def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return None


def _oracle_pattern(p):
    kind = {lcs.ATTN_FULL: "full", lcs.ATTN_ATTNSINK: "attnsink", lcs.ATTN_BLOCKSPARSE: "blocksparse",
            lcs.ATTN_SLIDING: "sliding"}[p.kind]
    return dict(kind=kind, block=p.block, sink_blocks=p.sink_blocks, local_blocks=p.local_blocks,
                stride=p.stride, causal=p.causal, window_tokens=p.window_tokens)


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def _host_head(L, d, seed, dtype):
    """One head's Q, K, V (and dO) generated on the host with the seed
    recipe, rounded to the workload's dtype."""
    g = torch.Generator().manual_seed(seed)
    return [torch.randn((1, 1, L, d), generator=g).to(dtype) for _ in range(4)]


def cpu_baseline(spec, budget_s=15.0):
    """Times the oracle, as it stands, on a bounded sample of the benched
    workload on the host cores, scaled to the workload's unit:
      prefill: random query rows of one head (float64 dense-masked rows),
               effective TFLOP/s over the computed blocks of those rows; the
               same rows of the GPU forward of that head are compared with
               the oracle's and the errors reported beside the rate;
      train:   random query blocks of one head, forward + backward of each
               block's exact sub-problem, TFLOP/s at 3.5x the forward count;
      decode:  random heads of one sequence at the benched position, tok/s
               of one layer (the time for all heads of one token)."""
    import oracle
    threads = _blas_threads()
    rng = np.random.default_rng(0)
    common = dict(kind="oracle", cores=threads, affinity_cpus=len(os.sched_getaffinity(0)),
                  cpu_model=cpu_model(), blas_threads=threads)

    def extrapolated(rate_tflops):
        # the benched work at the sampled rate, linear in its FLOPs (not run)
        if "work_tflop" not in spec or rate_tflops <= 0:
            return {}
        return dict(extrapolated_s=spec["work_tflop"] / rate_tflops,
                    extrapolated=f"{spec['work']} ({spec['work_tflop']:.1f} TFLOP) at the sampled rate, "
                                 "linear in FLOPs; not run")
    kind = spec["kind"]
    if kind in ("prefill", "train"):
        pat, L, d, dtype = spec["pattern"], spec["L"], spec.get("d", D), spec.get("dtype", torch.bfloat16)
        opat = _oracle_pattern(pat)
        qt, kt, vt, dot = _host_head(L, d, spec["seed"], dtype)
        q, k, v, do = (x[0, 0].double().numpy() for x in (qt, kt, vt, dot))
        host_ix = lcs.attn_index_build(pat, 1, L, with_csc=False)
        row_len = np.diff(host_ix.row_ptr[:L // BLK + 1])           # listed blocks per query block
        scale = 1.0 / math.sqrt(d)
        t_used, flops, n_done = 0.0, 0.0, 0
        if kind == "prefill":
            gpat = pat
            gq, gk, gv = (x.cuda() for x in (qt, kt, vt))
            ix = lcs.build_device_index(gpat, 1, L, gq.device, with_csc=False)
            go, glse = lcs.attn_sparse_fwd(gq, gk, gv, ix, gpat)
            go, glse = go[0, 0].double().cpu().numpy(), glse[0, 0].double().cpu().numpy()
            err_o = err_l = err_sum = 0.0
            n_el = 0
            t0 = time.perf_counter()
            lists = oracle.pattern_lists_for_head(opat, L // BLK, 0)     # the head's block lists, once
            t_used += time.perf_counter() - t0
            lo = min(L - 64, WINDOW_BLOCKS * BLK)
            while t_used < budget_s and n_done < 65536:
                rows = np.sort(rng.choice(np.arange(lo, L), size=64, replace=False))
                t0 = time.perf_counter()
                mask = oracle.pattern_token_mask(opat, 0, L, rows=rows, lists=lists)
                o, lse = oracle.attention_forward(q[rows], k, v, mask, scale)
                t_used += time.perf_counter() - t0
                d_o = np.abs(go[rows] - o)
                err_o = max(err_o, float(d_o.max()))
                err_l = max(err_l, float(np.abs(glse[rows] - lse).max()))
                err_sum += float(d_o.sum())
                n_el += d_o.size
                n_done += len(rows)
                flops += float(row_len[rows // BLK].sum()) / BLK * pair_flops(d)
            return dict(value=flops / t_used / 1e12, unit="TFLOP/s", **common,
                        sample=f"{n_done} query rows (random, past the first window) of one head of "
                               f"{spec['what']}, float64 dense-masked NumPy; {t_used:.1f} s",
                        sample_s=t_used, **extrapolated(flops / t_used / 1e12),
                        parity_vs_gpu=dict(rows=n_done, o_max_abs=err_o, o_mean_abs=err_sum / max(n_el, 1),
                                           lse_max_abs=err_l, tolerance="max 2e-2, mean 2e-3"))
        t0 = time.perf_counter()
        lists = oracle.pattern_lists_for_head(opat, L // BLK, 0)         # the head's block lists, once
        t_used += time.perf_counter() - t0
        blocks = rng.permutation(np.arange(WINDOW_BLOCKS, L // BLK))
        for i in blocks:
            if t_used >= budget_s or n_done >= 4096:
                break
            rows = np.arange(i * BLK, (i + 1) * BLK)
            keys = np.concatenate([np.arange(j * BLK, (j + 1) * BLK) for j in lists[i]])
            t0 = time.perf_counter()
            mask = oracle.pattern_token_mask(opat, 0, L, rows=rows, lists=lists)[:, keys]
            oracle.attention_backward(q[rows], k[keys], v[keys], do[rows], mask, scale)
            t_used += time.perf_counter() - t0
            n_done += 1
            flops += 3.5 * len(lists[i]) * pair_flops(d)
        return dict(value=flops / t_used / 1e12, unit="TFLOP/s", **common,
                    sample=f"{n_done} query blocks (random, past the first window) of one head of "
                           f"{spec['what']}: forward + backward of each block's exact sub-problem, "
                           f"float64 NumPy; {t_used:.1f} s",
                    sample_s=t_used, **extrapolated(flops / t_used / 1e12))
    if kind == "decode":
        t, d = spec["t"], D
        g = torch.Generator().manual_seed(spec["seed"])
        t_used, n_heads = 0.0, 0
        while t_used < budget_s and n_heads < 4 * H:
            h = int(rng.integers(0, H))
            kh = torch.randn((t + 1, d), generator=g).to(torch.bfloat16).double().numpy()
            vh = torch.randn((t + 1, d), generator=g).to(torch.bfloat16).double().numpy()
            qh = torch.randn((d,), generator=g).to(torch.bfloat16).double().numpy()
            t0 = time.perf_counter()
            keep = spec["positions"](t, h)
            oracle.decode_one(qh, kh, vh, keep, 1.0 / math.sqrt(d))
            t_used += time.perf_counter() - t0
            n_heads += 1
        return dict(value=(n_heads / H) / t_used, unit="tok/s (one layer)", **common,
                    sample=f"{n_heads} heads (random) of one sequence at t={t} in {spec['what']}, "
                           f"float64 NumPy over the token positions the token reads; {t_used:.1f} s")
    return None


def baseline_spec(name, wl):
    """What the CPU baseline samples for a benched workload (None: no
    oracle counterpart)."""
    import oracle
    if name == "hybrid128k":
        return dict(kind="prefill", pattern=lcs.attnsink_pattern(SINK_BLOCKS, WINDOW_BLOCKS), L=131072,
                    seed=seed_for(5, 0, "q"), what="one 128K AttnSink layer (the metric's sparse prefill)",
                    work_tflop=(N_LAYERS - (FULL_LAST - FULL_FIRST + 1)) * wl.nnz_sparse * pair_flops() / 1e12,
                    work="the step's 21 sparse prefill layers")
    if isinstance(wl, Prefill):
        fl = wl.pairs * pair_flops(wl.d) / 1e12
        return dict(kind="train" if wl.backward else "prefill", pattern=wl.pattern, L=wl.L, d=wl.d,
                    dtype=wl.dtype, seed=seed_for(9, 0, "q"), what=wl.describe(),
                    work_tflop=3.5 * fl if wl.backward else fl, work="one step of the workload")
    if name == "bsdecode128k":
        opat = _oracle_pattern(wl.pat)
        return dict(kind="decode", t=wl.t, seed=seed_for(6, 0, "cache"), what="a BlockSparse layer",
                    positions=lambda t, h: oracle.blocksparse_decode_positions(t, opat, h))
    if name == "pageddecode128k":
        return dict(kind="decode", t=wl.t, seed=seed_for(8, 0, "cache"), what="a full layer",
                    positions=lambda t, h: oracle.decode_positions(t))
    return None


# ----------------------------------------------------------------------------
# rocprofv3 CSV summaries (the text kept next to the measurements)
# ----------------------------------------------------------------------------
def _short(name, width=72):
    name = name.replace("(anonymous namespace)::", "")
    return name if len(name) <= width else name[:width - 3] + "..."


def summarize_stats(path, top=12):
    import csv
    rows = list(csv.DictReader(open(path)))
    out = [f"{'kernel':72s} {'calls':>6s} {'total ms':>10s} {'avg ms':>10s} {'min ms':>9s} "
           f"{'max ms':>9s} {'%':>6s}"]
    for r in rows[:top]:
        out.append(f"{_short(r['Name']):72s} {int(r['Calls']):6d} {float(r['TotalDurationNs']) / 1e6:10.3f} "
                   f"{float(r['AverageNs']) / 1e6:10.4f} {float(r['MinNs']) / 1e6:9.4f} "
                   f"{float(r['MaxNs']) / 1e6:9.4f} {float(r['Percentage']):6.2f}")
    return "\n".join(out)


def _counter_means(path, counter):
    import csv
    acc = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return acc


N_XCD, N_SIMD = 8, 1024   # MI355X: 8 XCDs, 256 CUs x 4 SIMDs


def summarize_mfma(path):
    """Per attention kernel, from one rocprofv3 --pmc run with
    SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE (optionally also
    SQ_ACTIVE_INST_VALU and SQ_VALU_MFMA_COEXEC_CYCLES): the matrix-core busy
    fraction (busy cycles summed over SIMDs / (GPU-active cycles of one XCD x
    SIMDs), the profiler's own MfmaUtil), the clock the kernel ran at
    (GPU-active cycles of one XCD / dispatch time), and -- when present --
    the fraction of SIMD cycles with a vector instruction at work
    (SQ_ACTIVE_INST_VALU counts quad-cycles) and the share of those cycles
    issued while the matrix core was busy (co-issue), averaged over
    dispatches."""
    import csv
    per = {}
    for r in csv.DictReader(open(path)):
        if "attn::" not in r["Kernel_Name"]:
            continue
        key = (r["Kernel_Name"], r["Dispatch_Id"])
        d = per.setdefault(key, {"ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    acc = {}
    extra = False
    for (name, _), d in per.items():
        if "SQ_VALU_MFMA_BUSY_CYCLES" not in d or "GRBM_GUI_ACTIVE" not in d:
            continue
        active = d["GRBM_GUI_ACTIVE"] / N_XCD
        row = [d["SQ_VALU_MFMA_BUSY_CYCLES"] / (active * N_SIMD), active / d["ns"], d["ns"] / 1e6]
        if "SQ_ACTIVE_INST_VALU" in d and "SQ_VALU_MFMA_COEXEC_CYCLES" in d:
            valu = 4 * d["SQ_ACTIVE_INST_VALU"]
            row += [valu / (active * N_SIMD), d["SQ_VALU_MFMA_COEXEC_CYCLES"] / valu if valu else 0.0]
            extra = True
        acc.setdefault(name, []).append(row)
    head = f"{'kernel':72s} {'n':>3s} {'avg ms':>8s} {'MFMA busy':>10s} {'clock GHz':>10s}"
    out = [head + (f" {'VALU active':>12s} {'co-issued':>10s}" if extra else "")]
    for name, v in sorted(acc.items(), key=lambda kv: -sum(x[2] for x in kv[1])):
        cols = [sum(x[i] for x in v) / len(v) for i in range(len(v[0]))]
        line = f"{_short(name):72s} {len(v):3d} {cols[2]:8.3f} {100 * cols[0]:9.1f}% {cols[1]:10.3f}"
        if len(cols) > 3:
            line += f" {100 * cols[3]:11.1f}% {100 * cols[4]:9.1f}%"
        out.append(line)
    return "\n".join(out)


def summarize_counters(paths):
    """Per attention kernel, from one or more rocprofv3 --pmc runs of the same
    command: every counter averaged over dispatches and, where a run also
    counted SQ_WAVES, divided by the waves of a dispatch (per-wave figures;
    the SQ_*_CYCLES and SQ_ACTIVE_* / SQ_WAIT_* counters are in quad-cycles)."""
    import csv
    sums = {}
    for path in paths:
        per = {}
        for r in csv.DictReader(open(path)):
            if "attn::" not in r["Kernel_Name"]:
                continue
            per.setdefault((r["Kernel_Name"], r["Dispatch_Id"]), {})[r["Counter_Name"]] = float(r["Counter_Value"])
        for (name, _), d in per.items():
            k = sums.setdefault(name, {})
            for c, x in d.items():
                k.setdefault(c, []).append(x)
    out = []
    for name, k in sorted(sums.items()):
        avg = {c: sum(v) / len(v) for c, v in k.items()}
        waves = avg.get("SQ_WAVES")
        out.append(_short(name))
        out.append(f"  {'counter':28s} {'per dispatch':>14s} {'per wave':>12s}")
        for c in sorted(avg):
            per_wave = f"{avg[c] / waves:12.1f}" if waves and c.startswith("SQ_") and c != "SQ_WAVES" else f"{'':12s}"
            out.append(f"  {c:28s} {avg[c]:14.5g} {per_wave}")
    return "\n".join(out)


def summarize_traffic(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) per kernel, scaled so that
    the copy1g kernel reads 1 GiB and writes 1 GiB."""
    cf = _counter_means(copy_fetch_csv, "FETCH_SIZE")
    cw = _counter_means(copy_write_csv, "WRITE_SIZE")
    neg = lambda d: max(d.items(), key=lambda kv: len(kv[1]))[1]   # the repeated copy kernel
    copy_kib = Copy1G.BYTES / 1024
    f_copy, w_copy = np.median(neg(cf)), np.median(neg(cw))
    kf, kw = copy_kib / f_copy, copy_kib / w_copy
    fe = _counter_means(fetch_csv, "FETCH_SIZE")
    wr = _counter_means(write_csv, "WRITE_SIZE")
    out = [f"calibration (copy1g, 1 GiB read + 1 GiB written): FETCH_SIZE {f_copy:.0f} KiB -> factor {kf:.4f}; "
           f"WRITE_SIZE {w_copy:.0f} KiB -> factor {kw:.4f}",
           f"{'kernel':72s} {'n':>4s} {'fetch KiB':>12s} {'write KiB':>12s} {'scaled GB/launch':>17s}"]
    per_kernel = {}
    for name in fe:
        if name not in wr or not name.startswith("void attn::"):
            continue
        f, w = float(np.mean(fe[name])), float(np.mean(wr[name]))
        gb = (f * kf + w * kw) * 1024 / 1e9
        per_kernel[name] = gb
        out.append(f"{_short(name):72s} {len(fe[name]):4d} {f:12.0f} {w:12.0f} {gb:17.3f}")
    return "\n".join(out), per_kernel


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="hybrid128k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="hybrid128k: skip timing the other configurations after the step")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--summarize-stats", metavar="KERNEL_STATS_CSV",
                    help="print a summary of a rocprofv3 --stats kernel_stats.csv and exit")
    ap.add_argument("--summarize-mfma", metavar="COUNTER_CSV",
                    help="print matrix-core busy fraction and clock per attention kernel from a "
                         "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE "
                         "counter_collection.csv, and exit")
    ap.add_argument("--summarize-counters", nargs="+", metavar="COUNTER_CSV",
                    help="print per-kernel counter averages (and per-wave figures) of rocprofv3 --pmc runs")
    ap.add_argument("--summarize-traffic", nargs=4,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="print per-kernel HBM bytes from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE "
                         "counter_collection.csv files of a workload and of copy1g, and exit")
    args = ap.parse_args()
    if args.summarize_stats:
        print(summarize_stats(args.summarize_stats))
        return
    if args.summarize_counters:
        print(summarize_counters(args.summarize_counters))
        return
    if args.summarize_mfma:
        print(summarize_mfma(args.summarize_mfma))
        return
    if args.summarize_traffic:
        print(summarize_traffic(*args.summarize_traffic)[0])
        return
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU; --gpus must be 1"}))
        raise SystemExit(2)
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    lcs.lib()
    log(f"[bench] setting up {args.workload}")
    wl = make_workload(args.workload)
    timer = Timer()
    for i in range(args.warmup):
        wl.step(timer)
        timer.collect()
        log(f"[bench] warmup {i + 1}/{args.warmup} done")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        wl.step(timer)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    times = timer.collect()
    log(f"[bench] timed {args.steps} steps in {wall:.2f} s")
    rep = wl.report(times, args.steps)
    spec = None if args.no_cpu_baseline else baseline_spec(args.workload, wl)
    del wl
    torch.cuda.empty_cache()
    configs = None
    if args.workload == "hybrid128k" and not args.no_configs:
        configs = config_sweep()
    line = {
        "metric": "effective TFLOP/s (computed blocks) sparse prefill @128K; decode tok/s",
        "value": rep["value"],
        "unit": rep.get("unit", "TFLOP/s"),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": rep["config"],
        "roofline": rep["roofline"],
        **rep["extra"],
        # every timed span (one launch of an op, or one layer's launches) by label
        "span_ms": {k: {"n": len(v), "median": float(np.median(v)), "min": float(min(v))}
                    for k, v in sorted(times.items())},
    }
    if configs is not None:
        # every configuration of the workload definitions, timed in this run
        line["configs"] = configs
    if spec is not None:
        log("[bench] timing the CPU oracle baseline")
        line["cpu_baseline"] = cpu_baseline(spec, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
