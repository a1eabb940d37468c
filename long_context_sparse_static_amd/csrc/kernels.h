// Internal launcher interface between the C ABI (api.cpp) and the HIP kernels.
// Every launcher assumes its arguments were validated by the ABI layer and
// returns a hipError_t from the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

constexpr int kBlock = 64;   // tokens per sparse block (the only size built)
constexpr int kNumXcd = 8;   // MI355X: 8 XCDs, workgroups dealt round-robin

struct IndexView {
  const int32_t *row_ptr;
  const int32_t *col_idx;
  const int32_t *col_ptr;
  const int32_t *row_idx;
  int32_t n_heads;     // 1 (broadcast) or H
  int32_t n_qblocks;
  int32_t n_kblocks;
  int32_t nnz;
};

// Element strides of one tensor indexed [b, h, l, e] (the d elements e of a
// token row are contiguous): element (b, h, l, e) sits at
// b * s.b + h * s.h + l * s.l + e.  Contiguous [B,H,L,d]: {H L d, L d, d};
// [B,L,H,d]: {L H d, d, H d}.
struct Strides {
  int64_t b, h;
  int32_t l;
  __host__ __device__ __forceinline__ size_t at(int bb, int hh) const {
    return (size_t)bb * b + (size_t)hh * h;
  }
};

// Whether s is the contiguous [B,H,L,d] layout.
inline bool dense_layout(const Strides &s, int32_t H, int32_t L, int32_t d) {
  return s.l == d && s.h == (int64_t)L * d && s.b == (int64_t)H * L * d;
}

struct FwdArgs {
  const void *q, *k, *v;
  void *o;
  float *lse;            // [B,H,L] contiguous
  Strides qs, ks, vs, os;
  IndexView ix;
  int32_t B, H, L, d;
  float scale;
  int32_t causal;
  // Token window (Sliding patterns; window 0: none): key k of a block
  // j >= sink_blk is masked for query q when k <= q - window.
  int32_t window, sink_blk;
};

struct BwdArgs {
  const void *q, *k, *v, *o, *dout;
  const float *lse;
  void *dq, *dk, *dv;
  Strides qs, ks, vs, os, dos, dqs, dks, dvs;
  float *delta;        // workspace: -D = -rowsum(dO * O), [B,H,L] fp32
  float *lse2;         // workspace: LSE * log2(e) (+inf for empty rows), [B,H,L] fp32
  IndexView ix;
  int32_t B, H, L, d;
  float scale;
  int32_t causal;
  int32_t window, sink_blk;  // token window, as in FwdArgs
  int32_t kgroup;      // dK/dV key-block grouping: 1, or the BlockSparse stride
};

struct DecodeArgs {
  const void *q, *k_new, *v_new;
  void *k_cache, *v_cache;
  void *o;
  float *lse;
  const int64_t *pos;
  float *part;         // workspace: [B*H, n_split, d + 2] fp32 partials
  int32_t B, H, d;
  int64_t cap;         // slots per (b, h) in the cache
  int32_t sink, window;  // sparse layers; sink < 0 marks a full layer
  int64_t max_pos;     // full layers: host bound on positions
  int32_t n_split, split_len;
  float scale;
  // BlockSparse layers (bs_stride > 0): compacted cache of bs_sink sink
  // blocks, a ring of bs_local blocks and bs_cap strided blocks; sink and
  // window are unused then.
  int32_t bs_sink, bs_local, bs_stride, bs_cap;
  // Paged full layers (table != nullptr): k_cache / v_cache are page pools
  // [n_pages, H, 64, d]; logical block j of sequence b lives in page
  // table[b * max_pages + j].  cap is unused then.
  const int32_t *table;
  int32_t max_pages, n_pages;
};

struct RingFillArgs {
  const void *k_src, *v_src;
  void *k_cache, *v_cache;
  const int64_t *len;
  int64_t src_len;
  int32_t B, H, d, sink, window;
};

hipError_t launch_fwd_bf16(const FwdArgs &a, hipStream_t s);
hipError_t launch_fwd_f32(const FwdArgs &a, hipStream_t s);
hipError_t launch_bwd_bf16(const BwdArgs &a, hipStream_t s);
hipError_t launch_decode_bf16(const DecodeArgs &a, hipStream_t s);
hipError_t launch_ring_fill_bf16(const RingFillArgs &a, hipStream_t s);

// Fill of a BlockSparse compacted cache from prefill K/V: the state decode
// would have reached after appending tokens 0 .. len-1.
struct BsFillArgs {
  const void *k_src, *v_src;
  void *k_cache, *v_cache;
  const int64_t *len;
  int64_t src_len;
  int32_t B, H, d;
  int32_t sink, local, stride, cap;  // blocks
};
hipError_t launch_bs_fill_bf16(const BsFillArgs &a, hipStream_t s);

// Fill of a page pool from prefill K/V [B,H,src_len,d]: tokens 0 .. len-1
// of sequence b into the pages its block table names.
struct PagedFillArgs {
  const void *k_src, *v_src;
  void *k_pages, *v_pages;
  const int32_t *table;
  const int64_t *len;
  int64_t src_len;
  int32_t B, H, d, max_pages, n_pages;
};
hipError_t launch_paged_fill_bf16(const PagedFillArgs &a, hipStream_t s);

// LDS bytes one forward workgroup needs (static tiles + union bitmap).
size_t fwd_bf16_lds_bytes(int d, int n_kblocks);
size_t bwd_bf16_lds_bytes(int d, int n_blocks);  // the larger (dK/dV) backward kernel
constexpr size_t kMaxLdsPerWorkgroup = 160 * 1024;

// Size of the fixed per-device decode scratch (split-KV partials of
// attn_full_decode_noalloc): B*H*n_split*(d+2) floats must fit.
constexpr size_t kDecodeScratchBytes = 8u << 20;
// Device address of the current device's decode scratch (looked up once per
// device, then cached).
hipError_t decode_scratch(void **ptr);

// Split-KV sizing shared by the workspace query and the decode launcher.
void decode_split_plan(int32_t B, int32_t H, int64_t n_keys, int32_t *n_split,
                       int32_t *split_len);
// Upper bound of decode_split_plan's n_split over all key counts <= n_keys.
int32_t decode_split_bound(int32_t B, int32_t H, int64_t n_keys);

}  // namespace attn
