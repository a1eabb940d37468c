// C ABI entry points: synchronous argument checks, then dispatch to the HIP
// launchers.  Nothing is enqueued when a check fails.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/attn_sparse.h"
#include "kernels.h"

namespace {

using attn::IndexView;

bool index_shape_ok(const attn_index_t *ix, int32_t H, int64_t L, bool need_csc) {
  if (!ix || !ix->row_ptr || !ix->col_idx) return false;
  if (ix->n_heads != 1 && ix->n_heads != H) return false;
  const int64_t nb = (L + attn::kBlock - 1) / attn::kBlock;   // the last block may be partial
  if (ix->n_qblocks != nb || ix->n_kblocks != nb) return false;
  if (ix->nnz < 0 || ix->nnz > INT32_MAX) return false;
  if (need_csc && (!ix->col_ptr || !ix->row_idx)) return false;
  return true;
}

IndexView view_of(const attn_index_t *ix) {
  IndexView v;
  v.row_ptr = ix->row_ptr;
  v.col_idx = ix->col_idx;
  v.col_ptr = ix->col_ptr;
  v.row_idx = ix->row_idx;
  v.n_heads = ix->n_heads;
  v.n_qblocks = ix->n_qblocks;
  v.n_kblocks = ix->n_kblocks;
  v.nnz = (int32_t)ix->nnz;
  return v;
}

bool prefill_dims_ok(int32_t B, int32_t H, int64_t L, int32_t d, float scale,
                     const attn_pattern_t *p) {
  if (B < 1 || H < 1 || L < 1) return false;
  if (!p || p->block != attn::kBlock) return false;
  if (p->kind == ATTN_SLIDING && (p->window_tokens < 1 || p->sink_blocks < 0 || !p->causal))
    return false;
  if (!(scale > 0.f) || !isfinite(scale)) return false;
  // int32 token / tile arithmetic inside the kernels (over whole blocks)
  const int64_t Lb = (L + attn::kBlock - 1) / attn::kBlock * attn::kBlock;
  if ((int64_t)B * H * Lb > INT32_MAX) return false;
  (void)d;
  return true;
}

attn_status_t hip_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

// Token window of a Sliding pattern (window 0: none).
void window_of(const attn_pattern_t *p, int32_t *window, int32_t *sink_blk) {
  const bool sl = p->kind == ATTN_SLIDING;
  *window = sl ? p->window_tokens : 0;
  *sink_blk = sl ? p->sink_blocks : 0;
}

size_t decode_ws_bytes(int32_t B, int32_t H, int64_t n_keys, int32_t d) {
  return (size_t)B * H * attn::decode_split_bound(B, H, n_keys) * (d + 2) * sizeof(float);
}

}  // namespace

extern "C" {

size_t attn_workspace_bytes(int32_t op, attn_dtype_t dtype, int32_t B, int32_t H,
                            int64_t L_or_cap, int32_t d) {
  (void)dtype;
  if (B < 1 || H < 1 || L_or_cap < 1 || d < 1) return 0;
  switch (op) {
    case ATTN_OP_FWD: return 0;
    case ATTN_OP_BWD: return 2 * (size_t)B * H * L_or_cap * sizeof(float);  // D, LSE2
    case ATTN_OP_SPARSE_DECODE:
    case ATTN_OP_FULL_DECODE:
    case ATTN_OP_BLOCKSPARSE_DECODE: return decode_ws_bytes(B, H, L_or_cap, d);
  }
  return 0;
}

}  // extern "C"

namespace {

// Contiguous [B,H,L,d] strides.
attn_strides_t dense_strides(int32_t H, int64_t L, int32_t d) {
  attn_strides_t s;
  s.token = d;
  s.head = L * d;
  s.batch = (int64_t)H * L * d;
  return s;
}

// Strides the kernels can address: non-negative, whole 16-byte vectors
// (vec elements), 64 token rows within int32 byte offsets, 16-byte aligned
// base.
bool strides_ok(const attn_strides_t *s, const void *p, int vec) {
  if (!s || !p || ((uintptr_t)p & 15) != 0) return false;
  if (s->batch < 0 || s->head < 0 || s->token < 0) return false;
  if (s->batch % vec || s->head % vec || s->token % vec) return false;
  return s->token <= INT32_MAX / (2 * attn::kBlock);  // 64 rows of bf16 in int32 bytes
}

attn::Strides to_kernel(const attn_strides_t *s) {
  attn::Strides k;
  k.b = s->batch;
  k.h = s->head;
  k.l = (int32_t)s->token;
  return k;
}

attn_status_t fwd_impl(attn_dtype_t dtype, int32_t B, int32_t H, int64_t L, int32_t d,
                       float scale, const attn_pattern_t *pattern, const attn_index_t *dev_index,
                       const void *q, const attn_strides_t *qs, const void *k,
                       const attn_strides_t *ks, const void *v, const attn_strides_t *vs,
                       void *o, const attn_strides_t *os, float *lse, void *stream) {
  if (!prefill_dims_ok(B, H, L, d, scale, pattern)) return ATTN_ERR_INVALID_ARG;
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_INVALID_ARG;
  const int vec = dtype == ATTN_F32 ? 4 : 8;
  if (!strides_ok(qs, q, vec) || !strides_ok(ks, k, vec) || !strides_ok(vs, v, vec) ||
      !strides_ok(os, o, vec))
    return ATTN_ERR_INVALID_ARG;
  if (!index_shape_ok(dev_index, H, L, false)) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_BF16 && dtype != ATTN_F32) return ATTN_ERR_UNSUPPORTED;
  if (L % attn::kBlock != 0 && !pattern->causal) return ATTN_ERR_UNSUPPORTED;  // keys past L unmasked
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (dtype == ATTN_BF16 && attn::fwd_bf16_lds_bytes(d, dev_index->n_kblocks) > attn::kMaxLdsPerWorkgroup)
    return ATTN_ERR_UNSUPPORTED;  // union bitmap of more than ~65K key blocks (~4M tokens)
  attn::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.qs = to_kernel(qs);
  a.ks = to_kernel(ks);
  a.vs = to_kernel(vs);
  a.os = to_kernel(os);
  a.ix = view_of(dev_index);
  a.B = B;
  a.H = H;
  a.L = (int32_t)L;
  a.d = d;
  a.scale = scale;
  a.causal = pattern->causal ? 1 : 0;
  window_of(pattern, &a.window, &a.sink_blk);
  hipStream_t s = (hipStream_t)stream;
  return hip_status(dtype == ATTN_BF16 ? attn::launch_fwd_bf16(a, s) : attn::launch_fwd_f32(a, s));
}

attn_status_t bwd_impl(attn_dtype_t dtype, int32_t B, int32_t H, int64_t L, int32_t d, float scale,
                       const attn_pattern_t *pattern, const attn_index_t *dev_index,
                       const void *q, const attn_strides_t *qs, const void *k,
                       const attn_strides_t *ks, const void *v, const attn_strides_t *vs,
                       const void *o, const attn_strides_t *os, const float *lse,
                       const void *dout, const attn_strides_t *dos, void *dq,
                       const attn_strides_t *dqs, void *dk, const attn_strides_t *dks, void *dv,
                       const attn_strides_t *dvs, void *workspace, size_t workspace_bytes,
                       void *stream) {
  if (!prefill_dims_ok(B, H, L, d, scale, pattern)) return ATTN_ERR_INVALID_ARG;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return ATTN_ERR_INVALID_ARG;
  if (!strides_ok(qs, q, 8) || !strides_ok(ks, k, 8) || !strides_ok(vs, v, 8) ||
      !strides_ok(os, o, 8) || !strides_ok(dos, dout, 8) || !strides_ok(dqs, dq, 8) ||
      !strides_ok(dks, dk, 8) || !strides_ok(dvs, dv, 8))
    return ATTN_ERR_INVALID_ARG;
  if (!index_shape_ok(dev_index, H, L, true)) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (L % attn::kBlock != 0 && !pattern->causal) return ATTN_ERR_UNSUPPORTED;  // keys past L unmasked
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (attn::bwd_bf16_lds_bytes(d, dev_index->n_qblocks) > attn::kMaxLdsPerWorkgroup)
    return ATTN_ERR_UNSUPPORTED;
  const size_t need = attn_workspace_bytes(ATTN_OP_BWD, dtype, B, H, L, d);
  if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  attn::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.qs = to_kernel(qs);
  a.ks = to_kernel(ks);
  a.vs = to_kernel(vs);
  a.os = to_kernel(os);
  a.dos = to_kernel(dos);
  a.dqs = to_kernel(dqs);
  a.dks = to_kernel(dks);
  a.dvs = to_kernel(dvs);
  a.delta = (float *)workspace;
  a.lse2 = (float *)workspace + (size_t)B * H * L;
  a.ix = view_of(dev_index);
  a.B = B;
  a.H = H;
  a.L = (int32_t)L;
  a.d = d;
  a.scale = scale;
  a.causal = pattern->causal ? 1 : 0;
  window_of(pattern, &a.window, &a.sink_blk);
  // Work grouping only (any grouping gives the same result): a per-head
  // BlockSparse index groups each head's strided key blocks together.
  a.kgroup = pattern->kind == ATTN_BLOCKSPARSE && dev_index->n_heads == H && pattern->stride >= 2 &&
                     pattern->stride <= dev_index->n_kblocks
                 ? pattern->stride
                 : 1;
  return hip_status(attn::launch_bwd_bf16(a, (hipStream_t)stream));
}

}  // namespace

extern "C" {

attn_status_t attn_sparse_fwd(attn_dtype_t dtype, int32_t B, int32_t H, int64_t L, int32_t d,
                              float scale, const attn_pattern_t *pattern,
                              const attn_index_t *dev_index, const void *q, const void *k,
                              const void *v, void *o, float *lse, void *workspace,
                              size_t workspace_bytes, void *stream) {
  (void)workspace;
  (void)workspace_bytes;
  const attn_strides_t s = dense_strides(H, L, d);
  return fwd_impl(dtype, B, H, L, d, scale, pattern, dev_index, q, &s, k, &s, v, &s, o, &s, lse,
                  stream);
}

attn_status_t attn_sparse_fwd_strided(attn_dtype_t dtype, int32_t B, int32_t H, int64_t L,
                                      int32_t d, float scale, const attn_pattern_t *pattern,
                                      const attn_index_t *dev_index, const void *q,
                                      const attn_strides_t *q_strides, const void *k,
                                      const attn_strides_t *k_strides, const void *v,
                                      const attn_strides_t *v_strides, void *o,
                                      const attn_strides_t *o_strides, float *lse,
                                      void *workspace, size_t workspace_bytes, void *stream) {
  (void)workspace;
  (void)workspace_bytes;
  return fwd_impl(dtype, B, H, L, d, scale, pattern, dev_index, q, q_strides, k, k_strides, v,
                  v_strides, o, o_strides, lse, stream);
}

attn_status_t attn_sparse_bwd(attn_dtype_t dtype, int32_t B, int32_t H, int64_t L, int32_t d,
                              float scale, const attn_pattern_t *pattern,
                              const attn_index_t *dev_index, const void *q, const void *k,
                              const void *v, const void *o, const float *lse, const void *dout,
                              void *dq, void *dk, void *dv, void *workspace,
                              size_t workspace_bytes, void *stream) {
  const attn_strides_t s = dense_strides(H, L, d);
  return bwd_impl(dtype, B, H, L, d, scale, pattern, dev_index, q, &s, k, &s, v, &s, o, &s, lse,
                  dout, &s, dq, &s, dk, &s, dv, &s, workspace, workspace_bytes, stream);
}

attn_status_t attn_sparse_bwd_strided(
    attn_dtype_t dtype, int32_t B, int32_t H, int64_t L, int32_t d, float scale,
    const attn_pattern_t *pattern, const attn_index_t *dev_index, const void *q,
    const attn_strides_t *q_strides, const void *k, const attn_strides_t *k_strides,
    const void *v, const attn_strides_t *v_strides, const void *o,
    const attn_strides_t *o_strides, const float *lse, const void *dout,
    const attn_strides_t *dout_strides, void *dq, const attn_strides_t *dq_strides, void *dk,
    const attn_strides_t *dk_strides, void *dv, const attn_strides_t *dv_strides,
    void *workspace, size_t workspace_bytes, void *stream) {
  return bwd_impl(dtype, B, H, L, d, scale, pattern, dev_index, q, q_strides, k, k_strides, v,
                  v_strides, o, o_strides, lse, dout, dout_strides, dq, dq_strides, dk, dk_strides,
                  dv, dv_strides, workspace, workspace_bytes, stream);
}

static attn_status_t decode_common(attn_dtype_t dtype, int32_t B, int32_t H, int32_t d,
                                   float scale, int64_t cap, int32_t sink, int32_t window,
                                   int64_t max_pos, const int64_t *dev_pos, const void *q,
                                   const void *k_new, const void *v_new, void *k_cache,
                                   void *v_cache, void *o, float *lse, void *workspace,
                                   size_t workspace_bytes, void *stream,
                                   const int32_t *table = nullptr, int32_t max_pages = 0,
                                   int32_t n_pages = 0) {
  if (B < 1 || H < 1 || !(scale > 0.f) || !isfinite(scale)) return ATTN_ERR_INVALID_ARG;
  if (!dev_pos || !q || !k_new || !v_new || !k_cache || !v_cache || !o || !lse)
    return ATTN_ERR_INVALID_ARG;
  if ((int64_t)B * H > 65535) return ATTN_ERR_INVALID_ARG;  // grid.y limit
  if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  const int64_t n_keys = sink >= 0 ? cap : max_pos + 1;
  const size_t need = decode_ws_bytes(B, H, n_keys, d);
  if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  attn::DecodeArgs a;
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.o = o;
  a.lse = lse;
  a.pos = dev_pos;
  a.part = (float *)workspace;
  a.B = B;
  a.H = H;
  a.d = d;
  a.cap = cap;
  a.sink = sink;
  a.window = window;
  a.max_pos = max_pos;
  attn::decode_split_plan(B, H, n_keys, &a.n_split, &a.split_len);
  a.scale = scale;
  a.bs_sink = a.bs_local = a.bs_stride = a.bs_cap = 0;
  a.table = table;
  a.max_pages = max_pages;
  a.n_pages = n_pages;
  return hip_status(attn::launch_decode_bf16(a, (hipStream_t)stream));
}

// BlockSparse compacted-cache geometry: blocks of 64 tokens, sink + local +
// strided capacity; all checked before anything is enqueued.
static bool bs_pattern_ok(const attn_pattern_t *p, int32_t strided_blocks) {
  if (!p || p->kind != ATTN_BLOCKSPARSE || p->block != attn::kBlock) return false;
  if (p->sink_blocks < 0 || p->local_blocks < 1 || p->stride < 1 || strided_blocks < 0) return false;
  const int64_t blocks = (int64_t)p->sink_blocks + p->local_blocks + strided_blocks;
  return blocks * attn::kBlock <= INT32_MAX;
}

static int64_t bs_slots(const attn_pattern_t *p, int32_t strided_blocks) {
  return ((int64_t)p->sink_blocks + p->local_blocks + strided_blocks) * attn::kBlock;
}

attn_status_t attn_sparse_decode(attn_dtype_t dtype, int32_t B, int32_t H, int32_t d, float scale,
                                 int32_t sink_tokens, int32_t window_tokens,
                                 const int64_t *dev_pos, const void *q, const void *k_new,
                                 const void *v_new, void *k_cache, void *v_cache, void *o,
                                 float *lse, void *workspace, size_t workspace_bytes,
                                 void *stream) {
  if (sink_tokens < 0 || window_tokens < 1) return ATTN_ERR_INVALID_ARG;
  const int64_t cap = (int64_t)sink_tokens + window_tokens;
  if (cap > INT32_MAX) return ATTN_ERR_INVALID_ARG;
  return decode_common(dtype, B, H, d, scale, cap, sink_tokens, window_tokens, 0, dev_pos, q,
                       k_new, v_new, k_cache, v_cache, o, lse, workspace, workspace_bytes,
                       stream);
}

attn_status_t attn_full_decode(attn_dtype_t dtype, int32_t B, int32_t H, int32_t d, float scale,
                               int64_t capacity, int64_t max_pos, const int64_t *dev_pos,
                               const void *q, const void *k_new, const void *v_new,
                               void *k_cache, void *v_cache, void *o, float *lse,
                               void *workspace, size_t workspace_bytes, void *stream) {
  if (capacity < 1 || max_pos < 0 || max_pos >= capacity) return ATTN_ERR_INVALID_ARG;
  if (max_pos + 1 > (int64_t)INT32_MAX * 256) return ATTN_ERR_INVALID_ARG;
  return decode_common(dtype, B, H, d, scale, capacity, -1, 0, max_pos, dev_pos, q, k_new, v_new,
                       k_cache, v_cache, o, lse, workspace, workspace_bytes, stream);
}

attn_status_t attn_full_decode_noalloc(attn_dtype_t dtype, int32_t B, int32_t H, int32_t d,
                                       float scale, int64_t capacity, int64_t max_pos,
                                       const int64_t *dev_pos, const void *q, const void *k_new,
                                       const void *v_new, void *k_cache, void *v_cache, void *o,
                                       float *lse, void *stream) {
  // Every other argument is checked first: without a workspace,
  // attn_full_decode returns ATTN_ERR_WORKSPACE exactly when all its other
  // checks pass (its workspace check comes last), and enqueues nothing.
  const attn_status_t st = attn_full_decode(dtype, B, H, d, scale, capacity, max_pos, dev_pos, q,
                                            k_new, v_new, k_cache, v_cache, o, lse, nullptr, 0,
                                            stream);
  if (st != ATTN_ERR_WORKSPACE) return st;
  void *ws = nullptr;
  if (attn::decode_scratch(&ws) != hipSuccess) return ATTN_ERR_HIP;
  // partials beyond the fixed scratch: ATTN_ERR_WORKSPACE, nothing enqueued
  return attn_full_decode(dtype, B, H, d, scale, capacity, max_pos, dev_pos, q, k_new, v_new,
                          k_cache, v_cache, o, lse, ws, attn::kDecodeScratchBytes, stream);
}

attn_status_t attn_paged_decode(attn_dtype_t dtype, int32_t B, int32_t H, int32_t d, float scale,
                                int32_t n_pages, int32_t max_pages,
                                const int32_t *dev_block_table, int64_t max_pos,
                                const int64_t *dev_pos, const void *q, const void *k_new,
                                const void *v_new, void *k_pages, void *v_pages, void *o,
                                float *lse, void *workspace, size_t workspace_bytes,
                                void *stream) {
  if (n_pages < 1 || max_pages < 1 || !dev_block_table) return ATTN_ERR_INVALID_ARG;
  if (max_pos < 0 || max_pos >= (int64_t)max_pages * attn::kBlock) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)B * max_pages > INT32_MAX) return ATTN_ERR_INVALID_ARG;
  return decode_common(dtype, B, H, d, scale, (int64_t)max_pages * attn::kBlock, -1, 0, max_pos,
                       dev_pos, q, k_new, v_new, k_pages, v_pages, o, lse, workspace,
                       workspace_bytes, stream, dev_block_table, max_pages, n_pages);
}

attn_status_t attn_paged_cache_fill(attn_dtype_t dtype, int32_t B, int32_t H, int32_t d,
                                    int32_t n_pages, int32_t max_pages,
                                    const int32_t *dev_block_table, const int64_t *dev_len,
                                    const void *k_src, const void *v_src, int64_t src_len,
                                    void *k_pages, void *v_pages, void *stream) {
  if (B < 1 || H < 1 || n_pages < 1 || max_pages < 1 || src_len < 0) return ATTN_ERR_INVALID_ARG;
  if (!dev_block_table || !dev_len || !k_src || !v_src || !k_pages || !v_pages)
    return ATTN_ERR_INVALID_ARG;
  if ((int64_t)B * H > 65535 || (int64_t)B * max_pages > INT32_MAX) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  attn::PagedFillArgs a;
  a.k_src = k_src;
  a.v_src = v_src;
  a.k_pages = k_pages;
  a.v_pages = v_pages;
  a.table = dev_block_table;
  a.len = dev_len;
  a.src_len = src_len;
  a.B = B;
  a.H = H;
  a.d = d;
  a.max_pages = max_pages;
  a.n_pages = n_pages;
  return hip_status(attn::launch_paged_fill_bf16(a, (hipStream_t)stream));
}

attn_status_t attn_blocksparse_decode(attn_dtype_t dtype, int32_t B, int32_t H, int32_t d,
                                      float scale, const attn_pattern_t *pattern,
                                      int32_t strided_blocks, const int64_t *dev_pos,
                                      const void *q, const void *k_new, const void *v_new,
                                      void *k_cache, void *v_cache, void *o, float *lse,
                                      void *workspace, size_t workspace_bytes, void *stream) {
  if (!bs_pattern_ok(pattern, strided_blocks)) return ATTN_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || !(scale > 0.f) || !isfinite(scale)) return ATTN_ERR_INVALID_ARG;
  if (!dev_pos || !q || !k_new || !v_new || !k_cache || !v_cache || !o || !lse)
    return ATTN_ERR_INVALID_ARG;
  if ((int64_t)B * H > 65535) return ATTN_ERR_INVALID_ARG;  // grid.y limit
  if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  const int64_t slots = bs_slots(pattern, strided_blocks);
  const size_t need = decode_ws_bytes(B, H, slots, d);
  if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  attn::DecodeArgs a;
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.o = o;
  a.lse = lse;
  a.pos = dev_pos;
  a.part = (float *)workspace;
  a.B = B;
  a.H = H;
  a.d = d;
  a.cap = slots;
  a.sink = 0;
  a.window = 0;
  a.max_pos = 0;
  attn::decode_split_plan(B, H, slots, &a.n_split, &a.split_len);
  a.scale = scale;
  a.bs_sink = pattern->sink_blocks;
  a.bs_local = pattern->local_blocks;
  a.bs_stride = pattern->stride;
  a.bs_cap = strided_blocks;
  a.table = nullptr;
  a.max_pages = a.n_pages = 0;
  return hip_status(attn::launch_decode_bf16(a, (hipStream_t)stream));
}

attn_status_t attn_blocksparse_cache_fill(attn_dtype_t dtype, int32_t B, int32_t H, int32_t d,
                                          const attn_pattern_t *pattern, int32_t strided_blocks,
                                          const int64_t *dev_len, const void *k_src,
                                          const void *v_src, int64_t src_len, void *k_cache,
                                          void *v_cache, void *stream) {
  if (!bs_pattern_ok(pattern, strided_blocks)) return ATTN_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || src_len < 0) return ATTN_ERR_INVALID_ARG;
  if (!dev_len || !k_src || !v_src || !k_cache || !v_cache) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)B * H > 65535) return ATTN_ERR_INVALID_ARG;  // grid.y limit
  if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  attn::BsFillArgs a;
  a.k_src = k_src;
  a.v_src = v_src;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.len = dev_len;
  a.src_len = src_len;
  a.B = B;
  a.H = H;
  a.d = d;
  a.sink = pattern->sink_blocks;
  a.local = pattern->local_blocks;
  a.stride = pattern->stride;
  a.cap = strided_blocks;
  return hip_status(attn::launch_bs_fill_bf16(a, (hipStream_t)stream));
}

attn_status_t attn_ring_fill(attn_dtype_t dtype, int32_t B, int32_t H, int32_t d,
                             int32_t sink_tokens, int32_t window_tokens, const int64_t *dev_len,
                             const void *k_src, const void *v_src, int64_t src_len,
                             void *k_cache, void *v_cache, void *stream) {
  if (B < 1 || H < 1 || sink_tokens < 0 || window_tokens < 1 || src_len < 0)
    return ATTN_ERR_INVALID_ARG;
  if (!dev_len || !k_src || !v_src || !k_cache || !v_cache) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)B * H > 65535) return ATTN_ERR_INVALID_ARG;  // grid.y limit
  if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  attn::RingFillArgs a;
  a.k_src = k_src;
  a.v_src = v_src;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.len = dev_len;
  a.src_len = src_len;
  a.B = B;
  a.H = H;
  a.d = d;
  a.sink = sink_tokens;
  a.window = window_tokens;
  return hip_status(attn::launch_ring_fill_bf16(a, (hipStream_t)stream));
}

}  // extern "C"
