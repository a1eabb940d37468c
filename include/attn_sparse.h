/*
 * attn_sparse.h -- C ABI of the MI355X (gfx950) static block-sparse attention
 * library (libattn_sparse.so).
 *
 * The method: LongGen ("A Little Goes a Long Way: Efficient Long Context
 * Training and Inference with Partial Contexts") keeps one third of the layers
 * on full attention and makes the other two thirds sparse with fixed,
 * GPU-friendly patterns: attention sink (initial tokens), window attention
 * (recent tokens) and blockwise sparse attention (strided token blocks)
 * [mlsanity index page, "Abstract (arXiv)"].  Sparse layers sit at the top and
 * bottom and full layers in the middle; the sparsity is static and block-wise
 * [atlas.scime.ai summary, "Approach"].  Sparse layers keep a reduced KV cache
 * during decoding [same summary, "Key results"].
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are contiguous, row-major [B, H, L, d] (batch, head, token,
 *    head dim).  LSE is float32 [B, H, L]: the natural log of the sum of
 *    exp(scale * q.k) over the keys a query may see.
 *  - A "block" is 64 consecutive tokens; a sequence of L tokens has
 *    ceil(L / 64) blocks, the last one partial when L % 64 != 0.  Keys past
 *    L do not exist; rows past L are never written.
 *  - Device pointers are HIP device (or managed) pointers; `stream` is a
 *    hipStream_t passed as void* (NULL = the default stream).
 *  - Ownership: the caller allocates and frees every buffer (tensors, index,
 *    workspace).  The library allocates no device memory and is reentrant.
 *    Its only global state belongs to attn_full_decode_noalloc: a fixed
 *    device array per GPU and the cached addresses of those arrays.
 *  - Errors: arguments are checked synchronously.  On a negative status
 *    nothing has been enqueued and no output has been touched.  A failed
 *    kernel launch returns ATTN_ERR_HIP.  Faults inside kernels surface at the
 *    caller's next synchronisation of `stream`.  No C++ exception crosses the
 *    ABI.
 *  - Streams and graphs: a device op only enqueues kernels on `stream`; it
 *    makes no allocation, synchronisation, memset or copy of its own, and
 *    its launch shapes depend on host arguments only (a decode's split count
 *    on the capacity or max_pos, never on the device-side positions).  So
 *    calls on different streams run concurrently, and a call can be captured
 *    in a HIP graph and replayed with new contents of the same buffers
 *    (positions included).
 *  - Kernels treat a malformed device index defensively: row pointers are
 *    clamped to [0, nnz] and out-of-range block ids are skipped, so a bad
 *    index gives wrong numbers, never an out-of-bounds access.  Use
 *    attn_index_validate on the host copy before uploading it.
 */
#ifndef ATTN_SPARSE_H
#define ATTN_SPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = -1, /* null pointer, bad size, bad stride, ...        */
  ATTN_ERR_UNSUPPORTED = -2, /* valid request the library does not implement */
  ATTN_ERR_BAD_INDEX = -3,   /* malformed block index (host validation)      */
  ATTN_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required   */
  ATTN_ERR_HIP = -5          /* HIP runtime error (launch / device query)    */
} attn_status_t;

typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype_t;

/* Pattern kinds.  Full: every key block up to the diagonal.  AttnSink: sink
 * blocks plus a window of the most recent blocks.  BlockSparse: AttnSink plus
 * strided earlier blocks whose phase depends on the head.  Sliding: a
 * token-granular window of the most recent window_tokens tokens (window
 * attention over recent tokens, LongGen's sparse-pattern family: mlsanity
 * index page "A Little Goes a Long Way...", "Abstract (arXiv)"), plus
 * optional sink blocks; sink_blocks = 0 is plain sliding-window attention. */
typedef enum {
  ATTN_FULL = 0,
  ATTN_ATTNSINK = 1,
  ATTN_BLOCKSPARSE = 2,
  ATTN_SLIDING = 3
} attn_kind_t;

/* Operation ids for attn_workspace_bytes. */
typedef enum {
  ATTN_OP_FWD = 0,
  ATTN_OP_BWD = 1,
  ATTN_OP_SPARSE_DECODE = 2,
  ATTN_OP_FULL_DECODE = 3,
  ATTN_OP_BLOCKSPARSE_DECODE = 4
} attn_op_t;

/* Static pattern description (host struct, passed by pointer).
 * AttnSink / BlockSparse: query block i (tokens 64i..64i+63) reads key
 * block j when
 *   j <  sink_blocks and j <= i                              (sink)
 *   i - local_blocks < j <= i                                (window; it
 *                                                             holds the diagonal)
 *   kind == BLOCKSPARSE, j < i and (j + h) % stride == 0     (strided; h = head)
 * Full ignores the other fields and reads every j <= i.  With causal != 0,
 * keys later than the query token are masked inside any block.
 * Sliding (causal must be 1): query token q reads key token k when k <= q
 * and (k < 64 sink_blocks or q - k < window_tokens) -- the same keys decode
 * of token q reads from a sink + window ring (attn_sparse_decode with
 * sink_tokens = 64 sink_blocks, window_tokens = window_tokens).  Its block
 * lists hold every block with such a key; the kernels mask keys outside
 * the window inside its edge blocks. */
typedef struct {
  int32_t kind;          /* attn_kind_t                                      */
  int32_t block;         /* tokens per block; must be 64                     */
  int32_t sink_blocks;   /* >= 0                                             */
  int32_t local_blocks;  /* >= 1 for AttnSink / BlockSparse; else ignored    */
  int32_t stride;        /* BlockSparse: >= 1; otherwise ignored             */
  int32_t causal;        /* 1: mask key position > query position            */
  int32_t window_tokens; /* Sliding: >= 1; otherwise ignored                 */
} attn_pattern_t;

/* Block index in CSR form (and its transpose, CSC, for the backward pass).
 * Offsets are global into col_idx / row_idx.  Head hh of the index owns
 *   row_ptr[hh*(n_qblocks+1) .. hh*(n_qblocks+1)+n_qblocks]
 *   col_ptr[hh*(n_kblocks+1) .. hh*(n_kblocks+1)+n_kblocks].
 * n_heads is either 1 (one pattern broadcast to every head) or H (attention
 * head h uses index head h).  Lists are strictly ascending.  For the kernels
 * every pointer is a device pointer; for attn_index_validate they are host
 * pointers. */
typedef struct {
  int32_t n_heads;
  int32_t n_qblocks;
  int32_t n_kblocks;
  int64_t nnz;            /* total entries in col_idx (== in row_idx)       */
  const int32_t *row_ptr; /* [n_heads*(n_qblocks+1)]                        */
  const int32_t *col_idx; /* [nnz]                                         */
  const int32_t *col_ptr; /* [n_heads*(n_kblocks+1)] or NULL (forward only) */
  const int32_t *row_idx; /* [nnz] or NULL                                  */
} attn_index_t;

/* Element strides of a tensor indexed [b, h, l, e] whose d elements e of a
 * token row are contiguous: element (b, h, l, e) sits at
 *   b * batch + h * head + l * token + e   (in elements, not bytes).
 * Contiguous [B,H,L,d] is {H*L*d, L*d, d}; [B,L,H,d] is {L*H*d, d, H*d}; the
 * Q of a fused [B,L,3,H,d] projection is {3*L*H*d, d, 3*H*d} at offset 0
 * (K at H*d, V at 2*H*d).  Strides must be >= 0 and whole 16-byte vectors
 * (multiples of 8 bf16 / 4 fp32 elements), token <= INT32_MAX / 128, and the
 * base pointer 16-byte aligned.  Input rows may overlap (a token stride
 * below d, or 0 to repeat one row).  Outputs must not overlap each other or
 * the inputs. */
typedef struct {
  int64_t batch;
  int64_t head;
  int64_t token;
} attn_strides_t;

/* Human-readable name of a status code (static string, never NULL). */
const char *attn_status_str(attn_status_t status);

/* ---------------------------------------------------------------------------
 * Host helpers: pure CPU, no HIP calls, caller-owned host buffers.
 * ------------------------------------------------------------------------- */

/* Total entries of the index of `pattern` for n_heads index heads and L
 * tokens (ceil(L / block) query and key blocks), written to *nnz_out.  The index is the static
 * block list of the sparse layers' fixed patterns -- sink, window and
 * strided blocks (mlsanity index page "A Little Goes a Long Way...",
 * "Abstract (arXiv)"), accessed block-wise and fixed ahead of time
 * (atlas.scime.ai summary, "Approach"): it is built once per shape.
 * ATTN_ERR_INVALID_ARG for a NULL pointer, n_heads < 1 or an invalid
 * pattern; ATTN_ERR_UNSUPPORTED if nnz exceeds INT32_MAX (int32 offsets). */
attn_status_t attn_index_nnz(const attn_pattern_t *pattern, int32_t n_heads,
                             int64_t L, int64_t *nnz_out);

/* Builds the index of `pattern` (the static block lists of the sparse
 * patterns: mlsanity index page, "Abstract (arXiv)"; atlas.scime.ai summary,
 * "Approach") into caller host buffers sized as in attn_index_t (nnz from
 * attn_index_nnz): CSR rows ascending, and the CSC transpose the backward
 * walks.  Index head hh uses stride phase hh.  col_ptr and row_idx may both
 * be NULL (forward-only index); one of them alone is ATTN_ERR_INVALID_ARG.
 * Errors as attn_index_nnz; nothing is written on an error. */
attn_status_t attn_index_build(const attn_pattern_t *pattern, int32_t n_heads,
                               int64_t L, int32_t *row_ptr, int32_t *col_idx,
                               int32_t *col_ptr, int32_t *row_idx);

/* Per-head mix of patterns in one index (for instance full-attention
 * retrieval heads beside sink + window streaming heads, the head split of
 * DuoAttention on the Hugging Face paper-search page "long-context decoding
 * latency"): head h's rows follow patterns[h] with stride phase h.
 * patterns: n_heads host structs that share `block` and `causal` (a launch
 * applies both to every head) and are not ATTN_SLIDING (whose token window
 * a launch would apply to every head); otherwise ATTN_ERR_INVALID_ARG.
 * Buffers and the NULL-CSC rule as for attn_index_build.  Pass any of the
 * patterns to the device ops: they read only its block and causal fields. */
attn_status_t attn_index_nnz_mixed(const attn_pattern_t *patterns, int32_t n_heads,
                                   int64_t L, int64_t *nnz_out);
attn_status_t attn_index_build_mixed(const attn_pattern_t *patterns, int32_t n_heads,
                                     int64_t L, int32_t *row_ptr, int32_t *col_idx,
                                     int32_t *col_ptr, int32_t *row_idx);

/* Checks a HOST copy of an index (the static block lists the sparse layers
 * walk: mlsanity index page, "Abstract (arXiv)"; atlas.scime.ai summary,
 * "Approach") before it is uploaded: monotone pointers within [0, nnz],
 * block ids in range and strictly ascending, and (when present) that the
 * CSC is exactly the transpose of the CSR.  Returns ATTN_ERR_BAD_INDEX
 * otherwise, ATTN_ERR_INVALID_ARG for missing pointers or bad sizes.  Reads
 * only; the caller owns the arrays. */
attn_status_t attn_index_validate(const attn_index_t *host_index);

/* Hybrid layer map: is_full[l] = 1 for full_first <= l <= full_last, else 0
 * (one third full layers in the middle, sparse at top and bottom:
 * atlas.scime.ai summary, "Approach"). */
attn_status_t attn_layer_map(int32_t n_layers, int32_t full_first,
                             int32_t full_last, uint8_t *is_full);

/* Workspace bytes needed by an operation (0 if none).  `L_or_cap` is L for
 * prefill ops and the cache capacity (full decode) or sink+window (sparse
 * decode) for decode ops. */
size_t attn_workspace_bytes(int32_t op, attn_dtype_t dtype, int32_t B,
                            int32_t H, int64_t L_or_cap, int32_t d);

/* ---------------------------------------------------------------------------
 * Device operations: validate synchronously, then enqueue on `stream`.
 * ------------------------------------------------------------------------- */

/* Prefill forward of the hybrid model's attention layers: the sparse layers
 * with their static block patterns (sink, window, strided blocks: mlsanity
 * index page "A Little Goes a Long Way...", "Abstract (arXiv)"; static
 * block-wise access and FlashAttention-2 style tiling: atlas.scime.ai
 * summary, "Approach"; prefill is where the pages report 1.67x: same
 * summary, "Key results"), and the full middle layers with a Full index.
 * For every (b, h) and query token i: O[i] = softmax(scale * q_i K_S^T) V_S
 * over the allowed key set S of i, LSE[i] = log sum exp(scale * q_i K_S^T).
 *   dtype: ATTN_BF16 (q/k/v/o bf16, fp32 accumulation) or ATTN_F32 (all
 *          fp32).  d in {64, 128}.  pattern->block == 64; B, H, L >= 1
 *          (an empty batch or sequence is ATTN_ERR_INVALID_ARG).  A partial
 *          last block (L % 64 != 0) needs a causal pattern (ATTN_ERR_UNSUPPORTED
 *          otherwise): causality is what keeps every query off the keys past L.
 *   dev_index: device CSR for ceil(L/64) query and key blocks (CSC unused).
 *   pattern: its causal flag applies to every head; for kind ATTN_SLIDING
 *   its token window (sink_blocks, window_tokens) also masks keys inside
 *   the listed blocks of every head.  Sliding with causal == 0 is
 *   ATTN_ERR_INVALID_ARG.
 *   q, k, v: [B,H,L,d] in; o: [B,H,L,d] out; lse: [B,H,L] fp32 out.
 *   Rows with no allowed key give O = 0, LSE = -inf.  No workspace.
 *   Length limit of the bf16 path (its per-workgroup LDS holds a bitmap
 *   over the key blocks): L <= 4,161,536 tokens at d = 128 and about 12.4M
 *   at d = 64; longer sequences give ATTN_ERR_UNSUPPORTED. */
attn_status_t attn_sparse_fwd(attn_dtype_t dtype, int32_t B, int32_t H,
                              int64_t L, int32_t d, float scale,
                              const attn_pattern_t *pattern,
                              const attn_index_t *dev_index, const void *q,
                              const void *k, const void *v, void *o,
                              float *lse, void *workspace,
                              size_t workspace_bytes, void *stream);

/* attn_sparse_fwd over tensors with explicit strides (attn_strides_t): for
 * instance [B,L,H,d] activations, or Q/K/V read in place from a fused QKV
 * projection.  LSE stays contiguous [B,H,L] fp32.  Same dtypes, patterns,
 * index and errors as attn_sparse_fwd; invalid strides or misaligned
 * pointers give ATTN_ERR_INVALID_ARG. */
attn_status_t attn_sparse_fwd_strided(attn_dtype_t dtype, int32_t B, int32_t H,
                                      int64_t L, int32_t d, float scale,
                                      const attn_pattern_t *pattern,
                                      const attn_index_t *dev_index,
                                      const void *q, const attn_strides_t *q_strides,
                                      const void *k, const attn_strides_t *k_strides,
                                      const void *v, const attn_strides_t *v_strides,
                                      void *o, const attn_strides_t *o_strides,
                                      float *lse, void *workspace,
                                      size_t workspace_bytes, void *stream);

/* Backward of the prefill forward, for context-extension training (the
 * LongGen sparse layers are trained during length extension: mlsanity index
 * page, "Abstract (arXiv)").  With P the masked softmax and loss gradients
 * dO: D = rowsum(dO*O), dV = P^T dO, dS = P*(dO V^T - D), dQ = scale dS K,
 * dK = scale dS^T Q.
 *   dtype: ATTN_BF16 only; d in {64, 128}.
 *   dev_index: CSR and CSC (col_ptr/row_idx must be set).
 *   pattern: as for attn_sparse_fwd (causal flag; Sliding token window).
 *   q, k, v, o, dout: [B,H,L,d] bf16 in; lse: [B,H,L] fp32 in (from the
 *   forward); dq, dk, dv: [B,H,L,d] bf16 out.
 *   workspace: attn_workspace_bytes(ATTN_OP_BWD, ...) = 2*B*H*L*4 bytes
 *   (device; holds D and the base-2 LSE per token). */
attn_status_t attn_sparse_bwd(attn_dtype_t dtype, int32_t B, int32_t H,
                              int64_t L, int32_t d, float scale,
                              const attn_pattern_t *pattern,
                              const attn_index_t *dev_index, const void *q,
                              const void *k, const void *v, const void *o,
                              const float *lse, const void *dout, void *dq,
                              void *dk, void *dv, void *workspace,
                              size_t workspace_bytes, void *stream);

/* attn_sparse_bwd over tensors with explicit strides (attn_strides_t), one
 * stride set per tensor; LSE stays contiguous [B,H,L] fp32 and the
 * workspace is as for attn_sparse_bwd.  Errors as attn_sparse_bwd, plus
 * ATTN_ERR_INVALID_ARG for invalid strides or misaligned pointers. */
attn_status_t attn_sparse_bwd_strided(
    attn_dtype_t dtype, int32_t B, int32_t H, int64_t L, int32_t d, float scale,
    const attn_pattern_t *pattern, const attn_index_t *dev_index,
    const void *q, const attn_strides_t *q_strides,
    const void *k, const attn_strides_t *k_strides,
    const void *v, const attn_strides_t *v_strides,
    const void *o, const attn_strides_t *o_strides, const float *lse,
    const void *dout, const attn_strides_t *dout_strides,
    void *dq, const attn_strides_t *dq_strides,
    void *dk, const attn_strides_t *dk_strides,
    void *dv, const attn_strides_t *dv_strides,
    void *workspace, size_t workspace_bytes, void *stream);

/* Decode one new token per sequence in a sparse (sink + window) layer,
 * against its reduced ring-buffer cache: the sparse layers keep only the
 * sink and the recent window (mlsanity index page, "Abstract (arXiv)"),
 * which is where the pages' KV-memory cut and decode speedup come from
 * (atlas.scime.ai summary, "Key results": 69.2 GB to 26.5 GB, 1.41x).
 *   Cache layout: k_cache, v_cache [B,H,S,d] with S = sink_tokens +
 *   window_tokens.  Token p lives in slot p if p < sink_tokens, else in slot
 *   sink_tokens + (p - sink_tokens) % window_tokens.
 *   dev_pos: [B] int64 device, the absolute position t >= 0 of the new token.
 *   The new token's k_new / v_new ([B,H,1,d]) are written to slot(t); then q
 *   ([B,H,1,d]) attends to tokens {0..sink-1} U {t-window+1..t}.  The cache
 *   must already hold those tokens (attn_ring_fill, or earlier decodes).
 *   o: [B,H,1,d] out; lse: [B,H] fp32 out.  dtype: ATTN_BF16; d in {64,128}.
 *   A negative position gives o = 0, lse = NaN and appends nothing.
 *   workspace: attn_workspace_bytes(ATTN_OP_SPARSE_DECODE, ..., S, d). */
attn_status_t attn_sparse_decode(attn_dtype_t dtype, int32_t B, int32_t H,
                                 int32_t d, float scale, int32_t sink_tokens,
                                 int32_t window_tokens, const int64_t *dev_pos,
                                 const void *q, const void *k_new,
                                 const void *v_new, void *k_cache,
                                 void *v_cache, void *o, float *lse,
                                 void *workspace, size_t workspace_bytes,
                                 void *stream);

/* Decode one new token per sequence in a full-attention layer -- the middle
 * third of the hybrid, which keeps direct access to every token (mlsanity
 * index page, "Abstract (arXiv)"; atlas.scime.ai summary, "Approach").
 *   k_cache, v_cache: [B,H,capacity,d]; token p lives in slot p.
 *   dev_pos: [B] int64 device positions t; k_new / v_new go to slot t and q
 *   attends to slots 0..t.  max_pos: a host-side upper bound on every t
 *   (sizes the split-KV grid; must be < capacity).  A position outside
 *   [0, max_pos] gives o = 0, lse = NaN and appends nothing.
 *   dtype: ATTN_BF16; d in {64, 128}.
 *   workspace: attn_workspace_bytes(ATTN_OP_FULL_DECODE, ..., max_pos+1, d). */
attn_status_t attn_full_decode(attn_dtype_t dtype, int32_t B, int32_t H,
                               int32_t d, float scale, int64_t capacity,
                               int64_t max_pos, const int64_t *dev_pos,
                               const void *q, const void *k_new,
                               const void *v_new, void *k_cache, void *v_cache,
                               void *o, float *lse, void *workspace,
                               size_t workspace_bytes, void *stream);

/* attn_full_decode without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The split-KV partials live in a fixed
 * 8 MiB device array inside the library (one copy per GPU, held until the
 * process ends; its address is looked up on the first call on each device,
 * with the caller's current device, which must be the one holding the
 * tensors).  The call allocates nothing.  Arguments, layouts and errors as
 * attn_full_decode; partials beyond 8 MiB -- B*H*n_split*(d+2)*4 bytes, at
 * most (4096 + B*H)*(d+2)*4: every B*H <= 12000 fits at d = 128 -- give
 * ATTN_ERR_WORKSPACE before anything is enqueued.  Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (other streams,
 * other threads) race and must be ordered by the caller.  Nothing in the
 * array needs clearing between calls (every partial read is written first
 * in the same call). */
attn_status_t attn_full_decode_noalloc(attn_dtype_t dtype, int32_t B, int32_t H,
                                       int32_t d, float scale, int64_t capacity,
                                       int64_t max_pos, const int64_t *dev_pos,
                                       const void *q, const void *k_new,
                                       const void *v_new, void *k_cache,
                                       void *v_cache, void *o, float *lse,
                                       void *stream);

/* Decode one new token per sequence in a full-attention layer whose cache
 * is paged: a pool of 64-token pages shared by the batch, each sequence
 * naming its pages in a block table (the block-table KV cache of
 * PagedAttention, listed among LongGen's foundations on the mlsanity index
 * page, "Builds on"; LongGen is served with vLLM: atlas.scime.ai summary,
 * "Approach").  No sequence needs a contiguous [capacity] slab.
 *   k_pages, v_pages: [n_pages, H, 64, d] device pools; token p of
 *   sequence b lives in page dev_block_table[b * max_pages + p / 64], row
 *   p % 64 (all heads of a token share the page id).
 *   dev_block_table: [B, max_pages] int32 device.  The caller allocates
 *   pages; the entry for the new token's block must be set before the call.
 *   dev_pos, k_new, v_new, q, o, lse: as for attn_full_decode (k_new / v_new
 *   are written to the new token's page row, q attends to tokens 0..t).
 *   max_pos: host upper bound on every t, < 64 * max_pages.
 *   A position outside [0, max_pos] or a page id outside [0, n_pages) in
 *   any block 0 .. t / 64 of a sequence gives that sequence o = 0, lse = NaN
 *   (such pages are never read or written).
 *   dtype: ATTN_BF16; d in {64, 128}.
 *   workspace: attn_workspace_bytes(ATTN_OP_FULL_DECODE, ..., max_pos+1, d). */
attn_status_t attn_paged_decode(attn_dtype_t dtype, int32_t B, int32_t H,
                                int32_t d, float scale, int32_t n_pages,
                                int32_t max_pages,
                                const int32_t *dev_block_table,
                                int64_t max_pos, const int64_t *dev_pos,
                                const void *q, const void *k_new,
                                const void *v_new, void *k_pages,
                                void *v_pages, void *o, float *lse,
                                void *workspace, size_t workspace_bytes,
                                void *stream);

/* Copies prefill K/V into a page pool: tokens 0 .. min(len[b], src_len,
 * 64 max_pages) - 1 of sequence b go to the pages its block table names
 * (entries outside [0, n_pages) are skipped).
 *   k_src, v_src: [B,H,src_len,d] bf16 device; dev_len: [B] int64 device.
 *   Pools and table as for attn_paged_decode.  dtype: ATTN_BF16. */
attn_status_t attn_paged_cache_fill(attn_dtype_t dtype, int32_t B, int32_t H,
                                    int32_t d, int32_t n_pages,
                                    int32_t max_pages,
                                    const int32_t *dev_block_table,
                                    const int64_t *dev_len, const void *k_src,
                                    const void *v_src, int64_t src_len,
                                    void *k_pages, void *v_pages, void *stream);

/* Sizing of a BlockSparse compacted cache (layout as in
 * attn_blocksparse_decode): the strided area keeps the strided blocks that
 * have left the window, the part of the block-wise sparse pattern a reduced
 * KV cache must still hold (mlsanity index page, "Abstract (arXiv)";
 * atlas.scime.ai summary, "Key results").  Pure host, no HIP calls.
 *   attn_blocksparse_strided_capacity: *strided_blocks_out = the largest
 *   number of strided blocks any position t < max_tokens reads outside its
 *   window, over every head's stride phase -- the strided_blocks argument
 *   that fits decode of every such position.
 *   attn_blocksparse_cache_slots: *slots_out = 64 (sink_blocks +
 *   local_blocks + strided_blocks), the S of the [B,H,S,d] cache.
 *   pattern: kind ATTN_BLOCKSPARSE, block 64, sink_blocks >= 0,
 *   local_blocks >= 1, stride >= 1; max_tokens >= 1; strided_blocks >= 0.
 *   ATTN_ERR_INVALID_ARG otherwise (or for a NULL pointer);
 *   ATTN_ERR_UNSUPPORTED if the result does not fit (strided blocks beyond
 *   INT32_MAX, slots beyond INT32_MAX).  Nothing is written on an error. */
attn_status_t attn_blocksparse_strided_capacity(const attn_pattern_t *pattern,
                                                int64_t max_tokens,
                                                int32_t *strided_blocks_out);
attn_status_t attn_blocksparse_cache_slots(const attn_pattern_t *pattern,
                                           int32_t strided_blocks,
                                           int64_t *slots_out);

/* Decode one new token per sequence in a BlockSparse layer against its
 * compacted cache (the block-wise sparse layers of LongGen: mlsanity index
 * page, "Abstract (arXiv)"; their reduced KV cache: atlas.scime.ai summary,
 * "Key results").  The token at position t (block i = t / 64) reads exactly
 * the keys of its row of the prefill mask: sink blocks j < sink_blocks, the
 * local blocks i-local_blocks+1 .. i (keys <= t inside block i) and the
 * strided blocks sink_blocks <= j < i-local_blocks+1 with
 * (j + h) % stride == 0, h = head index.
 *   pattern: kind ATTN_BLOCKSPARSE, block 64 (sink_blocks s, local_blocks w,
 *   stride st).  strided_blocks C: capacity of the strided area
 *   (attn_blocksparse_strided_capacity gives the C that fits every
 *   position below a bound; attn_blocksparse_cache_slots gives S).
 *   Cache layout: k_cache, v_cache [B,H,S,d], S = 64 (s + w + C):
 *     slots [0, 64 s)            sink blocks;
 *     slots [64 s, 64 (s + w))   ring of the w most recent blocks, block j at
 *                                ring block j mod w;
 *     slots [64 (s + w), S)      strided blocks that left the window, in
 *                                ascending order.
 *   When t starts a block (t % 64 == 0) and block j = t/64 - w is a strided
 *   block, it is first copied from the ring to the strided area; then
 *   k_new / v_new ([B,H,1,d]) are written to the new token's slot and q
 *   ([B,H,1,d]) attends.  dev_pos: [B] int64 device.  A position whose
 *   strided blocks exceed C (or t < 0) gives lse = NaN and touches nothing.
 *   o: [B,H,1,d] bf16, lse: [B,H] fp32.  workspace:
 *   attn_workspace_bytes(ATTN_OP_BLOCKSPARSE_DECODE, ..., S, d).
 *   dtype: ATTN_BF16, d in {64, 128}. */
attn_status_t attn_blocksparse_decode(attn_dtype_t dtype, int32_t B, int32_t H,
                                      int32_t d, float scale,
                                      const attn_pattern_t *pattern,
                                      int32_t strided_blocks,
                                      const int64_t *dev_pos, const void *q,
                                      const void *k_new, const void *v_new,
                                      void *k_cache, void *v_cache, void *o,
                                      float *lse, void *workspace,
                                      size_t workspace_bytes, void *stream);

/* Fills a BlockSparse compacted cache (layout as in attn_blocksparse_decode)
 * from prefill K/V [B,H,src_len,d]: the state decode would have reached
 * after appending tokens 0 .. len_b-1 of sequence b (len_b = dev_len[b],
 * int64 device, clamped to src_len).  Slots that hold no token yet are left
 * untouched.  dtype: ATTN_BF16. */
attn_status_t attn_blocksparse_cache_fill(attn_dtype_t dtype, int32_t B, int32_t H,
                                          int32_t d, const attn_pattern_t *pattern,
                                          int32_t strided_blocks,
                                          const int64_t *dev_len, const void *k_src,
                                          const void *v_src, int64_t src_len,
                                          void *k_cache, void *v_cache, void *stream);

/* Fills a sparse layer's ring cache from prefill K/V (the reduced cache of
 * the LongGen sparse layers: atlas.scime.ai summary, "Key results").
 *   k_src, v_src: [B,H,src_len,d]; sequence b holds tokens 0..len_b-1 with
 *   len_b = dev_len[b] (int64 device, 0 <= len_b <= src_len).
 *   Copies tokens 0..min(sink,len_b)-1 and the last `window_tokens` tokens
 *   (never below position sink_tokens) into their slots of k_cache/v_cache
 *   [B,H,sink+window,d] (slot rule as in attn_sparse_decode).  Slots of
 *   tokens that do not exist are left untouched.  dtype: ATTN_BF16. */
attn_status_t attn_ring_fill(attn_dtype_t dtype, int32_t B, int32_t H,
                             int32_t d, int32_t sink_tokens,
                             int32_t window_tokens, const int64_t *dev_len,
                             const void *k_src, const void *v_src,
                             int64_t src_len, void *k_cache, void *v_cache,
                             void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_SPARSE_H */
