// Host-side static block index: CSR (per query block) and CSC (per key block)
// lists of the LongGen sparse patterns, plus the hybrid layer map.
//
// Patterns: attention sink (initial tokens), window attention (recent tokens)
// and blockwise sparse attention (strided token blocks) [LongGen, mlsanity
// index page "A Little Goes a Long Way...", "Abstract (arXiv)"]; the access
// is static and block-wise, sparse layers at the top and bottom, full layers
// in the middle [atlas.scime.ai summary, "Approach"].
//
// Each row is generated directly in ascending order as
//   sink blocks [0, min(sink, i+1))
//   strided blocks in [sink, a) with (j + h) % stride == 0   (BlockSparse)
//   window blocks [max(a, sink), i]          with a = max(0, i - local + 1),
//                                            Sliding: a = the block of token
//                                            64 i - window + 1 (clamped at 0)
// which is a disjoint, sorted partition of the set the header defines.

#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "../../include/attn_sparse.h"

namespace {

// Blocks of a sequence of L tokens: the last one may hold fewer than
// `block` tokens.
int64_t n_blocks(int64_t L, int32_t block) { return (L + block - 1) / block; }

bool pattern_ok(const attn_pattern_t *p, int64_t L) {
  if (!p || p->block <= 0 || L <= 0) return false;
  if (n_blocks(L, p->block) > INT32_MAX - 1) return false;
  if (p->kind == ATTN_FULL) return true;
  if (p->kind == ATTN_SLIDING) return p->sink_blocks >= 0 && p->window_tokens >= 1 && p->causal;
  if (p->kind != ATTN_ATTNSINK && p->kind != ATTN_BLOCKSPARSE) return false;
  if (p->sink_blocks < 0 || p->local_blocks < 1) return false;
  if (p->kind == ATTN_BLOCKSPARSE && p->stride < 1) return false;
  return true;
}

// Appends the row of query block i for head h to `out`; returns its length.
template <class Sink>
int64_t emit_row(const attn_pattern_t *p, int64_t i, int32_t h, Sink &&sink) {
  int64_t n = 0;
  if (p->kind == ATTN_FULL) {
    for (int64_t j = 0; j <= i; ++j) sink(j), ++n;
    return n;
  }
  const int64_t s = p->sink_blocks;
  int64_t a;
  if (p->kind == ATTN_SLIDING) {
    // first key allowed for the block's first query: 64 i - window + 1
    const int64_t k0 = i * p->block - p->window_tokens + 1;
    a = k0 <= 0 ? 0 : k0 / p->block;
  } else {
    a = std::max<int64_t>(0, i - p->local_blocks + 1);
  }
  const int64_t sink_end = std::min<int64_t>(s, i + 1);
  for (int64_t j = 0; j < sink_end; ++j) sink(j), ++n;
  if (p->kind == ATTN_BLOCKSPARSE) {
    const int64_t st = p->stride;
    // first j >= s with (j + h) % st == 0
    int64_t r = ((-(int64_t)h) % st + st) % st;
    int64_t j0 = s <= r ? r : r + ((s - r + st - 1) / st) * st;
    for (int64_t j = j0; j < a; j += st) sink(j), ++n;
  }
  for (int64_t j = std::max(a, s); j <= i; ++j) sink(j), ++n;
  return n;
}

}  // namespace

extern "C" {

const char *attn_status_str(attn_status_t s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_BAD_INDEX: return "malformed block index";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

}  // extern "C"

namespace {

// Shared by the single-pattern and per-head builders: head h's rows follow
// pattern_of(h).
template <class PatternOf>
attn_status_t count_nnz(PatternOf &&pattern_of, int32_t n_heads, int64_t nb, bool same_rows,
                        int64_t *nnz_out) {
  int64_t total = 0;
  const int32_t distinct = same_rows ? 1 : n_heads;
  for (int32_t h = 0; h < distinct; ++h)
    for (int64_t i = 0; i < nb; ++i) total += emit_row(pattern_of(h), i, h, [](int64_t) {});
  if (same_rows) total *= n_heads;
  if (total > INT32_MAX) return ATTN_ERR_UNSUPPORTED;  // int32 offsets
  *nnz_out = total;
  return ATTN_OK;
}

template <class PatternOf>
void build_lists(PatternOf &&pattern_of, int32_t n_heads, int64_t nb, int32_t *row_ptr,
                 int32_t *col_idx, int32_t *col_ptr, int32_t *row_idx) {
  int64_t off = 0;
  for (int32_t h = 0; h < n_heads; ++h) {
    const attn_pattern_t *p = pattern_of(h);
    const int64_t head_start = off;
    int32_t *rp = row_ptr + (int64_t)h * (nb + 1);
    for (int64_t i = 0; i < nb; ++i) {
      rp[i] = (int32_t)off;
      emit_row(p, i, h, [&](int64_t j) { col_idx[off++] = (int32_t)j; });
    }
    rp[nb] = (int32_t)off;
    if (col_ptr) {
      int32_t *cp = col_ptr + (int64_t)h * (nb + 1);
      std::vector<int64_t> count(nb + 1, 0);
      for (int64_t e = head_start; e < off; ++e) count[col_idx[e]]++;
      int64_t acc = head_start;
      for (int64_t j = 0; j < nb; ++j) {
        cp[j] = (int32_t)acc;
        int64_t c = count[j];
        count[j] = acc;  // becomes the fill cursor
        acc += c;
      }
      cp[nb] = (int32_t)acc;
      for (int64_t i = 0; i < nb; ++i)  // rows visited in order -> ascending
        for (int64_t e = rp[i]; e < rp[i + 1]; ++e) row_idx[count[col_idx[e]]++] = (int32_t)i;
    }
  }
}

// Per-head patterns must agree on block size and causality (one kernel
// launch applies both to every head).
bool mixed_ok(const attn_pattern_t *patterns, int32_t n_heads, int64_t L) {
  if (!patterns || n_heads < 1) return false;
  for (int32_t h = 0; h < n_heads; ++h) {
    if (!pattern_ok(&patterns[h], L) || patterns[h].kind == ATTN_SLIDING) return false;
    if (patterns[h].block != patterns[0].block) return false;
    if ((patterns[h].causal != 0) != (patterns[0].causal != 0)) return false;
  }
  return true;
}

}  // namespace

extern "C" {

attn_status_t attn_index_nnz(const attn_pattern_t *p, int32_t n_heads, int64_t L,
                             int64_t *nnz_out) {
  if (!nnz_out || n_heads < 1 || !pattern_ok(p, L)) return ATTN_ERR_INVALID_ARG;
  return count_nnz([p](int32_t) { return p; }, n_heads, n_blocks(L, p->block),
                   p->kind != ATTN_BLOCKSPARSE, nnz_out);
}

attn_status_t attn_index_build(const attn_pattern_t *p, int32_t n_heads, int64_t L,
                               int32_t *row_ptr, int32_t *col_idx, int32_t *col_ptr,
                               int32_t *row_idx) {
  int64_t nnz = 0;
  attn_status_t st = attn_index_nnz(p, n_heads, L, &nnz);
  if (st != ATTN_OK) return st;
  if (!row_ptr || !col_idx) return ATTN_ERR_INVALID_ARG;
  if ((col_ptr == nullptr) != (row_idx == nullptr)) return ATTN_ERR_INVALID_ARG;
  build_lists([p](int32_t) { return p; }, n_heads, n_blocks(L, p->block), row_ptr, col_idx, col_ptr,
              row_idx);
  return ATTN_OK;
}

attn_status_t attn_index_nnz_mixed(const attn_pattern_t *patterns, int32_t n_heads, int64_t L,
                                   int64_t *nnz_out) {
  if (!nnz_out || !mixed_ok(patterns, n_heads, L)) return ATTN_ERR_INVALID_ARG;
  return count_nnz([patterns](int32_t h) { return &patterns[h]; }, n_heads,
                   n_blocks(L, patterns[0].block), false, nnz_out);
}

attn_status_t attn_index_build_mixed(const attn_pattern_t *patterns, int32_t n_heads, int64_t L,
                                     int32_t *row_ptr, int32_t *col_idx, int32_t *col_ptr,
                                     int32_t *row_idx) {
  int64_t nnz = 0;
  attn_status_t st = attn_index_nnz_mixed(patterns, n_heads, L, &nnz);
  if (st != ATTN_OK) return st;
  if (!row_ptr || !col_idx) return ATTN_ERR_INVALID_ARG;
  if ((col_ptr == nullptr) != (row_idx == nullptr)) return ATTN_ERR_INVALID_ARG;
  build_lists([patterns](int32_t h) { return &patterns[h]; }, n_heads, n_blocks(L, patterns[0].block),
              row_ptr, col_idx, col_ptr, row_idx);
  return ATTN_OK;
}

attn_status_t attn_index_validate(const attn_index_t *ix) {
  if (!ix || ix->n_heads < 1 || ix->n_qblocks < 1 || ix->n_kblocks < 1 || ix->nnz < 0 ||
      ix->nnz > INT32_MAX || !ix->row_ptr || (ix->nnz > 0 && !ix->col_idx))
    return ATTN_ERR_INVALID_ARG;
  if ((ix->col_ptr == nullptr) != (ix->row_idx == nullptr)) return ATTN_ERR_INVALID_ARG;
  const int64_t nq = ix->n_qblocks, nk = ix->n_kblocks, nnz = ix->nnz;
  for (int32_t h = 0; h < ix->n_heads; ++h) {
    const int32_t *rp = ix->row_ptr + (int64_t)h * (nq + 1);
    for (int64_t i = 0; i < nq; ++i) {
      if (rp[i] < 0 || rp[i + 1] < rp[i] || rp[i + 1] > nnz) return ATTN_ERR_BAD_INDEX;
      for (int64_t e = rp[i]; e < rp[i + 1]; ++e) {
        const int32_t j = ix->col_idx[e];
        if (j < 0 || j >= nk) return ATTN_ERR_BAD_INDEX;
        if (e > rp[i] && ix->col_idx[e - 1] >= j) return ATTN_ERR_BAD_INDEX;
      }
    }
  }
  if (!ix->col_ptr) return ATTN_OK;
  // CSC must be the exact transpose of the CSR, head by head.
  for (int32_t h = 0; h < ix->n_heads; ++h) {
    const int32_t *rp = ix->row_ptr + (int64_t)h * (nq + 1);
    const int32_t *cp = ix->col_ptr + (int64_t)h * (nk + 1);
    for (int64_t j = 0; j < nk; ++j) {
      if (cp[j] < 0 || cp[j + 1] < cp[j] || cp[j + 1] > nnz) return ATTN_ERR_BAD_INDEX;
      for (int64_t e = cp[j]; e < cp[j + 1]; ++e) {
        const int32_t i = ix->row_idx[e];
        if (i < 0 || i >= nq) return ATTN_ERR_BAD_INDEX;
        if (e > cp[j] && ix->row_idx[e - 1] >= i) return ATTN_ERR_BAD_INDEX;
      }
    }
    // same number of entries per head, and every (i, j) of the CSC is in the CSR
    if ((cp[nk] - cp[0]) != (rp[nq] - rp[0])) return ATTN_ERR_BAD_INDEX;
    for (int64_t j = 0; j < nk; ++j)
      for (int64_t e = cp[j]; e < cp[j + 1]; ++e) {
        const int32_t i = ix->row_idx[e];
        const int32_t *b = ix->col_idx + rp[i], *en = ix->col_idx + rp[i + 1];
        if (!std::binary_search(b, en, (int32_t)j)) return ATTN_ERR_BAD_INDEX;
      }
  }
  return ATTN_OK;
}

// BlockSparse compacted cache.  Position t (block i = t / block) reads the
// strided blocks j in [sink, i - local + 1) with (j + h) % stride == 0; the
// most any phase h can hold in a span of n blocks is ceil(n / stride), and
// the span only grows with t, so the last position below max_tokens sets the
// capacity.
static bool bs_sizing_ok(const attn_pattern_t *p) {
  return p && p->kind == ATTN_BLOCKSPARSE && p->block == 64 && p->sink_blocks >= 0 &&
         p->local_blocks >= 1 && p->stride >= 1;
}

attn_status_t attn_blocksparse_strided_capacity(const attn_pattern_t *p, int64_t max_tokens,
                                                int32_t *out) {
  if (!bs_sizing_ok(p) || !out || max_tokens < 1) return ATTN_ERR_INVALID_ARG;
  const int64_t last_block = (max_tokens - 1) / p->block;
  const int64_t first_local = std::max<int64_t>(0, last_block - p->local_blocks + 1);
  const int64_t span = std::max<int64_t>(0, first_local - p->sink_blocks);
  const int64_t cap = (span + p->stride - 1) / p->stride;
  if (cap > INT32_MAX) return ATTN_ERR_UNSUPPORTED;
  *out = (int32_t)cap;
  return ATTN_OK;
}

attn_status_t attn_blocksparse_cache_slots(const attn_pattern_t *p, int32_t strided_blocks,
                                           int64_t *out) {
  if (!bs_sizing_ok(p) || !out || strided_blocks < 0) return ATTN_ERR_INVALID_ARG;
  const int64_t slots = ((int64_t)p->sink_blocks + p->local_blocks + strided_blocks) * p->block;
  if (slots > INT32_MAX) return ATTN_ERR_UNSUPPORTED;
  *out = slots;
  return ATTN_OK;
}

attn_status_t attn_layer_map(int32_t n_layers, int32_t full_first, int32_t full_last,
                             uint8_t *is_full) {
  if (n_layers < 1 || !is_full) return ATTN_ERR_INVALID_ARG;
  for (int32_t l = 0; l < n_layers; ++l)
    is_full[l] = (l >= full_first && l <= full_last) ? 1 : 0;
  return ATTN_OK;
}

}  // extern "C"
