// Host-side harness for the index builder and validator, built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_host_sanitize.py.
// Every buffer is sized exactly to what the API reports, so any write past the
// entries the builder promises is caught; the corruption cases check that the
// validator rejects malformed indexes without reading out of bounds.
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "../../include/attn_sparse.h"

static int fails = 0;
#define CHECK(cond)                                                      \
  do {                                                                   \
    if (!(cond)) {                                                       \
      fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond);  \
      ++fails;                                                           \
    }                                                                    \
  } while (0)

struct Built {
  std::vector<int32_t> row_ptr, col_idx, col_ptr, row_idx;
  attn_index_t ix;
};

static attn_pattern_t pat(int kind, int s, int w, int st, int win = 0, int causal = 1) {
  attn_pattern_t p;
  p.kind = kind;
  p.block = 64;
  p.sink_blocks = s;
  p.local_blocks = w;
  p.stride = st;
  p.causal = causal;
  p.window_tokens = win;
  return p;
}

static bool build(const attn_pattern_t *ps, int n_pat, int32_t heads, int64_t L, bool csc, Built &b) {
  int64_t nnz = -1;
  const bool mixed = n_pat > 1;
  attn_status_t st = mixed ? attn_index_nnz_mixed(ps, heads, L, &nnz) : attn_index_nnz(ps, heads, L, &nnz);
  if (st != ATTN_OK) return false;
  const int64_t nb = L / 64;
  b.row_ptr.assign(heads * (nb + 1), -7);
  b.col_idx.assign(nnz, -7);
  if (csc) {
    b.col_ptr.assign(heads * (nb + 1), -7);
    b.row_idx.assign(nnz, -7);
  }
  int32_t *cp = csc ? b.col_ptr.data() : nullptr, *ri = csc ? b.row_idx.data() : nullptr;
  st = mixed ? attn_index_build_mixed(ps, heads, L, b.row_ptr.data(), b.col_idx.data(), cp, ri)
             : attn_index_build(ps, heads, L, b.row_ptr.data(), b.col_idx.data(), cp, ri);
  if (st != ATTN_OK) return false;
  b.ix.n_heads = heads;
  b.ix.n_qblocks = (int32_t)nb;
  b.ix.n_kblocks = (int32_t)nb;
  b.ix.nnz = nnz;
  b.ix.row_ptr = b.row_ptr.data();
  b.ix.col_idx = b.col_idx.data();
  b.ix.col_ptr = cp;
  b.ix.row_idx = ri;
  return true;
}

int main() {
  const attn_pattern_t pats[] = {
      pat(ATTN_ATTNSINK, 1, 4, 0),     pat(ATTN_ATTNSINK, 2, 3, 0),   pat(ATTN_ATTNSINK, 1, 64, 0),
      pat(ATTN_BLOCKSPARSE, 1, 16, 8), pat(ATTN_BLOCKSPARSE, 3, 5, 7), pat(ATTN_FULL, 0, 0, 0),
      pat(ATTN_SLIDING, 1, 0, 0, 4096), pat(ATTN_SLIDING, 0, 0, 0, 1000), pat(ATTN_SLIDING, 2, 0, 0, 65),
      pat(ATTN_ATTNSINK, 0, 1, 0),
  };
  const int64_t lens[] = {64, 64 * 37, 32768};
  for (const attn_pattern_t &p : pats)
    for (int64_t L : lens)
      for (int heads : {1, 9})
        for (bool csc : {false, true}) {
          Built b;
          CHECK(build(&p, 1, heads, L, csc, b));
          CHECK(attn_index_validate(&b.ix) == ATTN_OK);
        }

  // per-head mix
  const attn_pattern_t mix[] = {pat(ATTN_FULL, 0, 0, 0), pat(ATTN_ATTNSINK, 1, 4, 0),
                                pat(ATTN_BLOCKSPARSE, 1, 3, 4), pat(ATTN_ATTNSINK, 2, 3, 0)};
  {
    Built b;
    CHECK(build(mix, 4, 4, 64 * 37, true, b));
    CHECK(attn_index_validate(&b.ix) == ATTN_OK);
  }

  // corruptions of a valid index
  {
    const attn_pattern_t p = pat(ATTN_BLOCKSPARSE, 1, 3, 4);
    auto fresh = [&](Built &b) { CHECK(build(&p, 1, 2, 64 * 20, true, b)); };
    Built b;
    fresh(b);
    b.row_ptr[5] = b.row_ptr[4] - 1;  // non-monotone
    CHECK(attn_index_validate(&b.ix) == ATTN_ERR_BAD_INDEX);
    fresh(b);
    b.col_idx[3] = 1000;  // out of range
    CHECK(attn_index_validate(&b.ix) == ATTN_ERR_BAD_INDEX);
    fresh(b);
    b.col_idx[b.row_ptr[10]] = b.col_idx[b.row_ptr[10] + 1];  // not strictly ascending
    CHECK(attn_index_validate(&b.ix) == ATTN_ERR_BAD_INDEX);
    fresh(b);
    b.row_idx[7] = (b.row_idx[7] + 1) % 20;  // CSC no longer the transpose
    CHECK(attn_index_validate(&b.ix) == ATTN_ERR_BAD_INDEX);
    fresh(b);
    b.row_ptr[b.row_ptr.size() - 1] = (int32_t)b.ix.nnz + 5;  // past nnz
    CHECK(attn_index_validate(&b.ix) == ATTN_ERR_BAD_INDEX);
    CHECK(attn_index_validate(nullptr) != ATTN_OK);
  }

  // invalid patterns and arguments
  int64_t nnz = 0;
  attn_pattern_t bad = pat(7, 1, 1, 0);
  CHECK(attn_index_nnz(&bad, 1, 640, &nnz) != ATTN_OK);
  bad = pat(ATTN_ATTNSINK, 1, 0, 0);
  CHECK(attn_index_nnz(&bad, 1, 640, &nnz) != ATTN_OK);
  bad = pat(ATTN_SLIDING, 1, 0, 0, 0);
  CHECK(attn_index_nnz(&bad, 1, 640, &nnz) != ATTN_OK);
  bad = pat(ATTN_ATTNSINK, 1, 2, 0);
  CHECK(attn_index_nnz(&bad, 1, 0, &nnz) != ATTN_OK);    // empty sequence
  // a partial last block: ceil(650 / 64) = 11 blocks, the lists of 704 tokens
  int64_t nnz_ragged = 0, nnz_whole = 0;
  CHECK(attn_index_nnz(&bad, 1, 650, &nnz_ragged) == ATTN_OK);
  CHECK(attn_index_nnz(&bad, 1, 704, &nnz_whole) == ATTN_OK);
  CHECK(nnz_ragged == nnz_whole);
  CHECK(attn_index_nnz(&bad, 1, 640, nullptr) != ATTN_OK);

  // layer map
  uint8_t m[32];
  CHECK(attn_layer_map(32, 11, 21, m) == ATTN_OK);
  int full = 0;
  for (int i = 0; i < 32; ++i) full += m[i];
  CHECK(full == 11 && m[10] == 0 && m[11] == 1 && m[21] == 1 && m[22] == 0);
  CHECK(attn_layer_map(32, 21, 11, m) == ATTN_OK);  // empty full range: all sparse
  full = 0;
  for (int i = 0; i < 32; ++i) full += m[i];
  CHECK(full == 0);
  CHECK(attn_layer_map(0, 0, 0, m) != ATTN_OK);
  CHECK(attn_layer_map(4, 1, 2, nullptr) != ATTN_OK);
  for (int s = -6; s <= 0; ++s) CHECK(attn_status_str((attn_status_t)s) != nullptr);

  // BlockSparse cache sizing: extreme sizes stay in int64 arithmetic (UBSan
  // catches overflow), errors write nothing
  {
    const attn_pattern_t bs = pat(ATTN_BLOCKSPARSE, 1, 16, 8);
    int32_t cap = -7;
    int64_t slots = -7;
    CHECK(attn_blocksparse_strided_capacity(&bs, 131073, &cap) == ATTN_OK && cap == 254);
    CHECK(attn_blocksparse_cache_slots(&bs, cap, &slots) == ATTN_OK && slots == 17344);
    CHECK(attn_blocksparse_strided_capacity(&bs, INT64_MAX, &cap) == ATTN_ERR_UNSUPPORTED && cap == 254);
    const attn_pattern_t one = pat(ATTN_BLOCKSPARSE, INT32_MAX, INT32_MAX, 1);
    CHECK(attn_blocksparse_strided_capacity(&one, INT64_MAX, &cap) == ATTN_ERR_UNSUPPORTED && cap == 254);
    CHECK(attn_blocksparse_cache_slots(&one, INT32_MAX, &slots) == ATTN_ERR_UNSUPPORTED && slots == 17344);
    CHECK(attn_blocksparse_strided_capacity(&bs, 0, &cap) == ATTN_ERR_INVALID_ARG);
  }

  if (fails) return 1;
  printf("harness ok\n");
  return 0;
}
