// LDS staging of 64-token tiles and the CSR union walk, shared by the MFMA
// forward and backward kernels.
//
// Two LDS layouts of a 64 x D bf16 tile (64 tokens, D head dims):
//   row-major   [token][d], rows padded to D + 8 elements, read as the
//               row-operand of a 32x32x16 MFMA (16 contiguous bytes per lane);
//   transposed  [d][pos(token)], rows padded to 64 + 8 elements, read as the
//               operand whose k index runs over tokens.  pos() swaps bits 2
//               and 3 of the token index so that the 8 tokens one lane feeds
//               into a k-step sit in 16 contiguous bytes (they match the
//               register order of a 32x32 accumulator reused as an operand,
//               see pack_acc_operand()).
// Both paddings make 16 consecutive lanes of a 16-byte read hit distinct
// banks.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace attn {

__device__ __forceinline__ int tpos(int u) {
  return (u & ~0xC) | ((u & 4) << 1) | ((u & 8) >> 1);
}

template <int D>
struct TileGeom {
  static constexpr int ROW = D + 8;        // row-major LDS row (elements)
  static constexpr int TROW = kBlock + 8;  // transposed LDS row (elements)
  static constexpr int CPR = D / 8;        // 16-byte chunks per token row
  static constexpr int ROW_ELEMS = kBlock * ROW;
  static constexpr int T_ELEMS = D * TROW;
};

// Row-major staging of one 64 x D tile by NT threads.
template <int D, int NT>
struct RowStage {
  static constexpr int CPR = D / 8;
  static constexpr int N = kBlock * CPR / NT;
  static_assert(N >= 1 && kBlock * CPR % NT == 0, "row stage shape");
  u32x4 r[N];

  __device__ __forceinline__ void load(const bf16 *g) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int ch = threadIdx.x + i * NT;
      r[i] = *(const u32x4 *)(g + (ch / CPR) * D + (ch % CPR) * 8);
    }
  }
  __device__ __forceinline__ void store(bf16 *lds) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int ch = threadIdx.x + i * NT;
      *(u32x4 *)(lds + (ch / CPR) * TileGeom<D>::ROW + (ch % CPR) * 8) = r[i];
    }
  }
};

// Transposed staging of one 64 x D tile by NT threads: each thread loads KPT
// consecutive token rows of one 8-dim chunk and writes 8 transposed rows of
// KPT tokens.
template <int D, int NT>
struct TStage {
  static constexpr int CPR = D / 8;
  static constexpr int KPT = kBlock * CPR / NT;
  static_assert(KPT == 2 || KPT == 4, "transposed stage shape");
  u32x4 r[KPT];

  __device__ __forceinline__ void load(const bf16 *g) {
    const int c = threadIdx.x % CPR, grp = threadIdx.x / CPR;
#pragma unroll
    for (int kk = 0; kk < KPT; ++kk) r[kk] = *(const u32x4 *)(g + (grp * KPT + kk) * D + c * 8);
  }
  __device__ __forceinline__ void store(bf16 *lds) const {
    constexpr int TR = TileGeom<D>::TROW;
    const int c = threadIdx.x % CPR, grp = threadIdx.x / CPR;
    const int pos = tpos(grp * KPT);
#pragma unroll
    for (int w = 0; w < 4; ++w) {  // word w holds dims 8c+2w (low half), 8c+2w+1 (high half)
      if constexpr (KPT == 4) {
        u32x2 lo, hi;
        lo[0] = (r[0][w] & 0xffffu) | (r[1][w] << 16);
        lo[1] = (r[2][w] & 0xffffu) | (r[3][w] << 16);
        hi[0] = (r[0][w] >> 16) | (r[1][w] & 0xffff0000u);
        hi[1] = (r[2][w] >> 16) | (r[3][w] & 0xffff0000u);
        *(u32x2 *)(lds + (c * 8 + 2 * w) * TR + pos) = lo;
        *(u32x2 *)(lds + (c * 8 + 2 * w + 1) * TR + pos) = hi;
      } else {
        *(uint32_t *)(lds + (c * 8 + 2 * w) * TR + pos) = (r[0][w] & 0xffffu) | (r[1][w] << 16);
        *(uint32_t *)(lds + (c * 8 + 2 * w + 1) * TR + pos) = (r[0][w] >> 16) | (r[1][w] & 0xffff0000u);
      }
    }
  }
};

// Rows of a 32x32 accumulator pair (64 tokens x 32 columns, fp32) converted to
// the bf16 operand of a k-step that runs over those 64 tokens: k-step ks takes
// registers 8*(ks%2)..+7 of tile ks/2.  Logical k = 8*hh + 4*a + b is token
// 16*ks + 8*a + 4*hh + b, which tpos() places at 16*ks + 8*hh + 4*a + b.
__device__ __forceinline__ bf16x8 pack_acc_operand(const f32x16 &t, int half) {
  u32x4 w;
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(t[8 * half + 2 * e], t[8 * half + 2 * e + 1]);
  return __builtin_bit_cast(bf16x8, w);
}

// Ascending union of two sorted CSR (or CSC) lists -- the two 64-token
// blocks of a 128-token tile -- with defensive skipping of out-of-range ids.
// Every step advances at least one list, so the walk ends after at most the
// total list length.  Plain scalars (no arrays) keep the cursors in SGPRs.
struct PairWalk {
  int p0, e0, p1, e1;
  const int32_t *ids;
  int n_ids;

  __device__ __forceinline__ void init(const int32_t *ptr, int first, int n_rows, int nnz) {
    p0 = e0 = p1 = e1 = 0;
    if (first < n_rows) {
      p0 = clamp_i(ptr[first], 0, nnz);
      e0 = clamp_i(ptr[first + 1], p0, nnz);
    }
    if (first + 1 < n_rows) {
      p1 = clamp_i(ptr[first + 1], 0, nnz);
      e1 = clamp_i(ptr[first + 2], p1, nnz);
    }
  }
  __device__ __forceinline__ bool ok(int x) const { return x >= 0 && x < n_ids; }
  __device__ __forceinline__ int next() {
    while (p0 < e0 && !ok(ids[p0])) ++p0;
    while (p1 < e1 && !ok(ids[p1])) ++p1;
    int j = INT32_MAX;
    if (p0 < e0) j = ids[p0];
    if (p1 < e1) j = min(j, (int)ids[p1]);
    return j;
  }
  // Whether list `which` (0 or 1) holds j at its cursor.
  __device__ __forceinline__ bool has(int which, int j) const {
    return which == 0 ? (p0 < e0 && ids[p0] == j) : (p1 < e1 && ids[p1] == j);
  }
  __device__ __forceinline__ void advance(int j) {
    if (p0 < e0 && ids[p0] == j) ++p0;
    if (p1 < e1 && ids[p1] == j) ++p1;
  }
};

}  // namespace attn
