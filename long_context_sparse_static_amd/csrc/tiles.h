// LDS staging of 64-token tiles and the CSR union walk, shared by the MFMA
// forward and backward kernels.
//
// Two LDS layouts of a 64 x D bf16 tile (64 tokens, D head dims):
//   row-major   [token][d], rows padded to D + 8 elements, read as the
//               row-operand of a 32x32x16 MFMA (16 contiguous bytes per lane);
//               the padding puts 16 consecutive lanes on distinct banks.
//   transposed  [d][token], 128-byte rows (64 tokens) without padding, read
//               as the operand whose k index runs over tokens.  Within a row
//               the tokens are permuted by tpos() (bits 2 and 3 swapped) so
//               that the 8 tokens one lane feeds into a k-step are 16
//               contiguous bytes, matching the register order of a 32x32
//               accumulator reused as an operand (pack_acc_operand()); and
//               the eight 16-byte chunks of row d are XOR-swizzled by
//               tswz(d) so that both the 16-lane operand reads and the
//               transposing 8-byte writes spread over all 64 banks.  (With
//               plain padding the transposing writes ran ~25x slower than the
//               reads on gfx950 and stalled the whole CU's LDS.)
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace attn {

__host__ __device__ __forceinline__ int tpos(int u) {
  return (u & ~0xC) | ((u & 4) << 1) | ((u & 8) >> 1);
}

// XOR key of the 16-byte chunks of transposed row d (0..7).
__host__ __device__ __forceinline__ int tswz(int d) { return ((d >> 1) ^ (d >> 4)) & 7; }

// Element offset of logical 16-byte chunk q (0..7) of transposed row d.
__host__ __device__ __forceinline__ int t_off(int d, int q) { return d * kBlock + ((q ^ tswz(d)) << 3); }

template <int D>
struct TileGeom {
  static constexpr int ROW = D + 8;        // row-major LDS row (elements)
  static constexpr int CPR = D / 8;        // 16-byte chunks per token row
  static constexpr int ROW_ELEMS = kBlock * ROW;
  static constexpr int T_ELEMS = D * kBlock;
};

// Row-major staging of one 64 x D tile by NT threads into LDS rows of RS
// elements (RS >= D).
template <int D, int NT, int RS = TileGeom<D>::ROW>
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
      *(u32x4 *)(lds + (ch / CPR) * RS + (ch % CPR) * 8) = r[i];
    }
  }
};

// Transposed staging of one 64 x D tile by NT threads: each thread loads KPT
// consecutive token rows of one 8-dim chunk c and writes 8 transposed rows
// (dims 8c..8c+7) of KPT tokens.  Lanes with odd c write each pair of rows in
// the opposite order, so every store instruction covers both bank halves.
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
  // byte offset of this thread's KPT tokens inside transposed row d
  __device__ __forceinline__ static int unit_off(int d, int grp) {
    if constexpr (KPT == 4) {
      const int u = tpos(grp * 4) >> 2;               // 8-byte unit 0..15
      return (((u >> 1) ^ tswz(d)) << 4) + ((u & 1) << 3);
    } else {
      const int u = tpos(grp * 2) >> 1;               // 4-byte unit 0..31
      return (((u >> 2) ^ tswz(d)) << 4) + ((u & 3) << 2);
    }
  }
  __device__ __forceinline__ void store(bf16 *lds) const {
    const int c = threadIdx.x % CPR, grp = threadIdx.x / CPR;
    const bool odd = c & 1;
    // v_perm selectors: the low halves (dims 8c+2w) or the high halves
    // (dims 8c+2w+1) of two 32-bit words; odd lanes take them swapped.
    const uint32_t sel_a = odd ? 0x07060302u : 0x05040100u;
    const uint32_t sel_b = odd ? 0x05040100u : 0x07060302u;
    char *base = (char *)lds;
#pragma unroll
    for (int w = 0; w < 4; ++w) {  // word w holds dims 8c+2w (low half), 8c+2w+1 (high half)
      const int dA = c * 8 + 2 * w + (odd ? 1 : 0);
      const int dB = dA ^ 1;
      if constexpr (KPT == 4) {
        u32x2 va, vb;
        va[0] = __builtin_amdgcn_perm(r[1][w], r[0][w], sel_a);
        va[1] = __builtin_amdgcn_perm(r[3][w], r[2][w], sel_a);
        vb[0] = __builtin_amdgcn_perm(r[1][w], r[0][w], sel_b);
        vb[1] = __builtin_amdgcn_perm(r[3][w], r[2][w], sel_b);
        *(u32x2 *)(base + dA * (kBlock * 2) + unit_off(dA, grp)) = va;
        *(u32x2 *)(base + dB * (kBlock * 2) + unit_off(dB, grp)) = vb;
      } else {
        *(uint32_t *)(base + dA * (kBlock * 2) + unit_off(dA, grp)) = __builtin_amdgcn_perm(r[1][w], r[0][w], sel_a);
        *(uint32_t *)(base + dB * (kBlock * 2) + unit_off(dB, grp)) = __builtin_amdgcn_perm(r[1][w], r[0][w], sel_b);
      }
    }
  }
};

// Row-major 64 x D tile read through the gfx950 transposing LDS load
// (ds_read_b64_tr_b16) as the A operand of a 32x32x16 MFMA whose k index
// runs over the 64 tokens: A[m = d][k = token].  Within each 16-lane group
// the instruction hands output lane i element i%4 of the 8-byte chunks that
// source lanes i/4, 4 + i/4, 8 + i/4, 12 + i/4 address.  Source lane s of
// group gi (lane = 16*gi + s, plus 32*hh) therefore addresses token
// 16*ks + 8*r + 4*hh + s/4 at dims 32*mt + 16*gi + 4*(s%4); two reads
// (r = 0, 1) give the lane d = 32*mt + lane%32 and the 8 tokens that the
// register order of pack_acc_operand() assigns to logical k = 8*hh .. +7.
// Row stride TRS = D + 32 elements puts the 32 lanes of one read phase on
// all 64 banks (row r starts at bank 16*r mod 64).
template <int D>
struct TrRead {
  static constexpr int TRS = D + 32;           // row stride (elements)
  static constexpr int ELEMS = kBlock * TRS;
  int base;                                    // byte offset of this lane
  __device__ __forceinline__ void init(int lane) {
    const int s = lane & 15, gi = (lane >> 4) & 1, hh = lane >> 5;
    base = ((s >> 2) + 4 * hh) * TRS * 2 + (16 * gi + 4 * (s & 3)) * 2;
  }
  __device__ __forceinline__ bf16x8 load(const bf16 *tile, int mt, int ks) const {
    typedef short s4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s4 lds_s4;
    const char *p = (const char *)tile + base + (16 * ks) * TRS * 2 + 64 * mt;
    const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)p);
    const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(p + 8 * TRS * 2));
    typedef short s8 __attribute__((ext_vector_type(8)));
    const s8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
  }
};

// Byte offsets of one lane's reads of a transposed tile as the A operand of
// a 32x32x16 MFMA: row d = 32*mt + n (n = lane % 32), logical chunk
// q = 2*ks + hh.  Because tswz(32*mt + n) = tswz(n) ^ 2*mt for mt < 4, the
// physical chunk is (2*(ks ^ mt)) ^ sigma with a per-lane sigma, so four
// per-lane bases (one per value of ks ^ mt) plus the immediate mt * 4096
// cover every read: no address arithmetic inside the loop.
struct TReadBases {
  int b[4];
  __device__ __forceinline__ void init(int n, int hh) {
    const int sigma = (hh ^ tswz(n)) & 7;
#pragma unroll
    for (int x = 0; x < 4; ++x) b[x] = n * (kBlock * 2) + (((2 * x) ^ sigma) << 4);
  }
  // byte offset of (mt, ks)
  __device__ __forceinline__ int at(int mt, int ks) const { return b[ks ^ mt] + mt * 32 * kBlock * 2; }
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

// A 64 x D bf16 tile staged straight from global memory into LDS
// (buffer_load_dwordx4 ... lds) as 64 unpadded rows of RB = 2 D bytes whose
// 16-byte chunks are XOR-swizzled: chunk c of row r sits at chunk
// c ^ swz(r).  The swizzle is chosen by how the tile is read:
//   kRowRead  as the row operand of a 32x32x16 MFMA (lane = row, 16 bytes);
//             16 consecutive rows per phase must hit distinct bank groups.
//   kTrRead   through ds_read_b64_tr_b16 (lane = dim, 4 tokens); 4
//             consecutive rows x 64 bytes per phase must cover all banks.
//   kBothRead both ways; one swizzle satisfies both conditions.
// Every swizzle acts on the chunk index only, so one per-lane base XOR a
// constant addresses every k-step (row reads) or dim tile (transposing
// reads).
enum SwzKind { kRowRead = 0, kTrRead = 1, kBothRead = 2 };

template <int D, int KIND>
struct SwzTile {
  static constexpr int RB = 2 * D;          // bytes per token row
  static constexpr int CPR = RB / 16;       // 16-byte chunks per row
  static constexpr int TILE = kBlock * RB;  // bytes per tile
  static constexpr int RPI = 1024 / RB;     // rows per wave load instruction

  __host__ __device__ static int swz(int r) {
    if (KIND == kRowRead) return D == 128 ? (r & 15) : ((r >> 1) & 7);
    if (KIND == kTrRead) return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
    return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
  }

  // Loading: wave lw of NL loading waves fills rows lw * 64 / NL .. +64/NL.
  template <int NL>
  struct Loader {
    static constexpr int LPW = kBlock / NL / RPI;  // instructions per wave
    static_assert(LPW >= 1 && kBlock % (NL * RPI) == 0, "load shape");
    int goff[LPW];   // per-lane global byte offsets from the tile's first row
    int lds_row0;    // first LDS row of this wave's share
    // row_stride: elements between consecutive token rows in global memory
    __device__ __forceinline__ void init(int lw, int lane, int row_stride) {
      lds_row0 = lw * (kBlock / NL);
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int r = lds_row0 + i * RPI + lane / CPR;
        goff[i] = 2 * (r * row_stride + (((lane % CPR) ^ swz(r)) << 3));
      }
    }
    __device__ __forceinline__ void load(const bf16 *g, char *lds) const {
      const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(g);
#pragma unroll
      for (int i = 0; i < LPW; ++i) load_lds<16>(rs, goff[i], lds + (lds_row0 + i * RPI) * RB);
    }
  };

  // Row operand reads: lane (n, hh) reads row 32 t + n, dims 16 ks + 8 hh .. +7.
  int kbase;
  // Transposing reads: lane (hh, gi, s) = 32 hh + 16 gi + s addresses token
  // 16 ks + 8 h + 4 hh + s / 4 (h = 0, 1) at dims 32 mt + 16 gi + 4 (s % 4);
  // the two reads give lane d = 32 mt + lane % 32 the 8 tokens that
  // pack_acc_operand() assigns to logical k = 8 hh .. +7.
  int trb[2];
  __device__ __forceinline__ void init_reads(int lane) {
    const int n = lane & 31, hh = lane >> 5, s = lane & 15, gi = (lane >> 4) & 1;
    kbase = n * RB + ((hh ^ swz(n)) << 4);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 8 * h + 4 * hh + (s >> 2);
      trb[h] = r * RB + (((2 * gi + ((s & 3) >> 1)) ^ swz(r)) << 4) + ((s & 1) << 3);
    }
  }
  __device__ __forceinline__ bf16x8 row(const char *tile, int t, int ks) const {
    return *(const bf16x8 *)(tile + (kbase ^ (ks << 5)) + t * 32 * RB);
  }
  __device__ __forceinline__ bf16x8 tr(const char *tile, int mt, int ks) const {
    typedef short s4 __attribute__((ext_vector_type(4)));
    typedef short s8 __attribute__((ext_vector_type(8)));
    typedef __attribute__((address_space(3))) s4 lds_s4;
    const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s4 *)(tile + (trb[0] ^ (mt << 6)) + 16 * ks * RB));
    const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s4 *)(tile + (trb[1] ^ (mt << 6)) + 16 * ks * RB));
    return __builtin_bit_cast(bf16x8, (s8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
};

// Union of R consecutive CSR (or CSC) rows -- the 64-token blocks of one
// workgroup tile -- held as R LDS bitmaps over block ids plus a summary
// bitmap of the non-empty words.  Built once per workgroup (atomicOr per list
// entry, so row order, duplicates and out-of-range ids cannot matter: bad ids
// are dropped), then walked in ascending order by every wave with scalar bit
// tricks.
//   LDS layout (32-bit words): bm[r*nw .. r*nw+nw) row r, then sm[0..nsw)
//   (bit w set when word w of any row is non-zero).
template <int R>
struct RowsBitmap {
  uint32_t *bm;
  uint32_t *sm;
  int nw, nsw;

  __host__ __device__ static int words(int n_ids) { return (n_ids + 31) / 32; }
  __host__ __device__ static int summary_words(int n_ids) { return (words(n_ids) + 31) / 32; }
  __host__ __device__ static size_t lds_bytes(int n_ids) {
    return (size_t)(R * words(n_ids) + summary_words(n_ids)) * sizeof(uint32_t);
  }

  __device__ __forceinline__ void init(uint32_t *lds, int n_ids) {
    nw = words(n_ids);
    nsw = summary_words(n_ids);
    bm = lds;
    sm = lds + R * nw;
  }

  // Caller: every thread of the workgroup, nt threads.  Ends with a barrier.
  // Bitmap row r holds list rows[r] (none if rows[r] < 0).  The R row
  // extents are read first and the R lists then read as one flat range, kU
  // entries per thread in flight, so the build waits for two dependent
  // global reads rather than two per row (and one per entry and thread).
  __device__ void build_rows(const int32_t *ptr, const int (&rows)[R], int nnz, const int32_t *ids,
                             int n_ids, int nt) {
    constexpr int kU = R >= 4 ? 8 : 1;   // the two-row (backward) tiles gained nothing from more
    int beg[R], len[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = rows[r];
      const int p = row >= 0 ? clamp_i(ptr[row], 0, nnz) : 0;
      const int e = row >= 0 ? clamp_i(ptr[row + 1], p, nnz) : 0;
      beg[r] = p;
      len[r] = e - p;
    }
    for (int i = threadIdx.x; i < R * nw + nsw; i += nt) bm[i] = 0u;
    __syncthreads();
    int total = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) total += len[r];
    // flat entry x -> (row, global position)
    auto locate = [&](int x, int &row) -> int {
      int pos = beg[0] + x;
      row = 0;
#pragma unroll
      for (int r = 1; r < R; ++r) {
        if (row == r - 1 && x >= len[r - 1]) {   // past rows 0 .. r-1
          x -= len[r - 1];
          pos = beg[r] + x;
          row = r;
        }
      }
      return pos;
    };
    for (int x0 = threadIdx.x; x0 < total; x0 += kU * nt) {
      int jv[kU], rv[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int x = x0 + u * nt;
        jv[u] = -1;
        rv[u] = 0;
        if (x < total) jv[u] = ids[locate(x, rv[u])];
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int j = jv[u];
        if (j >= 0 && j < n_ids) atomicOr(&bm[rv[u] * nw + (j >> 5)], 1u << (j & 31));
      }
    }
    __syncthreads();
    for (int w = threadIdx.x; w < nw; w += nt) {
      uint32_t any = 0u;
#pragma unroll
      for (int r = 0; r < R; ++r) any |= bm[r * nw + w];
      if (any) atomicOr(&sm[w >> 5], 1u << (w & 31));
    }
    __syncthreads();
  }

  // Lists first .. first + R - 1 (those below n_rows).
  __device__ void build(const int32_t *ptr, int first, int n_rows, int nnz, const int32_t *ids,
                        int n_ids, int nt) {
    int rows[R];
#pragma unroll
    for (int r = 0; r < R; ++r) rows[r] = first + r < n_rows ? first + r : -1;
    build_rows(ptr, rows, nnz, ids, n_ids, nt);
  }
};

// Walk over a RowsBitmap: ids rot..n_ids-1 ascending, then 0..rot-1
// ascending (rot = 0: plain ascending order).  All state is wave-uniform
// (SGPRs).  A rotation shared by the workgroups that run side by side makes
// them touch the same key blocks at about the same time, so the tiles they
// stream are served from L2 instead of being refetched.
template <int R>
struct RowsIter {
  int sw, sw_last, w, lo, hi, rot;
  bool second;
  uint32_t sbits, rem;
  uint32_t b[R];
  int j;          // current block id
  uint32_t mask;  // bit r set: listed by row r

  __device__ __forceinline__ void start(int n_ids, int rotate = 0) {
    rot = rotate < 0 ? 0 : (rotate > n_ids ? n_ids : rotate);
    second = false;
    begin(rot, n_ids);
#pragma unroll
    for (int r = 0; r < R; ++r) b[r] = 0u;
  }
  // next pass covers ids [l, h)
  __device__ __forceinline__ void begin(int l, int h) {
    lo = l;
    hi = h;
    sbits = rem = 0u;
    if (l >= h) {
      sw = 0;
      sw_last = -1;
    } else {
      sw = ((l >> 5) >> 5) - 1;
      sw_last = ((h - 1) >> 5) >> 5;
    }
  }
  // bits of [first, last] inside the 32-bit word covering ids 32*word ..
  __device__ __forceinline__ static uint32_t span_mask(int word, int first, int last) {
    uint32_t m = ~0u;
    if (word == (first >> 5)) m &= ~0u << (first & 31);
    if (word == (last >> 5)) m &= (last & 31) == 31 ? ~0u : ((2u << (last & 31)) - 1u);
    return m;
  }
  __device__ __forceinline__ bool next(const RowsBitmap<R> &pb) {
    while (rem == 0u) {
      while (sbits == 0u) {
        if (++sw > sw_last) {
          if (second) return false;
          second = true;
          begin(0, rot);
          continue;
        }
        sbits = __builtin_amdgcn_readfirstlane(pb.sm[sw]) & span_mask(sw, lo >> 5, (hi - 1) >> 5);
      }
      const int wb = __builtin_ctz(sbits);
      sbits &= sbits - 1u;
      w = sw * 32 + wb;
      const uint32_t wm = span_mask(w, lo, hi - 1);
      rem = 0u;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        b[r] = __builtin_amdgcn_readfirstlane(pb.bm[r * pb.nw + w]) & wm;
        rem |= b[r];
      }
    }
    const int bit = __builtin_ctz(rem);
    rem &= rem - 1u;
    j = w * 32 + bit;
    mask = 0u;
#pragma unroll
    for (int r = 0; r < R; ++r) mask |= ((b[r] >> bit) & 1u) << r;
    return true;
  }
};

// Two-row forms used by the backward kernels.
using PairBitmap = RowsBitmap<2>;
struct PairIter : RowsIter<2> {
  bool in0, in1;
  __device__ __forceinline__ bool next(const PairBitmap &pb) {
    const bool ok = RowsIter<2>::next(pb);
    in0 = mask & 1u;
    in1 = (mask >> 1) & 1u;
    return ok;
  }
};

}  // namespace attn
