// LDS staging of 64-token tiles and the CSR union walk, shared by the MFMA
// forward and backward kernels.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace attn {

// Register order of a 32x32 fp32 accumulator pair (64 tokens x 32 columns)
// reused as the bf16 B operand of a k-step that runs over those 64 tokens:
// k-step ks takes registers 8 (ks % 2) .. +7 of tile ks / 2, so the lane's
// logical k = 8 hh + 4 a + b (hh = lane / 32) is token 16 ks + 8 a + 4 hh + b.
// Every transposing read below hands the A operand over in this same order.

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

// Descriptor for the 64-row tile at g (rows ld_bytes apart, row_bytes used
// per row) of a sequence with rows_left rows from the tile's first row: a
// partial last block's rows past the end load as zeros and are never read.
// The descriptor's base may sit `shift` bytes before g (the per-lane offsets
// then carry the shift): offsets stay non-negative when an instruction's
// immediate offset exceeds its rows' distance from g.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void *g, int rows_left, int ld_bytes,
                                                            int row_bytes, int shift = 0) {
  return buffer_rsrc_n((const char *)g - shift,
                       rows_left >= kBlock ? -1 : (rows_left - 1) * ld_bytes + row_bytes + shift);
}

// Descriptor for reading ROWS rows from g (ld_bytes apart, row_bytes used
// per row) of which rows_left exist (none if rows_left <= 0): loads past
// them return zeros, so a wave's operand rows load without a branch.
template <int ROWS>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void *g, int rows_left, int ld_bytes,
                                                            int row_bytes) {
  return buffer_rsrc_n(g, rows_left >= ROWS ? -1 : rows_left <= 0 ? 0 : (rows_left - 1) * ld_bytes + row_bytes);
}
// 16 bytes of a row operand through a rows_rsrc descriptor
__device__ __forceinline__ bf16x8 load_row16(__amdgpu_buffer_rsrc_t rs, int byte_off) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off, 0, 0));
}

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
    // Instruction i's LDS rows start i KB after the wave's first row: that
    // step is its immediate offset, which moves the global address too, so
    // it is taken back out of the lane offsets.  The descriptor base sits
    // SHIFT bytes before the tile, so those stay non-negative for any row
    // stride (also one below d).
    static constexpr int SHIFT = (LPW - 1) * RPI * RB;
    int goff[LPW];   // per-lane byte offsets from the descriptor base, less i KB
    int lds_row0;    // first LDS row of this wave's share
    // row_stride: elements between consecutive token rows in global memory
    __device__ __forceinline__ void init(int lw, int lane, int row_stride) {
      lds_row0 = lw * (kBlock / NL);
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int r = lds_row0 + i * RPI + lane / CPR;
        goff[i] = 2 * (r * row_stride + (((lane % CPR) ^ swz(r)) << 3)) + SHIFT - i * RPI * RB;
      }
    }
    // the tile at g of a sequence with rows_left rows from g on, row stride
    // ld elements (rows past the end load as zeros)
    __device__ __forceinline__ void load(const bf16 *g, int rows_left, int ld, char *lds) const {
      const __amdgpu_buffer_rsrc_t rs = tile_rsrc(g, rows_left, 2 * ld, RB, SHIFT);
      char *base = lds + lds_row0 * RB;
      static_for<LPW>([&](auto I) __attribute__((always_inline)) {
        constexpr int i = decltype(I)::value;
        load_lds<16, i * RPI * RB>(rs, goff[i], base);
      });
    }
  };

  // Row operand reads: lane (n, hh) reads row 32 t + n, dims 16 ks + 8 hh .. +7.
  int kbase;
  // Transposing reads: lane (hh, gi, s) = 32 hh + 16 gi + s addresses token
  // 16 ks + 8 h + 4 hh + s / 4 (h = 0, 1) at dims 32 mt + 16 gi + 4 (s % 4);
  // the two reads give lane d = 32 mt + lane % 32 the 8 tokens that
  // register order above assigns to logical k = 8 hh .. +7.
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

// Stores a wave's 32 x D fp32 accumulator (the transposed-product layout:
// lane (n, hh) = (lane % 32, lane / 32) holds row n, register r of tile mt
// holds column 32 mt + 8 (r / 4) + 4 hh + r % 4), times sc, rounded to bf16,
// to rows out[n * ld ..] through the wave's LDS area st (32 * 2 D bytes):
// written in that layout with the 16-byte chunks of a row XOR-swizzled by
// the row (the writes spread over the banks), read back as whole chunks of
// consecutive rows and stored as contiguous 1 KB runs -- not as 8-byte
// pieces of 32 different rows per store instruction.  With LIMIT, rows
// n_rows .. 31 (past the end of a partial last block) are not stored.
template <int D, bool LIMIT = false>
__device__ __forceinline__ void store_rows_staged(const f32x16 (&acc)[D / 32], float sc, char *st,
                                                  bf16 *out, int ld, int lane, int n_rows = 32) {
  constexpr int RB = 2 * D, CPR = RB / 16, RPS = 1024 / RB;
  const int n = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 w;
      w[0] = pack_bf16x2(acc[mt][4 * g] * sc, acc[mt][4 * g + 1] * sc);
      w[1] = pack_bf16x2(acc[mt][4 * g + 2] * sc, acc[mt][4 * g + 3] * sc);
      const int ch = 4 * mt + g;   // columns 8 ch + 4 hh .. +3
      *(u32x2 *)(st + n * RB + ((ch ^ (n & (CPR - 1))) << 4) + (hh << 3)) = w;
    }
#pragma unroll
  for (int i = 0; i < 32 / RPS; ++i) {
    const int r = i * RPS + lane / CPR, ch = lane % CPR;
    const u32x4 v = *(const u32x4 *)(st + r * RB + ((ch ^ (r & (CPR - 1))) << 4));
    if (!LIMIT || r < n_rows) *(u32x4 *)(out + (size_t)r * ld + ch * 8) = v;
  }
}

// Union of R consecutive CSR (or CSC) rows -- the 64-token blocks of one
// workgroup tile -- held as R LDS bitmaps over block ids plus a summary
// bitmap of the non-empty words.  Built once per workgroup (atomicOr per list
// entry into both, so row order, duplicates and out-of-range ids cannot
// matter: bad ids are dropped), then walked in ascending order by every wave
// with scalar bit tricks.
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
  // issue() runs once per thread after the first round of list reads is
  // issued and before any of them is used: loads it issues are not waited
  // for here (loads return in order, so a load issued before the list reads
  // would hold up the build until it landed).
  template <typename Issue>
  __device__ void build_rows(const int32_t *ptr, const int (&rows)[R], int nnz, const int32_t *ids,
                             int n_ids, int nt, Issue &&issue) {
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
    int jv[kU], rv[kU];
    auto read_round = [&](int x0) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int x = x0 + u * nt;
        jv[u] = -1;
        rv[u] = 0;
        if (x < total) jv[u] = ids[locate(x, rv[u])];
      }
    };
    // each entry sets its bit and its word's summary bit
    auto or_round = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int j = jv[u];
        if (j >= 0 && j < n_ids) {
          atomicOr(&bm[rv[u] * nw + (j >> 5)], 1u << (j & 31));
          atomicOr(&sm[j >> 10], 1u << ((j >> 5) & 31));
        }
      }
    };
    read_round(threadIdx.x);   // every thread, entries or not, so issue() runs once each
    issue();
    or_round();
    for (int x0 = threadIdx.x + kU * nt; x0 < total; x0 += kU * nt) {
      read_round(x0);
      or_round();
    }
    __syncthreads();
  }

  // Lists first .. first + R - 1 (those below n_rows).
  template <typename Issue>
  __device__ void build(const int32_t *ptr, int first, int n_rows, int nnz, const int32_t *ids,
                        int n_ids, int nt, Issue &&issue) {
    int rows[R];
#pragma unroll
    for (int r = 0; r < R; ++r) rows[r] = first + r < n_rows ? first + r : -1;
    build_rows(ptr, rows, nnz, ids, n_ids, nt, issue);
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

}  // namespace attn
