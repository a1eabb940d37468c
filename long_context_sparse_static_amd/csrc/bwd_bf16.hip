// Backward pass of static block-sparse causal attention (bf16 tensors, fp32
// accumulation) for context-extension training of LongGen's sparse layers
// (mlsanity index page "A Little Goes a Long Way...", "Abstract (arXiv)": the
// sparse architecture is what gets trained during length extension; the
// training kernel is FlashAttention-2 based: atlas.scime.ai summary,
// "Approach").
//
// With P = exp(scale * Q K^T - LSE) on the allowed (query, key) pairs:
//   D  = rowsum(dO * O)                       bwd_dq_kernel     (first; each query
//   dQ = scale * dS K                                              tile's own rows,
//        with dS = P * (dO V^T - D)                                walks the CSR)
//   dV = P^T dO,  dK = scale * dS^T Q          bwd_dkdv_kernel   (key-tile major,
//                                                                   walks the CSC)
// P and dS are recomputed per block pair from the forward's LSE, never stored.
// The dQ pass computes D and the base-2 LSE of its own rows and leaves them in
// the workspace for the dK/dV pass.  Splitting dQ into its own pass keeps
// every output written by exactly one workgroup: no atomics,
// bitwise-deterministic results.
//
// gfx950 mapping (both MFMA kernels): the streamed tiles (K and V for dQ; Q
// and dO for dK/dV) go straight from global memory into XOR-swizzled LDS
// rows (buffer_load_dwordx4 ... lds), double-buffered in slots that every load
// and read names at compile time, so the compiler never waits for a tile
// load in flight before reading the other slot.  A tile needed both as a row
// operand and transposed is read transposed through ds_read_b64_tr_b16;
// nothing is transposed on the way in.  The union of the workgroup's two
// CSR (CSC) lists is walked from a 64-block boundary, so the workgroups on
// one XCD stream the same blocks at the same time.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "tiles.h"

namespace attn {
namespace {

constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = kBwdWaves * 64;
constexpr int kBwdTB = kBwdWaves / 2;  // 64-token blocks per tile (32 rows per wave)

// A compile-time order of k-steps: KOrder<...>::value[i].
template <int... J>
struct KOrder {
  static constexpr int size = sizeof...(J);
  static constexpr int value[sizeof...(J)] = {J...};
};

// Packs registers 8 half .. 8 half + 7 of a 32x32 accumulator tile (scaled
// by nothing) into the B operand of a 32x32x16 MFMA whose k index runs over
// the tile's rows (the register order described at the top of tiles.h).
__device__ __forceinline__ bf16x8 pack_half(const f32x16 &t, int half) {
  u32x4 w;
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(t[8 * half + 2 * e], t[8 * half + 2 * e + 1]);
  return __builtin_bit_cast(bf16x8, w);
}

// Key blocks of the dK/dV tiles of one head.  g == 1: tile t holds blocks
// TB t .. TB t + TB - 1.  g > 1 (BlockSparse with stride g): the head's
// strided class, the blocks j = r0 (mod g) with r0 = -h mod g, comes first,
// TB class members per tile -- their CSC columns run from about j to the last
// query block, so the members of one tile list nearly the same query blocks
// and no wave idles through another member's long column; the remaining
// blocks follow, TB consecutive ones per tile.  Every head gets the same
// number of tiles (the class has ceil(nkb / g) members at most); a slot past
// a head's blocks holds -1.
template <int TB>
struct KeyTiles {
  int g, r0, n_cls, cls_tiles, nkb;

  __host__ __device__ static int cls_tiles_max(int nkb, int g) {
    return g > 1 ? ((nkb + g - 1) / g + TB - 1) / TB : 0;
  }
  __host__ __device__ static int per_head(int nkb, int g) {
    if (g <= 1) return (nkb + TB - 1) / TB;
    return cls_tiles_max(nkb, g) + (nkb - nkb / g + TB - 1) / TB;
  }
  // tiles of a head started before any other tile of any head (longest first)
  __host__ __device__ static int priority(int nkb, int g) {
    const int n = per_head(nkb, g);
    const int p = g > 1 ? cls_tiles_max(nkb, g) + 1 : 1;
    return p < n ? p : n;
  }

  __device__ __forceinline__ void init(int nkb_, int g_, int h) {
    nkb = nkb_;
    g = g_;
    r0 = g > 1 ? (g - h % g) % g : 0;
    n_cls = g > 1 && r0 < nkb ? (nkb - 1 - r0) / g + 1 : 0;
    cls_tiles = cls_tiles_max(nkb, g);
  }
  __device__ __forceinline__ int block(int tile, int r) const {
    if (g <= 1) {
      const int j = tile * TB + r;
      return j < nkb ? j : -1;
    }
    if (tile < cls_tiles) {
      const int idx = tile * TB + r;
      return idx < n_cls ? r0 + idx * g : -1;
    }
    const int idx = (tile - cls_tiles) * TB + r;
    const int p = idx / (g - 1), o = idx % (g - 1);
    const int j = p * g + o + (o >= r0 ? 1 : 0);
    return j < nkb ? j : -1;
  }
};

// One position of a union walk.
struct BwdPos {
  bool valid;
  int j;
  uint32_t mask;
};

// ----------------------------------------------------------------------------
// dQ: one workgroup per 128 query tokens (two query blocks), union of their
// CSR lists; two workgroups per CU.  Per wave (32 queries, lane = query):
//   S^T = K Q^T, dP^T = V dO^T, dS^T = P^T * (dP^T - D), dQ^T += K^T dS^T
// K is read as rows and transposed (kBothRead), V as rows.
// ----------------------------------------------------------------------------
// RAG: L is not a multiple of 64 (the last block is partial); the range
// checks compile away otherwise.
template <int D, bool WIN, bool DENSE, bool RAG>
__global__ __launch_bounds__(kBwdThreads, 2) void bwd_dq_kernel(BwdArgs a) {
  using KT = SwzTile<D, kBothRead>;
  using VT = SwzTile<D, kRowRead>;
  constexpr int KS = D / 16, MT = D / 32;
  __shared__ __attribute__((aligned(1024))) char k0[KT::TILE];
  __shared__ __attribute__((aligned(1024))) char k1[KT::TILE];
  __shared__ __attribute__((aligned(1024))) char v0[VT::TILE];
  __shared__ __attribute__((aligned(1024))) char v1[VT::TILE];
  extern __shared__ uint32_t dyn_lds[];

  const int nqb = a.ix.n_qblocks;
  const int n_tiles = (nqb + kBwdTB - 1) / kBwdTB;
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lin / n_tiles;
  const int tile = n_tiles - 1 - lin % n_tiles;   // heaviest tiles first
  const int hidx = a.ix.n_heads == 1 ? 0 : bh % a.H;
  // token-row strides: compile-time for contiguous [B,H,L,d] tensors
  const int bb = bh / a.H, head = bh % a.H;
  const size_t dense_base = (size_t)bh * a.L * D;
  const int lq = DENSE ? D : a.qs.l, lk = DENSE ? D : a.ks.l, lv = DENSE ? D : a.vs.l;
  const int ldo = DENSE ? D : a.dos.l, ldq = DENSE ? D : a.dqs.l, lo_ = DENSE ? D : a.os.l;
  const bf16 *kg = (const bf16 *)a.k + (DENSE ? dense_base : a.ks.at(bb, head));
  const bf16 *vg = (const bf16 *)a.v + (DENSE ? dense_base : a.vs.at(bb, head));

  const int wave = uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 31, hh = lane >> 5;
  const int my_r = wave >> 1;
  const int qb = tile * kBwdTB + my_r;
  const bool q_valid = qb < nqb;
  const int q_wave = qb * kBlock + (wave & 1) * 32;  // first query of this wave
  const int q_tok = q_wave + n;
  const bf16 *qw = (const bf16 *)a.q + (DENSE ? dense_base : a.qs.at(bb, head)) + (size_t)q_wave * lq;
  const bf16 *dow = (const bf16 *)a.dout + (DENSE ? dense_base : a.dos.at(bb, head)) + (size_t)q_wave * ldo;
  const bf16 *ow = (const bf16 *)a.o + (DENSE ? dense_base : a.os.at(bb, head)) + (size_t)q_wave * lo_;

  // The wave's operand rows, and the O rows and LSE of its queries (for D),
  // loaded inside the bitmap build behind the list reads.  Rows past L of a
  // partial last block (and every row of a query block past the last) load as
  // zeros, and P = 0 there (LSE2 = +inf).
  const bool q_in = q_valid && (!RAG || q_tok < a.L);
  const int rows_left = q_valid ? a.L - q_wave : 0;
  const size_t vrow = (size_t)bh * a.L + q_wave;   // the wave's first entry of [B,H,L] vectors
  bf16x8 bq[KS], bdo[KS], bo[KS];
  float lse;
  auto load_rows = [&]() __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rq = rows_rsrc<32>(qw, rows_left, 2 * lq, 2 * D);
    const __amdgpu_buffer_rsrc_t rg = rows_rsrc<32>(dow, rows_left, 2 * ldo, 2 * D);
    const __amdgpu_buffer_rsrc_t ro = rows_rsrc<32>(ow, rows_left, 2 * lo_, 2 * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bq[ks] = load_row16(rq, 2 * (n * lq + ks * 16 + hh * 8));
      bdo[ks] = load_row16(rg, 2 * (n * ldo + ks * 16 + hh * 8));
      bo[ks] = load_row16(ro, 2 * (n * lo_ + ks * 16 + hh * 8));
    }
    lse = __uint_as_float(
        __builtin_amdgcn_raw_buffer_load_b32(rows_rsrc<32>(a.lse + vrow, rows_left, 4, 4), 4 * n, 0, 0));
  };
  const float c = a.scale * kLog2e;

  KT kr;
  kr.init_reads(lane);
  VT vr;
  vr.init_reads(lane);
  typename KT::template Loader<kBwdWaves> kl;
  kl.init(wave, lane, lk);
  typename VT::template Loader<kBwdWaves> vl;
  vl.init(wave, lane, lv);

  RowsBitmap<kBwdTB> pb;
  pb.init(dyn_lds, a.ix.n_kblocks);
  pb.build(a.ix.row_ptr + (size_t)hidx * (nqb + 1), tile * kBwdTB, nqb, a.ix.nnz, a.ix.col_idx,
           a.ix.n_kblocks, kBwdThreads, load_rows);

  // D = rowsum(dO * O) of the lane's query: its 64 dims (d = 16 ks + 8 hh ..
  // +7), then the other 64 from lane n + 32 (the same sum on both lanes); and
  // the base-2 LSE (+inf for an empty row, so that P = 0 there).  Both go to
  // the workspace for the dK/dV pass (one writer per query).
  float lse2, dlt;
  {
    float dsum = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 o = __builtin_bit_cast(u32x4, bo[ks]), g = __builtin_bit_cast(u32x4, bdo[ks]);
#pragma unroll
      for (int i = 0; i < 4; ++i) dsum += bf16_lo(o[i]) * bf16_lo(g[i]) + bf16_hi(o[i]) * bf16_hi(g[i]);
    }
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(dsum), __float_as_uint(dsum), false, false);
    dsum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    lse2 = q_in && lse != -INFINITY ? lse * kLog2e : INFINITY;
    dlt = q_in ? dsum : 0.f;
    if (q_in && hh == 0) {
      a.delta[vrow + n] = -dsum;   // -D: the dK/dV kernel starts its dP accumulator from it
      a.lse2[vrow + n] = lse2;
    }
  }
  RowsIter<kBwdTB> it;
  it.start(a.ix.n_kblocks, min(tile * kBwdTB + kBwdTB - 1, nqb - 1) & ~63);
  auto advance = [&]() __attribute__((always_inline)) -> BwdPos {
    BwdPos p;
    p.valid = it.next(pb);
    p.j = it.j;
    p.mask = it.mask;
    return p;
  };
  auto listed = [&](const BwdPos &p) __attribute__((always_inline)) { return p.valid && q_valid && ((p.mask >> my_r) & 1u); };

  f32x16 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16{};

  auto block_work = [&](const char *kt, const char *vt, int j) __attribute__((always_inline)) {
    f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        s[t] = mfma_32x32x16(kr.row(kt, t, ks), bq[ks], s[t]);
        dp[t] = mfma_32x32x16(vr.row(vt, t, ks), bdo[ks], dp[t]);
      }
    // causal / token-window masks as -inf scores under one uniform branch
    // each (key offset in the block = 32 t + 8 (r / 4) + 4 hh + r % 4)
    const int lim = q_tok - j * kBlock - 4 * hh;   // later keys: offset > lim
    if (a.causal && j >= qb) {
      static_for<32>([&](auto E) __attribute__((always_inline)) {
        constexpr int t = decltype(E)::value / 16, r = decltype(E)::value % 16;
        s[t][r] = mask_neg_inf(s[t][r], lim - (32 * t + 8 * (r >> 2) + (r & 3)));
      });
    }
    if constexpr (WIN) {
      // token window: keys k <= q - window (offset <= lim - window) of blocks
      // past the sink blocks
      if (j >= a.sink_blk && j * kBlock <= q_wave + 31 - a.window) {
        const int lo = lim - a.window;
        static_for<32>([&](auto E) __attribute__((always_inline)) {
          constexpr int t = decltype(E)::value / 16, r = decltype(E)::value % 16;
          s[t][r] = mask_neg_inf(s[t][r], (32 * t + 8 * (r >> 2) + (r & 3)) - lo - 1);
        });
      }
    }
    static_for<32>([&](auto E) __attribute__((always_inline)) {
      constexpr int t = decltype(E)::value / 16, r = decltype(E)::value % 16;
      const float p = fast_exp2(__builtin_fmaf(s[t][r], c, -lse2));
      s[t][r] = p * (dp[t][r] - dlt);  // dS^T
    });
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 bds = pack_half(s[ks >> 1], ks & 1);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma_32x32x16(kr.tr(kt, mt, ks), bds, acc[mt]);
    }
  };

  BwdPos cur = advance(), nxt{false, 0, 0u};
  if (cur.valid) {
    nxt = advance();
    kl.load(kg + (size_t)cur.j * kBlock * lk, RAG ? a.L - cur.j * kBlock : kBlock, lk, k0);
    vl.load(vg + (size_t)cur.j * kBlock * lv, RAG ? a.L - cur.j * kBlock : kBlock, lv, v0);
  }
  // Block of walk step t lives in slot t & 1; the next block's tiles load into
  // the other slot while this one is computed.
  auto step = [&](auto PAR) __attribute__((always_inline)) -> bool {
    constexpr int P = decltype(PAR)::value;
    if (!cur.valid) return false;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (nxt.valid) {
      kl.load(kg + (size_t)nxt.j * kBlock * lk, RAG ? a.L - nxt.j * kBlock : kBlock, lk, P ? k0 : k1);
      vl.load(vg + (size_t)nxt.j * kBlock * lv, RAG ? a.L - nxt.j * kBlock : kBlock, lv, P ? v0 : v1);
    }
    if (listed(cur)) block_work(P ? k1 : k0, P ? v1 : v0, cur.j);
    cur = nxt;
    if (nxt.valid) nxt = advance();
    return true;
  };
  const std::integral_constant<int, 0> even;
  const std::integral_constant<int, 1> odd;
  while (step(even) && step(odd)) {
  }

  // every wave is done with the K slots (no loads in flight after the walk):
  // they stage the output rows, waves 0-1 in k0, 2-3 in k1
  __syncthreads();
  if (!q_valid) return;
  store_rows_staged<D, RAG>(acc, a.scale, (wave < 2 ? k0 : k1) + (wave & 1) * 32 * 2 * D,
                       (bf16 *)a.dq + (DENSE ? dense_base : a.dqs.at(bb, head)) + (size_t)q_wave * ldq, ldq,
                       lane, a.L - q_wave);
}

// ----------------------------------------------------------------------------
// dK, dV: NW waves as NW / 2 pairs; pair p (waves p and p + NW / 2) owns 32
// keys (lane = key) of key block p / 2 of the workgroup's tile and splits
// each listed query block by its 32-query halves: wave p takes half 0 and
// accumulates dV, its partner takes half 1 and accumulates dK.  The
// workgroup walks the union of its key blocks' CSC lists.
//   NW = 4: one key block per workgroup, two workgroups per CU, which run
//   unsynchronised, so one's vector work overlaps the other's matrix work.
//   NW = 8 (BlockSparse): two members of a head's strided class per
//   workgroup (KeyTiles), one workgroup per CU.  Every Q and dO tile loaded
//   serves both blocks: those columns run over nearly all later query
//   blocks, and with one key block per workgroup the 128K BlockSparse dK/dV
//   pass hit L2 on only 24% of its tile reads.
// Per block, each wave on its half:
//   S = Q K^T, dP = dO V^T - D (the accumulator starts at -D),
//   P = exp2(S c - LSE2) (masked), dS = P dP, both packed to bf16;
// then the pair trades through LDS what the other's product needs (wave p
// sends its dS, its partner its P) and, after the exchange barrier,
//   wave p:      dV^T += dO^T P       partner:     dK^T += Q^T dS
// over the whole block.  Each wave holds one accumulator set, so both fit
// on their SIMD at once (a single wave holding all of it needs about 400
// registers and runs alone), and the two halves of the vector work run on
// the two waves.  Q and dO are read as rows and transposed (kBothRead).
// ----------------------------------------------------------------------------
constexpr int kDkvMaxPairs = 4;   // of the NW = 8 form (LDS sizing)

template <int D, bool WIN, bool DENSE, bool RAG, int NW>
__global__ __launch_bounds__(NW * 64, 8 / NW) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int kDkvWaves = NW;
  constexpr int kDkvThreads = NW * 64;
  constexpr int kDkvPairs = NW / 2;
  constexpr int kDkvTB = kDkvPairs / 2;   // key blocks per workgroup (two pairs per block)
  using QT = SwzTile<D, kBothRead>;
  constexpr int KS = D / 16, MT = D / 32;
  __shared__ __attribute__((aligned(1024))) char q0[QT::TILE];
  __shared__ __attribute__((aligned(1024))) char q1[QT::TILE];
  __shared__ __attribute__((aligned(1024))) char o0[QT::TILE];
  __shared__ __attribute__((aligned(1024))) char o1[QT::TILE];
  __shared__ __attribute__((aligned(256))) float l0[kBlock];
  __shared__ __attribute__((aligned(256))) float l1[kBlock];
  __shared__ __attribute__((aligned(256))) float e0[kBlock];
  __shared__ __attribute__((aligned(256))) float e1[kBlock];
  // the pairs' exchange: xch[pair][side][j][lane] is packed operand j (the
  // B operand of k-step j of that half) sent by side 0 (dS of half 0) or
  // side 1 (P of half 1); consecutive lanes, consecutive 16 bytes
  __shared__ __attribute__((aligned(1024))) bf16x8 xch[kDkvPairs][2][2][64];
  extern __shared__ uint32_t dyn_lds[];

  const int nkb = a.ix.n_kblocks, nqb = a.ix.n_qblocks;
  using KTiles = KeyTiles<kDkvTB>;
  const int n_tiles = KTiles::per_head(nkb, a.kgroup);
  const int n_first = KTiles::priority(nkb, a.kgroup);
  const int BH = a.B * a.H;
  // The longest CSC columns (the sink block, early blocks of full attention,
  // the strided class of BlockSparse) are in the first n_first tiles of each
  // head: start those, round-robin over the XCD's heads, before anything
  // else on the XCD, then walk the heads' remaining tiles in order.
  int bh, tile;
  if (BH % kNumXcd == 0 && n_tiles > n_first) {
    const int hpx = BH / kNumXcd;
    const int xcd = blockIdx.x % kNumXcd;
    int s = blockIdx.x / kNumXcd;
    if (s < hpx * n_first) {
      bh = xcd * hpx + s % hpx;
      tile = s / hpx;
    } else {
      s -= hpx * n_first;
      bh = xcd * hpx + s / (n_tiles - n_first);
      tile = n_first + s % (n_tiles - n_first);
    }
  } else {
    bh = blockIdx.x / n_tiles;
    tile = blockIdx.x % n_tiles;
  }
  const int hidx = a.ix.n_heads == 1 ? 0 : bh % a.H;
  KTiles kt;
  kt.init(nkb, a.kgroup, bh % a.H);
  int krows[kDkvTB];
#pragma unroll
  for (int r = 0; r < kDkvTB; ++r) krows[r] = kt.block(tile, r);
  // token-row strides: compile-time for contiguous [B,H,L,d] tensors
  const int bb = bh / a.H, head = bh % a.H;
  const size_t dense_base = (size_t)bh * a.L * D;
  const int lq = DENSE ? D : a.qs.l, ldo_l = DENSE ? D : a.dos.l;
  const bf16 *qg = (const bf16 *)a.q + (DENSE ? dense_base : a.qs.at(bb, head));
  const bf16 *dog = (const bf16 *)a.dout + (DENSE ? dense_base : a.dos.at(bb, head));
  const float *lseg = a.lse2 + (size_t)bh * a.L;
  const float *ndltg = a.delta + (size_t)bh * a.L;   // -D

  const int wave = uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 31, hh = lane >> 5;
  const bool side0 = wave < kDkvPairs;   // query half 0 and dV (else half 1 and dK)
  const int pair = wave % kDkvPairs;
  const int my_r = pair >> 1;
  const int kb = krows[my_r];
  const bool k_valid = kb >= 0;
  const int k_wave = kb * kBlock + (pair & 1) * 32;  // first key of this pair
  const int k_tok = k_wave + n;

  // K and V of the pair's keys: the B operands of S and dP, loaded inside
  // the bitmap build behind the list reads (keys past L load as zeros when
  // rows do not overlap in memory; their dK and dV are never stored)
  bf16x8 bk[KS], bv[KS];
  auto load_kv = [&]() __attribute__((always_inline)) {
    const int lk = DENSE ? D : a.ks.l, lv = DENSE ? D : a.vs.l;
    const bf16 *kw = (const bf16 *)a.k + (DENSE ? dense_base : a.ks.at(bb, head)) + (size_t)k_wave * lk;
    const bf16 *vw = (const bf16 *)a.v + (DENSE ? dense_base : a.vs.at(bb, head)) + (size_t)k_wave * lv;
    const int rows_left = k_valid ? a.L - k_wave : 0;
    const __amdgpu_buffer_rsrc_t rk = rows_rsrc<32>(kw, rows_left, 2 * lk, 2 * D);
    const __amdgpu_buffer_rsrc_t rv = rows_rsrc<32>(vw, rows_left, 2 * lv, 2 * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bk[ks] = load_row16(rk, 2 * (n * lk + ks * 16 + hh * 8));
      bv[ks] = load_row16(rv, 2 * (n * lv + ks * 16 + hh * 8));
    }
  };
  const float c = a.scale * kLog2e;
  f32x16 acc[MT];   // dV^T (side 0) or dK^T (side 1) of the pair's keys
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16{};

  QT rd;
  rd.init_reads(lane);
  typename QT::template Loader<kDkvWaves> ldq, ldo;   // Q and dO tiles (own row strides)
  ldq.init(wave, lane, lq);
  ldo.init(wave, lane, ldo_l);
  // the two 64-float per-token vectors of a query block: wave 0 loads LSE2,
  // wave 1 the -D values (4 bytes per lane)
  // (a partial last block's vectors past L load as zeros, and its queries
  // past L are masked in the vector step, so they add nothing to dK or dV)
  auto load_vec = [&](int i, float *lv, float *ev) __attribute__((always_inline)) {
    const int bytes = RAG ? 4 * min(kBlock, a.L - i * kBlock) : -1;
    if (wave == 0)
      load_lds<4>(buffer_rsrc_n(lseg + (size_t)i * kBlock, bytes), 4 * lane, lv);
    else if (wave == 1)
      load_lds<4>(buffer_rsrc_n(ndltg + (size_t)i * kBlock, bytes), 4 * lane, ev);
  };
  auto load_block = [&](int i, char *qt, char *ot, float *lv, float *ev) __attribute__((always_inline)) {
    ldq.load(qg + (size_t)i * kBlock * lq, RAG ? a.L - i * kBlock : kBlock, lq, qt);
    ldo.load(dog + (size_t)i * kBlock * ldo_l, RAG ? a.L - i * kBlock : kBlock, ldo_l, ot);
    load_vec(i, lv, ev);
  };

  RowsBitmap<kDkvTB> pb;
  pb.init(dyn_lds, nqb);
  pb.build_rows(a.ix.col_ptr + (size_t)hidx * (nkb + 1), krows, a.ix.nnz, a.ix.row_idx, nqb,
                kDkvThreads, load_kv);
  RowsIter<kDkvTB> it;
  it.start(nqb, (krows[0] + 63) & ~63);
  auto advance = [&]() __attribute__((always_inline)) -> BwdPos {
    BwdPos p;
    p.valid = it.next(pb);
    p.j = it.j;
    p.mask = it.mask;
    return p;
  };
  auto listed = [&](const BwdPos &p) __attribute__((always_inline)) { return p.valid && k_valid && ((p.mask >> my_r) & 1u); };

  // An explicit stream of N MFMAs whose A operands come from LDS: the
  // operand of MFMA k + PF is read while MFMA k runs; a scheduling barrier
  // after each MFMA keeps this order.
  auto stream = [&](auto NN, auto fetch, auto mfma) __attribute__((always_inline)) {
    constexpr int N = decltype(NN)::value, PF = 4;
    bf16x8 op[PF + 1];
    static_for<PF>([&](auto K) __attribute__((always_inline)) { op[decltype(K)::value] = fetch(K); });
    static_for<N>([&](auto K) __attribute__((always_inline)) {
      constexpr int k = decltype(K)::value;
      if constexpr (k + PF < N) op[(k + PF) % (PF + 1)] = fetch(std::integral_constant<int, k + PF>{});
      mfma(K, op[k % (PF + 1)]);
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  // the exchange barrier: the pair's operand writes are complete in LDS (not
  // the tile loads in flight: no vmcnt wait)
  auto exchange_barrier = [&]() __attribute__((always_inline)) {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };

  // Half H of block i (tiles qt / ot, vectors lv / ev): S and dP, masks,
  // P and dS packed into bp / bds (the B operands of k-steps 2 H, 2 H + 1).
  // Element r of a score register set is query 32 H + 8 (r / 4) + 4 hh + r % 4.
  auto half_block = [&](auto HALF, const char *qt, const char *ot, const float *lv, const float *ev, int i,
                        bf16x8 (&bp)[2], bf16x8 (&bds)[2]) __attribute__((always_inline)) {
    constexpr int h = decltype(HALF)::value;
    f32x16 s = f32x16{}, dp;
    static_for<4>([&](auto G) __attribute__((always_inline)) {
      constexpr int g = decltype(G)::value;
      const f32x4 x = *(const f32x4 *)(ev + 32 * h + 8 * g + 4 * hh);
      static_for<4>([&](auto E) __attribute__((always_inline)) { dp[4 * g + decltype(E)::value] = x[decltype(E)::value]; });
    });
    // S and dP interleaved (two accumulator chains): MFMA k is S (k even) or
    // dP (k odd) of k-step k / 2
    stream(
        std::integral_constant<int, 2 * KS>{},
        [&](auto K) __attribute__((always_inline)) {
          constexpr int k = decltype(K)::value;
          return rd.row(k % 2 ? ot : qt, h, k / 2);
        },
        [&](auto K, const bf16x8 &op) __attribute__((always_inline)) {
          constexpr int k = decltype(K)::value;
          if constexpr (k % 2) dp = mfma_32x32x16(op, bv[k / 2], dp);
          else s = mfma_32x32x16(op, bk[k / 2], s);
        });
    // causal / token-window masks as -inf scores, one uniform branch each
    const int lim = k_tok - i * kBlock - 32 * h - 4 * hh;   // keys later than the query: offset < lim
    if (a.causal && kb >= i) {
      static_for<16>([&](auto R) __attribute__((always_inline)) {
        constexpr int r = decltype(R)::value;
        s[r] = mask_neg_inf(s[r], (8 * (r >> 2) + (r & 3)) - lim);
      });
    }
    if constexpr (RAG) {
      // queries past L of a partial last block: their Q and dO rows load as
      // zeros only when rows do not overlap in memory (row stride >= d), so
      // they are masked here as well
      if ((i + 1) * kBlock > a.L) {
        const int qlim = a.L - i * kBlock - 32 * h - 4 * hh;   // offsets below it are queries < L
        static_for<16>([&](auto R) __attribute__((always_inline)) {
          constexpr int r = decltype(R)::value;
          s[r] = mask_neg_inf(s[r], qlim - 1 - (8 * (r >> 2) + (r & 3)));
        });
      }
    }
    if constexpr (WIN) {
      // queries at or past key + window: offset >= lim + window
      if (kb >= a.sink_blk && i * kBlock + 63 >= k_wave + a.window) {
        const int hi = lim + a.window - 1;
        static_for<16>([&](auto R) __attribute__((always_inline)) {
          constexpr int r = decltype(R)::value;
          s[r] = mask_neg_inf(s[r], hi - (8 * (r >> 2) + (r & 3)));
        });
      }
    }
    static_for<4>([&](auto G) __attribute__((always_inline)) {
      constexpr int g = decltype(G)::value;
      const f32x4 l2 = *(const f32x4 *)(lv + 32 * h + 8 * g + 4 * hh);
      static_for<4>([&](auto E) __attribute__((always_inline)) {
        constexpr int e = decltype(E)::value, r = 4 * g + e;
        s[r] = fast_exp2(__builtin_fmaf(s[r], c, -l2[e]));   // P
        dp[r] = s[r] * dp[r];                                  // dS
      });
    });
    bp[0] = pack_half(s, 0);
    bp[1] = pack_half(s, 1);
    bds[0] = pack_half(dp, 0);
    bds[1] = pack_half(dp, 1);
  };
  // acc^T += tile^T X over k-steps ORDER of the block: x[j] is the B
  // operand of k-step j; MFMA k is k-step order[k / MT], dim tile k % MT
  auto accumulate = [&](const char *tile, const bf16x8 (&x)[4], auto ORDER) __attribute__((always_inline)) {
    stream(
        std::integral_constant<int, decltype(ORDER)::size * MT>{},
        [&](auto K) __attribute__((always_inline)) {
          constexpr int k = decltype(K)::value, j = decltype(ORDER)::value[k / MT];
          return rd.tr(tile, k % MT, j);
        },
        [&](auto K, const bf16x8 &op) __attribute__((always_inline)) {
          constexpr int k = decltype(K)::value, j = decltype(ORDER)::value[k / MT];
          acc[k % MT] = mfma_32x32x16(op, x[j], acc[k % MT]);
        });
  };

  BwdPos cur = advance(), nxt{false, 0, 0u};
  if (cur.valid) {
    nxt = advance();
    load_block(cur.j, q0, o0, l0, e0);
  }
  // Block of walk step t lives in slot t & 1; the next block's tiles load
  // into the other slot while this one is computed.  Per step: barrier
  // (tiles in, the previous exchange consumed), half block, exchange
  // barrier, dV / dK.  The two sides run separate copies of the loop, so
  // the register allocator never sees one side's values live in the other's.
  auto step = [&](auto PAR, auto SIDE1) __attribute__((always_inline)) -> bool {
    constexpr int P = decltype(PAR)::value;
    constexpr bool s1 = decltype(SIDE1)::value;
    if (!cur.valid) return false;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (nxt.valid) load_block(nxt.j, P ? q0 : q1, P ? o0 : o1, P ? l0 : l1, P ? e0 : e1);
    const char *qt = P ? q1 : q0, *ot = P ? o1 : o0;
    const float *lv = P ? l1 : l0, *ev = P ? e1 : e0;
    const bool lst = listed(cur);
    bf16x8 x[4];   // B operands of the block's k-steps (P for dV, dS for dK)
    const char *at = s1 ? qt : ot;   // A tile of the product: Q for dK, dO for dV
    if (lst) {
      bf16x8 bp[2], bds[2];
      half_block(std::integral_constant<int, s1 ? 1 : 0>{}, qt, ot, lv, ev, cur.j, bp, bds);
      // send what the partner's product needs, keep the own part and run
      // its k-steps before the exchange barrier (they overlap the partner's
      // vector work)
      xch[pair][s1][0][lane] = s1 ? bp[0] : bds[0];
      xch[pair][s1][1][lane] = s1 ? bp[1] : bds[1];
      x[2 * s1] = s1 ? bds[0] : bp[0];
      x[2 * s1 + 1] = s1 ? bds[1] : bp[1];
      if constexpr (s1)
        accumulate(at, x, KOrder<2, 3>{});
      else
        accumulate(at, x, KOrder<0, 1>{});
    }
    exchange_barrier();
    if (lst) {
      x[2 * !s1] = xch[pair][!s1][0][lane];
      x[2 * !s1 + 1] = xch[pair][!s1][1][lane];
      if constexpr (s1)
        accumulate(at, x, KOrder<0, 1>{});
      else
        accumulate(at, x, KOrder<2, 3>{});
    }
    cur = nxt;
    if (nxt.valid) nxt = advance();
    return true;
  };
  const std::integral_constant<int, 0> even;
  const std::integral_constant<int, 1> odd;
  if (side0) {
    while (step(even, std::false_type{}) && step(odd, std::false_type{})) {
    }
  } else {
    while (step(even, std::true_type{}) && step(odd, std::true_type{})) {
    }
  }

  // every wave is done with the tile slots (no loads in flight after the
  // walk): they stage the output rows, two waves per slot
  static_assert(kDkvWaves == 4 || kDkvWaves == 8, "output staging: waves 0-1 in q0, 2-3 q1, 4-5 o0, 6-7 o1");
  __syncthreads();
  if (!k_valid) return;
  const int ld_out = side0 ? (DENSE ? D : a.dvs.l) : (DENSE ? D : a.dks.l);
  bf16 *out = side0 ? (bf16 *)a.dv + (DENSE ? dense_base : a.dvs.at(bb, head)) + (size_t)k_wave * ld_out
                    : (bf16 *)a.dk + (DENSE ? dense_base : a.dks.at(bb, head)) + (size_t)k_wave * ld_out;
  char *stage = wave < 2 ? q0 : wave < 4 ? q1 : wave < 6 ? o0 : o1;
  store_rows_staged<D, RAG>(acc, side0 ? 1.0f : a.scale, stage + (wave & 1) * 32 * 2 * D, out, ld_out, lane,
                            a.L - k_wave);
}

// dK/dV launch with NW waves per workgroup (see bwd_dkdv_kernel)
template <int D, bool WIN, bool DENSE, bool RAG, int NW>
hipError_t launch_dkdv(const BwdArgs &a, hipStream_t s) {
  constexpr int TB = NW / 4;
  const int k_tiles = KeyTiles<TB>::per_head(a.ix.n_kblocks, a.kgroup);
  const size_t dyn_k = RowsBitmap<TB>::lds_bytes(a.ix.n_qblocks);
  hipError_t e = hipFuncSetAttribute((const void *)bwd_dkdv_kernel<D, WIN, DENSE, RAG, NW>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn_k);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, WIN, DENSE, RAG, NW>), dim3(a.B * a.H * k_tiles), dim3(NW * 64), dyn_k,
                     s, a);
  return hipSuccess;
}

template <int D, bool WIN, bool DENSE, bool RAG>
hipError_t launch_bwd(const BwdArgs &a, hipStream_t s) {
  const int q_tiles = (a.ix.n_qblocks + kBwdTB - 1) / kBwdTB;
  const int BH = a.B * a.H;
  const size_t dyn_q = RowsBitmap<kBwdTB>::lds_bytes(a.ix.n_kblocks);
  hipError_t e = hipFuncSetAttribute((const void *)bwd_dq_kernel<D, WIN, DENSE, RAG>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn_q);
  if (e != hipSuccess) return e;
  // dQ first: it leaves D and the base-2 LSE in the workspace
  hipLaunchKernelGGL((bwd_dq_kernel<D, WIN, DENSE, RAG>), dim3(BH * q_tiles), dim3(kBwdThreads), dyn_q, s, a);
  // BlockSparse (a per-head index grouped by strided class): two key blocks
  // per dK/dV workgroup; otherwise one
  if constexpr (!WIN) {
    e = a.kgroup > 1 ? launch_dkdv<D, WIN, DENSE, RAG, 8>(a, s) : launch_dkdv<D, WIN, DENSE, RAG, 4>(a, s);
  } else {
    e = launch_dkdv<D, WIN, DENSE, RAG, 4>(a, s);
  }
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace

size_t bwd_bf16_lds_bytes(int d, int n_blocks) {
  // dK/dV kernel: two Q and two dO slots, four 64-float vectors, the
  // packed-operand exchange (4 KB per pair), bitmaps
  const size_t tiles = 4 * (size_t)kBlock * 2 * d + 4 * kBlock * sizeof(float) + kDkvMaxPairs * 4 * 64 * 16;
  return tiles + RowsBitmap<2>::lds_bytes(n_blocks);
}

template <bool RAG>
static hipError_t launch_bwd_rag(const BwdArgs &a, bool dense, hipStream_t s) {
  if (a.window > 0) {
    if (dense) return a.d == 128 ? launch_bwd<128, true, true, RAG>(a, s) : launch_bwd<64, true, true, RAG>(a, s);
    return a.d == 128 ? launch_bwd<128, true, false, RAG>(a, s) : launch_bwd<64, true, false, RAG>(a, s);
  }
  if (dense) return a.d == 128 ? launch_bwd<128, false, true, RAG>(a, s) : launch_bwd<64, false, true, RAG>(a, s);
  return a.d == 128 ? launch_bwd<128, false, false, RAG>(a, s) : launch_bwd<64, false, false, RAG>(a, s);
}

hipError_t launch_bwd_bf16(const BwdArgs &a, hipStream_t s) {
  const bool dense = dense_layout(a.qs, a.H, a.L, a.d) && dense_layout(a.ks, a.H, a.L, a.d) &&
                     dense_layout(a.vs, a.H, a.L, a.d) && dense_layout(a.os, a.H, a.L, a.d) &&
                     dense_layout(a.dos, a.H, a.L, a.d) && dense_layout(a.dqs, a.H, a.L, a.d) &&
                     dense_layout(a.dks, a.H, a.L, a.d) && dense_layout(a.dvs, a.H, a.L, a.d);
  if (a.L % kBlock != 0) return launch_bwd_rag<true>(a, dense, s);
  return launch_bwd_rag<false>(a, dense, s);
}

}  // namespace attn
