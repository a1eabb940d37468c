// Backward pass of static block-sparse causal attention (bf16 tensors, fp32
// accumulation) for context-extension training of LongGen's sparse layers
// (mlsanity index page "A Little Goes a Long Way...", "Abstract (arXiv)": the
// sparse architecture is what gets trained during length extension; the
// training kernel is FlashAttention-2 based: atlas.scime.ai summary,
// "Approach").
//
// With P = exp(scale * Q K^T - LSE) on the allowed (query, key) pairs:
//   D  = rowsum(dO * O)                       bwd_delta_kernel
//   dV = P^T dO,  dK = scale * dS^T Q          bwd_dkdv_kernel   (key-tile major,
//        with dS = P * (dO V^T - D)                                 walks the CSC)
//   dQ = scale * dS K                          bwd_dq_kernel     (query-tile major,
//                                                                   walks the CSR)
// P and dS are recomputed per block pair from the forward's LSE, never stored.
// Splitting dQ into its own pass keeps every output written by exactly one
// workgroup: no atomics, bitwise-deterministic results.
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

// D = rowsum(dO * O) and the base-2 LSE (lse * log2 e; +inf for an empty
// row, so that P = exp2(s - lse2) = 0 there) per token.
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdArgs a) {
  constexpr int LPR = D / 8;      // lanes per row
  constexpr int RPB = 256 / LPR;  // rows per workgroup
  const size_t total = (size_t)a.B * a.H * a.L;
  const size_t row = (size_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int c = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < total) {
    const int bh = (int)(row / a.L), l = (int)(row % a.L);
    const int bb = bh / a.H, head = bh % a.H;
    const bf16 *op = (const bf16 *)a.o + a.os.at(bb, head) + (size_t)l * a.os.l;
    const bf16 *gp = (const bf16 *)a.dout + a.dos.at(bb, head) + (size_t)l * a.dos.l;
    const u32x4 o = *(const u32x4 *)(op + c * 8);
    const u32x4 g = *(const u32x4 *)(gp + c * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc += bf16_lo(o[i]) * bf16_lo(g[i]) + bf16_hi(o[i]) * bf16_hi(g[i]);
  }
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) acc += __shfl_xor(acc, off);
  if (row < total && c == 0) {
    a.delta[row] = acc;
    const float l = a.lse[row];
    a.lse2[row] = l == -INFINITY ? INFINITY : l * kLog2e;
  }
}

// Reads 16 consecutive fp32 values of a per-token vector laid out in LDS as
// the rows of a 32x32 accumulator tile: element r is token
// 32*tile + 8*(r/4) + 4*hh + r%4.
__device__ __forceinline__ void load_rows16(const float *lds, int tile, int hh, float out[16]) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const f32x4 v = *(const f32x4 *)(lds + 32 * tile + 8 * g + 4 * hh);
#pragma unroll
    for (int e = 0; e < 4; ++e) out[4 * g + e] = v[e];
  }
}

// Packs registers 8 half .. 8 half + 7 of a 32x32 accumulator tile (scaled
// by nothing) into the B operand of a 32x32x16 MFMA whose k index runs over
// the tile's rows (see pack_acc_operand in tiles.h).
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
template <int D, bool WIN, bool DENSE>
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
  const int ldo = DENSE ? D : a.dos.l, ldq = DENSE ? D : a.dqs.l;
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
  const bf16 *qp = (const bf16 *)a.q + (DENSE ? dense_base : a.qs.at(bb, head)) + (size_t)q_tok * lq;
  const bf16 *dop = (const bf16 *)a.dout + (DENSE ? dense_base : a.dos.at(bb, head)) + (size_t)q_tok * ldo;

  bf16x8 bq[KS], bdo[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    bq[ks] = q_valid ? *(const bf16x8 *)(qp + ks * 16 + hh * 8) : bf16x8{};
    bdo[ks] = q_valid ? *(const bf16x8 *)(dop + ks * 16 + hh * 8) : bf16x8{};
  }
  const float c = a.scale * kLog2e;
  float lse2 = INFINITY, dlt = 0.f;
  if (q_valid) {
    lse2 = a.lse2[(size_t)bh * a.L + q_tok];
    dlt = a.delta[(size_t)bh * a.L + q_tok];
  }

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
           a.ix.n_kblocks, kBwdThreads);
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
    const bool diag = a.causal && j >= qb;
    // key offset in the block = 32 t + 8 (r / 4) + 4 hh + r % 4
    const int lim = q_tok - j * kBlock - 4 * hh;
    // token window: keys k <= q - window of blocks past the sink blocks
    const bool wedge = WIN && j >= a.sink_blk && j * kBlock <= q_wave + 31 - a.window;
    const int lo = lim - a.window;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = fast_exp2(__builtin_fmaf(s[t][r], c, -lse2));
        if (diag && 32 * t + 8 * (r >> 2) + (r & 3) > lim) p = 0.f;
        if (wedge && 32 * t + 8 * (r >> 2) + (r & 3) <= lo) p = 0.f;
        s[t][r] = p * (dp[t][r] - dlt);  // dS^T
      }
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
    kl.load(kg + (size_t)cur.j * kBlock * lk, k0);
    vl.load(vg + (size_t)cur.j * kBlock * lv, v0);
  }
  // Block of walk step t lives in slot t & 1; the next block's tiles load into
  // the other slot while this one is computed.
  auto step = [&](auto PAR) __attribute__((always_inline)) -> bool {
    constexpr int P = decltype(PAR)::value;
    if (!cur.valid) return false;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (nxt.valid) {
      kl.load(kg + (size_t)nxt.j * kBlock * lk, P ? k0 : k1);
      vl.load(vg + (size_t)nxt.j * kBlock * lv, P ? v0 : v1);
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

  if (!q_valid) return;
  bf16 *out = (bf16 *)a.dq + (DENSE ? dense_base : a.dqs.at(bb, head)) + (size_t)q_tok * ldq;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 w;
      w[0] = pack_bf16x2(acc[mt][4 * g] * a.scale, acc[mt][4 * g + 1] * a.scale);
      w[1] = pack_bf16x2(acc[mt][4 * g + 2] * a.scale, acc[mt][4 * g + 3] * a.scale);
      *(u32x2 *)(out + 32 * mt + 8 * g + 4 * hh) = w;
    }
}

// ----------------------------------------------------------------------------
// dK, dV: one workgroup per 128 key tokens (two key blocks), union of their
// CSC lists.  Per wave (32 keys, lane = key), per 32-query half m of a listed
// query block:
//   S = Q K^T, dP = dO V^T, P = exp2(S c - LSE2), dS = P * (dP - D)
//   dV^T += dO^T P,  dK^T += Q^T dS
// Q and dO are read as rows and transposed (kBothRead).
// ----------------------------------------------------------------------------
template <int D, bool WIN, bool DENSE>
__global__ __launch_bounds__(kBwdThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_dkdv_kernel(BwdArgs a) {
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
  extern __shared__ uint32_t dyn_lds[];

  const int nkb = a.ix.n_kblocks, nqb = a.ix.n_qblocks;
  using KTiles = KeyTiles<kBwdTB>;
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
  int krows[kBwdTB];
#pragma unroll
  for (int r = 0; r < kBwdTB; ++r) krows[r] = kt.block(tile, r);
  // token-row strides: compile-time for contiguous [B,H,L,d] tensors
  const int bb = bh / a.H, head = bh % a.H;
  const size_t dense_base = (size_t)bh * a.L * D;
  const int lq = DENSE ? D : a.qs.l, ldo_l = DENSE ? D : a.dos.l;
  const bf16 *qg = (const bf16 *)a.q + (DENSE ? dense_base : a.qs.at(bb, head));
  const bf16 *dog = (const bf16 *)a.dout + (DENSE ? dense_base : a.dos.at(bb, head));
  const float *lseg = a.lse2 + (size_t)bh * a.L;
  const float *dltg = a.delta + (size_t)bh * a.L;

  const int wave = uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 31, hh = lane >> 5;
  const int my_r = wave >> 1;
  const int kb = krows[my_r];
  const bool k_valid = kb >= 0;
  const int k_wave = kb * kBlock + (wave & 1) * 32;  // first key of this wave
  const int k_tok = k_wave + n;
  const bf16 *kp = (const bf16 *)a.k + (DENSE ? dense_base : a.ks.at(bb, head)) +
                   (size_t)k_tok * (DENSE ? D : a.ks.l);
  const bf16 *vp = (const bf16 *)a.v + (DENSE ? dense_base : a.vs.at(bb, head)) +
                   (size_t)k_tok * (DENSE ? D : a.vs.l);

  bf16x8 bk[KS], bv[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    bk[ks] = k_valid ? *(const bf16x8 *)(kp + ks * 16 + hh * 8) : bf16x8{};
    bv[ks] = k_valid ? *(const bf16x8 *)(vp + ks * 16 + hh * 8) : bf16x8{};
  }
  const float c = a.scale * kLog2e;
  f32x16 dk[MT], dv[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) dk[mt] = dv[mt] = f32x16{};

  QT rd;
  rd.init_reads(lane);
  typename QT::template Loader<kBwdWaves> ldq, ldo;   // Q and dO tiles (own row strides)
  ldq.init(wave, lane, lq);
  ldo.init(wave, lane, ldo_l);
  // the two 64-float per-token vectors of a query block: wave 0 loads LSE2,
  // wave 1 the D values (4 bytes per lane)
  auto load_vec = [&](int i, float *lv, float *ev) __attribute__((always_inline)) {
    if (wave == 0)
      load_lds<4>(buffer_rsrc(lseg + (size_t)i * kBlock), 4 * lane, lv);
    else if (wave == 1)
      load_lds<4>(buffer_rsrc(dltg + (size_t)i * kBlock), 4 * lane, ev);
  };
  auto load_block = [&](int i, char *qt, char *ot, float *lv, float *ev) __attribute__((always_inline)) {
    ldq.load(qg + (size_t)i * kBlock * lq, qt);
    ldo.load(dog + (size_t)i * kBlock * ldo_l, ot);
    load_vec(i, lv, ev);
  };

  RowsBitmap<kBwdTB> pb;
  pb.init(dyn_lds, nqb);
  pb.build_rows(a.ix.col_ptr + (size_t)hidx * (nkb + 1), krows, a.ix.nnz, a.ix.row_idx, nqb,
                kBwdThreads);
  RowsIter<kBwdTB> it;
  it.start(nqb, (krows[0] + 63) & ~63);
  auto advance = [&]() __attribute__((always_inline)) -> BwdPos {
    BwdPos p;
    p.valid = it.next(pb);
    p.j = it.j;
    p.mask = it.mask;
    return p;
  };
  auto listed = [&](const BwdPos &p) __attribute__((always_inline)) { return p.valid && k_valid && ((p.mask >> my_r) & 1u); };

  // One query block as one explicit stream of 8 KS MFMAs (one wave per SIMD,
  // so the wave itself must keep the matrix core fed):
  //   i in [0, 2KS)      S and dP of query half 0 (row operands)
  //   i in [2KS, 4KS)    S and dP of half 1, with half 0's softmax-gradient
  //                      VALU spread between them
  //   i in [4KS, 6KS)    dV, dK of half 0 (transposed operands), with half
  //                      1's VALU spread between them
  //   i in [6KS, 8KS)    dV, dK of half 1
  // The LDS operand of MFMA i + PF is read while MFMA i runs; a scheduling
  // barrier after each MFMA keeps this order.
  auto block_work = [&](const char *qt, const char *ot, const float *lv, const float *ev, int i) __attribute__((always_inline)) {
    constexpr int NM = 8 * KS;       // MFMAs per query block
    constexpr int PF = 4;            // operand prefetch distance
    const bool diag = a.causal && kb >= i;
    // token window: queries q >= k + window, for keys past the sink blocks
    const bool wedge = WIN && kb >= a.sink_blk && i * kBlock + 63 >= k_wave + a.window;
    f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
    bf16x8 bp[2][2], bds[2][2];
    // LSE2 and D of both query halves, read from LDS during the score stage
    // (one 4-float read per MFMA slot), long before the gradient VALU needs
    // them: read right before their use, each read waited for every operand
    // read still in flight and stalled the matrix stream on every fourth
    // element.
    f32x4 l2v[2][4], dlv[2][4];
    bf16x8 opnd[PF + 1];
    // operand of MFMA k
    auto fetch = [&](int k) __attribute__((always_inline)) {
      bf16x8 v;
      if (k < 4 * KS) {                 // scores: k = 4 ks' + 2 m' + which
        const int m = k / (2 * KS), kk = k % (2 * KS), ks = kk >> 1;
        v = rd.row((kk & 1) ? ot : qt, m, ks);
      } else {                          // accumulation: half, mt, which
        const int kk = k - 4 * KS, m = kk / (4 * MT), r = kk % (4 * MT);
        const int half = r / (2 * MT), mt = (r % (2 * MT)) >> 1;
        v = rd.tr((r & 1) ? qt : ot, mt, 2 * m + half);
      }
      opnd[k % (PF + 1)] = v;
    };
    auto mfma_k = [&](int k) __attribute__((always_inline)) {
      const bf16x8 av = opnd[k % (PF + 1)];
      if (k < 4 * KS) {
        const int m = k / (2 * KS), kk = k % (2 * KS), ks = kk >> 1;
        if (kk & 1) dp[m] = mfma_32x32x16(av, bv[ks], dp[m]);
        else s[m] = mfma_32x32x16(av, bk[ks], s[m]);
      } else {
        const int kk = k - 4 * KS, m = kk / (4 * MT), r = kk % (4 * MT);
        const int half = r / (2 * MT), mt = (r % (2 * MT)) >> 1;
        if (r & 1) dk[mt] = mfma_32x32x16(av, bds[m][half], dk[mt]);
        else dv[mt] = mfma_32x32x16(av, bp[m][half], dv[mt]);
      }
    };
    // softmax-gradient VALU of half m, element r (query offset 32 m +
    // 8 (r / 4) + 4 hh + r % 4; masked when the key is later)
    // vector read v (0 .. 15) of the score stage: half v / 8, LSE2 or D,
    // group v % 4 (query offset 8 g + 4 hh .. +3 of the half)
    auto read_vec = [&](int v) __attribute__((always_inline)) {
      const int m = v >> 3, g = v & 3;
      const float *src = (v & 4) ? ev : lv;
      const f32x4 x = *(const f32x4 *)(src + 32 * m + 8 * g + 4 * hh);
      if (v & 4) dlv[m][g] = x;
      else l2v[m][g] = x;
    };
    // The softmax-gradient VALU of element r of half m in two parts, each a
    // short dependency chain; a slot runs part A of its elements and part B
    // of the previous slot's, so no slot waits on its own exp before the
    // next MFMA can issue.
    //   A: P = exp2(S c - LSE2), into s
    auto grad_a = [&](int m, int r) __attribute__((always_inline)) {
      s[m][r] = fast_exp2(__builtin_fmaf(s[m][r], c, -l2v[m][r >> 2][r & 3]));
    };
    //   B: masks, dS = P (dP - D) into dp; packing of each completed 8
    auto grad_b = [&](int m, int r) __attribute__((always_inline)) {
      const int lim = k_tok - i * kBlock - 32 * m - 4 * hh;
      float p = s[m][r];
      if (diag && 8 * (r >> 2) + (r & 3) < lim) p = 0.f;
      if (wedge && 8 * (r >> 2) + (r & 3) >= lim + a.window) p = 0.f;
      s[m][r] = p;
      dp[m][r] = p * (dp[m][r] - dlv[m][r >> 2][r & 3]);
      if (r == 7 || r == 15) {
        const int half = r >> 3;
        bp[m][half] = pack_half(s[m], half);
        bds[m][half] = pack_half(dp[m], half);
      }
    };
    constexpr int E = 16 / (2 * KS);   // gradient elements per MFMA slot
    auto stage = [&](auto STAGE) __attribute__((always_inline)) {
      constexpr int st = decltype(STAGE)::value;
#pragma unroll
      for (int kk = 0; kk < 2 * KS; ++kk) {
        const int k = st * 2 * KS + kk;
        if (k + PF < NM) fetch(k + PF);
        mfma_k(k);
        if constexpr (st == 0) {
#pragma unroll
          for (int v = kk * E; v < (kk + 1) * E; ++v) read_vec(v);
        }
        // the 16 elements of half st - 1 over the 2 KS slots of stages 1
        // and 2; part B of a stage's last slot runs in the next stage's
        // first slot (its packed P and dS are needed from that stage's
        // middle on)
        if constexpr (st == 1 || st == 2) {
#pragma unroll
          for (int r = kk * E; r < (kk + 1) * E; ++r) grad_a(st - 1, r);
        }
        if constexpr (st >= 1 && st <= 3) {
          if (kk > 0 && st <= 2) {
#pragma unroll
            for (int r = (kk - 1) * E; r < kk * E; ++r) grad_b(st - 1, r);
          }
          if (kk == 0 && st >= 2) {
#pragma unroll
            for (int r = 16 - E; r < 16; ++r) grad_b(st - 2, r);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
#pragma unroll
    for (int k = 0; k < PF; ++k) fetch(k);
    stage(std::integral_constant<int, 0>{});
    stage(std::integral_constant<int, 1>{});
    stage(std::integral_constant<int, 2>{});
    stage(std::integral_constant<int, 3>{});
  };

  BwdPos cur = advance(), nxt{false, 0, 0u};
  if (cur.valid) {
    nxt = advance();
    load_block(cur.j, q0, o0, l0, e0);
  }
  auto step = [&](auto PAR) __attribute__((always_inline)) -> bool {
    constexpr int P = decltype(PAR)::value;
    if (!cur.valid) return false;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (nxt.valid) load_block(nxt.j, P ? q0 : q1, P ? o0 : o1, P ? l0 : l1, P ? e0 : e1);
    if (listed(cur)) block_work(P ? q1 : q0, P ? o1 : o0, P ? l1 : l0, P ? e1 : e0, cur.j);
    cur = nxt;
    if (nxt.valid) nxt = advance();
    return true;
  };
  const std::integral_constant<int, 0> even;
  const std::integral_constant<int, 1> odd;
  while (step(even) && step(odd)) {
  }

  if (!k_valid) return;
  bf16 *dko = (bf16 *)a.dk + (DENSE ? dense_base : a.dks.at(bb, head)) + (size_t)k_tok * (DENSE ? D : a.dks.l);
  bf16 *dvo = (bf16 *)a.dv + (DENSE ? dense_base : a.dvs.at(bb, head)) + (size_t)k_tok * (DENSE ? D : a.dvs.l);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 wk, wv;
      wk[0] = pack_bf16x2(dk[mt][4 * g] * a.scale, dk[mt][4 * g + 1] * a.scale);
      wk[1] = pack_bf16x2(dk[mt][4 * g + 2] * a.scale, dk[mt][4 * g + 3] * a.scale);
      wv[0] = pack_bf16x2(dv[mt][4 * g], dv[mt][4 * g + 1]);
      wv[1] = pack_bf16x2(dv[mt][4 * g + 2], dv[mt][4 * g + 3]);
      *(u32x2 *)(dko + 32 * mt + 8 * g + 4 * hh) = wk;
      *(u32x2 *)(dvo + 32 * mt + 8 * g + 4 * hh) = wv;
    }
}

template <int D, bool WIN, bool DENSE>
hipError_t launch_bwd(const BwdArgs &a, hipStream_t s) {
  const size_t rows = (size_t)a.B * a.H * a.L;
  const int rpb = 256 / (D / 8);
  const int grid_delta = (int)((rows + rpb - 1) / rpb);
  const int q_tiles = (a.ix.n_qblocks + kBwdTB - 1) / kBwdTB;
  const int k_tiles = KeyTiles<kBwdTB>::per_head(a.ix.n_kblocks, a.kgroup);
  const int BH = a.B * a.H;
  const size_t dyn_k = RowsBitmap<kBwdTB>::lds_bytes(a.ix.n_qblocks);
  const size_t dyn_q = RowsBitmap<kBwdTB>::lds_bytes(a.ix.n_kblocks);
  hipError_t e = hipFuncSetAttribute((const void *)bwd_dkdv_kernel<D, WIN, DENSE>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn_k);
  if (e == hipSuccess)
    e = hipFuncSetAttribute((const void *)bwd_dq_kernel<D, WIN, DENSE>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn_q);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_delta_kernel<D>, dim3(grid_delta), dim3(256), 0, s, a);
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, WIN, DENSE>), dim3(BH * k_tiles), dim3(kBwdThreads), dyn_k, s, a);
  hipLaunchKernelGGL((bwd_dq_kernel<D, WIN, DENSE>), dim3(BH * q_tiles), dim3(kBwdThreads), dyn_q, s, a);
  return hipGetLastError();
}

}  // namespace

size_t bwd_bf16_lds_bytes(int d, int n_blocks) {
  // dK/dV kernel: two Q and two dO slots, four 64-float vectors, bitmaps
  const size_t tiles = 4 * (size_t)kBlock * 2 * d + 4 * kBlock * sizeof(float);
  return tiles + RowsBitmap<kBwdTB>::lds_bytes(n_blocks);
}

hipError_t launch_bwd_bf16(const BwdArgs &a, hipStream_t s) {
  const bool dense = dense_layout(a.qs, a.H, a.L, a.d) && dense_layout(a.ks, a.H, a.L, a.d) &&
                     dense_layout(a.vs, a.H, a.L, a.d) && dense_layout(a.os, a.H, a.L, a.d) &&
                     dense_layout(a.dos, a.H, a.L, a.d) && dense_layout(a.dqs, a.H, a.L, a.d) &&
                     dense_layout(a.dks, a.H, a.L, a.d) && dense_layout(a.dvs, a.H, a.L, a.d);
  if (a.window > 0) {
    if (dense) return a.d == 128 ? launch_bwd<128, true, true>(a, s) : launch_bwd<64, true, true>(a, s);
    return a.d == 128 ? launch_bwd<128, true, false>(a, s) : launch_bwd<64, true, false>(a, s);
  }
  if (dense) return a.d == 128 ? launch_bwd<128, false, true>(a, s) : launch_bwd<64, false, true>(a, s);
  return a.d == 128 ? launch_bwd<128, false, false>(a, s) : launch_bwd<64, false, false>(a, s);
}

}  // namespace attn
