// Prefill forward of static block-sparse causal attention, bf16 in / fp32
// accumulation / bf16 out, on the CDNA4 (gfx950) matrix cores.
//
// What it computes: for every query token, softmax attention restricted to
// the key blocks its query block lists in the static CSR index (sink, window
// and strided blocks of LongGen's sparse layers: mlsanity index page "A Little
// Goes a Long Way...", "Abstract (arXiv)"), with the FlashAttention-2 style
// tiled online softmax the pages name for their training kernel
// (atlas.scime.ai summary, "Approach").  Outputs O (bf16) and LSE (fp32,
// natural log of the sum of exp of the scaled scores).
//
// Work decomposition: one workgroup = 8 wave64s = 4 adjacent 64-token query
// blocks of one (batch, head); each wave owns 32 query rows.  Waves 0-3
// (group A, query blocks 0-1) and 4-7 (group B, query blocks 2-3) sit in
// pairs on the four SIMDs (wave w and w+4 share SIMD w).
//   * Ping-pong: per key block a wave runs a matrix-core step (P V and row
//     sum of the previous block and S of this block: 32 + 4 MFMAs) and a
//     vector step (mask, exp, pack, overflow test: ~100 VALU).  Group B runs one step behind group
//     A and every step ends at a workgroup barrier, so on each SIMD one wave
//     is in its matrix-core step while the other is in its vector step: the
//     two kinds of work overlap instead of queueing behind each other.
//   * The workgroup marks its four query blocks' KV-block lists in LDS
//     bitmaps and walks their union with scalar bit scans; a wave computes a
//     union block only if its own query block lists it.  The walk starts at
//     the 64-block boundary below the last query block and wraps around, so
//     the workgroups on one XCD stream the same key blocks at the same time
//     and L2 serves the repeats.
//   * K and V tiles go straight from global memory into LDS
//     (buffer_load_dwordx4 ... lds: no staging registers, no LDS store
//     instructions) into unpadded rows whose 16-byte chunks are XOR-swizzled
//     so the operand reads below hit all 64 banks.  Two K and two V slots;
//     the tiles of key block t+1 (K) and t (V) are issued two steps before
//     they are read, by the group that is in its vector step.
//   * Each wave computes S^T = K Q^T (keys x queries): a lane owns one query,
//     so row max / row sum need one swap between the two lane halves only.
//     V reaches the matrix cores through the transposing LDS read
//     (ds_read_b64_tr_b16) for O^T += V^T P^T; P goes fp32 -> bf16 (RNE).
//   * Online softmax in base 2 with scale*log2(e) folded into one FMA; the
//     running max is only moved when a block holds a P (against it) of 2^64
//     or more, found from the top exponent bit of the packed bf16 P (held
//     as 2^-63 P), so neither a per-block max nor the O rescale runs on most
//     blocks (exact: the final O / l uses the same reference point for both
//     sums).  The row sum l runs on the matrix cores (four 16x16x32 MFMAs
//     per block against a 0/1 selector) over the same bf16-rounded P that
//     enters the P V product, so numerator and denominator see identical
//     weights; on the vector units a row sum cost more than the MFMAs do.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "tiles.h"

namespace attn {
namespace {

constexpr int kFwdWaves = 8;                 // waves per workgroup
constexpr int kFwdThreads = kFwdWaves * 64;
constexpr int kFwdQB = 4;                    // query blocks per workgroup
constexpr int kFwdTileMajorTiles = 32;       // at most this many tiles per head (L <= 8192): tile-major block order
constexpr int kLoadWaves = 4;                // waves that issue the tile loads (group B)
constexpr float kFwdBias = 63.f;             // P is held as 2^-63 P (see the vector step; 0x1p63f below)

// LDS tile layout for direct global->LDS loads: 64 token rows of RB bytes,
// no padding; 16-byte chunk c of row r is stored at chunk c ^ swz(r).
template <int D>
struct FwdLayout {
  static constexpr int RB = 2 * D;                      // bytes per token row
  static constexpr int CPR = RB / 16;                   // chunks per row
  static constexpr int TILE = kBlock * RB;              // bytes per tile
  static constexpr int RPI = 1024 / RB;                 // rows per wave load instruction
  static constexpr int LPW = kBlock / kLoadWaves / RPI; // load instructions per loading wave per tile
  static_assert(LPW >= 1, "layout");
  // K is read as 16-byte row operands: 16 consecutive rows must use 16
  // distinct bank groups.
  __host__ __device__ static int kswz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  // V is read by ds_read_b64_tr_b16: 4 consecutive rows x 64 bytes per phase
  // must use all 64 banks.
  __host__ __device__ static int vswz(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

// Byte offset of the output staging inside the dynamic LDS (after the
// union bitmaps, 16-byte aligned).
__host__ __device__ inline size_t fwd_ostage_offset(int n_kblocks) {
  return (RowsBitmap<kFwdQB>::lds_bytes(n_kblocks) + 15) & ~(size_t)15;
}

// One position of the union walk.
struct WalkPos {
  bool valid;
  int j;          // key block
  uint32_t mask;  // bit r: listed by query block r of the workgroup
};

// RAG: L is not a multiple of 64 (the last block is partial); the range
// checks compile away otherwise.
template <int D, bool WIN, bool DENSE, bool RAG>
__global__ __launch_bounds__(kFwdThreads, 1) void fwd_bf16_kernel(FwdArgs a) {
  using Lay = FwdLayout<D>;
  constexpr int KS = D / 16;   // k-steps of S^T = K Q^T
  constexpr int MT = D / 32;   // 32-row tiles of O^T
  constexpr int RB = Lay::RB;
  constexpr int NS = 2 * KS;   // MFMAs of one block's scores (== MFMAs of its P V)
  static_assert(NS == 4 * MT, "step shape");
  // Two K and two V slots as four distinct objects: every load and read
  // below names its slot at compile time, so the compiler can see that the
  // tile loads in flight never touch the tile being read and does not wait
  // for them (a runtime-indexed slot made it wait for every load at once).
  __shared__ __attribute__((aligned(1024))) char k0[Lay::TILE];
  __shared__ __attribute__((aligned(1024))) char k1[Lay::TILE];
  __shared__ __attribute__((aligned(1024))) char v0[Lay::TILE];
  __shared__ __attribute__((aligned(1024))) char v1[Lay::TILE];
  // dynamic LDS: the union bitmaps, then each wave's 32 output rows on their
  // way to global memory (kept after the static tiles, whose offsets then
  // stay within the 16-bit immediates of the operand reads)
  extern __shared__ uint32_t dyn_lds[];

  const int nqb = a.ix.n_qblocks;
  const int n_tiles = (nqb + kFwdQB - 1) / kFwdQB;
  // Latest (heaviest) tiles first.  With many tiles per head, each XCD takes
  // a contiguous run of heads, tile by tile, so a head's tiles share its K/V
  // in that XCD's L2.  With few, that order would end each XCD's share on its
  // last head's heavy tiles, so blocks go tile-major over all heads instead:
  // the hardware deals consecutive blocks to the 8 XCDs in turn, so each XCD
  // holds every tile of the heads bh = x mod 8, heaviest first (3% faster at
  // 8K AttnSink; at 32K BlockSparse the L2 sharing weighs more, 1% slower).
  int bh, tile;
  if (n_tiles <= kFwdTileMajorTiles) {
    const int n_bh = gridDim.x / n_tiles;
    bh = blockIdx.x % n_bh;
    tile = n_tiles - 1 - blockIdx.x / n_bh;
  } else {
    const int lin = xcd_remap(blockIdx.x, gridDim.x);
    bh = lin / n_tiles;
    tile = n_tiles - 1 - lin % n_tiles;
  }
  const int hidx = a.ix.n_heads == 1 ? 0 : bh % a.H;

  // Token-row strides: compile-time for contiguous [B,H,L,d] tensors (so tile
  // addresses stay shifts and no stride is held in registers), else the
  // caller's strides.
  const int bb = bh / a.H, head = bh % a.H;
  const size_t dense_base = (size_t)bh * a.L * D;
  const int lq = DENSE ? D : a.qs.l, lk = DENSE ? D : a.ks.l, lv = DENSE ? D : a.vs.l;
  const int lo_ = DENSE ? D : a.os.l;
  const bf16 *qg = (const bf16 *)a.q + (DENSE ? dense_base : a.qs.at(bb, head));
  const bf16 *kg = (const bf16 *)a.k + (DENSE ? dense_base : a.ks.at(bb, head));
  const bf16 *vg = (const bf16 *)a.v + (DENSE ? dense_base : a.vs.at(bb, head));

  const int wave = uniform(threadIdx.x >> 6);
  const int grp = wave >> 2;                 // 0: group A, 1: group B (one step behind)
  const int lane = threadIdx.x & 63;
  const int n = lane & 31, hh = lane >> 5;
  const int my_r = 2 * grp + ((wave >> 1) & 1);
  const int qb = tile * kFwdQB + my_r;
  const bool q_valid = qb < nqb;
  const int q_wave = qb * kBlock + (wave & 1) * 32;  // first query of this wave
  const int q_tok = q_wave + n;

  // Q^T operand of S^T = K Q^T: lane holds query n, d = 16 ks + 8 hh .. +7
  // (loaded inside the bitmap build, behind the list reads; rows past L,
  // and every row of a query block past the last, load as zeros)
  bf16x8 bq[KS];
  auto load_q = [&]() __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rs =
        rows_rsrc<32>(qg + (size_t)q_wave * lq, q_valid ? a.L - q_wave : 0, 2 * lq, 2 * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) bq[ks] = load_row16(rs, 2 * (n * lq + ks * 16 + hh * 8));
  };

  // Per-lane byte offsets of this wave's share of a tile load (group B
  // waves load; a wave's share is 16 token rows).  Instruction i fills the
  // LDS rows i KB past the wave's first: that step is its immediate offset,
  // which moves the global address too, so it is taken out of the lane
  // offsets, and every instruction of a slot shares one LDS base.  The
  // descriptor base sits kShift bytes before the tile, so the offsets stay
  // non-negative for any row stride.
  constexpr int kShift = (Lay::LPW - 1) * Lay::RPI * RB;
  const int lw = wave & (kLoadWaves - 1);
  int goff_k[Lay::LPW], goff_v[Lay::LPW];
#pragma unroll
  for (int i = 0; i < Lay::LPW; ++i) {
    const int r = lw * (kBlock / kLoadWaves) + i * Lay::RPI + lane / Lay::CPR;
    const int pc = lane % Lay::CPR;
    goff_k[i] = 2 * (r * lk + ((pc ^ Lay::kswz(r)) << 3)) + kShift - i * Lay::RPI * RB;
    goff_v[i] = 2 * (r * lv + ((pc ^ Lay::vswz(r)) << 3)) + kShift - i * Lay::RPI * RB;
  }
  // tile of key block j of g (rows ld elements apart); the rows of a partial
  // last block past L load as zeros
  auto load_tile = [&](const bf16 *g, int j, int ld, char *lds, const int (&goff)[Lay::LPW])
                       __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rs =
        tile_rsrc(g + (size_t)j * kBlock * ld, RAG ? a.L - j * kBlock : kBlock, 2 * ld, RB, kShift);
    char *base = lds + lw * (kBlock / kLoadWaves) * RB;
    static_for<Lay::LPW>([&](auto I) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value;
      load_lds<16, i * Lay::RPI * RB>(rs, goff[i], base);
    });
  };

  // Per-lane LDS read offsets.  K row operand for k-step ks: row n (+32 t),
  // logical chunk 2 ks + hh.  V through the transposing read: source lane s
  // of 16-lane group gi addresses token 16 ks + 8 r + 4 hh + s/4 at dims
  // 32 mt + 16 gi + 4 (s % 4) (the lane algebra of SwzTile::tr in tiles.h).
  // The swizzles only touch chunk bits, so the offset of k-step ks (V:
  // dim tile mt) is one per-lane base XOR a constant: kofs(ks) = kbase ^
  // 32 ks, vofs(mt) = vbase ^ 64 mt (D = 128; D = 64 analogously).
  const int kbase = n * RB + ((hh ^ Lay::kswz(n)) << 4);
  auto kofs = [&](int ks) __attribute__((always_inline)) { return kbase ^ (ks << 5); };
  int vbase;
  {
    const int s = lane & 15, gi = (lane >> 4) & 1;
    vbase = (4 * hh + (s >> 2)) * RB + (((2 * gi + ((s & 3) >> 1)) ^ Lay::vswz(s >> 2)) << 4) +
            ((s & 1) << 3);
  }
  auto vofs = [&](int mt) __attribute__((always_inline)) { return vbase ^ (mt << 6); };
  auto v_operand = [&](const char *vt, int mt, int ks) __attribute__((always_inline)) -> bf16x8 {
    typedef short s4 __attribute__((ext_vector_type(4)));
    typedef short s8 __attribute__((ext_vector_type(8)));
    typedef __attribute__((address_space(3))) s4 lds_s4;
    const char *p = vt + vofs(mt) + 16 * ks * RB;
    const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)p);
    const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(p + 8 * RB));
    return __builtin_bit_cast(bf16x8, (s8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x16 oacc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) oacc[mt] = f32x16{};
  float m_run = -INFINITY;
  const float c = a.scale * kLog2e;
  // Row sums on the matrix cores: D += A P^T with v_mfma_f32_16x16x32_bf16,
  // P^T (the registers of one P V k-step) as its B operand and a 0/1
  // selector as A.  That B operand's k index 8 g + i (g = lane / 16) holds
  // key 8 (g / 2) + i of query 16 (g % 2) + lane % 16, so selector rows 0
  // and 8 take the groups with g even and rows 4 and 12 those with g odd;
  // D register 0 of lane l (rows 0, 4, 8, 12) is then the sum of its own
  // query l % 32.
  bf16x8 lsel;
  {
    const int m = lane & 15, g_odd = (lane >> 4) & 1;
    const bool one = g_odd ? (m == 4 || m == 12) : (m == 0 || m == 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) lsel[i] = one ? (bf16)1.0f : (bf16)0.0f;
  }
  f32x4 lacc = f32x4{};

  f32x16 sc[2];   // S^T of the current block (matrix-core step -> vector step)
  bf16x8 pk[4];   // packed P of the previous block (vector step -> matrix-core step)
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) pk[ks] = bf16x8{};

  // Matrix-core step: P V of the previous block (V tile vt, P in pk) and
  // S^T of the current block (K tile kt), interleaved.  It always issues all
  // 2 NS MFMAs, so the loop has no branches around matrix-core code: when
  // the previous block is not this wave's, pk is zero (P V adds zeros, as
  // the masked entries of a dense P would), and scores of a block that is
  // not this wave's are computed but never read.  The LDS operands of MFMA
  // pair i + PF are read while pair i runs; a scheduling barrier per pair
  // keeps the compiler from hoisting every read.
  // MFMA k of the step: the first 3 NS / 2 follow the pattern S, S, PV (S
  // MFMA number (k / 3) 2 + k % 3, PV MFMA number k / 3), the last NS / 2 are
  // PV MFMAs NS / 2 .. NS - 1.  Front-loading the scores lets the next vector
  // step start on them while the step's last P V products still run; every
  // accumulator's chain keeps at least 2 other MFMAs between its links.  The
  // LDS operand of MFMA k + PF is read while MFMA k runs.
  auto mfma_step = [&](const char *vt, const char *kt) __attribute__((always_inline)) {
    constexpr int NM = 2 * NS, NSP = 3 * NS / 2, PF = 4;
    constexpr int RS = NS / 8;   // one row-sum MFMA after every RS trailing P V MFMAs
    bf16x8 op[PF + 1];
    auto fetch = [&](auto K) __attribute__((always_inline)) {
      constexpr int k = decltype(K)::value;
      if constexpr (k < NSP && k % 3 != 2) {
        constexpr int si = (k / 3) * 2 + k % 3;
        op[k % (PF + 1)] = *(const bf16x8 *)(kt + kofs(si >> 1) + (si & 1) * 32 * RB);
      } else {
        constexpr int pi = k < NSP ? k / 3 : k - NS;
        op[k % (PF + 1)] = v_operand(vt, pi % MT, pi / MT);
      }
    };
    sc[0] = sc[1] = f32x16{};
    static_for<PF>(fetch);
    static_for<NM>([&](auto K) __attribute__((always_inline)) {
      constexpr int k = decltype(K)::value;
      if constexpr (k + PF < NM) fetch(std::integral_constant<int, k + PF>{});
      if constexpr (k < NSP && k % 3 != 2) {
        constexpr int si = (k / 3) * 2 + k % 3;
        sc[si & 1] = mfma_32x32x16(op[k % (PF + 1)], bq[si >> 1], sc[si & 1]);
      } else {
        constexpr int pi = k < NSP ? k / 3 : k - NS;
        oacc[pi % MT] = mfma_32x32x16(op[k % (PF + 1)], pk[pi / MT], oacc[pi % MT]);
      }
      if constexpr (k >= NSP && (k - NSP) % RS == RS - 1)
        lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lsel, pk[(k - NSP) / RS], lacc, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // Vector step of block j: causal mask, running max with rare rescale,
  // exps, packing of P and the row sum.
  auto vector_step = [&](int j) __attribute__((always_inline)) {
    // (the per-element loops below are expanded with static_for: in the
    // larger kernel variants a rolled loop would index the score registers
    // at run time and move them to scratch memory)
    if (a.causal && j >= qb) {
      // key offset in the block = 32 t + 8 (r / 4) + 4 hh + r % 4; compared
      // against a per-lane limit so the per-register part stays an immediate
      const int lim = q_tok - j * kBlock - 4 * hh;
      static_for<32>([&](auto E) __attribute__((always_inline)) {
        constexpr int t = decltype(E)::value / 16, r = decltype(E)::value % 16;
        sc[t][r] = mask_neg_inf(sc[t][r], lim - (32 * t + 8 * (r >> 2) + (r & 3)));
      });
    }
    if constexpr (WIN) {
      // token window: keys k <= q - window of blocks past the sink blocks
      // (only blocks holding such a key for one of this wave's queries)
      if (j >= a.sink_blk && j * kBlock <= q_wave + 31 - a.window) {
        const int lo = q_tok - a.window - j * kBlock - 4 * hh;
        static_for<32>([&](auto E) __attribute__((always_inline)) {
          constexpr int t = decltype(E)::value / 16, r = decltype(E)::value % 16;
          sc[t][r] = mask_neg_inf(sc[t][r], (32 * t + 8 * (r >> 2) + (r & 3)) - lo - 1);
        });
      }
    }
    // P' = exp2(s c - msub) of the block, packed into pk for the next P V;
    // returns the OR of the packed words.  k-step ks of P V takes registers
    // 8 (ks % 2) .. +7 of tile ks / 2.
    auto exps = [&](float msub) __attribute__((always_inline)) -> uint32_t {
      uint32_t o0 = 0u, o1 = 0u;   // two short OR chains
      static_for<4>([&](auto KS) __attribute__((always_inline)) {
        constexpr int ks = decltype(KS)::value;
        u32x4 w;
        static_for<4>([&](auto EE) __attribute__((always_inline)) {
          constexpr int e = decltype(EE)::value, r = 8 * (ks & 1) + 2 * e;
          const float p0 = fast_exp2(__builtin_fmaf(sc[ks >> 1][r], c, -msub));
          const float p1 = fast_exp2(__builtin_fmaf(sc[ks >> 1][r + 1], c, -msub));
          w[e] = pack_bf16x2(p0, p1);
          uint32_t &o = (e & 1) ? o1 : o0;
          o |= w[e];
        });
        pk[ks] = __builtin_bit_cast(bf16x8, w);
      });
      return o0 | o1;
    };
    // Lazy running max without a per-block max.  P is kept as
    // P' = 2^-kFwdBias P, P taken against the running max m_run, so the
    // top exponent bit of a packed bf16 P' (bit 14 of each half) is set
    // exactly when P >= 2^(kFwdBias + 1), and for inf and NaN.  A block with
    // such a P' takes the exact path: block max, rescale to it if it is
    // higher (so later blocks start from P <= 1 again), P' again.  A row with
    // no max yet needs no test of its own: m_run = -inf makes every P' +inf
    // (or NaN for a masked score), which sets that bit.  Between rescales P
    // stays below 2^64, far from fp32 overflow, and a P' of 2^-63 at the
    // running max keeps every P that matters (P >= 2^-63) a normal number.
    const uint32_t ow = exps(m_run + kFwdBias);
    if (__any((ow & 0x40004000u) != 0u)) {
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[t][r]);
      mx = xor32_max(mx);
      const float mc = mx * c;
      const bool need = mc > m_run;
      const float m_new = need ? mc : m_run;
      const float alpha = m_new == m_run ? 1.0f : fast_exp2(m_run - m_new);
      lacc[0] *= alpha;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) oacc[mt] *= alpha;
      m_run = m_new;
      exps(m_run == -INFINITY ? 0.f : m_run + kFwdBias);
    }
  };

  // The first matrix-core step multiplies pk = 0 by slot v1 before any
  // tile reached it: start it at zero so that product is exactly zero.
  for (int i = threadIdx.x; i < Lay::TILE / 16; i += kFwdThreads) ((u32x4 *)v1)[i] = u32x4{};
  RowsBitmap<kFwdQB> pb;
  pb.init(dyn_lds, a.ix.n_kblocks);
  pb.build(a.ix.row_ptr + (size_t)hidx * (nqb + 1), tile * kFwdQB, nqb, a.ix.nnz, a.ix.col_idx,
           a.ix.n_kblocks, kFwdThreads, load_q);
  RowsIter<kFwdQB> it;
  it.start(a.ix.n_kblocks, min(tile * kFwdQB + kFwdQB - 1, nqb - 1) & ~63);
  auto advance = [&]() __attribute__((always_inline)) -> WalkPos {
    WalkPos p;
    p.valid = it.next(pb);
    p.j = it.j;
    p.mask = it.mask;
    return p;
  };
  auto listed = [&](const WalkPos &p) __attribute__((always_inline)) { return p.valid && q_valid && ((p.mask >> my_r) & 1u); };

  // Walk window at even phase 2t: prev = block t-1, cur = t, nxt = t+1.
  WalkPos prev{false, 0, 0u}, cur = advance(), nxt{false, 0, 0u};
  if (cur.valid) {
    nxt = advance();
    if (grp == 1) load_tile(kg, cur.j, lk, k0, goff_k);
  }
  // Phases 2t and 2t+1 for t = 0 .. n (n = walk length): group A runs the
  // matrix-core step of walk block t in phase 2t and its vector step in
  // 2t+1; group B one phase later.  Both groups pass the same n+1 even and
  // n+1 odd barriers.  With P = t & 1, K of block t lives in slot k<P> and
  // V of block t in slot v<P>; K(t+1) and V(t) are issued at the start of
  // phase 2t and waited for at the start of phase 2t+2, where the barrier
  // also ends every read of the slots they overwrite.  The odd-phase barrier
  // only keeps the two groups a step apart: it orders no memory, so it does
  // not wait for tile loads in flight.  Each group has its own loop, unrolled
  // by two so that every slot is named at compile time, whose body is
  // "matrix-core step, then vector step": the register allocator then sees
  // straight-line state updates (a shared loop that switched roles by wave
  // made it copy the accumulators on every step).
  auto shift = [&]() __attribute__((always_inline)) {
    prev = cur;
    cur = nxt;
    if (nxt.valid) nxt = advance();
  };
  auto even_phase = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  // Tile loads of even phase 2t, issued by group B (in its vector step, so
  // the matrix-core waves never queue behind the address unit).
  auto issue_loads = [&](auto PAR) __attribute__((always_inline)) {
    constexpr int P = decltype(PAR)::value;
    if (nxt.valid) load_tile(kg, nxt.j, lk, P ? k0 : k1, goff_k);
    if (cur.valid) load_tile(vg, cur.j, lv, P ? v1 : v0, goff_v);
  };
  auto matrix_phase = [&](auto PAR) __attribute__((always_inline)) {
    constexpr int P = decltype(PAR)::value;
    mfma_step(P ? v0 : v1, P ? k1 : k0);
  };
  // vector step of a listed block; otherwise P = 0 for the next P V
  auto vector_or_zero = [&](const WalkPos &p) __attribute__((always_inline)) {
    if (listed(p)) {
      vector_step(p.j);
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) pk[ks] = bf16x8{};
    }
  };
  auto step_a = [&](auto PAR, int t) __attribute__((always_inline)) -> bool {
    if (t > 0) shift();
    if (!prev.valid && !cur.valid) return false;
    even_phase();
    matrix_phase(PAR);
    __builtin_amdgcn_s_barrier();
    vector_or_zero(cur);
    return true;
  };
  auto step_b = [&](auto PAR, int t) __attribute__((always_inline)) -> bool {
    if (t > 0) shift();
    if (!prev.valid && !cur.valid) return false;
    even_phase();
    issue_loads(PAR);
    vector_or_zero(prev);
    // this wave's tile loads land before its matrix step reads LDS, so the
    // compiler need not treat them as pending there
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    matrix_phase(PAR);
    return true;
  };
  const std::integral_constant<int, 0> even;
  const std::integral_constant<int, 1> odd;
  if (grp == 0) {
    for (int t = 0;; t += 2)
      if (!step_a(even, t) || !step_a(odd, t + 1)) break;
  } else {
    for (int t = 0;; t += 2)
      if (!step_b(even, t) || !step_b(odd, t + 1)) break;
  }

  if (!q_valid) return;
  const float l_tot = lacc[0];   // sum of P' of the row (bf16-rounded, as in P V)
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  // O leaves through the wave's own LDS area as contiguous row runs
  store_rows_staged<D, RAG>(oacc, inv, (char *)dyn_lds + fwd_ostage_offset(a.ix.n_kblocks) + wave * 32 * RB,
                       (bf16 *)a.o + (DENSE ? dense_base : a.os.at(bb, head)) + (size_t)q_wave * lo_, lo_,
                       lane, a.L - q_wave);
  if (hh == 0 && (!RAG || q_tok < a.L))
    // 2^63 l' = l exactly (a power-of-two scale): log2 of it, not of l', so
    // the LSE keeps full precision
    a.lse[(size_t)bh * a.L + q_tok] = l_tot > 0.f ? (m_run + fast_log2(l_tot * 0x1p63f)) * kLn2 : -INFINITY;
}

template <int D, bool WIN, bool DENSE, bool RAG>
hipError_t launch_fwd(const FwdArgs &a, hipStream_t s) {
  const int n_tiles = (a.ix.n_qblocks + kFwdQB - 1) / kFwdQB;
  const int grid = a.B * a.H * n_tiles;
  const size_t dyn = fwd_ostage_offset(a.ix.n_kblocks) + (size_t)kFwdWaves * 32 * FwdLayout<D>::RB;
  hipError_t e = hipFuncSetAttribute((const void *)fwd_bf16_kernel<D, WIN, DENSE, RAG>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, WIN, DENSE, RAG>), dim3(grid), dim3(kFwdThreads), dyn, s, a);
  return hipGetLastError();
}

template <int D, bool WIN>
hipError_t launch_fwd_layout(const FwdArgs &a, hipStream_t s) {
  return dense_layout(a.qs, a.H, a.L, D) && dense_layout(a.ks, a.H, a.L, D) &&
                 dense_layout(a.vs, a.H, a.L, D) && dense_layout(a.os, a.H, a.L, D)
             ? (a.L % kBlock ? launch_fwd<D, WIN, true, true>(a, s) : launch_fwd<D, WIN, true, false>(a, s))
             : (a.L % kBlock ? launch_fwd<D, WIN, false, true>(a, s) : launch_fwd<D, WIN, false, false>(a, s));
}

}  // namespace

size_t fwd_bf16_lds_bytes(int d, int n_kblocks) {
  // two K slots, two V slots, the waves' output staging, the union bitmaps
  return 4 * (size_t)kBlock * 2 * d + fwd_ostage_offset(n_kblocks) + (size_t)kFwdWaves * 32 * 2 * d;
}

hipError_t launch_fwd_bf16(const FwdArgs &a, hipStream_t s) {
  if (a.window > 0)
    return a.d == 128 ? launch_fwd_layout<128, true>(a, s) : launch_fwd_layout<64, true>(a, s);
  return a.d == 128 ? launch_fwd_layout<128, false>(a, s) : launch_fwd_layout<64, false>(a, s);
}

}  // namespace attn
