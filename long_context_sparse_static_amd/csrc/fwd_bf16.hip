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
// Work decomposition: one workgroup = 4 wave64s = 2 adjacent 64-token query
// blocks of one (batch, head); each wave owns 32 query rows; two workgroups
// per CU (two waves per SIMD).
//   * The workgroup marks both query blocks' KV-block lists in an LDS bitmap
//     and walks their ascending union with scalar bit scans; a wave computes
//     a union block only if its own query block lists it.
//   * K and V tiles go straight from global memory into LDS
//     (global_load_lds_dwordx4: no staging registers, no LDS store
//     instructions) into unpadded rows whose 16-byte chunks are XOR-swizzled
//     so the operand reads below hit all 64 banks.
//   * Each wave computes S^T = K Q^T (keys x queries): a lane owns one query,
//     so row max / row sum need one swap between the two lane halves only.
//     V reaches the matrix cores through the transposing LDS read
//     (ds_read_b64_tr_b16) for O^T += V^T P^T; P goes fp32 -> bf16 (RNE).
//   * Double buffering: the next block's tiles load while the current one is
//     computed.  Within a block the second half of the exps is interleaved
//     with the first half of P V; across the two waves of a SIMD the
//     matrix-core work of one overlaps the softmax of the other.
//   * Online softmax in base 2 with scale*log2(e) folded into one FMA; the
//     running max is only moved when a block raises it by more than 2^8, so
//     the O rescale is skipped on most blocks (exact: the final O / l uses
//     the same reference point for both sums).  The row sum l adds the same
//     bf16-rounded P that enters the P V product (two per dot2 instruction),
//     so numerator and denominator see identical weights.
//   * The union walk starts at the 64-block boundary below the workgroup's
//     last query block and wraps around, so neighbouring workgroups stream
//     the same key blocks at the same time and L2 serves the repeats.
#include "device_common.h"
#include "kernels.h"
#include "tiles.h"

namespace attn {
namespace {

constexpr int kFwdWaves = 4;                 // waves per workgroup
constexpr int kFwdThreads = kFwdWaves * 64;

// LDS tile layout for direct global->LDS loads: 64 token rows of RB bytes,
// no padding; 16-byte chunk c of row r is stored at chunk c ^ swz(r).
template <int D>
struct FwdLayout {
  static constexpr int RB = 2 * D;                      // bytes per token row
  static constexpr int CPR = RB / 16;                   // chunks per row
  static constexpr int TILE = kBlock * RB;              // bytes per tile
  static constexpr int RPI = 1024 / RB;                 // rows per wave load instruction
  static constexpr int LPW = kBlock / kFwdWaves / RPI;  // load instructions per wave per tile
  static_assert(LPW >= 1, "layout");
  // K is read as 16-byte row operands: 16 consecutive rows must use 16
  // distinct bank groups.
  __host__ __device__ static int kswz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  // V is read by ds_read_b64_tr_b16: 4 consecutive rows x 64 bytes per phase
  // must use all 64 banks.
  __host__ __device__ static int vswz(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

template <int D>
__global__ __launch_bounds__(kFwdThreads, 2) void fwd_bf16_kernel(FwdArgs a) {
  using Lay = FwdLayout<D>;
  constexpr int KS = D / 16;   // k-steps of S^T = K Q^T
  constexpr int MT = D / 32;   // 32-row tiles of O^T
  constexpr int RB = Lay::RB;
  constexpr int NS = 2 * KS;   // MFMAs of one block's scores
  __shared__ __attribute__((aligned(1024))) char klds[2][Lay::TILE];
  __shared__ __attribute__((aligned(1024))) char vlds[2][Lay::TILE];
  extern __shared__ uint32_t dyn_lds[];

  const int nqb = a.ix.n_qblocks;
  const int n_tiles = (nqb + 1) / 2;
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lin / n_tiles;
  const int tile = n_tiles - 1 - lin % n_tiles;  // heaviest (latest) tiles first
  const int hidx = a.ix.n_heads == 1 ? 0 : bh % a.H;

  const size_t base = (size_t)bh * a.L * D;
  const bf16 *qg = (const bf16 *)a.q + base;
  const bf16 *kg = (const bf16 *)a.k + base;
  const bf16 *vg = (const bf16 *)a.v + base;

  const int wave = uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 31, hh = lane >> 5;
  const int my_r = wave >> 1;
  const int qb = tile * 2 + my_r;
  const bool q_valid = qb < nqb;
  const int q_tok = qb * kBlock + (wave & 1) * 32 + n;

  // Q^T operand of S^T = K Q^T: lane holds query n, d = 16 ks + 8 hh .. +7.
  bf16x8 bq[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    bq[ks] = q_valid ? *(const bf16x8 *)(qg + (size_t)q_tok * D + ks * 16 + hh * 8) : bf16x8{};

  // Per-lane global element offsets of this wave's share of a tile load.
  int goff_k[Lay::LPW], goff_v[Lay::LPW];
#pragma unroll
  for (int i = 0; i < Lay::LPW; ++i) {
    const int r = wave * (kBlock / kFwdWaves) + i * Lay::RPI + lane / Lay::CPR;
    const int pc = lane % Lay::CPR;
    goff_k[i] = r * D + ((pc ^ Lay::kswz(r)) << 3);
    goff_v[i] = r * D + ((pc ^ Lay::vswz(r)) << 3);
  }
  auto load_tile = [&](const bf16 *g, char *lds, const int (&goff)[Lay::LPW]) {
#pragma unroll
    for (int i = 0; i < Lay::LPW; ++i)
      __builtin_amdgcn_global_load_lds(
          (const void *)(g + goff[i]),
          (__attribute__((address_space(3))) void *)(lds + (wave * (kBlock / kFwdWaves) + i * Lay::RPI) * RB),
          16, 0, 0);
  };

  // Per-lane LDS read offsets.  K row operand for k-step ks: row n (+32 t),
  // logical chunk 2 ks + hh.  V through the transposing read: source lane s
  // of 16-lane group gi addresses token 16 ks + 8 r + 4 hh + s/4 at dims
  // 32 mt + 16 gi + 4 (s % 4) (see TrRead in tiles.h for the lane algebra).
  int kofs[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) kofs[ks] = n * RB + (((2 * ks + hh) ^ Lay::kswz(n)) << 4);
  int vofs[MT];
  {
    const int s = lane & 15, gi = (lane >> 4) & 1;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      vofs[mt] = (4 * hh + (s >> 2)) * RB +
                 (((4 * mt + 2 * gi + ((s & 3) >> 1)) ^ Lay::vswz(s >> 2)) << 4) + ((s & 1) << 3);
  }
  auto v_operand = [&](const char *vt, int mt, int ks) -> bf16x8 {
    typedef short s4 __attribute__((ext_vector_type(4)));
    typedef short s8 __attribute__((ext_vector_type(8)));
    typedef __attribute__((address_space(3))) s4 lds_s4;
    const char *p = vt + vofs[mt] + 16 * ks * RB;
    const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)p);
    const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(p + 8 * RB));
    return __builtin_bit_cast(bf16x8, (s8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // i-th MFMA of S^T = K Q^T (i = 2 ks + t)
  auto s_step = [&](f32x16 (&s)[2], const char *kt, int i) {
    const int ks = i >> 1, t = i & 1;
    const bf16x8 ak = *(const bf16x8 *)(kt + kofs[ks] + t * 32 * RB);
    s[t] = mfma_32x32x16(ak, bq[ks], s[t]);
  };

  f32x16 oacc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) oacc[mt] = f32x16{};
  float m_run = -INFINITY, l_part = 0.f;
  const float c = a.scale * kLog2e;

  // Block j's causal mask, running max and rare rescale.  Returns the
  // exponent offset for the block's exps.
  auto softmax_pre = [&](f32x16 (&s)[2], int j) -> float {
    if (a.causal && j >= qb) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j * kBlock + 32 * t + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (key > q_tok) s[t][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
    mx = xor32_max(mx);
    const float mc = mx * c;
    const bool need = mc > m_run + 8.0f;
    if (__any(need)) {
      const float m_new = need ? mc : m_run;
      const float alpha = m_new == m_run ? 1.0f : fast_exp2(m_run - m_new);
      l_part *= alpha;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) oacc[mt] *= alpha;
      m_run = m_new;
    }
    return m_run == -INFINITY ? 0.f : m_run;
  };
  auto softmax_exp = [&](f32x16 (&s)[2], float msub, int e) {
    const int t = e >> 4, r = e & 15;
    s[t][r] = fast_exp2(__builtin_fmaf(s[t][r], c, -msub));
  };
  // k-step ks of O^T (D x 32 queries) += V^T (D x 64 keys) P^T (64 keys x 32 q)
  auto pv_ks = [&](f32x16 (&p)[2], const char *vt, int ks) {
    // The packed words are built here, not read back out of the bf16x8:
    // extracting 32-bit words of a bit-cast bf16x8 for the dot2 compiled to
    // four reads of word 0 (hipcc, ROCm 7.2).
    u32x4 pw;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 8 * (ks & 1) + 2 * e;
      const uint32_t w = pack_bf16x2(p[ks >> 1][r], p[ks >> 1][r + 1]);
      l_part = sum_bf16x2(w, l_part);
      pw[e] = w;
    }
    const bf16x8 pbk = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) oacc[mt] = mfma_32x32x16(v_operand(vt, mt, ks), pbk, oacc[mt]);
  };
  // Softmax + P V of block j (scores in s, V tile in vt): the exps of the
  // second 32 keys are interleaved with the first half of P V.
  auto block_work = [&](f32x16 (&s)[2], int j, const char *vt) {
    const float msub = softmax_pre(s, j);
#pragma unroll
    for (int e = 0; e < 16; ++e) softmax_exp(s, msub, e);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      pv_ks(s, vt, ks);
#pragma unroll
      for (int e = 16 + ks * 8; e < 24 + ks * 8; ++e) softmax_exp(s, msub, e);
    }
    pv_ks(s, vt, 2);
    pv_ks(s, vt, 3);
  };

  PairBitmap pb;
  pb.init(dyn_lds, a.ix.n_kblocks);
  pb.build(a.ix.row_ptr + (size_t)hidx * (nqb + 1), tile * 2, nqb, a.ix.nnz, a.ix.col_idx,
           a.ix.n_kblocks, kFwdThreads);
  RowsIter<2> it;
  it.start(a.ix.n_kblocks, min(tile * 2 + 1, nqb - 1) & ~63);
  auto listed_by_me = [&](uint32_t mask) { return q_valid && ((mask >> my_r) & 1u); };

  // ---- double-buffered walk: block j in buffers [ib] while block j+1 loads
  // straight into buffers [ib ^ 1] ----
  bool have = it.next(pb);
  int j = it.j;
  bool listed = listed_by_me(it.mask);
  if (have) {
    load_tile(kg + (size_t)j * kBlock * D, klds[0], goff_k);
    load_tile(vg + (size_t)j * kBlock * D, vlds[0], goff_v);
  }
  int ib = 0;
  while (have) {
    // every wave's loads of block j have landed and every wave is done with
    // the other buffers
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const bool have_n = it.next(pb);
    const int jn = it.j;
    const bool listed_n = listed_by_me(it.mask);
    if (have_n) {
      load_tile(kg + (size_t)jn * kBlock * D, klds[ib ^ 1], goff_k);
      load_tile(vg + (size_t)jn * kBlock * D, vlds[ib ^ 1], goff_v);
    }
    if (listed) {
      f32x16 sc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int i = 0; i < NS; ++i) s_step(sc, klds[ib], i);
      block_work(sc, j, vlds[ib]);
    }
    have = have_n;
    j = jn;
    listed = listed_n;
    ib ^= 1;
  }

  if (!q_valid) return;
  const float l_tot = xor32_sum(l_part);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  bf16 *orow = (bf16 *)a.o + base + (size_t)q_tok * D;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 w;
      w[0] = pack_bf16x2(oacc[mt][4 * g] * inv, oacc[mt][4 * g + 1] * inv);
      w[1] = pack_bf16x2(oacc[mt][4 * g + 2] * inv, oacc[mt][4 * g + 3] * inv);
      *(u32x2 *)(orow + 32 * mt + 8 * g + 4 * hh) = w;
    }
  if (hh == 0)
    a.lse[(size_t)bh * a.L + q_tok] = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
}

template <int D>
hipError_t launch_fwd(const FwdArgs &a, hipStream_t s) {
  const int n_tiles = (a.ix.n_qblocks + 1) / 2;
  const int grid = a.B * a.H * n_tiles;
  const size_t dyn = PairBitmap::lds_bytes(a.ix.n_kblocks);
  hipError_t e = hipFuncSetAttribute((const void *)fwd_bf16_kernel<D>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fwd_bf16_kernel<D>, dim3(grid), dim3(kFwdThreads), dyn, s, a);
  return hipGetLastError();
}

}  // namespace

size_t fwd_bf16_lds_bytes(int d, int n_kblocks) {
  return 4 * (size_t)kBlock * 2 * d + PairBitmap::lds_bytes(n_kblocks);
}

hipError_t launch_fwd_bf16(const FwdArgs &a, hipStream_t s) {
  return a.d == 128 ? launch_fwd<128>(a, s) : launch_fwd<64>(a, s);
}

}  // namespace attn
