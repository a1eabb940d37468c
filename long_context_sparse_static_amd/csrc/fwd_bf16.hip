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
// Work decomposition (one workgroup = 4 wave64s = 128 query tokens = two
// adjacent 64-token query blocks of one (batch, head)):
//   * the workgroup first marks both query blocks' KV-block lists in an LDS
//     bitmap and then walks their ascending union with scalar bit scans; a
//     wave computes a KV block only if its own query block lists it;
//   * per KV block, K and V are staged row-major in LDS once for the 4
//     waves, double-buffered: one barrier per block, the next block's global
//     loads in flight during the current block's math; V reaches the matrix
//     cores through the transposing LDS read (ds_read_b64_tr_b16), so no
//     transposition is ever written;
//   * each wave owns 32 query rows and computes S^T = K Q^T (keys x queries)
//     so that a lane owns one query: row max / row sum need no cross-lane
//     traffic except one swap between the two lane halves;
//   * O^T += V^T P^T accumulates in registers; P goes fp32 -> bf16 (RNE);
//   * online softmax in base 2 with scale*log2(e) folded into one FMA; the
//     running max is only moved when a block raises it by more than 2^8, so
//     the O rescale is skipped on most blocks (exact: the final O / l uses
//     the same reference point for both sums).
#include "device_common.h"
#include "kernels.h"
#include "tiles.h"

namespace attn {
namespace {

constexpr int kFwdWaves = 4;                 // waves per workgroup
constexpr int kFwdThreads = kFwdWaves * 64;

template <int D>
__global__ __launch_bounds__(kFwdThreads, 2) void fwd_bf16_kernel(FwdArgs a) {
  using G = TileGeom<D>;
  constexpr int KS = D / 16;   // k-steps of S^T = K Q^T
  constexpr int MT = D / 32;   // 32-row tiles of O^T
  __shared__ __attribute__((aligned(16))) bf16 klds[2][G::ROW_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 vlds[2][TrRead<D>::ELEMS];
  extern __shared__ uint32_t dyn_lds[];

  const int nqb = a.ix.n_qblocks;
  const int n_tiles = (nqb + 1) / 2;
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lin / n_tiles;
  const int tile = n_tiles - 1 - lin % n_tiles;  // heaviest (latest) tiles first
  const int h = bh % a.H;
  const int hidx = a.ix.n_heads == 1 ? 0 : h;

  const size_t base = (size_t)bh * a.L * D;
  const bf16 *qg = (const bf16 *)a.q + base;
  const bf16 *kg = (const bf16 *)a.k + base;
  const bf16 *vg = (const bf16 *)a.v + base;
  bf16 *og = (bf16 *)a.o + base;
  float *lg = a.lse + (size_t)bh * a.L;

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

  TrRead<D> vr;
  vr.init(lane);

  PairBitmap pb;
  pb.init(dyn_lds, a.ix.n_kblocks);
  pb.build(a.ix.row_ptr + (size_t)hidx * (nqb + 1), tile * 2, nqb, a.ix.nnz, a.ix.col_idx,
           a.ix.n_kblocks, kFwdThreads);
  PairIter it;
  it.start();

  f32x16 oacc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) oacc[mt] = f32x16{};
  float m_run = -INFINITY, l_part = 0.f;
  const float c = a.scale * kLog2e;

  RowStage<D, kFwdThreads> sk;
  RowStage<D, kFwdThreads, TrRead<D>::TRS> sv;
  bool have = it.next(pb);
  int j = it.j;
  bool act = q_valid && (my_r == 0 ? it.in0 : it.in1);
  if (have) {
    sk.load(kg + (size_t)j * kBlock * D);
    sv.load(vg + (size_t)j * kBlock * D);
    sk.store(klds[0]);
    sv.store(vlds[0]);
  }
  bool have_next = have && it.next(pb);
  if (have_next) {
    sk.load(kg + (size_t)it.j * kBlock * D);
    sv.load(vg + (size_t)it.j * kBlock * D);
  }
  int buf = 0;

  while (have) {
    // Block j is in buffer `buf`; every wave is done with the other buffer.
    __syncthreads();
    if (act) {
      const bf16 *kl = klds[buf];
      const bf16 *vl = vlds[buf];
      // S^T (64 keys x 32 queries) as two 32x32 tiles.
      f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const bf16x8 ak = *(const bf16x8 *)(kl + (32 * t + n) * G::ROW + ks * 16 + hh * 8);
          s[t] = mfma_32x32x16(ak, bq[ks], s[t]);
        }
      }
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
      const float msub = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(__builtin_fmaf(s[t][r], c, -msub));
          l_part += p;
          s[t][r] = p;
        }
      // O^T (D x 32 queries) += V^T (D x 64 keys) P^T (64 keys x 32 queries).
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 pbk = pack_acc_operand(s[ks >> 1], ks & 1);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const bf16x8 av = vr.load(vl, mt, ks);
          oacc[mt] = mfma_32x32x16(av, pbk, oacc[mt]);
        }
      }
    }
    if (have_next) {
      sk.store(klds[buf ^ 1]);
      sv.store(vlds[buf ^ 1]);
    }
    have = have_next;
    j = it.j;
    act = q_valid && (my_r == 0 ? it.in0 : it.in1);
    have_next = have && it.next(pb);
    if (have_next) {
      sk.load(kg + (size_t)it.j * kBlock * D);
      sv.load(vg + (size_t)it.j * kBlock * D);
    }
    buf ^= 1;
  }

  const float l_tot = xor32_sum(l_part);
  if (!q_valid) return;
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  bf16 *orow = og + (size_t)q_tok * D;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 w;
      w[0] = pack_bf16x2(oacc[mt][4 * g] * inv, oacc[mt][4 * g + 1] * inv);
      w[1] = pack_bf16x2(oacc[mt][4 * g + 2] * inv, oacc[mt][4 * g + 3] * inv);
      *(u32x2 *)(orow + 32 * mt + 8 * g + 4 * hh) = w;
    }
  if (hh == 0) lg[q_tok] = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
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
  const size_t stat = 2 * (kBlock * (d + 8) + kBlock * (d + 32)) * sizeof(uint16_t);
  return stat + PairBitmap::lds_bytes(n_kblocks);
}

hipError_t launch_fwd_bf16(const FwdArgs &a, hipStream_t s) {
  return a.d == 128 ? launch_fwd<128>(a, s) : launch_fwd<64>(a, s);
}

}  // namespace attn
