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
//   * the workgroup walks the ascending union of its query blocks' KV-block
//     lists; each wave computes a KV block only if its own query block lists
//     it (no wasted MFMA work on the other block's entries);
//   * per KV block, K (row-major) and V (transposed, [d][key]) are staged in
//     LDS once and shared by the 4 waves; the next block's global loads are
//     in flight while the current one is computed;
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
constexpr int kFwdQB = kFwdWaves / 2;        // 64-token query blocks per tile

template <int D>
__global__ __launch_bounds__(kFwdThreads, 2) void fwd_bf16_kernel(FwdArgs a) {
  using G = TileGeom<D>;
  constexpr int KS = D / 16;   // k-steps of S^T = K Q^T
  constexpr int MT = D / 32;   // 32-row tiles of O^T
  __shared__ __attribute__((aligned(16))) bf16 klds[G::ROW_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 vlds[G::T_ELEMS];

  const int nqb = a.ix.n_qblocks;
  const int n_tiles = (nqb + kFwdQB - 1) / kFwdQB;
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

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 31, hh = lane >> 5;
  const int my_r = wave >> 1;
  const int qb = tile * kFwdQB + my_r;
  const bool q_valid = qb < nqb;
  const int q_tok = qb * kBlock + (wave & 1) * 32 + n;

  PairWalk walk;
  walk.ids = a.ix.col_idx;
  walk.n_ids = a.ix.n_kblocks;
  walk.init(a.ix.row_ptr + (size_t)hidx * (nqb + 1), tile * kFwdQB, nqb, a.ix.nnz);

  // Q^T operand of S^T = K Q^T: lane holds query n, d = 16 ks + 8 hh .. +7.
  bf16x8 bq[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    bq[ks] = q_valid ? *(const bf16x8 *)(qg + (size_t)q_tok * D + ks * 16 + hh * 8) : bf16x8{};

  f32x16 oacc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) oacc[mt] = f32x16{};
  float m_run = -INFINITY, l_part = 0.f;
  const float c = a.scale * kLog2e;

  RowStage<D, kFwdThreads> sk;
  TStage<D, kFwdThreads> sv;
  int j = walk.next();
  if (j != INT32_MAX) {
    sk.load(kg + (size_t)j * kBlock * D);
    sv.load(vg + (size_t)j * kBlock * D);
  }

  while (j != INT32_MAX) {
    __syncthreads();
    sk.store(klds);
    sv.store(vlds);
    __syncthreads();
    const bool active = q_valid && walk.has(my_r, j);
    walk.advance(j);
    const int jn = walk.next();
    if (jn != INT32_MAX) {
      sk.load(kg + (size_t)jn * kBlock * D);
      sv.load(vg + (size_t)jn * kBlock * D);
    }

    if (active) {
      // S^T (64 keys x 32 queries) as two 32x32 tiles.
      f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const bf16x8 ak = *(const bf16x8 *)(klds + (32 * t + n) * G::ROW + ks * 16 + hh * 8);
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
      mx = fmaxf(mx, __shfl_xor(mx, 32));
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
        const bf16x8 pb = pack_acc_operand(s[ks >> 1], ks & 1);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const bf16x8 av = *(const bf16x8 *)(vlds + (32 * mt + n) * G::TROW + ks * 16 + hh * 8);
          oacc[mt] = mfma_32x32x16(av, pb, oacc[mt]);
        }
      }
    }
    j = jn;
  }

  const float l_tot = l_part + __shfl_xor(l_part, 32);
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

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs &a, hipStream_t s) {
  const int n_tiles = (a.ix.n_qblocks + kFwdQB - 1) / kFwdQB;
  const int grid = a.B * a.H * n_tiles;
  if (a.d == 128)
    hipLaunchKernelGGL(fwd_bf16_kernel<128>, dim3(grid), dim3(kFwdThreads), 0, s, a);
  else
    hipLaunchKernelGGL(fwd_bf16_kernel<64>, dim3(grid), dim3(kFwdThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace attn
