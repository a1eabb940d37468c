// Prefill forward in fp32 throughout (inputs, arithmetic and outputs), for
// the small exactness-checked workloads.  Same static block-sparse semantics
// as the bf16 kernel (LongGen sparse patterns: mlsanity index page "A Little
// Goes a Long Way...", "Abstract (arXiv)"), computed on the vector ALUs: one
// workgroup per (batch, head, 64-token query block), four lanes per query
// row, each lane owning a quarter of the head dimension.  Per listed KV block
// the 64 scores of a row are formed first, then one rescale, then P V.
// Exponentials use expf (full fp32 accuracy); this path is latency bound, not
// throughput bound.
#include "device_common.h"
#include "kernels.h"

namespace attn {
namespace {

template <int D>
__global__ __launch_bounds__(256) void fwd_f32_kernel(FwdArgs a) {
  constexpr int DP = D / 4;  // dims per lane
  __shared__ __attribute__((aligned(16))) float klds[kBlock * D];
  __shared__ __attribute__((aligned(16))) float vlds[kBlock * D];

  const int nqb = a.ix.n_qblocks;
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lin / nqb;
  const int qb = nqb - 1 - lin % nqb;
  const int h = bh % a.H;
  const int hidx = a.ix.n_heads == 1 ? 0 : h;
  const int bb = bh / a.H;
  const float *qg = (const float *)a.q + a.qs.at(bb, h);
  const float *kg = (const float *)a.k + a.ks.at(bb, h);
  const float *vg = (const float *)a.v + a.vs.at(bb, h);
  float *og = (float *)a.o + a.os.at(bb, h);

  const int t = threadIdx.x;
  const int qi = t >> 2, part = t & 3;
  const int q_tok = qb * kBlock + qi;
  float qv[DP], ov[DP];
  const bool q_in = q_tok < a.L;   // rows past L of a partial last block: computed, not stored
#pragma unroll
  for (int i = 0; i < DP; ++i) {
    qv[i] = q_in ? qg[(size_t)q_tok * a.qs.l + part * DP + i] : 0.f;
    ov[i] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;

  const int32_t *rp = a.ix.row_ptr + (size_t)hidx * (nqb + 1);
  const int e0 = clamp_i(rp[qb], 0, a.ix.nnz);
  const int e1 = clamp_i(rp[qb + 1], e0, a.ix.nnz);
  for (int e = e0; e < e1; ++e) {
    const int j = a.ix.col_idx[e];
    if (j < 0 || j >= a.ix.n_kblocks) continue;
    __syncthreads();
    for (int i = t; i < kBlock * D / 4; i += blockDim.x) {
      const size_t row = (size_t)j * kBlock + i / (D / 4), c4 = 4 * (i % (D / 4));
      const bool in = row < (size_t)a.L;   // keys past L: zeros (later than every query, so masked)
      ((f32x4 *)klds)[i] = in ? *(const f32x4 *)(kg + row * a.ks.l + c4) : f32x4{};
      ((f32x4 *)vlds)[i] = in ? *(const f32x4 *)(vg + row * a.vs.l + c4) : f32x4{};
    }
    __syncthreads();
    float s[kBlock];
    float mx = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < kBlock; ++kk) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < DP; ++i) acc = __builtin_fmaf(qv[i], klds[kk * D + part * DP + i], acc);
      acc += __shfl_xor(acc, 1);
      acc += __shfl_xor(acc, 2);
      acc *= a.scale;
      if (a.causal && j * kBlock + kk > q_tok) acc = -INFINITY;
      if (a.window > 0 && j >= a.sink_blk && j * kBlock + kk <= q_tok - a.window) acc = -INFINITY;
      s[kk] = acc;
      mx = fmaxf(mx, acc);
    }
    const float m_new = fmaxf(m_run, mx);
    if (m_new == -INFINITY) continue;  // nothing allowed yet in this row
    const float alpha = m_run == -INFINITY ? 0.f : expf(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < DP; ++i) ov[i] *= alpha;
    m_run = m_new;
#pragma unroll
    for (int kk = 0; kk < kBlock; ++kk) {
      const float p = expf(s[kk] - m_new);
      l_run += p;
#pragma unroll
      for (int i = 0; i < DP; ++i) ov[i] = __builtin_fmaf(p, vlds[kk * D + part * DP + i], ov[i]);
    }
  }
  if (!q_in) return;
  const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
#pragma unroll
  for (int i = 0; i < DP; ++i) og[(size_t)q_tok * a.os.l + part * DP + i] = ov[i] * inv;
  if (part == 0) a.lse[(size_t)bh * a.L + q_tok] = l_run > 0.f ? m_run + logf(l_run) : -INFINITY;
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs &a, hipStream_t s) {
  const int grid = a.B * a.H * a.ix.n_qblocks;
  if (a.d == 128)
    hipLaunchKernelGGL(fwd_f32_kernel<128>, dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(fwd_f32_kernel<64>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace attn
