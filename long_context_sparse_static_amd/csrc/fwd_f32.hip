// Prefill forward in fp32 throughout (inputs, arithmetic and outputs), for
// the small exactness-checked workloads.  Same static block-sparse semantics
// as the bf16 kernel (LongGen sparse patterns: mlsanity index page "A Little
// Goes a Long Way...", "Abstract (arXiv)"), computed on the vector ALUs.
// 4 KG lanes per query row: 4 quarters of the head dimension x KG groups of
// 64 / KG keys of each block, so a workgroup of 256 lanes holds 64 / KG rows
// of one (batch, head, 64-token query block).  Each key group keeps its own
// running max, sum and output over the row's listed blocks; the groups are
// merged at the end.  Small grids take KG = 4 (four times the workgroups,
// each row's blocks four times shorter to walk); large ones KG = 1.  K and V of the
// listed blocks are staged in LDS, double-buffered: the next block's loads
// are in flight while the current one is computed.  Exponentials use expf
// (full fp32 accuracy); the path is latency bound, not throughput bound.
#include "device_common.h"
#include "kernels.h"

namespace attn {
namespace {

// LDS float offset of (key, column) of a staged 64 x D block: key group g
// (keys g * 64 / KG ..) is shifted by 4 g floats so the groups' reads fall in
// distinct banks.
template <int D, int KG>
__device__ __forceinline__ int f32_lds(int key, int col) {
  return key * D + (key / (kBlock / KG)) * 4 + col;
}

template <int D, int KG>
__global__ __launch_bounds__(256) void fwd_f32_kernel(FwdArgs a) {
  constexpr int DP = D / 4;                  // dims per lane
  constexpr int kF32Rows = 64 / KG;          // query rows per workgroup
  constexpr int kF32Keys = kBlock / KG;      // keys per group
  constexpr int SZ = kBlock * D + 4 * KG;
  constexpr int NL = kBlock * D / 4 / 256;   // 16-byte pieces of K (and of V) per thread per block
  __shared__ __attribute__((aligned(16))) float klds[2][SZ];
  __shared__ __attribute__((aligned(16))) float vlds[2][SZ];

  const int nqb = a.ix.n_qblocks;
  constexpr int QPB = kBlock / kF32Rows;     // workgroups per query block
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lin / (nqb * QPB);
  const int rem = lin % (nqb * QPB);
  const int qb = nqb - 1 - rem / QPB;        // later (longer) rows first
  const int h = bh % a.H;
  const int hidx = a.ix.n_heads == 1 ? 0 : h;
  const int bb = bh / a.H;
  const float *qg = (const float *)a.q + a.qs.at(bb, h);
  const float *kg = (const float *)a.k + a.ks.at(bb, h);
  const float *vg = (const float *)a.v + a.vs.at(bb, h);
  float *og = (float *)a.o + a.os.at(bb, h);

  const int t = threadIdx.x;
  const int r = t / (4 * KG), part = t & 3, grp = (t >> 2) & (KG - 1);
  const int q_tok = qb * kBlock + (rem % QPB) * kF32Rows + r;
  const bool q_in = q_tok < a.L;   // rows past L of a partial last block: computed, not stored
  float qv[DP], ov[DP];
#pragma unroll
  for (int i = 0; i < DP; ++i) {
    qv[i] = q_in ? qg[(size_t)q_tok * a.qs.l + part * DP + i] : 0.f;
    ov[i] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;

  // staging: piece x = t + 256 i of a block is key x / (D/4), columns
  // 4 (x % (D/4)) .. +3; keys past L are zeros (later than every query)
  f32x4 kreg[NL], vreg[NL];
  auto fetch = [&](int j) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int x = t + 256 * i, key = x / (D / 4), c4 = 4 * (x % (D / 4));
      const size_t row = (size_t)j * kBlock + key;
      const bool in = row < (size_t)a.L;
      kreg[i] = in ? *(const f32x4 *)(kg + row * a.ks.l + c4) : f32x4{};
      vreg[i] = in ? *(const f32x4 *)(vg + row * a.vs.l + c4) : f32x4{};
    }
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int x = t + 256 * i, key = x / (D / 4), c4 = 4 * (x % (D / 4));
      *(f32x4 *)&klds[buf][f32_lds<D, KG>(key, c4)] = kreg[i];
      *(f32x4 *)&vlds[buf][f32_lds<D, KG>(key, c4)] = vreg[i];
    }
  };
  // this lane's keys of block j (staged in buffer buf)
  auto compute = [&](int j, int buf) {
    float s[kF32Keys];
    float mx = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < kF32Keys; ++kk) {
      const int key = grp * kF32Keys + kk;
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < DP; ++i) acc = __builtin_fmaf(qv[i], klds[buf][f32_lds<D, KG>(key, part * DP + i)], acc);
      acc += __shfl_xor(acc, 1);
      acc += __shfl_xor(acc, 2);
      acc *= a.scale;
      const int kpos = j * kBlock + key;
      if (a.causal && kpos > q_tok) acc = -INFINITY;
      if (a.window > 0 && j >= a.sink_blk && kpos <= q_tok - a.window) acc = -INFINITY;
      s[kk] = acc;
      mx = fmaxf(mx, acc);
    }
    const float m_new = fmaxf(m_run, mx);
    if (m_new == -INFINITY) return;  // nothing allowed yet for this key group
    const float alpha = m_run == -INFINITY ? 0.f : expf(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < DP; ++i) ov[i] *= alpha;
    m_run = m_new;
#pragma unroll
    for (int kk = 0; kk < kF32Keys; ++kk) {
      const int key = grp * kF32Keys + kk;
      const float p = expf(s[kk] - m_new);
      l_run += p;
#pragma unroll
      for (int i = 0; i < DP; ++i) ov[i] = __builtin_fmaf(p, vlds[buf][f32_lds<D, KG>(key, part * DP + i)], ov[i]);
    }
  };

  const int32_t *rp = a.ix.row_ptr + (size_t)hidx * (nqb + 1);
  const int e0 = clamp_i(rp[qb], 0, a.ix.nnz);
  const int e1 = clamp_i(rp[qb + 1], e0, a.ix.nnz);
  auto next_valid = [&](int &e) -> int {   // key block of the first valid entry at or after e, or -1
    for (; e < e1; ++e) {
      const int j = a.ix.col_idx[e];
      if (j >= 0 && j < a.ix.n_kblocks) return j;
    }
    return -1;
  };
  int e = e0;
  int j = next_valid(e);
  if (j >= 0) {
    fetch(j);
    commit(0);
  }
  __syncthreads();
  int buf = 0;
  while (j >= 0) {
    ++e;
    const int jn = next_valid(e);
    if (jn >= 0) fetch(jn);   // in flight while block j is computed
    compute(j, buf);
    if (jn >= 0) commit(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    j = jn;
  }

  // merge the key groups of the row (lanes 4, 8, ... apart)
#pragma unroll
  for (int off = 4; off < 4 * KG; off <<= 1) {
    const float m2 = __shfl_xor(m_run, off);
    const float l2 = __shfl_xor(l_run, off);
    const float mn = fmaxf(m_run, m2);
    const float a1 = mn == -INFINITY ? 0.f : expf(m_run - mn);
    const float a2 = mn == -INFINITY ? 0.f : expf(m2 - mn);
#pragma unroll
    for (int i = 0; i < DP; ++i) ov[i] = ov[i] * a1 + __shfl_xor(ov[i], off) * a2;
    l_run = l_run * a1 + l2 * a2;
    m_run = mn;
  }
  if (!q_in || grp != 0) return;
  const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
#pragma unroll
  for (int i = 0; i < DP; ++i) og[(size_t)q_tok * a.os.l + part * DP + i] = ov[i] * inv;
  if (part == 0) a.lse[(size_t)bh * a.L + q_tok] = l_run > 0.f ? m_run + logf(l_run) : -INFINITY;
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs &a, hipStream_t s) {
  // four key groups (four workgroups per query block) while the grid would
  // not fill the chip with one workgroup per query block
  const int qblocks = a.B * a.H * a.ix.n_qblocks;
  const bool small = qblocks < 256;
  const int grid = qblocks * (small ? 4 : 1);
  if (a.d == 128) {
    if (small)
      hipLaunchKernelGGL((fwd_f32_kernel<128, 4>), dim3(grid), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((fwd_f32_kernel<128, 1>), dim3(grid), dim3(256), 0, s, a);
  } else {
    if (small)
      hipLaunchKernelGGL((fwd_f32_kernel<64, 4>), dim3(grid), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((fwd_f32_kernel<64, 1>), dim3(grid), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace attn
