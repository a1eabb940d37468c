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
#include "device_common.h"
#include "kernels.h"
#include "tiles.h"

namespace attn {
namespace {

constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = kBwdWaves * 64;
constexpr int kBwdTB = kBwdWaves / 2;  // 64-token blocks per tile (32 rows per wave)

template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdArgs a) {
  constexpr int LPR = D / 8;      // lanes per row
  constexpr int RPB = 256 / LPR;  // rows per workgroup
  const size_t total = (size_t)a.B * a.H * a.L;
  const size_t row = (size_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int c = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < total) {
    const u32x4 o = *(const u32x4 *)((const bf16 *)a.o + row * D + c * 8);
    const u32x4 g = *(const u32x4 *)((const bf16 *)a.dout + row * D + c * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc += bf16_lo(o[i]) * bf16_lo(g[i]) + bf16_hi(o[i]) * bf16_hi(g[i]);
  }
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) acc += __shfl_xor(acc, off);
  if (row < total && c == 0) a.delta[row] = acc;
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

// ----------------------------------------------------------------------------
// dQ: one workgroup per 128 query tokens (two query blocks), union of their
// CSR lists.  Per wave (32 queries, lane = query):
//   S^T = K Q^T, dP^T = V dO^T, dS^T = P^T * (dP^T - D), dQ^T += K^T dS^T
// ----------------------------------------------------------------------------
template <int D>
struct DqBuf {
  bf16 k[TileGeom<D>::ROW_ELEMS];
  bf16 v[TileGeom<D>::ROW_ELEMS];
  bf16 kt[TileGeom<D>::T_ELEMS];
};

template <int D>
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_dq_kernel(BwdArgs a) {
  using G = TileGeom<D>;
  constexpr int KS = D / 16, MT = D / 32;
  __shared__ __attribute__((aligned(16))) DqBuf<D> lds[2];
  extern __shared__ uint32_t dyn_lds[];

  const int nqb = a.ix.n_qblocks;
  const int n_tiles = (nqb + kBwdTB - 1) / kBwdTB;
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lin / n_tiles;
  const int tile = n_tiles - 1 - lin % n_tiles;
  const int hidx = a.ix.n_heads == 1 ? 0 : bh % a.H;
  const size_t base = (size_t)bh * a.L * D;
  const bf16 *kg = (const bf16 *)a.k + base;
  const bf16 *vg = (const bf16 *)a.v + base;

  const int wave = uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 31, hh = lane >> 5;
  const int my_r = wave >> 1;
  const int qb = tile * kBwdTB + my_r;
  const bool q_valid = qb < nqb;
  const int q_tok = qb * kBlock + (wave & 1) * 32 + n;
  const size_t qrow = base + (size_t)q_tok * D;

  bf16x8 bq[KS], bdo[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    bq[ks] = q_valid ? *(const bf16x8 *)((const bf16 *)a.q + qrow + ks * 16 + hh * 8) : bf16x8{};
    bdo[ks] = q_valid ? *(const bf16x8 *)((const bf16 *)a.dout + qrow + ks * 16 + hh * 8) : bf16x8{};
  }
  const float c = a.scale * kLog2e;
  float lse2 = INFINITY, dlt = 0.f;
  if (q_valid) {
    const float l = a.lse[(size_t)bh * a.L + q_tok];
    lse2 = l == -INFINITY ? INFINITY : l * kLog2e;  // empty row: P = 0
    dlt = a.delta[(size_t)bh * a.L + q_tok];
  }

  TReadBases tb;
  tb.init(n, hh);

  PairBitmap pb;
  pb.init(dyn_lds, a.ix.n_kblocks);
  pb.build(a.ix.row_ptr + (size_t)hidx * (nqb + 1), tile * kBwdTB, nqb, a.ix.nnz, a.ix.col_idx,
           a.ix.n_kblocks, kBwdThreads);
  PairIter it;
  it.start(a.ix.n_kblocks);

  f32x16 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16{};

  RowStage<D, kBwdThreads> sk, sv;
  TStage<D, kBwdThreads> skt;
  auto load = [&](int jj) {
    const size_t off = (size_t)jj * kBlock * D;
    sk.load(kg + off);
    sv.load(vg + off);
    skt.load(kg + off);
  };
  auto store = [&](DqBuf<D> &b) {
    sk.store(b.k);
    sv.store(b.v);
    skt.store(b.kt);
  };
  bool have = it.next(pb);
  int j = it.j;
  bool act = q_valid && (my_r == 0 ? it.in0 : it.in1);
  if (have) {
    load(j);
    store(lds[0]);
  }
  bool have_next = have && it.next(pb);
  if (have_next) load(it.j);
  int buf = 0;
  while (have) {
    __syncthreads();
    if (act) {
      const DqBuf<D> &bb = lds[buf];
      f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const bf16x8 ak = *(const bf16x8 *)(bb.k + (32 * t + n) * G::ROW + ks * 16 + hh * 8);
          const bf16x8 av = *(const bf16x8 *)(bb.v + (32 * t + n) * G::ROW + ks * 16 + hh * 8);
          s[t] = mfma_32x32x16(ak, bq[ks], s[t]);
          dp[t] = mfma_32x32x16(av, bdo[ks], dp[t]);
        }
      const bool diag = a.causal && j >= qb;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(__builtin_fmaf(s[t][r], c, -lse2));
          if (diag) {
            const int key = j * kBlock + 32 * t + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (key > q_tok) p = 0.f;
          }
          s[t][r] = p * (dp[t][r] - dlt);  // dS^T
        }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 bds = pack_acc_operand(s[ks >> 1], ks & 1);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const bf16x8 akt = *(const bf16x8 *)((const char *)bb.kt + tb.at(mt, ks));
          acc[mt] = mfma_32x32x16(akt, bds, acc[mt]);
        }
      }
    }
    if (have_next) store(lds[buf ^ 1]);
    have = have_next;
    j = it.j;
    act = q_valid && (my_r == 0 ? it.in0 : it.in1);
    have_next = have && it.next(pb);
    if (have_next) load(it.j);
    buf ^= 1;
  }
  if (!q_valid) return;
  bf16 *out = (bf16 *)a.dq + qrow;
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
// ----------------------------------------------------------------------------
template <int D>
struct DkvBuf {
  bf16 q[TileGeom<D>::ROW_ELEMS];
  bf16 dout[TileGeom<D>::ROW_ELEMS];
  bf16 qt[TileGeom<D>::T_ELEMS];
  bf16 dot[TileGeom<D>::T_ELEMS];
  float lse2[kBlock];
  float dlt[kBlock];
};

template <int D>
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_dkdv_kernel(BwdArgs a) {
  using G = TileGeom<D>;
  constexpr int KS = D / 16, MT = D / 32;
  __shared__ __attribute__((aligned(16))) DkvBuf<D> lds[2];
  extern __shared__ uint32_t dyn_lds[];

  const int nkb = a.ix.n_kblocks, nqb = a.ix.n_qblocks;
  const int n_tiles = (nkb + kBwdTB - 1) / kBwdTB;
  const int BH = a.B * a.H;
  // Long CSC columns (the sink block, early blocks of full attention) are the
  // first tiles of each head: start every head's tile 0 before anything else
  // on its XCD, then walk the heads' remaining tiles in order.
  int bh, tile;
  if (BH % kNumXcd == 0 && n_tiles > 1) {
    const int hpx = BH / kNumXcd;
    const int xcd = blockIdx.x % kNumXcd;
    int s = blockIdx.x / kNumXcd;
    if (s < hpx) {
      bh = xcd * hpx + s;
      tile = 0;
    } else {
      s -= hpx;
      bh = xcd * hpx + s / (n_tiles - 1);
      tile = 1 + s % (n_tiles - 1);
    }
  } else {
    bh = blockIdx.x / n_tiles;
    tile = blockIdx.x % n_tiles;
  }
  const int hidx = a.ix.n_heads == 1 ? 0 : bh % a.H;
  const size_t base = (size_t)bh * a.L * D;
  const bf16 *qg = (const bf16 *)a.q + base;
  const bf16 *dog = (const bf16 *)a.dout + base;
  const float *lseg = a.lse + (size_t)bh * a.L;
  const float *dltg = a.delta + (size_t)bh * a.L;

  const int wave = uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 31, hh = lane >> 5;
  const int my_r = wave >> 1;
  const int kb = tile * kBwdTB + my_r;
  const bool k_valid = kb < nkb;
  const int k_tok = kb * kBlock + (wave & 1) * 32 + n;
  const size_t krow = base + (size_t)k_tok * D;

  bf16x8 bk[KS], bv[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    bk[ks] = k_valid ? *(const bf16x8 *)((const bf16 *)a.k + krow + ks * 16 + hh * 8) : bf16x8{};
    bv[ks] = k_valid ? *(const bf16x8 *)((const bf16 *)a.v + krow + ks * 16 + hh * 8) : bf16x8{};
  }
  const float c = a.scale * kLog2e;
  f32x16 dk[MT], dv[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) dk[mt] = dv[mt] = f32x16{};

  TReadBases tb;
  tb.init(n, hh);

  PairBitmap pb;
  pb.init(dyn_lds, nqb);
  pb.build(a.ix.col_ptr + (size_t)hidx * (nkb + 1), tile * kBwdTB, nkb, a.ix.nnz, a.ix.row_idx, nqb,
           kBwdThreads);
  PairIter it;
  it.start(nqb);

  RowStage<D, kBwdThreads> sq, sdo;
  TStage<D, kBwdThreads> sqt, sdot;
  float lse_st = 0.f, dlt_st = 0.f;
  auto load = [&](int ii) {
    const size_t off = (size_t)ii * kBlock * D;
    sq.load(qg + off);
    sdo.load(dog + off);
    sqt.load(qg + off);
    sdot.load(dog + off);
    if (threadIdx.x < kBlock) {
      lse_st = lseg[(size_t)ii * kBlock + threadIdx.x];
      dlt_st = dltg[(size_t)ii * kBlock + threadIdx.x];
    }
  };
  auto store = [&](DkvBuf<D> &b) {
    sq.store(b.q);
    sdo.store(b.dout);
    sqt.store(b.qt);
    sdot.store(b.dot);
    if (threadIdx.x < kBlock) {
      b.lse2[threadIdx.x] = lse_st == -INFINITY ? INFINITY : lse_st * kLog2e;
      b.dlt[threadIdx.x] = dlt_st;
    }
  };
  bool have = it.next(pb);
  int i = it.j;
  bool act = k_valid && (my_r == 0 ? it.in0 : it.in1);
  if (have) {
    load(i);
    store(lds[0]);
  }
  bool have_next = have && it.next(pb);
  if (have_next) load(it.j);
  int buf = 0;
  while (have) {
    __syncthreads();
    if (act) {
      const DkvBuf<D> &bb = lds[buf];
      const bool diag = a.causal && kb >= i;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 aq = *(const bf16x8 *)(bb.q + (32 * m + n) * G::ROW + ks * 16 + hh * 8);
          const bf16x8 ado = *(const bf16x8 *)(bb.dout + (32 * m + n) * G::ROW + ks * 16 + hh * 8);
          s = mfma_32x32x16(aq, bk[ks], s);
          dp = mfma_32x32x16(ado, bv[ks], dp);
        }
        float l2[16], dl[16];
        load_rows16(bb.lse2, m, hh, l2);
        load_rows16(bb.dlt, m, hh, dl);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(__builtin_fmaf(s[r], c, -l2[r]));
          if (diag) {
            const int q_tok = i * kBlock + 32 * m + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (k_tok > q_tok) p = 0.f;
          }
          s[r] = p;
          dp[r] = p * (dp[r] - dl[r]);
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int ks = 2 * m + half;
          const bf16x8 bp = pack_acc_operand(s, half);
          const bf16x8 bds = pack_acc_operand(dp, half);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const bf16x8 adot = *(const bf16x8 *)((const char *)bb.dot + tb.at(mt, ks));
            const bf16x8 aqt = *(const bf16x8 *)((const char *)bb.qt + tb.at(mt, ks));
            dv[mt] = mfma_32x32x16(adot, bp, dv[mt]);
            dk[mt] = mfma_32x32x16(aqt, bds, dk[mt]);
          }
        }
      }
    }
    if (have_next) store(lds[buf ^ 1]);
    have = have_next;
    i = it.j;
    act = k_valid && (my_r == 0 ? it.in0 : it.in1);
    have_next = have && it.next(pb);
    if (have_next) load(it.j);
    buf ^= 1;
  }
  if (!k_valid) return;
  bf16 *dko = (bf16 *)a.dk + krow;
  bf16 *dvo = (bf16 *)a.dv + krow;
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

template <int D>
hipError_t launch_bwd(const BwdArgs &a, hipStream_t s) {
  const size_t rows = (size_t)a.B * a.H * a.L;
  const int rpb = 256 / (D / 8);
  const int grid_delta = (int)((rows + rpb - 1) / rpb);
  const int q_tiles = (a.ix.n_qblocks + kBwdTB - 1) / kBwdTB;
  const int k_tiles = (a.ix.n_kblocks + kBwdTB - 1) / kBwdTB;
  const int BH = a.B * a.H;
  const size_t dyn_k = PairBitmap::lds_bytes(a.ix.n_qblocks);
  const size_t dyn_q = PairBitmap::lds_bytes(a.ix.n_kblocks);
  hipError_t e = hipFuncSetAttribute((const void *)bwd_dkdv_kernel<D>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn_k);
  if (e == hipSuccess)
    e = hipFuncSetAttribute((const void *)bwd_dq_kernel<D>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn_q);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_delta_kernel<D>, dim3(grid_delta), dim3(256), 0, s, a);
  hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3(BH * k_tiles), dim3(kBwdThreads), dyn_k, s, a);
  hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3(BH * q_tiles), dim3(kBwdThreads), dyn_q, s, a);
  return hipGetLastError();
}

}  // namespace

size_t bwd_bf16_lds_bytes(int d, int n_blocks) {
  const size_t buf = d == 128 ? sizeof(DkvBuf<128>) : sizeof(DkvBuf<64>);
  return 2 * buf + PairBitmap::lds_bytes(n_blocks);
}

hipError_t launch_bwd_bf16(const BwdArgs &a, hipStream_t s) {
  return a.d == 128 ? launch_bwd<128>(a, s) : launch_bwd<64>(a, s);
}

}  // namespace attn
