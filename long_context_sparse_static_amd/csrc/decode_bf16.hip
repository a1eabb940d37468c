// Single-token decode against a KV cache, bf16 storage / fp32 arithmetic.
//
// LongGen's sparse layers keep only their sink and window tokens, which is
// where its KV-memory saving and decode speedup come from (atlas.scime.ai
// summary of "A Little Goes a Long Way...", "Key results"; mlsanity index
// page, "Abstract (arXiv)"); its full layers keep every token.  Decode reads
// each cached K/V row once, so it is bound by HBM bandwidth: the kernels are
// written for wide coalesced streaming, not for the matrix cores.
//
//   decode_split_kernel  grid (n_split, B*H): one workgroup streams a
//                        contiguous slot range of one (b, h) and writes a
//                        partial (m, l, o) in base 2; the workgroup owning
//                        the new token's slot also appends k_new / v_new
//                        (every workgroup reads that slot from k_new / v_new,
//                        so no ordering between them is needed).
//   decode_combine_kernel grid (B*H): merges the partials, writes o and lse.
//   ring_fill_kernel     copies prefill K/V into the sink + window ring.
//   paged_fill_kernel    copies prefill K/V into the pages of a block table.
//
// Ring slot of token p: p if p < sink, else sink + (p - sink) % window.
// Paged full layers (a block-table cache in the manner of PagedAttention,
// listed among LongGen's foundations on the mlsanity index page, "Builds
// on"; LongGen is served with vLLM: atlas.scime.ai summary, "Approach"): pools
// [n_pages, H, 64, d], token p of sequence b in page table[b][p / 64] at
// row p % 64; a page id outside [0, n_pages) reads nothing and makes the
// result NaN.
#include <mutex>

#include "device_common.h"
#include "kernels.h"

// Fixed split-KV partial buffer for callers that cannot allocate device
// memory (attn_full_decode_noalloc).  Each GPU the library runs on holds its
// own copy, at its own address, until the process ends; host code reaches it
// only through the address hipGetSymbolAddress returns for the current device
// (the name itself is a host-side stand-in, not a device address).
static __device__ __align__(256) float scratch[attn::kDecodeScratchBytes / sizeof(float)];

namespace attn {
namespace {

constexpr int kDecThreads = 256;
constexpr int kDecUnroll = 4;       // keys in flight per lane group
constexpr int kDecTargetWgs = 4096;  // split-KV workgroups aimed for per launch

__device__ __forceinline__ int64_t ring_slot(int64_t p, int sink, int window) {
  return p < sink ? p : sink + (p - sink) % window;
}

// BlockSparse compacted cache of one (b, h), block size 64 (the BlockSparse
// pattern of LongGen's sparse layers: mlsanity index page "A Little Goes a
// Long Way...", "Abstract (arXiv)"; the token at position t reads exactly
// the keys its row of the prefill mask allows):
//   slots [0, 64 s)              sink blocks 0 .. s-1
//   slots [64 s, 64 (s + w))     ring of the w most recent blocks (block j
//                                at ring block j mod w)
//   slots [64 (s + w), ...)      strided blocks j >= s, (j + h) % stride == 0,
//                                that have left the window, ascending
// A strided block moves from the ring to the strided area when the block w
// places later starts (bs_move_kernel, before the split kernel).
__host__ __device__ __forceinline__ int64_t bs_strided_before(int64_t x, int64_t s, int64_t st,
                                                               int64_t h) {
  // number of j in [s, x) with (j + h) % st == 0
  const int64_t r0 = ((-h) % st + st) % st;
  const int64_t j0 = s <= r0 ? r0 : r0 + ((s - r0 + st - 1) / st) * st;
  return j0 >= x ? 0 : (x - 1 - j0) / st + 1;
}

// Block held by ring block pb when the newest block is i (i >= 0).
__device__ __forceinline__ int64_t bs_ring_block(int64_t i, int64_t pb, int64_t w) {
  return i - (((i - pb) % w) + w) % w;
}

// Whether slot `slot` of a BlockSparse cache holds a key the token at
// position t reads (t = 64 i + r, a = first window block, cnt strided blocks).
__device__ __forceinline__ bool bs_slot_valid(const DecodeArgs &a, int64_t slot, int64_t t) {
  const int64_t s = a.bs_sink, w = a.bs_local;
  if (slot < 64 * s) return slot <= t;
  if (slot < 64 * (s + w)) {
    const int64_t q = slot - 64 * s, i = t >> 6;
    const int64_t j = bs_ring_block(i, q >> 6, w);
    return j >= s && j >= 0 && (j < i || (q & 63) <= (t & 63));
  }
  return true;  // strided blocks below the valid count
}

// Valid slot count and the new token's slot for position t; false if t is
// outside what the layer accepts.
__device__ __forceinline__ bool decode_geometry(const DecodeArgs &a, int64_t t, int h,
                                                int64_t *n_valid, int64_t *slot_new) {
  if (a.bs_stride > 0) {
    if (t < 0) return false;
    const int64_t s = a.bs_sink, w = a.bs_local, i = t >> 6;
    const int64_t first = i - w + 1 > 0 ? i - w + 1 : 0;
    const int64_t cnt = bs_strided_before(first, s, a.bs_stride, h);
    if (cnt > a.bs_cap) return false;
    *n_valid = 64 * (s + w + cnt);
    *slot_new = i < s ? t : 64 * s + 64 * (i % w) + (t & 63);
    return true;
  }
  if (a.table) {
    if (t < 0 || t > a.max_pos) return false;
    *n_valid = t + 1;
    *slot_new = t;
    return true;
  }
  if (a.sink >= 0) {
    if (t < 0) return false;
    const int64_t cap = (int64_t)a.sink + a.window;
    *n_valid = t + 1 < cap ? t + 1 : cap;
    *slot_new = ring_slot(t, a.sink, a.window);
  } else {
    if (t < 0 || t > a.max_pos || t >= a.cap) return false;
    *n_valid = t + 1;
    *slot_new = t;
  }
  return true;
}

template <int D>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(DecodeArgs a) {
  constexpr int LPK = D / 8;          // lanes per key row (16 bytes each)
  constexpr int KPW = 64 / LPK;       // keys per wave per step
  constexpr int NWAVE = kDecThreads / 64;
  __shared__ float red[NWAVE][D + 2];

  const int split = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.H;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane / LPK, c = lane % LPK;
  float *part = a.part + ((size_t)bh * a.n_split + split) * (D + 2);

  const int64_t t = a.pos[b];
  int64_t n_valid = 0, slot_new = -1;
  const bool ok = decode_geometry(a, t, bh % a.H, &n_valid, &slot_new);
  const bool bs = a.bs_stride > 0;
  const int64_t s0 = (int64_t)split * a.split_len;
  const int64_t s1 = ok ? (s0 + a.split_len < n_valid ? s0 + a.split_len : n_valid) : 0;

  const bool paged = a.table != nullptr;
  const int h = bh % a.H;
  const int32_t *tab = paged ? a.table + (size_t)b * a.max_pages : nullptr;
  // element offset of (page, h) and whether the page id is in range
  auto page_base = [&](int64_t blk, bool &valid) -> size_t {
    const int pg = tab[blk];
    valid = pg >= 0 && pg < a.n_pages;
    return ((size_t)(valid ? pg : 0) * a.H + h) * kBlock * D;
  };
  const size_t row0 = paged ? 0 : (size_t)bh * a.cap;
  const bf16 *kc = (const bf16 *)a.k_cache + row0 * D;
  const bf16 *vc = (const bf16 *)a.v_cache + row0 * D;
  const bf16 *kn = (const bf16 *)a.k_new + (size_t)bh * D;
  const bf16 *vn = (const bf16 *)a.v_new + (size_t)bh * D;

  // Append the new token (one workgroup per (b, h) owns its slot).
  if (ok && slot_new >= s0 && slot_new < s1 && threadIdx.x < LPK) {
    bool valid = true;
    const size_t dst = paged ? page_base(slot_new >> 6, valid) + (size_t)(slot_new & 63) * D
                             : (row0 + slot_new) * D;
    if (valid) {
      *(u32x4 *)((bf16 *)a.k_cache + dst + threadIdx.x * 8) = *(const u32x4 *)(kn + threadIdx.x * 8);
      *(u32x4 *)((bf16 *)a.v_cache + dst + threadIdx.x * 8) = *(const u32x4 *)(vn + threadIdx.x * 8);
    }
  }

  const float cs = a.scale * kLog2e;
  float qf[8];
  {
    const u32x4 qw = *(const u32x4 *)((const bf16 *)a.q + (size_t)bh * D + c * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qf[2 * i] = bf16_lo(qw[i]) * cs;
      qf[2 * i + 1] = bf16_hi(qw[i]) * cs;
    }
  }
  float m = -INFINITY, l = 0.f, o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.f;

  constexpr int STEP = NWAVE * KPW * kDecUnroll;
  static_assert(KPW * kDecUnroll <= kBlock && kBlock % (KPW * kDecUnroll) == 0,
                "the keys of one wave iteration lie in one 64-token page");
  for (int64_t kb = s0 + (int64_t)wave * KPW * kDecUnroll; kb < s1; kb += STEP) {
    u32x4 kw[kDecUnroll], vw[kDecUnroll];
    // paged: this iteration's keys (KPW * kDecUnroll aligned ones) share a
    // page, looked up once per wave
    bool pvalid = true;
    const size_t pbase = paged ? page_base(__builtin_amdgcn_readfirstlane((int)(kb >> 6)), pvalid) : 0;
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const int64_t key = kb + u * KPW + g;
      const int64_t safe = key < s1 ? key : s0;
      const size_t off = paged ? pbase + (size_t)(safe & 63) * D : (size_t)safe * D;
      const bool use_new = safe == slot_new || !pvalid;
      const bf16 *kp = use_new ? kn : kc + off;
      const bf16 *vp = use_new ? vn : vc + off;
      kw[u] = __builtin_nontemporal_load((const u32x4 *)(kp + c * 8));
      vw[u] = __builtin_nontemporal_load((const u32x4 *)(vp + c * 8));
    }
    float sc[kDecUnroll];
    float mx = m;
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc = __builtin_fmaf(qf[2 * i], bf16_lo(kw[u][i]), acc);
        acc = __builtin_fmaf(qf[2 * i + 1], bf16_hi(kw[u][i]), acc);
      }
#pragma unroll
      for (int off = 1; off < LPK; off <<= 1) acc += __shfl_xor(acc, off);
      const int64_t key = kb + u * KPW + g;
      sc[u] = key < s1 && pvalid && (!bs || bs_slot_valid(a, key, t)) ? acc : -INFINITY;
      mx = fmaxf(mx, sc[u]);
    }
    if (mx == -INFINITY) continue;
    const float alpha = fast_exp2(m - mx);  // m = -inf -> 0
    l *= alpha;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] *= alpha;
    m = mx;
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const float p = fast_exp2(sc[u] - m);
      l += p;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[2 * i] = __builtin_fmaf(p, bf16_lo(vw[u][i]), o[2 * i]);
        o[2 * i + 1] = __builtin_fmaf(p, bf16_hi(vw[u][i]), o[2 * i + 1]);
      }
    }
  }

  // Merge the KPW lane groups of this wave (lanes with equal c).
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(m, off);
    const float l2 = __shfl_xor(l, off);
    const float mn = fmaxf(m, m2);
    const float a1 = mn == -INFINITY ? 0.f : fast_exp2(m - mn);
    const float a2 = mn == -INFINITY ? 0.f : fast_exp2(m2 - mn);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = o[i] * a1 + __shfl_xor(o[i], off) * a2;
    l = l * a1 + l2 * a2;
    m = mn;
  }
  if (g == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) red[wave][c * 8 + i] = o[i];
    if (c == 0) {
      red[wave][D] = m;
      red[wave][D + 1] = l;
    }
  }
  __syncthreads();
  if (threadIdx.x < D) {
    const int dd = threadIdx.x;
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) mm = fmaxf(mm, red[w][D]);
    float acc = 0.f, ll = 0.f;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) {
      const float sc = mm == -INFINITY ? 0.f : fast_exp2(red[w][D] - mm);
      acc += red[w][dd] * sc;
      ll += red[w][D + 1] * sc;
    }
    part[dd] = acc;
    if (dd == 0) {
      part[D] = mm;
      part[D + 1] = ll;
    }
  }
}

template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeArgs a) {
  const int bh = blockIdx.x, b = bh / a.H;
  const int dd = threadIdx.x;
  const float *part = a.part + (size_t)bh * a.n_split * (D + 2);
  int64_t n_valid = 0, slot_new = 0;
  bool ok = decode_geometry(a, a.pos[b], bh % a.H, &n_valid, &slot_new);
  if (a.table && ok) {
    // every page the position reads must be in range, else the result is NaN
    const int32_t *tab = a.table + (size_t)b * a.max_pages;
    bool bad = false;
    for (int64_t j = dd; j <= a.pos[b] >> 6; j += D) bad |= tab[j] < 0 || tab[j] >= a.n_pages;
    ok = !__syncthreads_or(bad);
  }
  const int used = ok ? (int)((n_valid + a.split_len - 1) / a.split_len) : 0;
  float mm = -INFINITY;
  for (int s = 0; s < used; ++s) mm = fmaxf(mm, part[(size_t)s * (D + 2) + D]);
  float acc = 0.f, ll = 0.f;
  for (int s = 0; s < used; ++s) {
    const float *ps = part + (size_t)s * (D + 2);
    const float sc = mm == -INFINITY ? 0.f : fast_exp2(ps[D] - mm);
    acc += ps[dd] * sc;
    ll += ps[D + 1] * sc;
  }
  const float out = ll > 0.f ? acc / ll : 0.f;
  ((bf16 *)a.o)[(size_t)bh * D + dd] = (bf16)out;
  if (dd == 0) a.lse[bh] = !ok ? NAN : (ll > 0.f ? (mm + fast_log2(ll)) * kLn2 : -INFINITY);
}

template <int D>
__global__ __launch_bounds__(256) void ring_fill_kernel(RingFillArgs a) {
  constexpr int CPR = D / 8;
  const int bh = blockIdx.y, b = bh / a.H;
  const int64_t ring = (int64_t)a.sink + a.window;
  const int64_t ci = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (ci >= ring * CPR) return;
  const int64_t r = ci / CPR;
  const int c = (int)(ci % CPR);
  int64_t n = a.len[b];
  if (n < 0) return;
  if (n > a.src_len) n = a.src_len;
  int64_t p;
  if (r < a.sink) {
    p = r;
  } else {
    const int64_t first = n - a.window > a.sink ? n - a.window : (int64_t)a.sink;
    p = first + (r - a.sink);
  }
  if (p >= n) return;
  const int64_t slot = ring_slot(p, a.sink, a.window);
  const size_t src = ((size_t)bh * a.src_len + p) * D + c * 8;
  const size_t dst = ((size_t)bh * ring + slot) * D + c * 8;
  *(u32x4 *)((bf16 *)a.k_cache + dst) = *(const u32x4 *)((const bf16 *)a.k_src + src);
  *(u32x4 *)((bf16 *)a.v_cache + dst) = *(const u32x4 *)((const bf16 *)a.v_src + src);
}

// Moves a strided block out of the ring when the block w places later
// starts at position t (first token of its block), before the ring block is
// overwritten.  One workgroup per (b, h).
template <int D>
__global__ __launch_bounds__(256) void bs_move_kernel(DecodeArgs a) {
  constexpr int CPR = D / 8;
  const int bh = blockIdx.x, b = bh / a.H, h = bh % a.H;
  const int64_t t = a.pos[b];
  const int64_t s = a.bs_sink, w = a.bs_local, st = a.bs_stride;
  if (t < 0 || (t & 63) != 0) return;
  const int64_t j = (t >> 6) - w;
  if (j < s || (j + h) % st != 0) return;
  const int64_t m = bs_strided_before(j, s, st, h);
  if (m >= a.bs_cap) return;
  const size_t src = (size_t)bh * a.cap + 64 * (s + j % w);
  const size_t dst = (size_t)bh * a.cap + 64 * (s + w + m);
  for (int ci = threadIdx.x; ci < 64 * CPR; ci += blockDim.x) {
    const size_t r = ci / CPR, c = ci % CPR;
    *(u32x4 *)((bf16 *)a.k_cache + (dst + r) * D + c * 8) =
        *(const u32x4 *)((const bf16 *)a.k_cache + (src + r) * D + c * 8);
    *(u32x4 *)((bf16 *)a.v_cache + (dst + r) * D + c * 8) =
        *(const u32x4 *)((const bf16 *)a.v_cache + (src + r) * D + c * 8);
  }
}

// Fills a BlockSparse compacted cache from prefill K/V [B,H,src_len,D]: slot
// by slot, the token decode would hold there after appending tokens
// 0 .. len-1.  Slots that hold nothing yet are left untouched.
template <int D>
__global__ __launch_bounds__(256) void bs_fill_kernel(BsFillArgs a) {
  constexpr int CPR = D / 8;
  const int bh = blockIdx.y, b = bh / a.H, h = bh % a.H;
  const int64_t s = a.sink, w = a.local, st = a.stride;
  const int64_t slots = 64 * (s + w + a.cap);
  const int64_t ci = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (ci >= slots * CPR) return;
  const int64_t slot = ci / CPR;
  const int c = (int)(ci % CPR);
  int64_t n = a.len[b];
  if (n > a.src_len) n = a.src_len;
  if (n <= 0) return;
  const int64_t last = (n - 1) >> 6;
  int64_t p;
  if (slot < 64 * s) {
    p = slot;
  } else if (slot < 64 * (s + w)) {
    const int64_t q = slot - 64 * s;
    const int64_t j = last - ((((last - (q >> 6)) % w) + w) % w);
    if (j < s || j < 0) return;
    p = 64 * j + (q & 63);
  } else {
    const int64_t m = (slot - 64 * (s + w)) >> 6;
    const int64_t r0 = ((-(int64_t)h) % st + st) % st;
    const int64_t j0 = s <= r0 ? r0 : r0 + ((s - r0 + st - 1) / st) * st;
    const int64_t j = j0 + m * st;
    if (j > last - w) return;  // still in the ring
    p = 64 * j + (slot & 63);
  }
  if (p >= n) return;
  const size_t src = ((size_t)bh * a.src_len + p) * D + c * 8;
  const size_t dst = ((size_t)bh * slots + slot) * D + c * 8;
  *(u32x4 *)((bf16 *)a.k_cache + dst) = *(const u32x4 *)((const bf16 *)a.k_src + src);
  *(u32x4 *)((bf16 *)a.v_cache + dst) = *(const u32x4 *)((const bf16 *)a.v_src + src);
}

// Copies tokens 0 .. min(len, src_len) - 1 of prefill K/V [B,H,src_len,D]
// into the pages the block table names (pages with an id outside
// [0, n_pages) are skipped).
template <int D>
__global__ __launch_bounds__(256) void paged_fill_kernel(PagedFillArgs a) {
  constexpr int CPR = D / 8;
  const int bh = blockIdx.y, b = bh / a.H, h = bh % a.H;
  const int64_t ci = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t n = a.len[b];
  if (n > a.src_len) n = a.src_len;
  if (n > (int64_t)a.max_pages * kBlock) n = (int64_t)a.max_pages * kBlock;
  if (ci >= n * CPR) return;
  const int64_t p = ci / CPR;
  const int c = (int)(ci % CPR);
  const int pg = a.table[(size_t)b * a.max_pages + (p >> 6)];
  if (pg < 0 || pg >= a.n_pages) return;
  const size_t src = ((size_t)bh * a.src_len + p) * D + c * 8;
  const size_t dst = (((size_t)pg * a.H + h) * kBlock + (p & 63)) * D + c * 8;
  *(u32x4 *)((bf16 *)a.k_pages + dst) = *(const u32x4 *)((const bf16 *)a.k_src + src);
  *(u32x4 *)((bf16 *)a.v_pages + dst) = *(const u32x4 *)((const bf16 *)a.v_src + src);
}

}  // namespace

void decode_split_plan(int32_t B, int32_t H, int64_t n_keys, int32_t *n_split, int32_t *split_len) {
  // Aim for >= 16 workgroups per CU across 256 CUs, but keep each split at
  // >= 512 keys so a workgroup streams >= 256 KB (d = 128).  (Measured at
  // 16 x 32 heads x 131073 keys: 1536 to 16384 workgroups and 2 to 8 keys in
  // flight per lane group all land within 2% of each other, 6.66-6.79 TB/s.)
  const int64_t bh = (int64_t)B * H;
  int64_t want = (kDecTargetWgs + bh - 1) / bh;
  int64_t len = (n_keys + want - 1) / want;
  if (len < 512) len = 512;
  len = (len + 255) / 256 * 256;
  int64_t ns = (n_keys + len - 1) / len;
  if (ns < 1) ns = 1;
  *n_split = (int32_t)ns;
  *split_len = (int32_t)len;
}

int32_t decode_split_bound(int32_t B, int32_t H, int64_t n_keys) {
  // decode_split_plan gives ceil(n / len) splits with len >= 512 and
  // len >= ceil(n / want): at most min(want, ceil(n / 512)), which never
  // decreases as n grows (so a workspace sized for a capacity fits every
  // position below it).
  const int64_t bh = (int64_t)B * H;
  const int64_t want = (kDecTargetWgs + bh - 1) / bh;
  int64_t ns = (n_keys + 511) / 512;
  if (ns > want) ns = want;
  return (int32_t)(ns < 1 ? 1 : ns);
}

hipError_t decode_scratch(void **ptr) {
  // one lookup per device, with that device current; kept for the process
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_decode_bf16(const DecodeArgs &a, hipStream_t s) {
  dim3 grid(a.n_split, a.B * a.H);
  if (a.bs_stride > 0) {
    if (a.d == 128)
      hipLaunchKernelGGL(bs_move_kernel<128>, dim3(a.B * a.H), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(bs_move_kernel<64>, dim3(a.B * a.H), dim3(256), 0, s, a);
  }
  if (a.d == 128) {
    hipLaunchKernelGGL(decode_split_kernel<128>, grid, dim3(kDecThreads), 0, s, a);
    hipLaunchKernelGGL(decode_combine_kernel<128>, dim3(a.B * a.H), dim3(128), 0, s, a);
  } else {
    hipLaunchKernelGGL(decode_split_kernel<64>, grid, dim3(kDecThreads), 0, s, a);
    hipLaunchKernelGGL(decode_combine_kernel<64>, dim3(a.B * a.H), dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_ring_fill_bf16(const RingFillArgs &a, hipStream_t s) {
  const int64_t ring = (int64_t)a.sink + a.window;
  const int64_t chunks = ring * (a.d / 8);
  dim3 grid((unsigned)((chunks + 255) / 256), a.B * a.H);
  if (a.d == 128)
    hipLaunchKernelGGL(ring_fill_kernel<128>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(ring_fill_kernel<64>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bs_fill_bf16(const BsFillArgs &a, hipStream_t s) {
  const int64_t slots = 64 * ((int64_t)a.sink + a.local + a.cap);
  const int64_t chunks = slots * (a.d / 8);
  dim3 grid((unsigned)((chunks + 255) / 256), a.B * a.H);
  if (a.d == 128)
    hipLaunchKernelGGL(bs_fill_kernel<128>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(bs_fill_kernel<64>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_paged_fill_bf16(const PagedFillArgs &a, hipStream_t s) {
  int64_t n = a.src_len < (int64_t)a.max_pages * kBlock ? a.src_len : (int64_t)a.max_pages * kBlock;
  const int64_t chunks = n * (a.d / 8);
  if (chunks == 0) return hipSuccess;
  dim3 grid((unsigned)((chunks + 255) / 256), a.B * a.H);
  if (a.d == 128)
    hipLaunchKernelGGL(paged_fill_kernel<128>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(paged_fill_kernel<64>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace attn
