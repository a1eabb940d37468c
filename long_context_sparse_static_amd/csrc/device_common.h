// Device-side helpers shared by the gfx950 kernels: vector types, the bf16
// MFMA wrapper, wave reductions and the XCD-aware workgroup remap.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>
#include <stdint.h>

#include "kernels.h"

namespace attn {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D(32x32, f32) += A(32x16, bf16) * B(16x32, bf16) on the CDNA4 matrix cores.
// Lane l holds A row (l % 32), k = 8*(l/32) .. +7; B column (l % 32) with the
// same k range; and D column (l % 32), rows 8*(r/4) + 4*(l/32) + r%4 for its
// 16 registers r.
__device__ __forceinline__ f32x16 mfma_32x32x16(const bf16x8 &a, const bf16x8 &b,
                                                const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (bf16)lo;
  v[1] = (bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Workgroups are dealt to the 8 XCDs round-robin (bid % 8).  Remap so that
// each XCD receives a contiguous range of logical work items, which keeps one
// head's neighbouring query tiles -- and so its K/V blocks -- in one L2.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  const int xcd = bid % kNumXcd;
  const int slot = bid / kNumXcd;
  const int q = total / kNumXcd, r = total % kNumXcd;
  return xcd < r ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

// max of x over lane l and lane l ^ 32 (the two halves of a wave64).
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Direct global -> LDS loads through a raw buffer descriptor: lane i's BYTES
// (4 or 16) from base + byte_off land at lds + i * BYTES (lds wave-uniform).
// Unlike global_load_lds, the compiler counts this form on vmcnt alone, so
// LDS reads issued while it is in flight keep exact lgkmcnt waits (with a
// global_load_lds pending it waits for every outstanding LDS read instead).
// Descriptor: stride 0 (raw bytes), data format 32 (the untyped-buffer
// setting of the gfx9 descriptor word 3), limited to `bytes` (-1: no limit):
// loads at offsets >= bytes return zeros without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc_n(const void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}
// IMM, the instruction's immediate offset, moves the global and the LDS
// address alike: lane i's bytes come from base + byte_off + IMM and land at
// lds + IMM + i * BYTES.  Loads that differ only in IMM share one LDS base,
// so they need no M0 value (and no SGPR) each.
template <int BYTES, int IMM = 0>
__device__ __forceinline__ void load_lds(__amdgpu_buffer_rsrc_t rs, int byte_off, void *lds) {
  static_assert(BYTES == 4 || BYTES == 16, "4- or 16-byte lanes");
  static_assert(IMM >= 0 && IMM < 4096, "12-bit immediate offset");
  auto *l = (__attribute__((address_space(3))) void *)lds;
  // the builtin wants its size and offset as literals
  if constexpr (BYTES == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, l, 16, byte_off, 0, IMM, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, l, 4, byte_off, 0, IMM, 0);
}

// x if keep >= 0, else -inf: one bitfield insert keyed on keep's sign bit,
// so a run of masks needs no per-element condition registers.
__device__ __forceinline__ float mask_neg_inf(float x, int keep) {
  const uint32_t sel = (uint32_t)(keep >> 31);  // all ones when keep < 0
  return __uint_as_float((sel & 0xff800000u) | (~sel & __float_as_uint(x)));
}

// f(std::integral_constant<int, K>{}) for K = 0 .. N-1, fully expanded at
// compile time (a #pragma unroll is only a hint, and a loop left rolled
// turns register arrays indexed by its counter into scratch memory).
template <class F, int... K>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, K...>) {
  (f(std::integral_constant<int, K>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// A wave-uniform copy of a value every lane holds (kept in an SGPR).
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__host__ __device__ __forceinline__ int clamp_i(int x, int lo, int hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

}  // namespace attn
