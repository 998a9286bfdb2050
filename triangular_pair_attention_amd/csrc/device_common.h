// Device helpers for gfx950 (CDNA4): matrix-core fragments, conversions,
// wave reductions. Used by both kernels of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct bf16_t {  // storage type tag for bfloat16 tensors
  uint16_t bits;
};

template <typename T>
struct is_bf16 {
  static constexpr bool value = false;
};
template <>
struct is_bf16<bf16_t> {
  static constexpr bool value = true;
};

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- MFMA
// 16x16x32 bf16 -> f32. Lane l holds A[l%16][8(l/16)..+7], B[8(l/16)..+7][l%16];
// the result lane l holds C[4(l/16)+r][l%16], r = 0..3.
__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// 16x16x16 bf16 -> f32 (A[l%16][4(l/16)..+3]).
__device__ __forceinline__ f32x4 mfma(bf16x4 a, bf16x4 b, f32x4 c) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                   0, 0, 0);
}
// 16x16x4 f32. Lane l holds A[l%16][l/16], B[l/16][l%16].
__device__ __forceinline__ f32x4 mfma(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
__device__ __forceinline__ float bflo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bfhi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// Round-to-nearest-even float -> bf16 (the hardware conversion on gfx950).
// Converted as one two-element vector: a single packed conversion, where two
// scalar conversions would cost two conversions, a shift and an OR.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}
__device__ __forceinline__ uint16_t f2bf(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

// Three-way bf16 split of two floats: a = a1 + a2 + a3 exactly (likewise b),
// with a1 = bf16(a), a2 = bf16(a - a1), a3 = a - a1 - a2 (each rounded to
// nearest even). a - a1 is exact in float32 and has at most 16 significant
// bits, so a2 keeps its top 8 and a3 the rest exactly. Returned as packed
// pairs (low half a, high half b) of the first, second and third parts.
__device__ __forceinline__ void split3(float a, float b, uint32_t &p1, uint32_t &p2, uint32_t &p3) {
  p1 = pack_bf16x2(a, b);
  const float ra = a - bflo(p1), rb = b - bfhi(p1);
  p2 = pack_bf16x2(ra, rb);
  p3 = pack_bf16x2(ra - bflo(p2), rb - bfhi(p2));
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ uint4 as_u4(bf16x8 v) { return __builtin_bit_cast(uint4, v); }

// ---------------------------------------------------------------- loads / stores
template <typename V>
__device__ __forceinline__ V ldg(const void *p) {
  return *reinterpret_cast<const V *>(p);
}
template <typename V>
__device__ __forceinline__ void stg(void *p, V v) {
  *reinterpret_cast<V *>(p) = v;
}

// ---------------------------------------------------------------- wave reductions
__device__ __forceinline__ float xor_sum(float v, int m) { return v + __shfl_xor(v, m, 64); }
__device__ __forceinline__ float xor_max(float v, int m) { return fmaxf(v, __shfl_xor(v, m, 64)); }

// Sum over each aligned group of W lanes (W = 4 or 8: lanes Wk .. Wk+W-1),
// every lane getting its group's sum, with DPP lane moves on the VALU instead
// of round trips through the LDS crossbar: swap neighbours (quad_perm
// 1,0,3,2), swap pairs (quad_perm 2,3,0,1) and, for 8, add the other quad
// (row_half_mirror: lane i of the 8 reads lane 7 - i).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(W == 4 || W == 8, "groups of 4 or 8 lanes");
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  if constexpr (W == 8) v += dpp_mov<0x141>(v);
  return v;
}

// Sum / max over the four lanes that share l % 16 (lane groups l / 16).
__device__ __forceinline__ float group4_sum(float v) { return xor_sum(xor_sum(v, 16), 32); }
__device__ __forceinline__ float group4_max(float v) { return xor_max(xor_max(v, 16), 32); }
// Max over the 16 lanes of one lane group.
__device__ __forceinline__ float row16_max(float v) {
  v = xor_max(v, 1);
  v = xor_max(v, 2);
  v = xor_max(v, 4);
  return xor_max(v, 8);
}

// Workgroup barrier for data exchanged through LDS only. It waits for this
// wave's LDS operations (lgkmcnt) and then for the other waves; unlike
// __syncthreads() it does not drain the wave's outstanding global loads and
// stores, so a prefetch or a burst of output stores stays in flight across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Wait until at most N of this wave's vector-memory operations are outstanding.
template <int N>
__device__ __forceinline__ void vmcnt_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Direct global -> LDS copy, 16 bytes per lane: lane l's bytes land at
// lds_base + 16*l (lds_base is the same for the whole wave). Issued through
// inline assembly so that the compiler does not hold later LDS reads of other
// ring stages behind it; the caller tracks completion with vmcnt_wait (vector
// memory operations complete in issue order for vmcnt). The assembly sets
// M0, a register the compiler reserves and does not let an asm statement
// declare as clobbered; these kernels make no other use of M0 (no indexed
// register access, no message or GDS instructions), which a host-side test
// checks on the generated code.
__device__ __forceinline__ void dma16_to_lds(const void *gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds_base)
               : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)p;
}

// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011): ten rounds on a 4-word counter and a 2-word key,
// with the published multipliers and key increments. The dropout decisions of
// the training-mode kernels come from it.
// Each round's two 32x32 -> 64-bit products are written as 64-bit products,
// one v_mad_u64_u32 each (measured 1.3x the throughput of a mul_hi/mul_lo pair),
// and each three-way exclusive or as one gfx950 three-input bit operation
// (truth table 0x96: the parity of the three input bits).
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x, p1 = (uint64_t)0xCD9E8D57u * c.z;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    c = make_uint4(xor3(hi1, c.y, k0), lo1, xor3(hi0, c.w, k1), lo0);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// One element of a float32 or bf16 tensor, as float.
template <typename T>
__device__ __forceinline__ float ld_elem(const void *p, size_t i) {
  if constexpr (is_bf16<T>::value)
    return bf2f(reinterpret_cast<const uint16_t *>(p)[i]);
  else
    return reinterpret_cast<const float *>(p)[i];
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

}  // namespace tpa
