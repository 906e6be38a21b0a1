// Shared device helpers for the gfx950 kernels of libtokengate.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#define TG_LOG2E 1.4426950408889634f
#define TG_LN2 0.6931471805599453f

#pragma clang diagnostic ignored "-Winline-asm"

namespace tg {

// 16-byte direct global -> LDS load (gfx950 global_load_lds_dwordx4) for the
// active lanes of a wave: lane l's 16 bytes land at lds_base + 16*l, with m0
// carrying the wave's LDS byte address. Issued from asm so that the compiler
// does not add its conservative vmcnt(0) before every later LDS read; the
// callers order these loads with wait_vmcnt<> and a barrier themselves.
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_base), "v"(g)
               : "memory", "m0");
}

// 4-byte variant: lane l's dword lands at lds_base + 4*l
__device__ __forceinline__ void lds_dma4(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(lds_base), "v"(g)
               : "memory", "m0");
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource (gfx9 family): 48-bit base, stride 0, `bytes` of range.
// Loads whose byte offset is at or past `bytes` return zeros.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

// 16-byte buffer load straight into LDS: lane l reads rsrc at byte offset
// voff (range-checked, zero past the end) and lands at lds_base + 16*l.
__device__ __forceinline__ void buf_dma16(const i32x4& rsrc, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds_base),
               "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// Same with a wave-uniform byte offset in the instruction's scalar offset
// (added to the address; the range check sees the per-lane offset).
__device__ __forceinline__ void buf_dma16_soff(const i32x4& rsrc, uint32_t voff, uint32_t soff,
                                               uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds_base),
               "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}

// 4-byte variant: lane l's dword lands at lds_base + 4*l
__device__ __forceinline__ void buf_dma4(const i32x4& rsrc, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(lds_base),
               "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// wait until at most N vector-memory loads of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

__device__ __forceinline__ float bf2f(bf16 x) { return static_cast<float>(x); }
__device__ __forceinline__ bf16 f2bf(float x) { return static_cast<bf16>(x); }  // RNE

// 32x32x16 bf16 MFMA, fp32 accumulate (gfx950). Lane l supplies row (l % 32)
// of A and column (l % 32) of B for the k-slots owned by lane group l / 32;
// A and B use the same k-slot order, so any fixed k permutation cancels.
// Result: lane l holds column l % 32, rows 8*(r/4) + 4*(l/32) + r%4, r < 16.
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// erf without branches: Abramowitz and Stegun, Handbook of Mathematical
// Functions, formula 7.1.26: erf(a) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 +
// a5 t^5) exp(-a^2), t = 1 / (1 + p a), a = |x|, absolute error <= 1.5e-7;
// odd in x. Hardware reciprocal and exp2 (each ~1 ulp).
__device__ __forceinline__ float erf_fast(float x) {
  const float a = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, a, 1.0f));
  const float poly =
      t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, 1.061405429f, -1.453152027f), 1.421413741f), -0.284496736f),
               0.254829592f);
  const float e = __builtin_amdgcn_exp2f(-a * a * TG_LOG2E);
  return copysignf(fmaf(-poly, e, 1.0f), x);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = static_cast<bf16>(0.0f);
  return z;
}

__device__ __forceinline__ f32x16 zero_f32x16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

}  // namespace tg
