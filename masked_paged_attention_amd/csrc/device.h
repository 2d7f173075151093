// Device-side helpers shared by the gfx950 kernels: vector types, the MFMA
// wrappers, the LDS transpose read, cross-half wave reductions and conversions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mpa {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Vec;
template <>
struct Vec<_Float16> {
  typedef f16x8 x8;
  typedef f16x4 x4;
};
template <>
struct Vec<__bf16> {
  typedef bf16x8 x8;
  typedef bf16x4 x4;
};

// D(32x32, fp32) += A(32x16) * B(16x32).  Lane l supplies A row l%32 and B column
// l%32, each with the 8 contraction indices of half l/32; lane l receives
// D[8*(r/4) + 4*(l/32) + r%4][l%32] in register r (layout checked on gfx950).
__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D(32x32, int32) += A(32x32) * B(32x32), int8 operands.  Lane l supplies A row
// l%32 and B column l%32, each with the 16 contraction indices 16*(l/32) ..
// +15; D in the layout of mfma32 (checked on gfx950).
__device__ __forceinline__ i32x16 mfma32_i8(i32x4 a, i32x4 b, i32x16 c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// LDS transpose read of 8-bit data.  In each group of 16 lanes, source lane s
// points at 8 consecutive bytes (row s/2, bytes 8*(s%2)..+7 of an 8 x 16 block;
// the rows may lie anywhere); lane i of the group receives byte column i of
// the 8 rows, row e in byte e (checked on gfx950).
__device__ __forceinline__ i32x2 lds_read_tr8(const void* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((i32x2 __attribute__((address_space(3)))*)p);
}

// LDS transpose read of 16-bit data.  In each group of 16 lanes, source lane s
// points at 4 consecutive elements (row s/4, columns 4*(s%4)..+3 of a 4 x 16
// block); lane i of the group receives column i of the block's 4 rows.
__device__ __forceinline__ s16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)p);
}

// x combined with the value lane l^32 holds (one permlane32 swap).
__device__ __forceinline__ float max_with_other_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_other_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup barrier for data exchanged through LDS by ordinary LDS stores: waits
// for this wave's LDS operations only, so direct global->LDS loads issued
// earlier stay in flight across it.  The memory clobber keeps the compiler from
// moving memory operations across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 16-byte direct load global -> LDS (gfx950 global_load_lds_dwordx4): lane i of
// the wave writes its 16 bytes to lds_base + 16 * i, lds_base being wave-uniform.
// Issued through inline asm so that the compiler's wait tracking does not see an
// asynchronous LDS write: the caller orders it with explicit vmcnt waits and
// barriers (the LDS base is latched at issue, so M0 is restored right after).
__device__ __forceinline__ void dma16(const void* gsrc, const void* lds_base) {
  const unsigned m = (unsigned)(unsigned long)(const __attribute__((address_space(3))) void*)lds_base;
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gsrc), "s"(m)
      : "memory");
}

// Same, with a wave-uniform 64-bit base in SGPRs and a per-lane 32-bit byte
// offset: lane i reads sbase + voffset_i and writes its 16 bytes to
// lds_base + 16 * i.
__device__ __forceinline__ void dma16s_m0(const void* sbase, unsigned voffset, unsigned m) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voffset), "s"(sbase), "s"(m)
      : "memory");
}

// Same, without a memory clobber: the compiler may move ordinary memory
// accesses across it.  For callers whose every ordering constraint on the
// loaded LDS bytes runs through other volatile asm statements (waits and
// barriers), which keep their order relative to this one.
__device__ __forceinline__ void dma16s_m0_nomem(const void* sbase, unsigned voffset, unsigned m) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voffset), "s"(sbase), "s"(m));
}

// Same, with the LDS destination given as a pointer.
__device__ __forceinline__ void dma16s(const void* sbase, unsigned voffset, const void* lds_base) {
  dma16s_m0(sbase, voffset,
            (unsigned)(unsigned long)(const __attribute__((address_space(3))) void*)lds_base);
}

// Scalar load of 16 read-only bytes (a plan record) at a wave-uniform address,
// waited for inside the same asm block.  Scalar loads never wait on vector
// memory, so reading the plan does not drain direct loads in flight.
__device__ __forceinline__ int4 sload_int4(const int4* ptr) {
  typedef int v4i __attribute__((ext_vector_type(4)));
  v4i v;
  asm volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(ptr) : "memory");
  return make_int4(v[0], v[1], v[2], v[3]);
}

// Lane index 0..63 computed where it is used: the compiler cannot hoist
// values derived from it out of a loop, so per-lane addresses needed only now
// and then do not stay live (and occupy registers) across the loop.
__device__ __forceinline__ int opaque_lane() {
  int v;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(v));
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_sqrt(float x) { return __builtin_amdgcn_sqrtf(x); }

template <typename T>
__device__ __forceinline__ T to_elem(float x) {
  return (T)x;  // round to nearest even (v_cvt_f16_f32 / v_cvt_pk_bf16_f32)
}

// Rounds 8 fp32 values to one MFMA operand (round to nearest even).
template <typename T>
__device__ __forceinline__ typename Vec<T>::x8 pack8(const float* x) {
  typename Vec<T>::x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (T)x[e];
  return v;
}

}  // namespace mpa
