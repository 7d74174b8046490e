// Shared device helpers for the gfx950 frame-wise GDN kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair (a in the low half), round to nearest even.
// gfx950 does this in one instruction (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t cvt2bf(float a, float b) {
  const bf16x2 h = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, h);
}

// float -> bfloat16 bits (round to nearest even) in the low 16 bits.
__device__ __forceinline__ uint32_t f2bf(float f) { return cvt2bf(f, 0.f) & 0xffffu; }

__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }

// Split the pair (a, b) into a packed bf16 hi word (.x) and lo word (.y) with
// hi + lo equal to the inputs to about 2^-17 relative: hi = bf16(x),
// lo = bf16(x - hi).
__device__ __forceinline__ u32x2 split2(float a, float b) {
  const uint32_t hi = cvt2bf(a, b);
  const uint32_t lo = cvt2bf(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
  return (u32x2){hi, lo};
}

__device__ __forceinline__ uint32_t pack2(uint32_t lo16, uint32_t hi16) {
  return (lo16 & 0xffffu) | (hi16 << 16);
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, not for its outstanding global loads, so prefetches issued
// before the barrier stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// D = A(16x32) * B(32x16) + C.  Lane l supplies A[l%16][8(l/16)+e] and
// B[8(l/16)+e][l%16] (e = 0..7) and holds D[4(l/16)+i][l%16] (i = 0..3).
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// ds_read_b64_tr_b16 (gfx950): each lane names an 8-byte-aligned LDS
// address; within every 16-lane group, lane i receives as its element e
// (e = 0..3) element i % 4 of the 8 bytes named by lane 4e + i / 4.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
  return __builtin_bit_cast(u32x2, r);
}

template <typename T>
__device__ __forceinline__ T ld_nt(const T* p) { return __builtin_nontemporal_load(p); }
template <typename T>
__device__ __forceinline__ void st_nt(T* p, T v) { __builtin_nontemporal_store(v, p); }

}  // namespace gdn
