// Device-side helpers shared by the gfx950 GQA kernels: vector types, MFMA
// wrappers, wavefront reductions and LDS transpose reads.
//
// Matrix-core layouts used throughout (CDNA4, wave64), for lane l:
//   v_mfma_f32_16x16x32_bf16  A[i][k]: i = l%16, k-group l/16 (8 values)
//                             B[k][j]: j = l%16, k-group l/16 (8 values)
//                             D[i][j]: j = l%16, i = 4*(l/16) + r, r = 0..3
//   v_mfma_f32_32x32x16_bf16  A[i][k]: i = l%32, k-group l/32 (8 values)
//                             B[k][j]: j = l%32, k-group l/32
//                             D[i][j]: j = l%32, i = 8*(r/4) + 4*(l/32) + r%4,
//                             r = 0..15
// The contraction index may be permuted freely as long as A and B use the
// same permutation, which the kernels exploit to keep loads contiguous.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 2^x on the hardware exponential unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor(v, m));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor(v, m);
  return v;
}

// Orders LDS traffic between lanes of one wavefront (no cross-wave effect).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// ds_read_b64_tr_b16: every lane of a 16-lane block names an 8-byte word in
// LDS; lane i receives element i%4 of the words named by lanes 4e + i/4,
// e = 0..3.  With lane L naming row (r0 + L/4), columns c0 + 4*(L%4) .. +3
// of a row-major bf16 tile, lane i receives column c0 + i of rows r0..r0+3:
// a 4 x 16 tile read transposed.
__device__ __forceinline__ bf16x4 lds_read_tr16(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_bf16x4*)(__attribute__((address_space(3))) void*)(p));
}

__device__ __forceinline__ bf16x8 concat(const bf16x4& a, const bf16x4& b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Raw buffer resource over [base, base + bytes): loads whose per-lane byte
// offset (plus the instruction's immediate offset) is past `bytes` return
// zeros instead of touching memory; the uniform SGPR offset is NOT range
// checked, so callers keep it 0.  Dword 3 selects the 32-bit data format
// that untyped gfx9 buffer loads require.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// Cache-policy bits of buffer loads: 2 marks the access non-temporal (nt),
// for data read exactly once, such as a decode step's sweep of the KV cache.
constexpr int kCacheDefault = 0;
constexpr int kCacheStream = 2;

// 16-byte buffer load at byte offset voff (per lane) + soff (uniform).
template <int kPolicy = kCacheDefault>
__device__ __forceinline__ bf16x8 buffer_load_bf16x8(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kPolicy));
}

__device__ __forceinline__ bf16x8 load_bf16x8(const __bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ void store_bf16x8(__bf16* p, const bf16x8& v) {
  *reinterpret_cast<bf16x8*>(p) = v;
}

}  // namespace gqa
