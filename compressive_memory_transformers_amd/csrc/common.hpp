// Shared device helpers of the gfx950 kernels: element types, 32x32 MFMA
// fragments and the feature map. Device code only; no host state.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace infini {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <typename T> struct VecT;
template <> struct VecT<bf16> { typedef bf16x4 v4; typedef bf16x8 v8; };
template <> struct VecT<float> { typedef f32x4 v4; typedef f32x8 v8; };

// One MFMA operand fragment: 8 elements of the K dimension held by one lane.
template <typename T> using frag_t = typename VecT<T>::v8;
template <typename T> using vec4_t = typename VecT<T>::v4;

constexpr float kLog2e = 1.4426950408889634f;

// 32x32 output tile, K = 16 per call, float accumulation.
//
// Operand layout (both element types): lane l = 32*h + i holds, for A, row i
// and k = 8h + e (e = 0..7 the fragment element); for B, column i and the same
// k. The accumulator holds, in register r, row (r/4)*8 + 4h + (r%4) of
// column i. bf16 uses one v_mfma_f32_32x32x16_bf16. float uses eight
// v_mfma_f32_32x32x2_f32; call e takes element e of every lane, so it sums
// k in {e, 8 + e}, and the eight calls together cover the same 16 k as the
// bf16 instruction, with the same accumulator layout.
__device__ __forceinline__ void mma32(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma32(f32x16& acc, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], acc, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}

template <typename T> __device__ __forceinline__ float to_f32(T x) { return static_cast<float>(x); }
template <typename T> __device__ __forceinline__ T from_f32(float x) { return static_cast<T>(x); }

// A workgroup barrier for LDS only: this wave's LDS accesses have completed
// (lgkmcnt(0)), then s_barrier. Unlike __syncthreads() it does not wait for
// the wave's global loads and stores in flight (vmcnt), so stores that no
// other wave of the workgroup reads, and loads issued ahead for later use,
// stay in flight across it. The memory clobber keeps the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Lanes i and i ^ 32 combined, every lane getting the result: one
// v_permlane32_swap (gfx950) exchanges the two half-waves' copies in
// registers, where a shuffle would go through the LDS crossbar. The sum adds
// the two values in the same order for both halves' lanes as x + x[i ^ 32]
// would (the lower half's value first in the upper half is the commuted
// addend), so the results are identical to the shuffle form.
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Row of the 32x32 accumulator tile that register r of a lane in half h holds.
__device__ __forceinline__ constexpr int acc_row(int r, int h) { return (r >> 2) * 8 + 4 * h + (r & 3); }

// sigma(x) = ELU(x) + 1 with alpha = 1 ("Infini-Attention" (AI Wiki), "What
// happens inside the Infini-attention block?"): x + 1 above zero, e^x below.
__device__ __forceinline__ float feature_map(float x) {
  return x > 0.f ? x + 1.f : __builtin_amdgcn_exp2f(x * kLog2e);
}

template <typename T> __device__ __forceinline__ frag_t<T> load8(const T* p) {
  return *reinterpret_cast<const frag_t<T>*>(p);
}
template <typename T> __device__ __forceinline__ vec4_t<T> load4(const T* p) {
  return *reinterpret_cast<const vec4_t<T>*>(p);
}
template <typename T> __device__ __forceinline__ void store4(T* p, const vec4_t<T>& v) {
  *reinterpret_cast<vec4_t<T>*>(p) = v;
}
template <typename T> __device__ __forceinline__ void store8(T* p, const frag_t<T>& v) {
  *reinterpret_cast<frag_t<T>*>(p) = v;
}
// Two groups of four contiguous elements as one fragment (elements 0..3, 4..7).
template <typename T> __device__ __forceinline__ frag_t<T> load4x2(const T* p0, const T* p1) {
  vec4_t<T> lo = load4<T>(p0), hi = load4<T>(p1);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
template <typename T> __device__ __forceinline__ frag_t<T> zero_frag() {
  frag_t<T> f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = from_f32<T>(0.f);
  return f;
}
template <typename T> __device__ __forceinline__ vec4_t<T> zero4() {
  vec4_t<T> f;
#pragma unroll
  for (int e = 0; e < 4; ++e) f[e] = from_f32<T>(0.f);
  return f;
}

// Bytes of LDS padding per row that keep 16-byte alignment and spread rows
// over banks.
template <typename T> constexpr int pad16() { return 16 / (int)sizeof(T); }

}  // namespace infini
