// Device helpers shared by the gfx950 kernels of the GQA decode step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// bfloat16 is the upper half of a binary32: widening is a 16-bit shift.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// binary32 -> bfloat16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Streaming 16-byte load: K/V rows are read once per call, so they are fetched
// with the non-temporal hint and do not push reusable lines out of the caches.
__device__ __forceinline__ u32x4 load_nt16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ uint32_t load_nt4(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}
__device__ __forceinline__ uint16_t load_nt2(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p));
}

// Storage traits: element size and widening of 1, 4 or 8 consecutive elements.
template <int DT> struct Store;
template <> struct Store<0> {  // float32
  static constexpr int kBytes = 4;
  __device__ static __forceinline__ float load1(const void* base, int64_t i) {
    return __uint_as_float(load_nt4(reinterpret_cast<const uint32_t*>(base) + i));
  }
  __device__ static __forceinline__ float load1_cached(const void* base, int64_t i) {
    return reinterpret_cast<const float*>(base)[i];
  }
  __device__ static __forceinline__ void store1(void* base, int64_t i, float x) {
    reinterpret_cast<float*>(base)[i] = x;
  }
};
template <> struct Store<1> {  // bfloat16
  static constexpr int kBytes = 2;
  __device__ static __forceinline__ float load1(const void* base, int64_t i) {
    return bf16_to_f32(load_nt2(reinterpret_cast<const uint16_t*>(base) + i));
  }
  __device__ static __forceinline__ float load1_cached(const void* base, int64_t i) {
    return bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[i]);
  }
  __device__ static __forceinline__ void store1(void* base, int64_t i, float x) {
    reinterpret_cast<uint16_t*>(base)[i] = f32_to_bf16_rne(x);
  }
};

// Widen one 16-byte vector of storage into floats (8 bf16 or 4 f32).
template <int DT> __device__ __forceinline__ void widen16(u32x4 w, float* out);
template <> __device__ __forceinline__ void widen16<0>(u32x4 w, float* out) {
  out[0] = __uint_as_float(w.x); out[1] = __uint_as_float(w.y);
  out[2] = __uint_as_float(w.z); out[3] = __uint_as_float(w.w);
}
template <> __device__ __forceinline__ void widen16<1>(u32x4 w, float* out) {
  out[0] = bf16_lo(w.x); out[1] = bf16_hi(w.x); out[2] = bf16_lo(w.y); out[3] = bf16_hi(w.y);
  out[4] = bf16_lo(w.z); out[5] = bf16_hi(w.z); out[6] = bf16_lo(w.w); out[7] = bf16_hi(w.w);
}

// Fast base-2 exponential (v_exp_f32).  exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace gqa
