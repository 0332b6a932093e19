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
  __device__ static __forceinline__ void copy1(void* dst, int64_t i, const void* src, int64_t j) {
    reinterpret_cast<uint32_t*>(dst)[i] = reinterpret_cast<const uint32_t*>(src)[j];
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
  __device__ static __forceinline__ void copy1(void* dst, int64_t i, const void* src, int64_t j) {
    reinterpret_cast<uint16_t*>(dst)[i] = reinterpret_cast<const uint16_t*>(src)[j];
  }
};

template <> struct Store<2> {  // int8 codes (read only; the value is code * row scale)
  static constexpr int kBytes = 1;
  __device__ static __forceinline__ float load1(const void* base, int64_t i) {
    return (float)__builtin_nontemporal_load(reinterpret_cast<const int8_t*>(base) + i);
  }
  __device__ static __forceinline__ float load1_cached(const void* base, int64_t i) {
    return (float)reinterpret_cast<const int8_t*>(base)[i];
  }
};

// Widen one 16-byte vector of storage into floats (8 bf16, 4 f32 or 16 int8).
template <int DT> __device__ __forceinline__ void widen16(u32x4 w, float* out);
template <> __device__ __forceinline__ void widen16<0>(u32x4 w, float* out) {
  out[0] = __uint_as_float(w.x); out[1] = __uint_as_float(w.y);
  out[2] = __uint_as_float(w.z); out[3] = __uint_as_float(w.w);
}
template <> __device__ __forceinline__ void widen16<1>(u32x4 w, float* out) {
  out[0] = bf16_lo(w.x); out[1] = bf16_hi(w.x); out[2] = bf16_lo(w.y); out[3] = bf16_hi(w.y);
  out[4] = bf16_lo(w.z); out[5] = bf16_hi(w.z); out[6] = bf16_lo(w.w); out[7] = bf16_hi(w.w);
}
template <> __device__ __forceinline__ void widen16<2>(u32x4 w, float* out) {
  const uint32_t v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) out[4 * i + j] = (float)(int32_t)((int32_t)(v[i] << (24 - 8 * j)) >> 24);
}

// Reductions over the four 16-lane rows of a wave (lanes c, c + 16, c + 32,
// c + 48), result in every lane, with gfx950's cross-row swaps
// (v_permlane16_swap, v_permlane32_swap): vector-ALU only, no LDS round trip.
// With both operands x, permlane16_swap returns rows (0,0,2,2) and (1,1,3,3),
// permlane32_swap returns halves (lo,lo) and (hi,hi); the sums associate as
// (r0 + r1) + (r2 + r3).  All 64 lanes must be active.
__device__ __forceinline__ float rows_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float rows_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Reductions over the 16 lanes of each row with DPP lane permutations (quad
// xor 1, quad xor 2, half-row mirror, row mirror): vector-ALU only, every lane
// ends with its row's result.  All 64 lanes must be active.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f32<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp_f32<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp_f32<0x141>(x);  // row_half_mirror: lane i <-> 7 - i
  return x + dpp_f32<0x140>(x);  // row_mirror: lane i <-> 15 - i
}
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f32<0xB1>(x));
  x = fmaxf(x, dpp_f32<0x4E>(x));
  x = fmaxf(x, dpp_f32<0x141>(x));
  return fmaxf(x, dpp_f32<0x140>(x));
}
// Whole-wave sum / maximum from the row results and the cross-row swaps; all
// 64 lanes active.
__device__ __forceinline__ float wave_sum_dpp(float x) { return rows_sum(row16_sum(x)); }
__device__ __forceinline__ float wave_max_dpp(float x) { return rows_max(row16_max(x)); }

// Butterfly reductions over the 64 lanes of a wave, result in every lane.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// OCP 8-bit floating-point code (E4M3: bias 7, three mantissa bits,
// subnormals below 2^-6, largest finite 448) of a float32 value of magnitude at
// most 448: the nearest representable magnitude, ties to the even code, with
// the value's sign bit.  Normal range: the top three mantissa bits rounded on
// the 20 below (a carry moves into the exponent field); below 2^-6 the
// subnormal step 2^-9, i.e. rint(|x| * 512) (exact scaling, ties to even; 8
// is the code of 2^-6).
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(x);
  if (a < 0.015625f) return sign | (uint32_t)__builtin_rintf(a * 512.f);
  const uint32_t au = u & 0x7fffffffu;
  uint32_t m3 = (au >> 20) & 7u;
  const uint32_t rest = au & 0xfffffu;
  if (rest > 0x80000u || (rest == 0x80000u && (m3 & 1u))) ++m3;
  return sign | ((((au >> 23) - 120u) << 3) + m3);   // exponent field = unbiased + 7 = biased - 120
}

// Fast base-2 exponential (v_exp_f32).  exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace gqa
