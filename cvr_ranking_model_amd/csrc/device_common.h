// Device-side types and helpers shared by the gfx950 kernels of libcvr.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 f16;
typedef __bf16 bf16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void raise_flag(int32_t* flag, int32_t bits) {
  // Global-memory atomic through the vector memory path.
  atomicOr(flag, bits);
}

// Low-precision element traits.  The 32x32x16 MFMA on gfx950 takes 8 K-consecutive
// 16-bit values per lane for each operand: lane l holds row (l % 32) of A and
// column (l % 32) of B, k = 8*(l/32) .. 8*(l/32)+7; the 16 fp32 results of lane l
// are D[8*(v/4) + 4*(l/32) + (v%4)][l % 32] for v = 0..15.
template <typename T> struct Lowp;

template <> struct Lowp<f16> {
  typedef f16x8 vec8;
  typedef f16x4 vec4;
  static __device__ __forceinline__ f32x16 mfma32(const vec8& a, const vec8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f16 from_f32(float x) { return (f16)x; }
  static __device__ __forceinline__ float to_f32(f16 x) { return (float)x; }
};

template <> struct Lowp<bf16> {
  typedef bf16x8 vec8;
  typedef bf16x4 vec4;
  static __device__ __forceinline__ f32x16 mfma32(const vec8& a, const vec8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ bf16 from_f32(float x) { return (bf16)x; }
  static __device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
};

// The 32-bit finaliser of MurmurHash3 (Appleby): maps a row id to its cache set.
__device__ __forceinline__ uint32_t fmix32(uint32_t h) {
  h ^= h >> 16;
  h *= 0x85EBCA6Bu;
  h ^= h >> 13;
  h *= 0xC2B2AE35u;
  h ^= h >> 16;
  return h;
}

// IEEE 754-2019 maximum and minimum (v_maximum3_f32 / v_minimum3_f32 on gfx950): a NaN operand
// gives NaN, where fmaxf / fminf and a compare-and-select would return the other operand.  Every
// operator of the path lets NaN through, as the method's plain definition does.
__device__ __forceinline__ float max_nan(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float min_nan(float a, float b) { return __builtin_elementwise_minimum(a, b); }

// Clamp to [-c, c]; NaN passes through.
__device__ __forceinline__ float clamp_keep_nan(float v, float c) { return min_nan(max_nan(v, -c), c); }

// ReLU; NaN passes through.
__device__ __forceinline__ float relu_f32(float v) { return max_nan(v, 0.f); }

// Logistic sigmoid in fp32 from the device exp.
__device__ __forceinline__ float sigmoid_f32(float z) { return 1.0f / (1.0f + expf(-z)); }

// SplitMix64 output function (Steele, Lea & Flood 2014).
__device__ __forceinline__ uint64_t splitmix64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

template <typename T>
__device__ __forceinline__ typename Lowp<T>::vec8 load8(const T* p) {
  return *reinterpret_cast<const typename Lowp<T>::vec8*>(p);
}
