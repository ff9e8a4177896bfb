// Device-side helpers shared by the gfx950 kernels: vector types, storage
// formats, 16-lane DPP reductions and rounding to the output format.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Storage formats.  kBytes is the element size; a 16-byte chunk holds
// 16 / kBytes elements.
struct TF32 {
  static constexpr int kBytes = 4;
};
struct TF16 {
  static constexpr int kBytes = 2;
};
struct TBF16 {
  static constexpr int kBytes = 2;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(f16x2_t, w)[0]);
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(f16x2_t, w)[1]);
}

// Widen one 16-byte chunk of storage elements to float.
template <class T>
struct Unpack;
template <>
struct Unpack<TF32> {
  static constexpr int kE = 4;
  __device__ __forceinline__ static void run(u32x4_t w, float* o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __uint_as_float(w[i]);
  }
};
template <>
struct Unpack<TBF16> {
  static constexpr int kE = 8;
  __device__ __forceinline__ static void run(u32x4_t w, float* o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = bf16_lo(w[i]);
      o[2 * i + 1] = bf16_hi(w[i]);
    }
  }
};
template <>
struct Unpack<TF16> {
  static constexpr int kE = 8;
  __device__ __forceinline__ static void run(u32x4_t w, float* o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = f16_lo(w[i]);
      o[2 * i + 1] = f16_hi(w[i]);
    }
  }
};

// Read-only int32 data (block tables, context lengths) viewed through the
// constant address space: a wave-uniform index then compiles to a scalar
// load, whose wait (lgkmcnt) does not drain the vector loads in flight --
// a vector load of a table entry would need vmcnt(0), which is in order and
// so would wait for every K/V load issued before it.
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
__device__ __forceinline__ const_i32_ptr as_const(const int32_t* p) {
  return (const_i32_ptr)(p);  // address-space cast
}

__device__ __forceinline__ u32x4_t load16(const uint8_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

// Streaming load for data read once (the KV cache in decode): the
// nontemporal hint keeps it from displacing reusable lines in the caches.
__device__ __forceinline__ u32x4_t load16_stream(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

// DPP move within rows of 16 lanes.  quad_perm(1,0,3,2) = 0xB1,
// quad_perm(2,3,0,1) = 0x4E, row_ror:4 = 0x124, row_ror:8 = 0x128.
template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, 0xF, 0xF, false));
}

// Every lane of a 16-lane row receives the row's maximum / sum.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));
  v = fmaxf(v, dpp_mov<0x4E>(v));
  v = fmaxf(v, dpp_mov<0x124>(v));
  v = fmaxf(v, dpp_mov<0x128>(v));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x124>(v);
  v += dpp_mov<0x128>(v);
  return v;
}

__device__ __forceinline__ float uniform(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Round-to-nearest-even narrowing for the output formats.
__device__ __forceinline__ uint16_t to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ uint16_t to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// Store one float as an element of the output tensor (f32, or the input's
// 16-bit format).
template <class T>
__device__ __forceinline__ void store_out(void* base, int64_t idx, float v, bool out_f32) {
  if (out_f32) {
    static_cast<float*>(base)[idx] = v;
  } else if constexpr (T::kBytes == 4) {
    static_cast<float*>(base)[idx] = v;
  } else if constexpr (__is_same(T, TBF16)) {
    static_cast<uint16_t*>(base)[idx] = to_bf16_bits(v);
  } else {
    static_cast<uint16_t*>(base)[idx] = to_f16_bits(v);
  }
}

}  // namespace pa
