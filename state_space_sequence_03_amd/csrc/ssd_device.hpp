// ssd_device.hpp -- device-side types and MFMA fragment helpers for gfx950.
//
// Fragment convention used by every kernel here: an MFMA "K-step" covers 32
// values of the contraction index k.  Lane l of a wave (64 lanes) holds 8 of
// them for one row (A operand) or one column (B operand): row/col = l % 16,
// k = 8 * (l / 16) + e, e = 0..7.  The 16x16 fp32 accumulator holds, in lane
// l, column l % 16 and rows 4 * (l / 16) + r, r = 0..3.
//
//   bf16: one v_mfma_f32_16x16x32_bf16 per K-step.
//   fp32: eight v_mfma_f32_16x16x4_f32; in the s-th one lane group g = l / 16
//         supplies k = 8g + s, so the eight together cover the same 32 k's.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWave = 64;

template <typename T> struct FragOf;
template <> struct FragOf<bf16> { typedef bf16x8 type; };
template <> struct FragOf<float> { typedef floatx8 type; };

__device__ __forceinline__ floatx4 mma(floatx4 c, bf16x8 a, bf16x8 b) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mma(floatx4 c, floatx8 a, floatx8 b) {
#pragma unroll
  for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], c, 0, 0, 0);
  return c;
}

template <typename T> __device__ __forceinline__ T to_io(float v);
template <> __device__ __forceinline__ bf16 to_io<bf16>(float v) { return static_cast<bf16>(v); }
template <> __device__ __forceinline__ float to_io<float>(float v) { return v; }

__device__ __forceinline__ float to_f32(bf16 v) { return static_cast<float>(v); }
__device__ __forceinline__ float to_f32(float v) { return v; }

// Hardware base-2 exponential (v_exp_f32).  exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte vector of io elements: 8 bf16 or 4 fp32.
typedef uint4 vec16;
template <typename T> struct Vec16 { static constexpr int n = 16 / sizeof(T); };

__device__ __forceinline__ vec16 zero16() { return make_uint4(0u, 0u, 0u, 0u); }

template <typename T>
__device__ __forceinline__ vec16 load16(const T* p) { return *reinterpret_cast<const vec16*>(p); }
template <typename T>
__device__ __forceinline__ void store16(T* p, vec16 v) { *reinterpret_cast<vec16*>(p) = v; }

// Load one fragment (8 consecutive k values) from memory where k is contiguous.
__device__ __forceinline__ bf16x8 load_frag(const bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ floatx8 load_frag(const float* p) {
  // two 16-byte halves: rows are only guaranteed 16-byte aligned
  const floatx4 lo = *reinterpret_cast<const floatx4*>(p);
  const floatx4 hi = *reinterpret_cast<const floatx4*>(p + 4);
  floatx8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}
template <typename T> __device__ __forceinline__ typename FragOf<T>::type zero_frag() {
  typename FragOf<T>::type z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = static_cast<T>(0.0f);
  return z;
}

}  // namespace ssd
