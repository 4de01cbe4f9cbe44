// Device-side helpers shared by the xattn kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// v_exp_f32 computes 2^x; v_log_f32 computes log2(x).
__device__ __forceinline__ float exp2_approx(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_approx(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Load EPL consecutive elements of storage type T as float.
template <typename T, int EPL>
struct Load;

template <>
struct Load<uint16_t, 8> {
  __device__ __forceinline__ static void run(const uint16_t* p, float* out) {
    uint4 u = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

template <>
struct Load<uint16_t, 4> {
  __device__ __forceinline__ static void run(const uint16_t* p, float* out) {
    uint2 u = *reinterpret_cast<const uint2*>(p);
    out[0] = __uint_as_float(u.x << 16);
    out[1] = __uint_as_float(u.x & 0xffff0000u);
    out[2] = __uint_as_float(u.y << 16);
    out[3] = __uint_as_float(u.y & 0xffff0000u);
  }
};

template <>
struct Load<float, 8> {
  __device__ __forceinline__ static void run(const float* p, float* out) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  }
};

template <>
struct Load<float, 4> {
  __device__ __forceinline__ static void run(const float* p, float* out) {
    float4 a = *reinterpret_cast<const float4*>(p);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  }
};

// Map a hardware block index to a logical work index so that logical
// neighbours run on the same XCD (blocks are dealt round-robin to the 8 XCDs,
// each with its own L2). `grid` must be a multiple of 8. Returns -1 for the
// padding blocks beyond `n_logical`.
__device__ __forceinline__ int64_t xcd_logical_block(int64_t bid, int64_t grid, int64_t n_logical) {
  const int64_t per_xcd = grid >> 3;
  const int64_t logical = (bid & 7) * per_xcd + (bid >> 3);
  return logical < n_logical ? logical : -1;
}

}  // namespace xattn
