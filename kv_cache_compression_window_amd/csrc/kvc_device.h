// Device-side helpers shared by the gfx950 kernels of libkvc.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();
constexpr float kPosInf = __builtin_inff();

// One MFMA step of a 32x32 output block.  bf16 operands hold 8 consecutive
// contraction elements per lane (v_mfma_f32_32x32x16_bf16); fp32 operands hold
// one (v_mfma_f32_32x32x2_f32).  Lane l supplies row/column l % 32 and the
// contraction half l / 32 of every step, for A and B alike, so any fixed
// assignment of head_dim channels to (half, step, element) pairs that is the
// same for both operands forms every product q_d * k_d exactly once.
template <typename T> struct Mfma;

template <> struct Mfma<__bf16> {
  using op_t = bf16x8_t;
  static constexpr int KPL = 8;  // contraction elements per lane per step
  __device__ static inline f32x16_t run(op_t a, op_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline op_t zero() {
    op_t z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = (__bf16)0.0f;
    return z;
  }
};

template <> struct Mfma<float> {
  using op_t = float;
  static constexpr int KPL = 1;
  __device__ static inline f32x16_t run(op_t a, op_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static inline op_t zero() { return 0.0f; }
};

// Row (within the 32x32 output block) of accumulator register v in lane l;
// the column is l % 32.
__device__ inline int acc_row(int v, int lane) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Combine two (max, sum-of-exp2) pairs in base-2 log units.
__device__ inline void lse2_merge(float& m, float& z, float m2, float z2) {
  float mn = fmaxf(m, m2);
  if (mn == kNegInf) return;  // both empty
  z = z * exp2f(m - mn) + z2 * exp2f(m2 - mn);
  m = mn;
}

// Order-preserving map from float32 to uint32 (larger float -> larger key);
// -0.0 is mapped like +0.0.
__device__ inline uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace kvc
