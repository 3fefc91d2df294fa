// fa_common.h -- device helpers shared by the attention kernels (gfx950 only).
//
// Matrix-core conventions used throughout (CDNA 32x32 MFMA family):
//   * A operand (M x K): lane l supplies row m = l % 32 and KPL consecutive
//     k-elements of the lane group g = l / 32.
//   * B operand (K x N): lane l supplies column n = l % 32 and the same KPL
//     k-elements of group g.  Only the agreement between A and B matters for
//     the sum over k, so any k-assignment that both operands share is valid.
//   * C/D (32 x 32 fp32, 16 registers): register i of lane l holds
//     row acc_row(i, g) = 8*(i/4) + 4*g + (i%4), column l % 32.
// bf16 uses v_mfma_f32_32x32x16_bf16 (KPL = 8); fp32 uses
// v_mfma_f32_32x32x2_f32 (KPL = 1).  Accumulation is always fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

template <typename T> struct Mfma;

template <> struct Mfma<bf16> {
  static constexpr int KPL = 8;   // k elements per lane per instruction
  static constexpr int KC = 16;   // k per instruction
  using Frag = bf16x8;
  __device__ __forceinline__ static f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static Frag zero() { return Frag{}; }
  // 8 consecutive elements (16 bytes) from global or LDS memory
  __device__ __forceinline__ static Frag load(const bf16* p) { return *reinterpret_cast<const Frag*>(p); }
  // registers i = KPL*t .. KPL*t+KPL-1 of an accumulator, rounded to bf16
  __device__ __forceinline__ static Frag pack(const f32x16& x, int t) {
    Frag f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (bf16)x[8 * t + e];
    return f;
  }
};

template <> struct Mfma<float> {
  static constexpr int KPL = 1;
  static constexpr int KC = 2;
  using Frag = float;
  __device__ __forceinline__ static f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static Frag zero() { return 0.f; }
  __device__ __forceinline__ static Frag load(const float* p) { return *p; }
  __device__ __forceinline__ static Frag pack(const f32x16& x, int t) { return x[t]; }
};

// Row of accumulator register i for lane group g (see the header comment).
__device__ __forceinline__ constexpr int acc_row(int i, int g) { return 8 * (i >> 2) + 4 * g + (i & 3); }

// Both lanes l and l^32 receive f(x[l & 31], x[(l & 31) + 32]) with the
// operands in the same order, so the two halves of a wave agree bit for bit.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Exponent domain of the softmax.  bf16 inputs: base 2 with scale*log2(e)
// folded into one FMA and the hardware v_exp_f32.  fp32 inputs: base e with
// the accurate expf, so that the fp32 path keeps about 1e-7 relative error
// in every probability (the fp32 tolerance is 1e-5 absolute).
template <typename T> struct ExpDomain;
template <> struct ExpDomain<bf16> {
  __device__ __forceinline__ static float factor(float scale, float scale_log2) { return scale_log2; }
  __device__ __forceinline__ static float ex(float x) { return fast_exp2(x); }
  __device__ __forceinline__ static float from_lse(float lse) { return lse * kLog2e; }
};
template <> struct ExpDomain<float> {
  __device__ __forceinline__ static float factor(float scale, float) { return scale; }
  __device__ __forceinline__ static float ex(float x) { return expf(x); }
  __device__ __forceinline__ static float from_lse(float lse) { return lse; }
};

// 16-byte vector of elements, used for coalesced global<->LDS staging.
template <typename T> struct Vec16 {
  static constexpr int N = 16 / sizeof(T);
  uint4 raw;
  __device__ __forceinline__ T get(int e) const {
    union { uint4 u; T t[N]; } c;
    c.u = raw;
    return c.t[e];
  }
};

}  // namespace fa
