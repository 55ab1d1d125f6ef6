// Device helpers shared by the KDA kernels: element types, bfloat16
// conversion, and 16x16 MFMA tiles for gfx950 (CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int kWave = 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// bfloat16 is carried as its 16-bit pattern.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// float -> bfloat16, round to nearest even (the hardware conversion).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
// Two floats -> two bfloat16 in one 32-bit word (lo in the low half).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = __builtin_convertvector((f32x2){lo, hi}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}

// Element-type traits.  `Elem` is how a value of the type sits in memory.
template <typename T> struct Ty;
template <> struct Ty<float> {
  using Elem = float;
  static constexpr int kBytes = 4;
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static float to_f32(float x) { return x; }
  __device__ __forceinline__ static float from_f32(float x) { return x; }
};
template <> struct Ty<bf16_t> {
  using Elem = uint16_t;
  static constexpr int kBytes = 2;
  __device__ __forceinline__ static float to_f32(uint16_t x) { return bf16_to_f32(x); }
  __device__ __forceinline__ static uint16_t from_f32(float x) { return f32_to_bf16(x); }
};

// ---------------------------------------------------------------------------
// Input prologue: the recurrence's inputs from raw projections.
//   gate:     alpha = exp(-softplus(g)) = 1 / (1 + e^g)   (0 at g = +inf, 1 at -inf)
//   strength: beta = sigmoid(b) = 1 / (1 + e^-b)
//   feature:  silu(x) = x sigmoid(x), then x / max(||x||_2, 1e-12) per row
// The SiLU and the sigmoid of the write strength follow the DeltaNet module on
// "22580: от GPT-2 до Kimi K3, объяснение", section "DeltaNet, или Fast Weight
// Programmers"; the gate form keeps every real logit inside (0, 1), as the
// gate of section "Gated Delta Net" of "From GPT-2 to Kimi K3, Explained"
// must be.  Hardware exp2 and reciprocal, each within about one ulp.
// ---------------------------------------------------------------------------
enum QkMap : int { kQkAsGiven = 0, kQkL2 = 1, kQkSiluL2 = 2 };

__device__ __forceinline__ float gate_from_logit(float g) {
  return __builtin_amdgcn_rcpf(1.f + __expf(g));
}
__device__ __forceinline__ float sigmoid_f(float x) {
  return __builtin_amdgcn_rcpf(1.f + __expf(-x));
}
__device__ __forceinline__ float silu_f(float x) { return x * sigmoid_f(x); }
// 1 / max(sqrt(sum of squares), 1e-12).
__device__ __forceinline__ float inv_l2(float sumsq) {
  return sumsq < 1e-24f ? 1e12f : __builtin_amdgcn_rsqf(sumsq);
}

// ---------------------------------------------------------------------------
// 16x16 output tiles on the matrix cores (used by the prefill kernel).
//
// Every operand is read from a row-major array whose rows are indexed by the
// tile's M (for A) or N (for B) coordinate and whose columns run along the
// contraction index K ("K-contiguous").  For D = A * B with A [M][K] and
// B [K][N], the A array is A itself and the B array is B^T [N][K].
//
// Lane layouts (wave64), lane l, g = l / 16, i = l % 16:
//   f32 16x16x4    a = A[i][k0+g],           b = Bt[i][k0+g]
//   bf16 16x16x16  a = A[i][k0+4g .. +3],    b = Bt[i][k0+4g .. +3]
//   bf16 16x16x32  a = A[i][k0+8g .. +7],    b = Bt[i][k0+8g .. +7]
//   result         acc[r] = D[4g + r][i],  r = 0..3
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

}  // namespace kda
