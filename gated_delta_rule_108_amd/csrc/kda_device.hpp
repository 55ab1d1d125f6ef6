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

// Round-to-nearest-even float -> bfloat16; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
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
// 16x16 output tiles on the matrix cores.
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
template <typename OpT> struct Mma;

template <> struct Mma<float> {
  static constexpr int kStep = 4;
  // acc += A[a0.., k0..k0+16) * B[k0..k0+16), b0..]  (four K=4 steps)
  __device__ __forceinline__ static void k16(f32x4& acc, const float* A, int lda,
                                             const float* Bt, int ldb, int k0) {
    const int l = threadIdx.x % kWave;
    const int g = l >> 4, i = l & 15;
#pragma unroll
    for (int s = 0; s < 16; s += 4) {
      float a = A[i * lda + k0 + s + g];
      float b = Bt[i * ldb + k0 + s + g];
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
    }
  }
  __device__ __forceinline__ static void k32(f32x4& acc, const float* A, int lda,
                                             const float* Bt, int ldb, int k0) {
    k16(acc, A, lda, Bt, ldb, k0);
    k16(acc, A, lda, Bt, ldb, k0 + 16);
  }
};

template <> struct Mma<bf16_t> {
  static constexpr int kStep = 32;
  __device__ __forceinline__ static void k16(f32x4& acc, const uint16_t* A, int lda,
                                             const uint16_t* Bt, int ldb, int k0) {
    const int l = threadIdx.x % kWave;
    const int g = l >> 4, i = l & 15;
    bf16x4 a = *reinterpret_cast<const bf16x4*>(A + i * lda + k0 + 4 * g);
    bf16x4 b = *reinterpret_cast<const bf16x4*>(Bt + i * ldb + k0 + 4 * g);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, acc, 0, 0, 0);
  }
  __device__ __forceinline__ static void k32(f32x4& acc, const uint16_t* A, int lda,
                                             const uint16_t* Bt, int ldb, int k0) {
    const int l = threadIdx.x % kWave;
    const int g = l >> 4, i = l & 15;
    bf16x8 a = *reinterpret_cast<const bf16x8*>(A + i * lda + k0 + 8 * g);
    bf16x8 b = *reinterpret_cast<const bf16x8*>(Bt + i * ldb + k0 + 8 * g);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
  }
};

// acc += A[.., kb..ke) * B[kb..ke), ..]; kb, ke multiples of 16.
template <typename OpT>
__device__ __forceinline__ void mma_range(f32x4& acc, const typename Ty<OpT>::Elem* A, int lda,
                                          const typename Ty<OpT>::Elem* Bt, int ldb,
                                          int kb, int ke) {
  int k = kb;
  for (; k + 32 <= ke; k += 32) Mma<OpT>::k32(acc, A, lda, Bt, ldb, k);
  if (k < ke) Mma<OpT>::k16(acc, A, lda, Bt, ldb, k);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

}  // namespace kda
