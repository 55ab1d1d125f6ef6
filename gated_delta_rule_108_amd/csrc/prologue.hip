// The input prologue on its own, forward and adjoint, for training from raw
// projections: the forward writes the recurrence's inputs (q_hat, k_hat,
// alpha, beta) that the prefill backward takes, and the adjoint turns the
// gradients with respect to them into gradients with respect to the raw
// inputs.
//
// Forward, per row (one token of one head): alpha = 1 / (1 + e^g) per key
// channel, beta = sigmoid(b), and q, k mapped as given, by x / max(||x||,
// 1e-12), or by that after SiLU (the SiLU output rounded to the I/O type, as
// the fused prologue of the chunk and decode kernels does).  Sources: "From
// GPT-2 to Kimi K3, Explained", section "Gated Delta Net" (a gate in [0, 1]);
// "22580: от GPT-2 до Kimi K3, объяснение", section "DeltaNet, или Fast
// Weight Programmers" (SiLU, L2 normalisation over the head dimension, a
// sigmoid for the write strength).
//
// Adjoint (the chain rule of those maps):
//   dg = -dalpha alpha (1 - alpha),   db = dbeta beta (1 - beta)
//   normalize, y = x / max(||x||, eps):  dx = (dy - y (y . dy)) / ||x||   if ||x|| > eps
//                                        dx = dy / eps                     otherwise
//   SiLU:  dq = dx sigmoid(q) (1 + q (1 - sigmoid(q)))
//
// Both are bound by HBM: one wave per row, lane l holding channels
// l * EPL .. l * EPL + EPL - 1 (two at dk = 128, so each access is one wider
// load or store); the row sums (||x||^2, y . dy) are wave butterflies.
#include <type_traits>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {
namespace {

constexpr int kRowsPerBlock = 4;   // one wave per row

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// N consecutive channels of a row as float: two bf16 are one 32-bit load and
// two fp32 one 64-bit load (the rows start 16-byte aligned and a lane's
// first channel is even).
template <typename T, int N>
__device__ __forceinline__ void load_vec(const typename Ty<T>::Elem* p, float* out) {
  if constexpr (N == 2 && std::is_same<T, bf16_t>::value) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
    out[0] = __uint_as_float(w << 16);
    out[1] = __uint_as_float(w & 0xFFFF0000u);
  } else if constexpr (N == 2) {
    const float2 w = *reinterpret_cast<const float2*>(p);
    out[0] = w.x;
    out[1] = w.y;
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = Ty<T>::to_f32(p[i]);
  }
}
template <typename T, int N>
__device__ __forceinline__ void store_vec(typename Ty<T>::Elem* p, const float* v) {
  if constexpr (N == 2 && std::is_same<T, bf16_t>::value) {
    *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(v[0], v[1]);
  } else if constexpr (N == 2) {
    *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) p[i] = Ty<T>::from_f32(v[i]);
  }
}

// Value of a feature after the map's element-wise part (SiLU rounded to the
// I/O type, or the value itself).
template <typename IO>
__device__ __forceinline__ float feature_fwd(float x, int qk_map) {
  return qk_map == kQkSiluL2 ? Ty<IO>::to_f32(Ty<IO>::from_f32(silu_f(x))) : x;
}

template <typename IO, int DK>
__global__ void __launch_bounds__(kRowsPerBlock * kWave)
kda_prologue_forward_kernel(const typename Ty<IO>::Elem* __restrict__ q,
                            const typename Ty<IO>::Elem* __restrict__ k,
                            const typename Ty<IO>::Elem* __restrict__ g,
                            const float* __restrict__ b, typename Ty<IO>::Elem* __restrict__ qh,
                            typename Ty<IO>::Elem* __restrict__ kh, float* __restrict__ alpha,
                            float* __restrict__ beta, int rows, int qk_map) {
  constexpr int EPL = (DK + kWave - 1) / kWave;   // channels per lane
  const int row = blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (row >= rows) return;   // whole waves: the row is wave-uniform
  const size_t base = static_cast<size_t>(row) * DK + lane * EPL;
  const bool has = DK >= kWave || lane < DK;   // lanes past dk hold no channel
  float xq[EPL] = {}, xk[EPL] = {}, gl[EPL] = {}, sq = 0.f, sk = 0.f;
  if (has) {
    load_vec<IO, EPL>(q + base, xq);
    load_vec<IO, EPL>(k + base, xk);
    load_vec<IO, EPL>(g + base, gl);
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    xq[e] = feature_fwd<IO>(xq[e], qk_map);
    xk[e] = feature_fwd<IO>(xk[e], qk_map);
    gl[e] = gate_from_logit(gl[e]);
    sq += xq[e] * xq[e];
    sk += xk[e] * xk[e];
  }
  float iq = 1.f, ik = 1.f;
  if (qk_map != kQkAsGiven) {
    iq = inv_l2(wave_sum(sq));
    ik = inv_l2(wave_sum(sk));
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    xq[e] *= iq;
    xk[e] *= ik;
  }
  if (has) {
    store_vec<IO, EPL>(qh + base, xq);
    store_vec<IO, EPL>(kh + base, xk);
    store_vec<float, EPL>(alpha + base, gl);
  }
  if (lane == 0) beta[row] = sigmoid_f(b[row]);
}

// Adjoint of one feature row: x the raw row (EPL values per lane), dy the
// gradient with respect to the mapped row; returns dx in dy.
template <typename IO, int EPL>
__device__ __forceinline__ void feature_bwd(const float* x, float* dy, int qk_map) {
  if (qk_map == kQkAsGiven) return;
  float f[EPL], ss = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    f[e] = feature_fwd<IO>(x[e], qk_map);
    ss += f[e] * f[e];
  }
  ss = wave_sum(ss);
  if (ss < 1e-24f) {   // the norm floor: y = x / 1e-12, linear
#pragma unroll
    for (int e = 0; e < EPL; ++e) dy[e] *= 1e12f;
  } else {
    const float inv = __builtin_amdgcn_rsqf(ss);
    float proj = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) proj += f[e] * inv * dy[e];
    proj = wave_sum(proj);
#pragma unroll
    for (int e = 0; e < EPL; ++e) dy[e] = (dy[e] - f[e] * inv * proj) * inv;
  }
  if (qk_map == kQkSiluL2) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float s = sigmoid_f(x[e]);
      dy[e] *= s * (1.f + x[e] * (1.f - s));
    }
  }
}

template <typename IO, int DK>
__global__ void __launch_bounds__(kRowsPerBlock * kWave)
kda_prologue_backward_kernel(const typename Ty<IO>::Elem* __restrict__ q,
                             const typename Ty<IO>::Elem* __restrict__ k,
                             const typename Ty<IO>::Elem* __restrict__ g,
                             const float* __restrict__ b, const float* __restrict__ dqh,
                             const float* __restrict__ dkh, const float* __restrict__ dalpha,
                             const float* __restrict__ dbeta, float* __restrict__ dq,
                             float* __restrict__ dk, float* __restrict__ dg,
                             float* __restrict__ db, int rows, int qk_map) {
  constexpr int EPL = (DK + kWave - 1) / kWave;
  const int row = blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (row >= rows) return;
  const size_t base = static_cast<size_t>(row) * DK + lane * EPL;
  const bool has = DK >= kWave || lane < DK;
  float xq[EPL] = {}, xk[EPL] = {}, gq[EPL] = {}, gk[EPL] = {}, gl[EPL] = {}, da[EPL] = {};
  if (has) {
    load_vec<IO, EPL>(q + base, xq);
    load_vec<IO, EPL>(k + base, xk);
    load_vec<IO, EPL>(g + base, gl);
    load_vec<float, EPL>(dqh + base, gq);
    load_vec<float, EPL>(dkh + base, gk);
    load_vec<float, EPL>(dalpha + base, da);
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const float a = gate_from_logit(gl[e]);
    da[e] = -da[e] * a * (1.f - a);
  }
  feature_bwd<IO, EPL>(xq, gq, qk_map);
  feature_bwd<IO, EPL>(xk, gk, qk_map);
  if (has) {
    store_vec<float, EPL>(dq + base, gq);
    store_vec<float, EPL>(dk + base, gk);
    store_vec<float, EPL>(dg + base, da);
  }
  if (lane == 0) {
    const float be = sigmoid_f(b[row]);
    db[row] = dbeta[row] * be * (1.f - be);
  }
}

template <typename IO, int DK>
hipError_t run(const PrologueArgs& a) {
  using E = typename Ty<IO>::Elem;
  if (a.rows == 0) return hipSuccess;
  const unsigned grid = static_cast<unsigned>((a.rows + kRowsPerBlock - 1) / kRowsPerBlock);
  const hipStream_t stream = static_cast<hipStream_t>(a.stream);
  if (a.backward) {
    kda_prologue_backward_kernel<IO, DK><<<grid, kRowsPerBlock * kWave, 0, stream>>>(
        static_cast<const E*>(a.q), static_cast<const E*>(a.k), static_cast<const E*>(a.g), a.b,
        a.dq_hat, a.dk_hat, a.dalpha, a.dbeta, a.d_q, a.d_k, a.d_g, a.d_b, a.rows, a.qk_map);
  } else {
    kda_prologue_forward_kernel<IO, DK><<<grid, kRowsPerBlock * kWave, 0, stream>>>(
        static_cast<const E*>(a.q), static_cast<const E*>(a.k), static_cast<const E*>(a.g), a.b,
        static_cast<E*>(a.q_hat), static_cast<E*>(a.k_hat), a.alpha, a.beta, a.rows, a.qk_map);
  }
  return hipGetLastError();
}

template <typename IO>
hipError_t run_dk(const PrologueArgs& a) {
  switch (a.dk) {
    case 16: return run<IO, 16>(a);
    case 32: return run<IO, 32>(a);
    case 64: return run<IO, 64>(a);
    case 128: return run<IO, 128>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_prologue(const PrologueArgs& a) {
  return a.bf16 ? run_dk<bf16_t>(a) : run_dk<float>(a);
}

}  // namespace kda
