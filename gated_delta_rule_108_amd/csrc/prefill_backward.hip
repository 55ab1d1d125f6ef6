// KDA prefill backward: for B sequences x H heads of T tokens, the gradients
// of a loss L with respect to q, k, v, alpha, beta and the initial state,
// given dL/do for every token and dL/dS_T for the final state.
//
// The forward recurrence ("From GPT-2 to Kimi K3, Explained", sections
// "DeltaNet (Fast Weight Programmers)", "Gated Delta Net" and "KDA/Kimi
// Linear") applies, per token, S' = Diag(alpha) S, r = k S',
// u = beta (v - r), S = S' + k^T u, o = q S.  Its adjoint, token by token
// from the last to the first, with G = dS + q^T dO:
//   per value column j:  du_j = (k G)_j,  dv_j = beta du_j,  dr_j = -beta du_j
//   per element:         dS' = G + k^T dr,  dS (before the token) = Diag(alpha) dS'
//   row sums over j:     dq = S_new dO^T,  dk = G u^T + S' dr^T,
//                        dalpha = rowsum(dS' (.) S_before)
//   over j:              dbeta = sum_j du_j (v_j - r_j)
//
// Every value column of S (and of dS) evolves on its own in both directions;
// only the row sums and dbeta mix columns.  So one wave owns a slab of 8
// value columns of one (sequence, head) for the whole sequence: lane
// (rg = lane / 8, j = lane % 8) holds rows rg, rg + 8, ... of column j in
// registers.  Column sums (r, du) are an in-lane sum plus three exchanges
// across the 8 row-group lanes; row sums of the three per-row quantities are
// one transposed butterfly over the 8 column lanes (each exchange halves the
// values a lane holds), after which every lane adds its share to the fp32
// gradient rows with hardware float atomics (the slabs of a head add into the
// same rows).
//
// The backward needs the state before every token.  Kernel 1 runs the
// recurrence forward and stores the slab's state every kCk tokens into the
// workspace; kernel 2 walks those pieces from the last to the first: it
// restores the piece's first state, runs the kCk tokens forward again keeping
// each state in LDS, then runs them backward.  Per piece the token rows (k,
// alpha, q; v and dO of the slab; beta) are staged into LDS with 16-byte
// loads issued one piece ahead.
//
// The work is sequential in tokens (a latency-bound walk per wave, about
// 2 dk dv flops of VALU per element per token), unlike the chunked forward:
// the chunk form of the adjoint, on the matrix cores, is the next step.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {
namespace {

constexpr int kSlab = 8;    // value columns per wave
constexpr int kCk = 16;     // tokens between stored states

// Element x of a 16-byte word of IO values, as float.
template <typename IO> struct Word;
template <> struct Word<float> {
  static constexpr int kVec = 4;
  __device__ __forceinline__ static float get(const uint4& w, int x) {
    const uint32_t u = x == 0 ? w.x : x == 1 ? w.y : x == 2 ? w.z : w.w;
    return __uint_as_float(u);
  }
};
template <> struct Word<bf16_t> {
  static constexpr int kVec = 8;
  __device__ __forceinline__ static float get(const uint4& w, int x) {
    const uint32_t u = (x >> 1) == 0 ? w.x : (x >> 1) == 1 ? w.y : (x >> 1) == 2 ? w.z : w.w;
    return __uint_as_float((x & 1) ? (u & 0xFFFF0000u) : (u << 16));
  }
};

// LDS position of key row c in a staged row vector: the RPT rows of row
// group c % 8 sit together, so a lane reads its rows contiguously.
template <int DK>
__device__ __forceinline__ int kpos(int c) { return (c % kSlab) * (DK / kSlab) + c / kSlab; }

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int PATTERN>
__device__ __forceinline__ float swz(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), PATTERN));
}
// Lane exchanges.  xor 1 and 2: quad_perm; xor 8: row_ror:8 (within a row
// of 16 lanes, rotating by 8 is xor 8); xor 4 and 16: ds_swizzle in bit mode
// (and-mask 31, xor-mask 4 or 16); xor 32: the lane crossbar.
__device__ __forceinline__ float xor1(float v) { return dpp<0xB1>(v); }
__device__ __forceinline__ float xor2(float v) { return dpp<0x4E>(v); }
__device__ __forceinline__ float xor4(float v) { return swz<(4 << 10) | 0x1F>(v); }
__device__ __forceinline__ float xor8(float v) { return dpp<0x128>(v); }
__device__ __forceinline__ float xor16(float v) { return swz<(16 << 10) | 0x1F>(v); }

// Sum over the 8 row-group lanes of a column (lane bits 3..5), to all of them.
__device__ __forceinline__ float col_sum(float x) {
  x += xor8(x);
  x += xor16(x);
  x += __shfl_xor(x, 32);
  return x;
}
// Sum over the 8 column lanes of a row group (lane bits 0..2), to all of them.
__device__ __forceinline__ float row_sum(float x) {
  x += xor1(x);
  x += xor2(x);
  x += xor4(x);
  return x;
}

// One halving step of the transposed butterfly: of the first 2n values, the
// lane keeps the half its bit selects, summed with the partner's copy of it.
template <int N, class X>
__device__ __forceinline__ void halve(float* a, bool hi, X exch) {
#pragma unroll
  for (int m = 0; m < N; ++m) {
    const float keep = hi ? a[m + N] : a[m];
    const float send = hi ? a[m] : a[m + N];
    a[m] = keep + exch(send);
  }
}

// Token rows of one piece of kCk tokens, loaded into registers (one piece
// ahead) and then stored to LDS as float.
template <typename IO, int DK, bool kBwd>
struct Stage {
  using E = typename Ty<IO>::Elem;
  static constexpr int VEC = Word<IO>::kVec;
  static constexpr int NRI = (kCk * DK + kWave * VEC - 1) / (kWave * VEC);   // k, q words
  static constexpr int NRA = (kCk * DK + kWave * 4 - 1) / (kWave * 4);       // alpha float4s
  static constexpr int NCV = kCk / kSlab;                                      // v, dO per lane
  uint4 kr[NRI];
  uint4 qr[kBwd ? NRI : 1];
  float4 ar[NRA];
  float vc[NCV], oc[kBwd ? NCV : 1];
  float bb;

  // Tokens t0 .. t0 + n - 1 of chain (b, h); row offsets in elements.
  __device__ __forceinline__ void load(const E* k, const E* q, const float* alpha, const E* v,
                                       const E* dO, const float* beta, size_t tok0, int H,
                                       int DV, int n, int col, int lane) {
#pragma unroll
    for (int it = 0; it < NRI; ++it) {
      const int e = (it * kWave + lane) * VEC, s = e / DK, c = e % DK;
      const bool ok = e < kCk * DK && s < n;
      const size_t off = (tok0 + static_cast<size_t>(s) * H) * DK + c;
      kr[it] = ok ? *reinterpret_cast<const uint4*>(k + off) : make_uint4(0, 0, 0, 0);
      if constexpr (kBwd)
        qr[it] = ok ? *reinterpret_cast<const uint4*>(q + off) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int it = 0; it < NRA; ++it) {
      const int e = (it * kWave + lane) * 4, s = e / DK, c = e % DK;
      const bool ok = e < kCk * DK && s < n;
      const size_t off = (tok0 + static_cast<size_t>(s) * H) * DK + c;
      ar[it] = ok ? *reinterpret_cast<const float4*>(alpha + off) : make_float4(0, 0, 0, 0);
    }
#pragma unroll
    for (int m = 0; m < NCV; ++m) {
      const int s = lane / kSlab + kSlab * m;
      const bool ok = s < n;
      const size_t off = (tok0 + static_cast<size_t>(s) * H) * DV + col;
      vc[m] = ok ? Ty<IO>::to_f32(v[off]) : 0.f;
      if constexpr (kBwd) oc[m] = ok ? Ty<IO>::to_f32(dO[off]) : 0.f;
    }
    bb = (lane < kCk && lane < n) ? beta[tok0 + static_cast<size_t>(lane) * H] : 0.f;
  }

  __device__ __forceinline__ void store(float* kS, float* qS, float* aS, float* vS, float* oS,
                                        float* bS, int lane) const {
#pragma unroll
    for (int it = 0; it < NRI; ++it) {
      const int e = (it * kWave + lane) * VEC, s = e / DK, c = e % DK;
      if (e < kCk * DK) {
#pragma unroll
        for (int x = 0; x < VEC; ++x) {
          kS[s * DK + kpos<DK>(c + x)] = Word<IO>::get(kr[it], x);
          if constexpr (kBwd) qS[s * DK + kpos<DK>(c + x)] = Word<IO>::get(qr[it], x);
        }
      }
    }
#pragma unroll
    for (int it = 0; it < NRA; ++it) {
      const int e = (it * kWave + lane) * 4, s = e / DK, c = e % DK;
      if (e < kCk * DK) {
        aS[s * DK + kpos<DK>(c + 0)] = ar[it].x;
        aS[s * DK + kpos<DK>(c + 1)] = ar[it].y;
        aS[s * DK + kpos<DK>(c + 2)] = ar[it].z;
        aS[s * DK + kpos<DK>(c + 3)] = ar[it].w;
      }
    }
#pragma unroll
    for (int m = 0; m < NCV; ++m) {
      const int s = lane / kSlab + kSlab * m, j = lane % kSlab;
      vS[s * kSlab + j] = vc[m];
      if constexpr (kBwd) oS[s * kSlab + j] = oc[m];
    }
    if (lane < kCk) bS[lane] = bb;
  }
};

// One forward token on the lane's rows of column j.  Returns r_j; u_j in *u.
template <int RPT>
__device__ __forceinline__ float fwd_token(float* S, const float* kr, const float* ar, float vj,
                                           float bt, float* u) {
  float sp[RPT], acc = 0.f;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    sp[i] = ar[i] * S[i];
    acc += kr[i] * sp[i];
  }
  const float r = col_sum(acc);
  const float uj = bt * (vj - r);
#pragma unroll
  for (int i = 0; i < RPT; ++i) S[i] = sp[i] + kr[i] * uj;
  *u = uj;
  return r;
}

// Stored state layout: [chain][piece][slab][RPT][64 lanes] floats.
__device__ __forceinline__ size_t ck_off(size_t chain, int piece, int npiece, int slab, int NS,
                                         int DK) {
  return ((chain * npiece + piece) * NS + slab) * static_cast<size_t>(DK) * kSlab;
}

template <typename IO, int DK>
__global__ void __launch_bounds__(64)
kda_pb_forward_kernel(const typename Ty<IO>::Elem* __restrict__ k,
                      const typename Ty<IO>::Elem* __restrict__ v,
                      const float* __restrict__ alpha, const float* __restrict__ beta,
                      const float* __restrict__ S0, float* __restrict__ ck, int T, int H,
                      int DV) {
  constexpr int RPT = DK / kSlab;
  const int NS = DV / kSlab;
  const int chain = blockIdx.x / NS, slab = blockIdx.x % NS;
  const int b = chain / H, h = chain % H;
  const int lane = threadIdx.x, j = lane % kSlab, rg = lane / kSlab;
  const int col = slab * kSlab + j;
  const int npiece = (T + kCk - 1) / kCk;

  __shared__ float kS[kCk * DK], aS[kCk * DK], vS[kCk * kSlab], bS[kCk];
  float S[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    S[i] = S0 ? S0[(static_cast<size_t>(chain) * DK + rg + kSlab * i) * DV + col] : 0.f;

  Stage<IO, DK, false> st;
  auto tok0 = [&](int p) { return static_cast<size_t>(b) * T * H + static_cast<size_t>(p) * kCk * H + h; };
  auto count = [&](int p) { return min(kCk, T - p * kCk); };
  st.load(k, nullptr, alpha, v, nullptr, beta, tok0(0), H, DV, count(0), col, lane);
  for (int p = 0; p < npiece; ++p) {
    st.store(kS, nullptr, aS, vS, nullptr, bS, lane);
    __syncthreads();
    if (p + 1 < npiece)
      st.load(k, nullptr, alpha, v, nullptr, beta, tok0(p + 1), H, DV, count(p + 1), col, lane);
    float* out = ck + ck_off(chain, p, npiece, slab, NS, DK);
#pragma unroll
    for (int i = 0; i < RPT; ++i) out[i * kWave + lane] = S[i];
    const int n = count(p);
    for (int s = 0; s < n; ++s) {
      float u;
      fwd_token<RPT>(S, kS + s * DK + rg * RPT, aS + s * DK + rg * RPT, vS[s * kSlab + j], bS[s],
                     &u);
    }
    __syncthreads();
  }
}

template <typename IO, int DK>
__global__ void __launch_bounds__(64)
kda_pb_backward_kernel(const typename Ty<IO>::Elem* __restrict__ q,
                       const typename Ty<IO>::Elem* __restrict__ k,
                       const typename Ty<IO>::Elem* __restrict__ v,
                       const float* __restrict__ alpha, const float* __restrict__ beta,
                       const typename Ty<IO>::Elem* __restrict__ dO,
                       const float* __restrict__ dS_T, const float* __restrict__ ck,
                       float* __restrict__ g_q, float* __restrict__ g_k,
                       float* __restrict__ g_v, float* __restrict__ g_alpha,
                       float* __restrict__ g_beta, float* __restrict__ g_S0, int T, int H,
                       int DV) {
  constexpr int RPT = DK / kSlab;
  constexpr int NV = 3 * RPT;                     // (dq, dk, dalpha) per row
  constexpr int VP = (NV + kSlab - 1) / kSlab * kSlab;
  constexpr int PER = VP / kSlab;                 // values per lane after the butterfly
  const int NS = DV / kSlab;
  const int chain = blockIdx.x / NS, slab = blockIdx.x % NS;
  const int b = chain / H, h = chain % H;
  const int lane = threadIdx.x, j = lane % kSlab, rg = lane / kSlab;
  const int col = slab * kSlab + j;
  const int npiece = (T + kCk - 1) / kCk;

  __shared__ float kS[kCk * DK], qS[kCk * DK], aS[kCk * DK];
  __shared__ float vS[kCk * kSlab], oS[kCk * kSlab], uS[kCk * kSlab], rS[kCk * kSlab], bS[kCk];
  __shared__ float hist[kCk * RPT * kWave];     // state before each token of the piece

  float dS[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    dS[i] = dS_T ? dS_T[(static_cast<size_t>(chain) * DK + rg + kSlab * i) * DV + col] : 0.f;

  Stage<IO, DK, true> st;
  auto tok0 = [&](int p) { return static_cast<size_t>(b) * T * H + static_cast<size_t>(p) * kCk * H + h; };
  auto count = [&](int p) { return min(kCk, T - p * kCk); };
  if (npiece > 0)
    st.load(k, q, alpha, v, dO, beta, tok0(npiece - 1), H, DV, count(npiece - 1), col, lane);
  for (int p = npiece - 1; p >= 0; --p) {
    st.store(kS, qS, aS, vS, oS, bS, lane);
    __syncthreads();
    if (p > 0) st.load(k, q, alpha, v, dO, beta, tok0(p - 1), H, DV, count(p - 1), col, lane);
    const int n = count(p);
    float S[RPT];
    const float* in = ck + ck_off(chain, p, npiece, slab, NS, DK);
#pragma unroll
    for (int i = 0; i < RPT; ++i) S[i] = in[i * kWave + lane];
    // forward again over the piece, keeping the state before each token
    for (int s = 0; s < n; ++s) {
#pragma unroll
      for (int i = 0; i < RPT; ++i) hist[(s * RPT + i) * kWave + lane] = S[i];
      float u;
      const float r = fwd_token<RPT>(S, kS + s * DK + rg * RPT, aS + s * DK + rg * RPT,
                                     vS[s * kSlab + j], bS[s], &u);
      if (rg == 0) {
        uS[s * kSlab + j] = u;
        rS[s * kSlab + j] = r;
      }
    }
    __syncthreads();
    // backward over the piece
    for (int s = n - 1; s >= 0; --s) {
      const float* kr = kS + s * DK + rg * RPT;
      const float* qr = qS + s * DK + rg * RPT;
      const float* ar = aS + s * DK + rg * RPT;
      const float uj = uS[s * kSlab + j], rj = rS[s * kSlab + j];
      const float vj = vS[s * kSlab + j], oj = oS[s * kSlab + j], bt = bS[s];
      float Sb[RPT], G[RPT], acc = 0.f;
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        Sb[i] = hist[(s * RPT + i) * kWave + lane];
        G[i] = dS[i] + qr[i] * oj;
        acc += kr[i] * G[i];
      }
      const float du = col_sum(acc);
      const size_t row = tok0(p) + static_cast<size_t>(s) * H;   // (b, t, h)
      if (rg == 0) g_v[row * DV + col] = bt * du;
      const float pb = row_sum(du * (vj - rj));
      if (lane == 0) unsafeAtomicAdd(g_beta + row, pb);
      const float dr = -bt * du;
      float val[VP];
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const float sp = ar[i] * Sb[i];
        const float sn = sp + kr[i] * uj;
        const float dsp = G[i] + kr[i] * dr;
        val[3 * i + 0] = sn * oj;                 // dq
        val[3 * i + 1] = G[i] * uj + sp * dr;     // dk
        val[3 * i + 2] = dsp * Sb[i];             // dalpha
        dS[i] = ar[i] * dsp;
      }
#pragma unroll
      for (int m = NV; m < VP; ++m) val[m] = 0.f;
      halve<VP / 2>(val, (lane & 4) != 0, xor4);
      halve<VP / 4>(val, (lane & 2) != 0, xor2);
      halve<VP / 8>(val, (lane & 1) != 0, xor1);
      // lane j now holds the sums of values j * PER .. j * PER + PER - 1
#pragma unroll
      for (int w = 0; w < PER; ++w) {
        const int m = j * PER + w;
        if (m < NV) {
          const int i = m / 3, qn = m % 3;
          float* dst = qn == 0 ? g_q : (qn == 1 ? g_k : g_alpha);
          unsafeAtomicAdd(dst + row * DK + rg + kSlab * i, val[w]);
        }
      }
    }
    __syncthreads();
  }
  if (g_S0) {
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      g_S0[(static_cast<size_t>(chain) * DK + rg + kSlab * i) * DV + col] = dS[i];
  }
}

__global__ void zero_fill_kernel(float* a, size_t na, float* b, size_t nb, float* c, size_t nc,
                                 float* d, size_t nd) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
       i < na + nb + nc + nd; i += stride) {
    if (i < na) a[i] = 0.f;
    else if (i < na + nb) b[i - na] = 0.f;
    else if (i < na + nb + nc) c[i - na - nb] = 0.f;
    else d[i - na - nb - nc] = 0.f;
  }
}

template <typename IO, int DK>
hipError_t run(const PrefillBwdArgs& a) {
  using E = typename Ty<IO>::Elem;
  const int NS = a.dv / kSlab;
  const unsigned grid = static_cast<unsigned>(a.B) * a.H * NS;
  const hipStream_t stream = static_cast<hipStream_t>(a.stream);
  if (a.T > 0) {
    const size_t nk = static_cast<size_t>(a.B) * a.T * a.H * a.dk;
    const size_t nb = static_cast<size_t>(a.B) * a.T * a.H;
    const size_t tot = 3 * nk + nb;
    const size_t zb = (tot + 255) / 256;
    const unsigned zg = static_cast<unsigned>(zb < 4096 ? zb : 4096);
    zero_fill_kernel<<<zg, 256, 0, stream>>>(a.g_q, nk, a.g_k, nk, a.g_alpha, nk, a.g_beta,
                                               nb);
    kda_pb_forward_kernel<IO, DK><<<grid, kWave, 0, stream>>>(
        static_cast<const E*>(a.k), static_cast<const E*>(a.v), a.alpha, a.beta, a.S0,
        static_cast<float*>(a.workspace), a.T, a.H, a.dv);
  }
  kda_pb_backward_kernel<IO, DK><<<grid, kWave, 0, stream>>>(
      static_cast<const E*>(a.q), static_cast<const E*>(a.k), static_cast<const E*>(a.v),
      a.alpha, a.beta, static_cast<const E*>(a.dO), a.dS_T,
      static_cast<const float*>(a.workspace), a.g_q, a.g_k, a.g_v, a.g_alpha, a.g_beta, a.g_S0,
      a.T, a.H, a.dv);
  return hipGetLastError();
}

template <typename IO>
hipError_t run_dk(const PrefillBwdArgs& a) {
  switch (a.dk) {
    case 16: return run<IO, 16>(a);
    case 32: return run<IO, 32>(a);
    case 64: return run<IO, 64>(a);
    case 128: return run<IO, 128>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t prefill_backward_workspace(int B, int T, int H, int dk, int dv) {
  const size_t npiece = (static_cast<size_t>(T) + kCk - 1) / kCk;
  return static_cast<size_t>(B) * H * npiece * dk * dv * sizeof(float);
}

hipError_t launch_prefill_backward(const PrefillBwdArgs& a) {
  if (a.dv % kSlab != 0) return hipErrorInvalidValue;
  return a.bf16 ? run_dk<bf16_t>(a) : run_dk<float>(a);
}

}  // namespace kda
