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
// only the row sums and dbeta mix columns.  A workgroup of four waves (one
// per SIMD) owns WGC value columns of one (sequence, head) for the whole
// sequence; each wave holds CPW of them (2, or 4 at dk = 16): lane
// (rg = lane / CPW, j = lane % CPW) keeps rows rg, rg + RG, ... of its column
// in registers.  Column sums (r, du) are an in-lane sum plus exchanges across
// the RG row-group lanes; the row sums of the three per-row quantities are a
// transposed butterfly over the CPW column lanes, then plain stores into the
// wave's slots of the workgroup's row buffer; every half piece the four waves'
// sums are added to the fp32 gradient rows with coalesced global float
// atomics (the workgroups of a head add into the same rows).
//
// The backward needs the state before every token.  Kernel 1 runs the
// recurrence forward and stores the state every kCk tokens, and every token's
// write u and read r per column, into the workspace; kernel 2 walks those
// pieces from the last to the first: it restores the piece's first state,
// rebuilds the piece's states from it and the stored u (S = Diag(alpha) S +
// k^T u, no column sum) keeping each in LDS, then runs the tokens backward.
// Per piece the token rows (k, alpha, q; v, dO, u and r of the workgroup's
// columns; beta) and the next piece's first state are staged into LDS,
// shared by the four waves, with loads issued one piece ahead.
//
// The work is sequential in tokens (a latency-bound walk, about ten VALU
// flops per state element per token), unlike the chunked forward: the chunk
// form of the adjoint, on the matrix cores, is the next step.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {
namespace {

constexpr int kWaves = 4;   // waves per workgroup, one per SIMD
constexpr int kThreads = kWaves * kWave;
constexpr int kCk = 16;     // tokens between stored states
constexpr int kHalf = kCk / 2;   // tokens per row-sum flush

template <int DK>
struct Geo {
  static constexpr int CPW = DK >= 32 ? 2 : kWave / DK;   // value columns per wave
  static constexpr int RG = kWave / CPW;                   // row groups per wave
  static constexpr int RPT = DK / RG;                      // key rows per lane
  static constexpr int WGC = kWaves * CPW;                 // value columns per workgroup
  static constexpr int NV = 3 * RPT;                       // (dq, dk, dalpha) per row
  static constexpr int VP = (NV + CPW - 1) / CPW * CPW;    // padded for the butterfly
  static constexpr int PER = VP / CPW;                     // values per lane after it
  static_assert(RPT >= 1 && RG * RPT == DK, "rows must split evenly");
};

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
// group c % RG sit together, so a lane reads its rows contiguously.
template <int DK>
__device__ __forceinline__ int kpos(int c) {
  return (c % Geo<DK>::RG) * Geo<DK>::RPT + c / Geo<DK>::RG;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Value of lane (lane xor X), X = 1 or 2: quad_perm moves.
template <int X>
__device__ __forceinline__ float xr(float v) {
  static_assert(X == 1 || X == 2, "column lanes sit within a quad");
  return X == 1 ? dpp<0xB1>(v) : dpp<0x4E>(v);
}

// Sum over the row-group lanes of a column (the lanes equal to it modulo
// CPW), to all of them, on the VALU only: within each 16-lane row, adding
// the row rotated by CPW, 2 CPW, ... 8 sums the lanes of the same residue;
// permlane16_swap then pairs rows 0-1 and 2-3 and permlane32_swap the two
// halves of the wave (each swap exchanges the rows of two copies of x, so
// the sum of the two results is the sum over both rows).
template <int X>
__device__ __forceinline__ float ror_sum(float x) {
  if constexpr (X < 16) return ror_sum<2 * X>(x + dpp<0x120 + X>(x));
  else return x;
}
template <int CPW>
__device__ __forceinline__ float col_sum(float x) {
  x = ror_sum<CPW>(x);
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Sum over the CPW column lanes of a row group (lane bits below CPW), to all.
template <int CPW>
__device__ __forceinline__ float row_sum(float x) {
  x += xr<1>(x);
  if constexpr (CPW == 4) x += xr<2>(x);
  return x;
}

// Transposed butterfly over the CPW column lanes: each step keeps the half of
// the values that the lane's bit X selects, summed with the partner's copy of
// it.  Afterwards lane j holds the sums of values j * PER .. j * PER + PER - 1.
template <int N, int X>
__device__ __forceinline__ void halve(float* a, bool hi) {
#pragma unroll
  for (int m = 0; m < N; ++m) {
    const float keep = hi ? a[m + N] : a[m];
    const float send = hi ? a[m] : a[m + N];
    a[m] = keep + xr<X>(send);
  }
}
template <int CPW, int VP>
__device__ __forceinline__ void butterfly(float* a, int lane) {
  if constexpr (CPW == 4) {
    halve<VP / 2, 2>(a, (lane & 2) != 0);
    halve<VP / 4, 1>(a, (lane & 1) != 0);
  } else {
    halve<VP / 2, 1>(a, (lane & 1) != 0);
  }
}

// Token rows of one piece of kCk tokens for the whole workgroup, loaded into
// registers (one piece ahead) and then stored to LDS as float.
template <typename IO, int DK, bool kBwd, int kIn>
struct Stage {
  using E = typename Ty<IO>::Elem;
  static constexpr int VEC = Word<IO>::kVec;
  static constexpr int WGC = Geo<DK>::WGC;
  static constexpr int NRI = (kCk * DK + kThreads * VEC - 1) / (kThreads * VEC);  // k, q words
  static constexpr int NRA = (kCk * DK + kThreads * 4 - 1) / (kThreads * 4);      // alpha float4s
  static_assert(kCk * WGC <= kThreads, "one thread per (token, column)");
  uint4 kr[NRI];
  uint4 qr[kBwd ? NRI : 1];
  float4 ar[NRA];
  float vc, oc, uc, rc, bb;
  float sc[kBwd ? Geo<DK>::RPT : 1];   // the piece's first state, this lane's rows

  // Tokens of rows tok0, tok0 + H, ... (n of them); columns col0 .. col0 + WGC - 1.
  __device__ __forceinline__ void load(const E* k, const E* q, const float* alpha, const E* v,
                                       const E* dO, const float* beta, const float* uw,
                                       const float* rw, size_t tok0, int H, int DV, int n,
                                       int col0, int tid) {
#pragma unroll
    for (int it = 0; it < NRI; ++it) {
      const int e = (it * kThreads + tid) * VEC, s = e / DK, c = e % DK;
      const bool ok = e < kCk * DK && s < n;
      const size_t off = (tok0 + static_cast<size_t>(s) * H) * DK + c;
      kr[it] = ok ? *reinterpret_cast<const uint4*>(k + off) : make_uint4(0, 0, 0, 0);
      if constexpr (kBwd)
        qr[it] = ok ? *reinterpret_cast<const uint4*>(q + off) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int it = 0; it < NRA; ++it) {
      const int e = (it * kThreads + tid) * 4, s = e / DK, c = e % DK;
      const bool ok = e < kCk * DK && s < n;
      const size_t off = (tok0 + static_cast<size_t>(s) * H) * DK + c;
      if constexpr (kIn == kGateScalar) {   // one gate per token and head, or none (1)
        const float a = ok ? (alpha ? alpha[tok0 + static_cast<size_t>(s) * H] : 1.f) : 0.f;
        ar[it] = make_float4(a, a, a, a);
      } else {
        ar[it] = ok ? *reinterpret_cast<const float4*>(alpha + off) : make_float4(0, 0, 0, 0);
      }
    }
    {
      const int s = tid / WGC, cc = tid % WGC;
      const bool ok = tid < kCk * WGC && s < n;
      const size_t off = (tok0 + static_cast<size_t>(s) * H) * DV + col0 + cc;
      vc = ok ? Ty<IO>::to_f32(v[off]) : 0.f;
      if constexpr (kBwd) {
        oc = ok ? Ty<IO>::to_f32(dO[off]) : 0.f;
        uc = ok ? uw[off] : 0.f;
        rc = ok ? rw[off] : 0.f;
      }
    }
    bb = (tid < kCk && tid < n) ? beta[tok0 + static_cast<size_t>(tid) * H] : 0.f;
  }
  // The piece's stored state (backward only), this lane's RPT values.
  __device__ __forceinline__ void load_state(const float* in, int lane) {
#pragma unroll
    for (int i = 0; i < Geo<DK>::RPT; ++i) sc[i] = in[i * kWave + lane];
  }

  __device__ __forceinline__ void store(float* kS, float* qS, float* aS, float* vS, float* oS,
                                        float* uS, float* rS, float* bS, int tid) const {
#pragma unroll
    for (int it = 0; it < NRI; ++it) {
      const int e = (it * kThreads + tid) * VEC, s = e / DK, c = e % DK;
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
      const int e = (it * kThreads + tid) * 4, s = e / DK, c = e % DK;
      if (e < kCk * DK) {
        aS[s * DK + kpos<DK>(c + 0)] = ar[it].x;
        aS[s * DK + kpos<DK>(c + 1)] = ar[it].y;
        aS[s * DK + kpos<DK>(c + 2)] = ar[it].z;
        aS[s * DK + kpos<DK>(c + 3)] = ar[it].w;
      }
    }
    if (tid < kCk * WGC) {
      vS[tid] = vc;   // [token][column]
      if constexpr (kBwd) {
        oS[tid] = oc;
        uS[tid] = uc;
        rS[tid] = rc;
      }
    }
    if (tid < kCk) bS[tid] = bb;
  }
};

// One forward token on the lane's rows of its column.  Returns r; u in *u.
template <int DK>
__device__ __forceinline__ float fwd_token(float* S, const float* kr, const float* ar, float vj,
                                           float bt, float* u) {
  constexpr int RPT = Geo<DK>::RPT;
  float sp[RPT], acc = 0.f;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    sp[i] = ar[i] * S[i];
    acc += kr[i] * sp[i];
  }
  const float r = col_sum<Geo<DK>::CPW>(acc);
  const float uj = bt * (vj - r);
#pragma unroll
  for (int i = 0; i < RPT; ++i) S[i] = sp[i] + kr[i] * uj;
  *u = uj;
  return r;
}

// Stored state layout: [chain][piece][workgroup][wave][RPT][64 lanes] floats
// (DK x WGC floats per workgroup and piece).
__device__ __forceinline__ size_t ck_off(size_t chain, int piece, int npiece, int wg, int NWG,
                                         int block) {
  return ((chain * npiece + piece) * NWG + wg) * static_cast<size_t>(block);
}

template <typename IO, int DK, int kIn>
__global__ void __launch_bounds__(kThreads)
kda_pb_forward_kernel(const typename Ty<IO>::Elem* __restrict__ k,
                      const typename Ty<IO>::Elem* __restrict__ v,
                      const float* __restrict__ alpha, const float* __restrict__ beta,
                      const float* __restrict__ S0, float* __restrict__ ck,
                      float* __restrict__ uw, float* __restrict__ rw, int T, int H, int DV) {
  using G = Geo<DK>;
  constexpr int RPT = G::RPT, CPW = G::CPW, RG = G::RG, WGC = G::WGC;
  const int NWG = DV / WGC;
  const int chain = blockIdx.x / NWG, wg = blockIdx.x % NWG;
  const int b = chain / H, h = chain % H;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int j = lane % CPW, rg = lane / CPW, cw = wave * CPW + j;
  const int col = wg * WGC + cw;
  const int npiece = (T + kCk - 1) / kCk;

  __shared__ float kS[kCk * DK], aS[kCk * DK], vS[kCk * WGC], bS[kCk];
  __shared__ float uO[kCk * WGC], rO[kCk * WGC];   // the piece's writes and reads, [token][column]
  __shared__ float s0[kWaves * RPT * kWave];
  // The initial state goes through LDS: values that enter the token loop
  // straight from a global load make the compiler wait for every vector
  // memory operation (stores included) in each iteration.
  float S[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    s0[(wave * RPT + i) * kWave + lane] =
        S0 ? S0[(static_cast<size_t>(chain) * DK + rg + RG * i) * DV + col] : 0.f;
#pragma unroll
  for (int i = 0; i < RPT; ++i) S[i] = s0[(wave * RPT + i) * kWave + lane];

  Stage<IO, DK, false, kIn> st;
  auto tok0 = [&](int p) {
    return static_cast<size_t>(b) * T * H + static_cast<size_t>(p) * kCk * H + h;
  };
  auto count = [&](int p) { return min(kCk, T - p * kCk); };
  st.load(k, nullptr, alpha, v, nullptr, beta, nullptr, nullptr, tok0(0), H, DV, count(0),
          wg * WGC, tid);
  for (int p = 0; p < npiece; ++p) {
    st.store(kS, nullptr, aS, vS, nullptr, nullptr, nullptr, bS, tid);
    __syncthreads();
    if (p + 1 < npiece)
      st.load(k, nullptr, alpha, v, nullptr, beta, nullptr, nullptr, tok0(p + 1), H, DV,
              count(p + 1), wg * WGC, tid);
    float* out = ck + ck_off(chain, p, npiece, wg, NWG, DK * WGC) + wave * RPT * kWave;
#pragma unroll
    for (int i = 0; i < RPT; ++i) out[i * kWave + lane] = S[i];
    const int n = count(p);
    for (int s = 0; s < n; ++s) {
      float u;
      const float r = fwd_token<DK>(S, kS + s * DK + rg * RPT, aS + s * DK + rg * RPT,
                                    vS[s * WGC + cw], bS[s], &u);
      if (rg == 0) {   // the token's write and read, for the backward's rebuild
        uO[s * WGC + cw] = u;
        rO[s * WGC + cw] = r;
      }
    }
    __syncthreads();
    if (tid < n * WGC) {   // one coalesced store per thread for the piece
      const size_t o = (tok0(p) + static_cast<size_t>(tid / WGC) * H) * DV + wg * WGC + tid % WGC;
      uw[o] = uO[tid];
      rw[o] = rO[tid];
    }
  }
}

template <typename IO, int DK, int kIn>
__global__ void __launch_bounds__(kThreads)
kda_pb_backward_kernel(const typename Ty<IO>::Elem* __restrict__ q,
                       const typename Ty<IO>::Elem* __restrict__ k,
                       const typename Ty<IO>::Elem* __restrict__ v,
                       const float* __restrict__ alpha, const float* __restrict__ beta,
                       const typename Ty<IO>::Elem* __restrict__ dO,
                       const float* dS_T, const float* __restrict__ ck,
                       const float* __restrict__ uw, const float* __restrict__ rw,
                       float* __restrict__ g_q, float* __restrict__ g_k,
                       float* __restrict__ g_v, float* __restrict__ g_alpha,
                       float* __restrict__ g_beta, float* g_S0, int T, int H,
                       int DV) {
  using G = Geo<DK>;
  constexpr int RPT = G::RPT, CPW = G::CPW, RG = G::RG, WGC = G::WGC;
  constexpr int NV = G::NV, VP = G::VP, PER = G::PER;
  const int NWG = DV / WGC;
  const int chain = blockIdx.x / NWG, wg = blockIdx.x % NWG;
  const int b = chain / H, h = chain % H;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int j = lane % CPW, rg = lane / CPW, cw = wave * CPW + j;
  const int col = wg * WGC + cw;
  const int npiece = (T + kCk - 1) / kCk;

  __shared__ float kS[kCk * DK], qS[kCk * DK], aS[kCk * DK];
  __shared__ float vS[kCk * WGC], oS[kCk * WGC], uS[kCk * WGC], rS[kCk * WGC], bS[kCk];
  __shared__ float hist[kWaves * kCk * RPT * kWave];   // state before each token, per wave
  // Row sums of each wave, for half a piece: [wave][token][dq, dk, dalpha][row].
  // Plain stores (each slot has one writer); the flush adds the four waves.
  __shared__ float part[kWaves * kHalf * 3 * DK];
  __shared__ float partb[kWaves][kCk];                 // dbeta, per wave
  __shared__ float parta[kWaves][kCk];                 // the scalar gate's gradient, per wave
  __shared__ float dvS[kHalf * WGC];                   // dv of the half piece, [token][column]
  float* mypart = part + wave * kHalf * 3 * DK;
  float* myhist = hist + wave * kCk * RPT * kWave;

  // The incoming state gradient and each piece's first state go through LDS:
  // values that enter a token loop straight from a global load make the
  // compiler wait for every vector memory operation (the dv stores included)
  // in each iteration.
  float dS[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    myhist[i * kWave + lane] =
        dS_T ? dS_T[(static_cast<size_t>(chain) * DK + rg + RG * i) * DV + col] : 0.f;
#pragma unroll
  for (int i = 0; i < RPT; ++i) dS[i] = myhist[i * kWave + lane];

  Stage<IO, DK, true, kIn> st;
  auto tok0 = [&](int p) {
    return static_cast<size_t>(b) * T * H + static_cast<size_t>(p) * kCk * H + h;
  };
  auto count = [&](int p) { return min(kCk, T - p * kCk); };
  auto state_at = [&](int p) {
    return ck + ck_off(chain, p, npiece, wg, NWG, DK * WGC) + wave * RPT * kWave;
  };
  if (npiece > 0) {
    st.load(k, q, alpha, v, dO, beta, uw, rw, tok0(npiece - 1), H, DV, count(npiece - 1),
            wg * WGC, tid);
    st.load_state(state_at(npiece - 1), lane);
  }
  for (int p = npiece - 1; p >= 0; --p) {
    st.store(kS, qS, aS, vS, oS, uS, rS, bS, tid);
#pragma unroll
    for (int i = 0; i < RPT; ++i) myhist[i * kWave + lane] = st.sc[i];
    __syncthreads();
    if (p > 0) {
      st.load(k, q, alpha, v, dO, beta, uw, rw, tok0(p - 1), H, DV, count(p - 1), wg * WGC,
              tid);
      st.load_state(state_at(p - 1), lane);
    }
    const int n = count(p);
    float S[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) S[i] = myhist[i * kWave + lane];
    // rebuild the piece's states from its first one and the stored writes u
    // (S = Diag(alpha) S + k^T u: no column sum), keeping the state before
    // each token
    for (int s = 0; s < n; ++s) {
      const float* kr = kS + s * DK + rg * RPT;
      const float* ar = aS + s * DK + rg * RPT;
      const float uj = uS[s * WGC + cw];
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        myhist[(s * RPT + i) * kWave + lane] = S[i];
        S[i] = ar[i] * S[i] + kr[i] * uj;
      }
    }
    __syncthreads();
    // backward over the piece, in two halves of kHalf tokens (last half first)
    for (int half = 1; half >= 0; --half) {
      const int lo = half * kHalf, hi = min(n, lo + kHalf);
      for (int s = hi - 1; s >= lo; --s) {
        const float* kr = kS + s * DK + rg * RPT;
        const float* qr = qS + s * DK + rg * RPT;
        const float* ar = aS + s * DK + rg * RPT;
        const float uj = uS[s * WGC + cw], rj = rS[s * WGC + cw];
        const float vj = vS[s * WGC + cw], oj = oS[s * WGC + cw], bt = bS[s];
        float Sb[RPT], Gm[RPT], acc = 0.f;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
          Sb[i] = myhist[(s * RPT + i) * kWave + lane];
          Gm[i] = dS[i] + qr[i] * oj;
          acc += kr[i] * Gm[i];
        }
        const float du = col_sum<CPW>(acc);
        if (rg == 0) dvS[(s - lo) * WGC + cw] = bt * du;
        const float pb = row_sum<CPW>(du * (vj - rj));
        if (lane == 0) partb[wave][s] = pb;
        const float dr = -bt * du;
        float val[VP];
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
          const float sp = ar[i] * Sb[i];
          const float sn = sp + kr[i] * uj;
          const float dsp = Gm[i] + kr[i] * dr;
          val[3 * i + 0] = sn * oj;                  // dq
          val[3 * i + 1] = Gm[i] * uj + sp * dr;     // dk
          val[3 * i + 2] = dsp * Sb[i];              // dalpha
          dS[i] = ar[i] * dsp;
        }
#pragma unroll
        for (int m = NV; m < VP; ++m) val[m] = 0.f;
        if constexpr (kIn == kGateScalar) {   // d(gate) = sum over the slab of dS' (.) S
          float pa = 0.f;
#pragma unroll
          for (int i = 0; i < RPT; ++i) pa += val[3 * i + 2];
          pa = col_sum<CPW>(row_sum<CPW>(pa));
          if (lane == 0) parta[wave][s] = pa;
        }
        butterfly<CPW, VP>(val, lane);
#pragma unroll
        for (int w = 0; w < PER; ++w) {
          const int m = j * PER + w;
          if (m < NV) {
            const int i = m / 3, qn = m % 3;
            mypart[((s - lo) * 3 + qn) * DK + rg + RG * i] = val[w];
          }
        }
      }
      __syncthreads();
      // this half's row sums of the workgroup's columns into the gradient
      // rows: thread slot x = (quantity, row) adds token s's sum (four waves)
      constexpr int NSLOT = 3 * DK;
#pragma unroll
      for (int x0 = 0; x0 < NSLOT; x0 += kThreads) {
        const int x = x0 + tid;
        if (x < NSLOT) {
          const int qn = x / DK, c = x % DK;
          if (kIn == kGateScalar && qn == 2) continue;   // the gate's gradient goes below
          float* dst = (qn == 0 ? g_q : (qn == 1 ? g_k : g_alpha)) + tok0(p) * DK + c;
          const size_t step = static_cast<size_t>(H) * DK;
#pragma unroll
          for (int e = 0; e < kHalf; ++e) {
            if (lo + e < hi) {
              float sum = 0.f;
#pragma unroll
              for (int w = 0; w < kWaves; ++w) sum += part[(w * kHalf + e) * NSLOT + x];
              unsafeAtomicAdd(dst + (lo + e) * step, sum);
            }
          }
        }
      }
      if (tid < (hi - lo) * WGC) {   // dv: one coalesced store per thread
        const size_t o =
            (tok0(p) + static_cast<size_t>(lo + tid / WGC) * H) * DV + wg * WGC + tid % WGC;
        g_v[o] = dvS[tid];
      }
      if (tid >= lo && tid < hi) {
        float sb = 0.f, sa = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          sb += partb[w][tid];
          sa += parta[w][tid];
        }
        unsafeAtomicAdd(g_beta + tok0(p) + static_cast<size_t>(tid) * H, sb);
        if (kIn == kGateScalar && g_alpha)
          unsafeAtomicAdd(g_alpha + tok0(p) + static_cast<size_t>(tid) * H, sa);
      }
      __syncthreads();
    }
  }
  if (g_S0) {
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      g_S0[(static_cast<size_t>(chain) * DK + rg + RG * i) * DV + col] = dS[i];
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

template <typename IO, int DK, int kIn>
hipError_t run(const PrefillBwdArgs& a) {
  using E = typename Ty<IO>::Elem;
  constexpr int WGC = Geo<DK>::WGC;
  if (a.dv % WGC != 0) return hipErrorInvalidValue;
  const unsigned grid = static_cast<unsigned>(a.B) * a.H * (a.dv / WGC);
  const hipStream_t stream = static_cast<hipStream_t>(a.stream);
  // workspace: stored states, then u and r [B, T, H, dv] each
  float* ck = static_cast<float*>(a.workspace);
  const size_t npiece = (static_cast<size_t>(a.T) + kCk - 1) / kCk;
  float* uw = ck + static_cast<size_t>(a.B) * a.H * npiece * a.dk * a.dv;
  float* rw = uw + static_cast<size_t>(a.B) * a.T * a.H * a.dv;
  if (a.T > 0) {
    const size_t nk = static_cast<size_t>(a.B) * a.T * a.H * a.dk;
    const size_t nb = static_cast<size_t>(a.B) * a.T * a.H;
    const size_t tot = 3 * nk + 2 * nb;
    const size_t zb = (tot + 255) / 256;
    const unsigned zg = static_cast<unsigned>(zb < 4096 ? zb : 4096);
    // the gate's gradient: one per channel, one per token and head, or none
    const size_t na = kIn == kGateScalar ? (a.g_alpha ? nb : 0) : nk;
    zero_fill_kernel<<<zg, 256, 0, stream>>>(a.g_q, nk, a.g_k, nk, a.g_alpha, na, a.g_beta, nb);
    kda_pb_forward_kernel<IO, DK, kIn><<<grid, kThreads, 0, stream>>>(
        static_cast<const E*>(a.k), static_cast<const E*>(a.v), a.alpha, a.beta, a.S0, ck, uw,
        rw, a.T, a.H, a.dv);
  }
  kda_pb_backward_kernel<IO, DK, kIn><<<grid, kThreads, 0, stream>>>(
      static_cast<const E*>(a.q), static_cast<const E*>(a.k), static_cast<const E*>(a.v),
      a.alpha, a.beta, static_cast<const E*>(a.dO), a.dS_T,
      ck, uw, rw, a.g_q, a.g_k, a.g_v, a.g_alpha, a.g_beta, a.g_S0,
      a.T, a.H, a.dv);
  return hipGetLastError();
}

template <typename IO, int kIn>
hipError_t run_dk(const PrefillBwdArgs& a) {
  switch (a.dk) {
    case 16: return run<IO, 16, kIn>(a);
    case 32: return run<IO, 32, kIn>(a);
    case 64: return run<IO, 64, kIn>(a);
    case 128: return run<IO, 128, kIn>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t prefill_backward_workspace(int B, int T, int H, int dk, int dv) {
  const size_t npiece = (static_cast<size_t>(T) + kCk - 1) / kCk;
  return (static_cast<size_t>(B) * H * npiece * dk * dv +
          2 * static_cast<size_t>(B) * T * H * dv) * sizeof(float);
}

hipError_t launch_prefill_backward(const PrefillBwdArgs& a) {
  if (a.gate_in == kGateScalar)
    return a.bf16 ? run_dk<bf16_t, kGateScalar>(a) : run_dk<float, kGateScalar>(a);
  if (a.gate_in != kGateAlpha) return hipErrorInvalidValue;
  return a.bf16 ? run_dk<bf16_t, kGateAlpha>(a) : run_dk<float, kGateAlpha>(a);
}

}  // namespace kda
