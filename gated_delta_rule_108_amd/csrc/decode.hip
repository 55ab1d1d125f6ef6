// KDA decode step: one token for N sequences x H heads.
//
// For each (n, h) and each state column j (columns are independent):
//   S'[c][j]  = alpha[c] S[c][j]
//   rk[j]     = sum_c k[c] S'[c][j]        read at the key
//   rq[j]     = sum_c q[c] S'[c][j]
//   u[j]      = beta (v[j] - rk[j])         the delta
//   o[j]      = rq[j] + (q . k) u[j]        = q S_new, read after the write
//   S_new     = S' + k^T u
// ("From GPT-2 to Kimi K3, Explained", sections "DeltaNet (Fast Weight
// Programmers)" and "KDA/Kimi Linear"; decode is the t = 1 call with the
// cached state, section "Linear Attention".)
//
// The step is bound by HBM: each head's dk x dv fp32 state is read once and
// written once, ~0.9 flop per byte.  A workgroup owns a CW-column slab of one
// head's state.  Each thread holds RPT rows x 4 columns of it in registers
// (one 16-byte load per row), so the two column reductions and the update
// happen in a single pass; reductions over rows go through cross-lane
// exchanges inside a wave and a small LDS exchange between waves.
//
// kIn (GateIn) says how the gate arrives: one fp32 alpha per key channel; one
// per token and head (Gated DeltaNet), or none (DeltaNet) when the pointer is
// null; or, with kGateLogit, the input prologue on the fly: the gate
// comes as logits g in the I/O type, beta as its logit, and q, k pass through
// qk_map.  Each row's mapped gate, key and query are computed once per
// workgroup and staged in LDS.  The row norms of q and k ride along the same
// reductions (two more sums), and since every use of k and q is linear in
// them they are applied after the reductions: r_k, r_q and q.k are rescaled,
// k^T u uses k / |k|.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

template <int DK, int CW>
struct DecodeCfg {
  static constexpr int CG = CW / 4;                                   // float4 column groups
  static constexpr int NTH = (CG * DK < 256) ? CG * DK : 256;         // threads
  static constexpr int RG = NTH / CG;                                  // row groups
  static constexpr int RPT = DK / RG;                                  // rows per thread
  static constexpr int NWV = NTH / kWave;
  static_assert(NTH % kWave == 0, "decode block must be whole waves");
  static_assert(RPT * RG == DK, "rows must split evenly");
};

// The new state goes out with non-temporal stores: nothing reads it again in
// this step, and keeping it from allocating in the caches lets the reads of
// the old state stream at a higher rate (256 x 32 heads: 216 -> 161 us).
// Non-temporal loads of the old state measured slower (198 us).
__device__ __forceinline__ void store_streaming(float* p, const float4& w) {
  typedef float f4v __attribute__((ext_vector_type(4)));
  f4v t;
  t.x = w.x;
  t.y = w.y;
  t.z = w.z;
  t.w = w.w;
  __builtin_nontemporal_store(t, reinterpret_cast<f4v*>(p));
}

template <typename IO, int DK, int CW, int kIn>
__global__ void __launch_bounds__(256)
kda_decode_kernel(const typename Ty<IO>::Elem* __restrict__ q,
                  const typename Ty<IO>::Elem* __restrict__ k,
                  const typename Ty<IO>::Elem* __restrict__ v,
                  const void* __restrict__ gate, const float* __restrict__ beta,
                  const float* S_in, typename Ty<IO>::Elem* __restrict__ o, float* S_out,
                  int NH, int DV, int qk_map) {
  using Cf = DecodeCfg<DK, CW>;
  using E = typename Ty<IO>::Elem;
  constexpr int CG = Cf::CG, RG = Cf::RG, RPT = Cf::RPT, NWV = Cf::NWV;
  constexpr bool kLogit = kIn == kGateLogit;
  constexpr bool kScalar = kIn == kGateScalar;

  const int tiles = DV / CW;
  const int nh = blockIdx.x / tiles;            // (n, h) flattened
  const int col0 = (blockIdx.x % tiles) * CW;
  const int tid = threadIdx.x;
  const int cg = tid % CG, rg = tid / CG;
  const int lane = tid % kWave, wave = tid / kWave;

  const size_t sbase = static_cast<size_t>(nh) * DK * DV;
  const E* qh = q + static_cast<size_t>(nh) * DK;
  const E* kh = k + static_cast<size_t>(nh) * DK;
  const float* ah = static_cast<const float*>(gate) + static_cast<size_t>(nh) * DK;
  const E* gh = static_cast<const E*>(gate) + static_cast<size_t>(nh) * DK;
  const float bt = kLogit ? sigmoid_f(beta[nh]) : beta[nh];
  const bool qk_silu = kLogit && qk_map == kQkSiluL2;
  const bool qk_norm = kLogit && qk_map != kQkAsGiven;

  float4 s[RPT];
  float kr[RPT];
  float rk[4] = {0.f, 0.f, 0.f, 0.f}, rq[4] = {0.f, 0.f, 0.f, 0.f}, qk = 0.f;
  float nk = 0.f, nq = 0.f;   // sums of squares of k and q (prologue)
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg + RG * i;
    s[i] = *reinterpret_cast<const float4*>(S_in + sbase + static_cast<size_t>(r) * DV + col0 + 4 * cg);
  }
  // Row r's gate, key and query are read (and, with the prologue, mapped)
  // once per workgroup, by thread r (NTH >= DK), and staged in LDS while the
  // state loads are in flight, instead of by each of the CG threads that hold
  // a piece of row r.
  __shared__ float pro[3][DK];
  if (tid < DK) {
    float kv = Ty<IO>::to_f32(kh[tid]), qv = Ty<IO>::to_f32(qh[tid]);
    if (qk_silu) {   // rounded back to the I/O type, as the prefill does
      kv = Ty<IO>::to_f32(Ty<IO>::from_f32(silu_f(kv)));
      qv = Ty<IO>::to_f32(Ty<IO>::from_f32(silu_f(qv)));
    }
    float a;
    if constexpr (kLogit) a = gate_from_logit(Ty<IO>::to_f32(gh[tid]));
    else if constexpr (kScalar) a = gate != nullptr ? static_cast<const float*>(gate)[nh] : 1.f;
    else a = ah[tid];
    pro[0][tid] = a;
    pro[1][tid] = kv;
    pro[2][tid] = qv;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg + RG * i;
    const float a = pro[0][r], kv = pro[1][r], qv = pro[2][r];
    if constexpr (kLogit) {
      nk += kv * kv;
      nq += qv * qv;
    }
    kr[i] = kv;
    s[i].x *= a; s[i].y *= a; s[i].z *= a; s[i].w *= a;
    rk[0] += kv * s[i].x; rk[1] += kv * s[i].y; rk[2] += kv * s[i].z; rk[3] += kv * s[i].w;
    rq[0] += qv * s[i].x; rq[1] += qv * s[i].y; rq[2] += qv * s[i].z; rq[3] += qv * s[i].w;
    qk += qv * kv;
  }
  // Sum over the row groups of this wave (lanes that share cg).
#pragma unroll
  for (int off = CG; off < kWave; off <<= 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      rk[j] += __shfl_xor(rk[j], off);
      rq[j] += __shfl_xor(rq[j], off);
    }
    qk += __shfl_xor(qk, off);
    if constexpr (kLogit) {
      nk += __shfl_xor(nk, off);
      nq += __shfl_xor(nq, off);
    }
  }
  if constexpr (NWV > 1) {
    __shared__ float red[NWV][CG][kLogit ? 11 : 9];
    if (lane < CG) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        red[wave][cg][j] = rk[j];
        red[wave][cg][4 + j] = rq[j];
      }
      red[wave][cg][8] = qk;
      if constexpr (kLogit) {
        red[wave][cg][9] = nk;
        red[wave][cg][10] = nq;
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) { rk[j] = 0.f; rq[j] = 0.f; }
    qk = 0.f;
    nk = 0.f;
    nq = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        rk[j] += red[w][cg][j];
        rq[j] += red[w][cg][4 + j];
      }
      qk += red[w][cg][8];
      if constexpr (kLogit) {
        nk += red[w][cg][9];
        nq += red[w][cg][10];
      }
    }
  }
  float sk = 1.f;   // 1 / |k| (prologue)
  if (qk_norm) {
    sk = inv_l2(nk);
    const float sq = inv_l2(nq);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      rk[j] *= sk;
      rq[j] *= sq;
    }
    qk *= sk * sq;
  }
  const E* vh = v + static_cast<size_t>(nh) * DV + col0 + 4 * cg;
  float u[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) u[j] = bt * (Ty<IO>::to_f32(vh[j]) - rk[j]);
  if (rg == 0) {
    E* oh = o + static_cast<size_t>(nh) * DV + col0 + 4 * cg;
#pragma unroll
    for (int j = 0; j < 4; ++j) oh[j] = Ty<IO>::from_f32(rq[j] + qk * u[j]);
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg + RG * i;
    float4 w = s[i];
    const float kn = kr[i] * sk;
    w.x += kn * u[0]; w.y += kn * u[1]; w.z += kn * u[2]; w.w += kn * u[3];
    store_streaming(S_out + sbase + static_cast<size_t>(r) * DV + col0 + 4 * cg, w);
  }
}

// Column-slab width: whole rows when there are enough heads to fill the chip,
// narrower slabs (more workgroups) when there are few.
static int pick_cw(long nh, int dv) {
  int cw = dv;
  while (cw > 16 && nh * (dv / cw) < 2048) cw /= 2;
  return cw;
}

template <typename IO, int DK, int CW, int kIn>
static hipError_t launch_dec(const DecodeArgs& a) {
  using Cf = DecodeCfg<DK, CW>;
  using E = typename Ty<IO>::Elem;
  const long nh = static_cast<long>(a.N) * a.H;
  dim3 grid(static_cast<unsigned>(nh * (a.dv / CW)));
  hipLaunchKernelGGL((kda_decode_kernel<IO, DK, CW, kIn>), grid, dim3(Cf::NTH), 0,
                     static_cast<hipStream_t>(a.stream),
                     static_cast<const E*>(a.q), static_cast<const E*>(a.k),
                     static_cast<const E*>(a.v), a.gate, a.beta, a.S_in,
                     static_cast<E*>(a.o), a.S_out, static_cast<int>(nh), a.dv, a.qk_map);
  return hipGetLastError();
}

template <typename IO, int DK, int kIn>
static hipError_t dispatch_cw(const DecodeArgs& a, int cw) {
  switch (cw) {
    case 16: return launch_dec<IO, DK, 16, kIn>(a);
    case 32: return launch_dec<IO, DK, 32, kIn>(a);
    case 64: return launch_dec<IO, DK, 64, kIn>(a);
    case 128: return launch_dec<IO, DK, 128, kIn>(a);
  }
  return hipErrorInvalidValue;
}

template <typename IO, int kIn>
static hipError_t dispatch_dk(const DecodeArgs& a, int cw) {
  switch (a.dk) {
    case 16: return dispatch_cw<IO, 16, kIn>(a, cw);
    case 32: return dispatch_cw<IO, 32, kIn>(a, cw);
    case 64: return dispatch_cw<IO, 64, kIn>(a, cw);
    case 128: return dispatch_cw<IO, 128, kIn>(a, cw);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a) {
  const int cw = pick_cw(static_cast<long>(a.N) * a.H, a.dv);
  switch (a.gate_in) {
    case kGateAlpha:
      return a.bf16 ? dispatch_dk<bf16_t, kGateAlpha>(a, cw) : dispatch_dk<float, kGateAlpha>(a, cw);
    case kGateLogit:
      return a.bf16 ? dispatch_dk<bf16_t, kGateLogit>(a, cw) : dispatch_dk<float, kGateLogit>(a, cw);
    case kGateScalar:
      return a.bf16 ? dispatch_dk<bf16_t, kGateScalar>(a, cw)
                    : dispatch_dk<float, kGateScalar>(a, cw);
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
