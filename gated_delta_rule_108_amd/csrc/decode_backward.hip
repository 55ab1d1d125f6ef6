// KDA step adjoint: for one token of N sequences x H heads, the gradients of
// a loss L with respect to q, k, v, alpha, beta and the state before the
// step, given dL/do and dL/dS_new.
//
// Forward step (decode.hip; "From GPT-2 to Kimi K3, Explained", sections
// "DeltaNet (Fast Weight Programmers)" and "KDA/Kimi Linear"):
//   S' = Diag(alpha) S,  r = k S',  u = beta (v - r),  S_new = S' + k^T u,
//   o = q S_new.
// Backward, with G = dS_new + q^T dO (everything that reaches S_new):
//   column sums over the key rows c:  r_j = sum_c k_c S'_cj,
//                                     (k G)_j = sum_c k_c dS_new_cj + (q.k) dO_j
//   per value column j:  du = k G,  dv = beta du,  dr = -beta du,
//                        dbeta = sum_j du_j (v_j - r_j)
//   per element:         S_new, G, dS' = G + k_c dr_j, dS = alpha_c dS'
//   row sums over the value columns j:  dq_c = sum_j S_new_cj dO_j,
//                        dk_c = sum_j (G_cj u_j + S'_cj dr_j),
//                        dalpha_c = sum_j dS'_cj S_cj
//
// Like the forward step it is bound by HBM: per head it reads the state and
// the incoming state gradient and writes the outgoing one (3 dk dv fp32).
// The row sums need every column, so a workgroup owns one head's whole state:
// thread (row group rg, column group cg) holds RPT rows x 4 columns of S and
// of dS_new, one 16-byte load per row each.  256 threads (16 rows each at
// dk = dv = 128) leave room for two workgroups per CU, two heads' loads in
// flight (512 threads fit one and ran 5% slower).  Column sums run over the row
// groups (lane exchanges, then LDS across waves); row sums over the CG lanes
// of a row group, which are consecutive lanes of one wave (DPP moves within
// 16-lane rows).
#include <type_traits>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

template <int DK, int DV>
struct BwdCfg {
  static constexpr int CG = DV / 4;                                   // float4 column groups
  static constexpr int NTH = (CG * DK < 256) ? CG * DK : 256;         // threads
  static constexpr int RG = NTH / CG;                                  // row groups
  static constexpr int RPT = DK / RG;                                  // rows per thread
  static constexpr int NWV = NTH / kWave;
  static_assert(NTH % kWave == 0, "whole waves");
  static_assert(RPT * RG == DK, "rows must split evenly");
  static_assert(NTH >= DK, "one thread per key row stages the row vectors");
};

// Sum of x over the CG consecutive lanes of a row group (CG a power of two,
// 4..32), returned to every one of them.  Within a 16-lane row the steps are
// DPP moves (quad_perm for lane xor 1 and 2; row rotations by 4 and 8, which
// after the quad sums add the other three quads of the row); lane xor 4 for
// groups of 8, and xor 16 across rows, go through the lane crossbar.
template <int CG>
__device__ __forceinline__ float sum_row_group(float x) {
  auto dpp = [](float v, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), decltype(ctrl)::value, 0xF,
                                                    0xF, false));
  };
  x += dpp(x, std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]: lane xor 1
  x += dpp(x, std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]: lane xor 2
  if constexpr (CG == 8) x += __shfl_xor(x, 4);
  if constexpr (CG >= 16) {
    x += dpp(x, std::integral_constant<int, 0x124>{});  // row_ror:4
    x += dpp(x, std::integral_constant<int, 0x128>{});  // row_ror:8
  }
  if constexpr (CG >= 32) x += __shfl_xor(x, 16);
  return x;
}

// State and state-gradient rows are read once: non-temporal loads measured
// 291-292 us against 300-316 us at 256 x 32 heads (the decode kernel, which
// re-reads nothing either, measured slower with them: 201 against 162 us).
__device__ __forceinline__ float4 load_nt(const float* p) {
  typedef float f4v __attribute__((ext_vector_type(4)));
  const f4v t = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(p));
  return make_float4(t.x, t.y, t.z, t.w);
}

__device__ __forceinline__ void store_nt(float* p, float a, float b, float c, float d) {
  typedef float f4v __attribute__((ext_vector_type(4)));
  f4v t;
  t.x = a;
  t.y = b;
  t.z = c;
  t.w = d;
  __builtin_nontemporal_store(t, reinterpret_cast<f4v*>(p));
}

// kIn: kGateAlpha (one gate per key channel) or kGateScalar (one per head,
// or none: Gated DeltaNet / DeltaNet; its gradient is the sum over the rows).
template <typename IO, int DK, int DV, int kIn>
__global__ void __launch_bounds__(256)   // BwdCfg::NTH <= 256
kda_decode_backward_kernel(const typename Ty<IO>::Elem* __restrict__ q,
                           const typename Ty<IO>::Elem* __restrict__ k,
                           const typename Ty<IO>::Elem* __restrict__ v,
                           const float* __restrict__ alpha, const float* __restrict__ beta,
                           const float* __restrict__ S_in,
                           const typename Ty<IO>::Elem* __restrict__ dO, const float* dS_new,
                           typename Ty<IO>::Elem* __restrict__ dq,
                           typename Ty<IO>::Elem* __restrict__ dk,
                           typename Ty<IO>::Elem* __restrict__ dv,
                           float* __restrict__ dalpha, float* __restrict__ dbeta, float* dS) {
  using Cf = BwdCfg<DK, DV>;
  using E = typename Ty<IO>::Elem;
  constexpr int CG = Cf::CG, RG = Cf::RG, RPT = Cf::RPT, NWV = Cf::NWV;

  const int nh = blockIdx.x;   // (n, h) flattened
  const int tid = threadIdx.x;
  const int cg = tid % CG, rg = tid / CG;
  const int lane = tid % kWave, wave = tid / kWave;
  const size_t sbase = static_cast<size_t>(nh) * DK * DV;
  const size_t vbase = static_cast<size_t>(nh) * DV + 4 * cg;

  // State and incoming gradient rows first: the long loads go out before
  // anything waits.  dS may equal dS_new: every element is read here by the
  // thread that writes it at the end.
  float4 s[RPT], gs[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const size_t off = sbase + static_cast<size_t>(rg + RG * i) * DV + 4 * cg;
    s[i] = load_nt(S_in + off);
    gs[i] = load_nt(dS_new + off);
  }
  // Row vectors (gate, key, query) once per workgroup, by thread r.
  __shared__ float pro[3][DK];
  if (tid < DK) {
    if constexpr (kIn == kGateScalar)
      pro[0][tid] = alpha ? alpha[nh] : 1.f;
    else
      pro[0][tid] = alpha[static_cast<size_t>(nh) * DK + tid];
    pro[1][tid] = Ty<IO>::to_f32(k[static_cast<size_t>(nh) * DK + tid]);
    pro[2][tid] = Ty<IO>::to_f32(q[static_cast<size_t>(nh) * DK + tid]);
  }
  const float bt = beta[nh];
  float vv[4], dov[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    vv[j] = Ty<IO>::to_f32(v[vbase + j]);
    dov[j] = Ty<IO>::to_f32(dO[vbase + j]);
  }
  __syncthreads();

  // ---- column sums over the key rows: r = k S', kd = k dS_new, and q.k
  float rk[4] = {0.f, 0.f, 0.f, 0.f}, kd[4] = {0.f, 0.f, 0.f, 0.f}, qk = 0.f;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg + RG * i;
    const float a = pro[0][r], kv = pro[1][r], qv = pro[2][r];
    const float ka = kv * a;
    rk[0] += ka * s[i].x; rk[1] += ka * s[i].y; rk[2] += ka * s[i].z; rk[3] += ka * s[i].w;
    kd[0] += kv * gs[i].x; kd[1] += kv * gs[i].y; kd[2] += kv * gs[i].z; kd[3] += kv * gs[i].w;
    qk += qv * kv;
  }
#pragma unroll
  for (int off = CG; off < kWave; off <<= 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      rk[j] += __shfl_xor(rk[j], off);
      kd[j] += __shfl_xor(kd[j], off);
    }
    qk += __shfl_xor(qk, off);
  }
  if constexpr (NWV > 1) {
    __shared__ float red[NWV][CG][9];
    if (lane < CG) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        red[wave][cg][j] = rk[j];
        red[wave][cg][4 + j] = kd[j];
      }
      red[wave][cg][8] = qk;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) { rk[j] = 0.f; kd[j] = 0.f; }
    qk = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        rk[j] += red[w][cg][j];
        kd[j] += red[w][cg][4 + j];
      }
      qk += red[w][cg][8];
    }
  }

  // ---- per value column: u, du, dr; dv and dbeta from the first row group
  float u[4], dr[4], pb = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float du = kd[j] + qk * dov[j];
    u[j] = bt * (vv[j] - rk[j]);
    dr[j] = -bt * du;
    pb += du * (vv[j] - rk[j]);
    if (rg == 0) dv[vbase + j] = Ty<IO>::from_f32(bt * du);
  }
  pb = sum_row_group<CG>(pb);
  if (tid == 0) dbeta[nh] = pb;

  // ---- per element, then row sums over the value columns
  float ta = 0.f;   // scalar gate: this row group's share of sum_c dalpha_c
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg + RG * i;
    const float a = pro[0][r], kv = pro[1][r], qv = pro[2][r];
    const float sv[4] = {s[i].x, s[i].y, s[i].z, s[i].w};
    const float gv[4] = {gs[i].x, gs[i].y, gs[i].z, gs[i].w};
    float pq = 0.f, pk = 0.f, pa = 0.f, out[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float sp = a * sv[j];
      const float sn = sp + kv * u[j];
      const float G = gv[j] + qv * dov[j];
      const float dsp = G + kv * dr[j];
      pq += sn * dov[j];
      pk += G * u[j] + sp * dr[j];
      pa += dsp * sv[j];
      out[j] = a * dsp;
    }
    store_nt(dS + sbase + static_cast<size_t>(r) * DV + 4 * cg, out[0], out[1], out[2], out[3]);
    pq = sum_row_group<CG>(pq);
    pk = sum_row_group<CG>(pk);
    pa = sum_row_group<CG>(pa);
    ta += pa;
    if (cg == 0) {
      const size_t ro = static_cast<size_t>(nh) * DK + r;
      dq[ro] = Ty<IO>::from_f32(pq);
      dk[ro] = Ty<IO>::from_f32(pk);
      if constexpr (kIn != kGateScalar) dalpha[ro] = pa;
    }
  }
  if constexpr (kIn == kGateScalar) {
    // the rows' sum: over the row groups of the wave (lanes CG apart), then
    // over the waves through LDS
#pragma unroll
    for (int off = CG; off < kWave; off <<= 1) ta += __shfl_xor(ta, off);
    __shared__ float reda[NWV];
    if (lane == 0) reda[wave] = ta;
    __syncthreads();
    if (tid == 0 && dalpha) {
      float t = 0.f;
#pragma unroll
      for (int w = 0; w < NWV; ++w) t += reda[w];
      dalpha[nh] = t;
    }
  }
}

template <typename IO, int DK, int DV, int kIn>
static hipError_t launch_bwd(const DecodeBwdArgs& a) {
  using Cf = BwdCfg<DK, DV>;
  using E = typename Ty<IO>::Elem;
  const long nh = static_cast<long>(a.N) * a.H;
  hipLaunchKernelGGL((kda_decode_backward_kernel<IO, DK, DV, kIn>), dim3(static_cast<unsigned>(nh)),
                     dim3(Cf::NTH), 0, static_cast<hipStream_t>(a.stream),
                     static_cast<const E*>(a.q), static_cast<const E*>(a.k),
                     static_cast<const E*>(a.v), a.alpha, a.beta, a.S_in,
                     static_cast<const E*>(a.dO), a.dS_new, static_cast<E*>(a.g_q),
                     static_cast<E*>(a.g_k), static_cast<E*>(a.g_v), a.g_alpha, a.g_beta, a.g_S);
  return hipGetLastError();
}

template <typename IO, int DK, int kIn>
static hipError_t bwd_dv(const DecodeBwdArgs& a) {
  switch (a.dv) {
    case 16: return launch_bwd<IO, DK, 16, kIn>(a);
    case 32: return launch_bwd<IO, DK, 32, kIn>(a);
    case 64: return launch_bwd<IO, DK, 64, kIn>(a);
    case 128: return launch_bwd<IO, DK, 128, kIn>(a);
  }
  return hipErrorInvalidValue;
}

template <typename IO, int kIn>
static hipError_t bwd_dk(const DecodeBwdArgs& a) {
  switch (a.dk) {
    case 16: return bwd_dv<IO, 16, kIn>(a);
    case 32: return bwd_dv<IO, 32, kIn>(a);
    case 64: return bwd_dv<IO, 64, kIn>(a);
    case 128: return bwd_dv<IO, 128, kIn>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_backward(const DecodeBwdArgs& a) {
  if (a.gate_in == kGateScalar)
    return a.bf16 ? bwd_dk<bf16_t, kGateScalar>(a) : bwd_dk<float, kGateScalar>(a);
  if (a.gate_in != kGateAlpha) return hipErrorInvalidValue;
  return a.bf16 ? bwd_dk<bf16_t, kGateAlpha>(a) : bwd_dk<float, kGateAlpha>(a);
}

}  // namespace kda
