// KDA chunk scan: the sequential half of the split prefill.
//
// The prep kernel (kda_prefill_kernel<..., kPrep = true>) has already written,
// for every chunk of every chain, the column-free chunk quantities
//   W = Y Diag(beta)(K.E),  Q.E,  (K.E')^T,  P (gated Q K^T, lower),  Y,
//   and the chunk decay E_{C-1}
// to a workspace record (RecCfg).  This kernel walks the chunks of one chain
// in order.  Each computing wave owns a 16-column tile of the state and does
// all of its column work alone:
//   U~ = Y Diag(beta) V,  U = U~ - W S,  O = (Q.E) S + P U,
//   S <- Diag(E_{C-1}) S + (K.E')^T U
// (the chunk algebra of "From GPT-2 to Kimi K3, Explained", section "DeltaNet
// (Parallelizing Linear Transformers with Delta Rule)", with the per-channel
// decay of section "KDA/Kimi Linear").  The only data the waves share, the
// chunk record, is staged in LDS once per chunk, and the next chunk's record
// is fetched into registers while the current one is consumed; a chunk costs
// two workgroup barriers.
#pragma once

#include "prefill_kernel.hpp"

namespace kda {

template <typename OpT, int DK, int C, int NJ>
struct SCfg {
  static constexpr int NTH = 512, NW = 8;
  static_assert(NJ >= 1 && NJ <= NW, "computing waves");
  static constexpr int NB = C / 16, NCB = DK / 16;
  static constexpr int EB = Ty<OpT>::kBytes, PADE = 16 / EB;
  static constexpr int LDK = DK + PADE, LDC = C + PADE;
  static constexpr int kW = align16(C * LDK * EB);
  static constexpr int kKG = align16(DK * LDC * EB);
  static constexpr int kP = align16(C * LDC * EB);
  static constexpr int oW = 0, oQ = kW, oKG = oQ + kW, oP = oKG + kKG, oY = oP + kP;
  static constexpr int oGC = oY + kP;
  static constexpr int oBE = oGC + align16(DK * 4);
  static constexpr int oWV = oBE + align16(C * 4);
  static constexpr int kST = align16(16 * LDK * EB), kUT = align16(16 * LDC * EB);
  static constexpr int kPW = kST + 2 * kUT;          // per wave: S^T, U^T, (beta V)^T
  static constexpr int kLds = oWV + NJ * kPW;
  using RC = RecCfg<OpT, DK, C>;
  // the record as 16-byte vectors, and its segments
  static constexpr int vK = DK * EB / 16, vC = C * EB / 16;
  static constexpr int nW = C * vK, nKG = DK * vC, nP = C * vC, nGC = DK * 4 / 16;
  static constexpr int NVEC = 2 * nW + nKG + 2 * nP + nGC;
  static constexpr int NPV = (NVEC + NTH - 1) / NTH;
  // the wave's value tile, C rows x 16 columns, as 16-byte vectors
  static constexpr int VPR = 16 * EB / 16;           // vectors per value row
  static constexpr int NVV = C * VPR;
  static constexpr int NVL = (NVV + kWave - 1) / kWave;
};

// LDS byte offset of record vector x (row padding applied per segment).
template <class Cf>
__device__ __forceinline__ int rec_vec_lds(int x) {
  constexpr int EB = Cf::EB;
  if (x < Cf::nW) return Cf::oW + (x / Cf::vK) * Cf::LDK * EB + (x % Cf::vK) * 16;
  x -= Cf::nW;
  if (x < Cf::nW) return Cf::oQ + (x / Cf::vK) * Cf::LDK * EB + (x % Cf::vK) * 16;
  x -= Cf::nW;
  if (x < Cf::nKG) return Cf::oKG + (x / Cf::vC) * Cf::LDC * EB + (x % Cf::vC) * 16;
  x -= Cf::nKG;
  if (x < Cf::nP) return Cf::oP + (x / Cf::vC) * Cf::LDC * EB + (x % Cf::vC) * 16;
  x -= Cf::nP;
  if (x < Cf::nP) return Cf::oY + (x / Cf::vC) * Cf::LDC * EB + (x % Cf::vC) * 16;
  x -= Cf::nP;
  return Cf::oGC + x * 16;
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Element q of a 16-byte vector holding 16 / sizeof(E) values.
template <typename OpT>
__device__ __forceinline__ float vec_elem(const u32x4& v, int q) {
  if constexpr (Ty<OpT>::kBytes == 2)
    return bf16_to_f32(static_cast<uint16_t>((v[q >> 1] >> (16 * (q & 1))) & 0xffffu));
  else
    return __uint_as_float(v[q]);
}

template <typename OpT, int DK, int C, int NJ>
__global__ void __launch_bounds__(512)
kda_scan_kernel(const typename Ty<OpT>::Elem* __restrict__ gv, const float* __restrict__ gbeta,
                const float* gS0, typename Ty<OpT>::Elem* __restrict__ go, float* gST,
                const char* __restrict__ gws, int B, int T, int H, int DV) {
  using Cf = SCfg<OpT, DK, C, NJ>;
  using RC = typename Cf::RC;
  using E = typename Ty<OpT>::Elem;
  constexpr int NB = Cf::NB, NCB = Cf::NCB, NTH = Cf::NTH;
  constexpr int LDK = Cf::LDK, LDC = Cf::LDC, EB = Cf::EB;
  static_assert(Cf::kLds <= kMaxLds, "scan LDS plan exceeds 160 KiB");

  __shared__ __attribute__((aligned(16))) char smem[Cf::kLds];
  const E* Wm = reinterpret_cast<const E*>(smem + Cf::oW);
  const E* Qg = reinterpret_cast<const E*>(smem + Cf::oQ);
  const E* KgT = reinterpret_cast<const E*>(smem + Cf::oKG);
  const E* PP = reinterpret_cast<const E*>(smem + Cf::oP);
  const E* Yb = reinterpret_cast<const E*>(smem + Cf::oY);
  const float* sGC = reinterpret_cast<const float*>(smem + Cf::oGC);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const bool comp = wave < NJ;

  // Workgroup -> (chain, slab of 16*NJ columns), all slabs of a chain on one XCD.
  const int ntiles = DV / (16 * NJ);
  const int total = gridDim.x;
  int L = blockIdx.x;
  if (ntiles > 1 && (total % 8) == 0) L = (blockIdx.x % 8) * (total / 8) + blockIdx.x / 8;
  const int chain = L / ntiles;
  const int jw = (L % ntiles) * 16 * NJ + 16 * (comp ? wave : 0);   // this wave's columns
  const int b = chain / H, h = chain % H;
  const int NC = (T + C - 1) / C;
  const size_t row0 = static_cast<size_t>(b) * T * H + h;

  E* ST = reinterpret_cast<E*>(smem + Cf::oWV + (comp ? wave : 0) * Cf::kPW);   // [16][LDK]
  E* UT = ST + Cf::kST / EB;                                                      // [16][LDC]
  E* VbT = UT + Cf::kUT / EB;                                                     // [16][LDC]
  float* sBE = reinterpret_cast<float*>(smem + Cf::oBE);

  // state tiles (Cb, this wave's columns) in registers
  f32x4 S[NCB];
  {
    const Lane ln = lane_now();
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      S[cb] = zero4();
      if (comp && gS0 != nullptr) {
        const float* src = gS0 + static_cast<size_t>(chain) * DK * DV + jw;
#pragma unroll
        for (int r = 0; r < 4; ++r) S[cb][r] = src[(16 * cb + 4 * ln.g + r) * DV + ln.i];
      }
    }
  }

  // next chunk, fetched into registers one chunk ahead
  u32x4 pf[Cf::NPV];
  u32x4 pv[Cf::NVL];
  float pbe = 0.f;
  const char* rec0 = gws + static_cast<size_t>(chain) * NC * RC::kBytes;
  auto fetch = [&](int ch) {
    const u32x4* rv = reinterpret_cast<const u32x4*>(rec0 + static_cast<size_t>(ch) * RC::kBytes);
#pragma unroll
    for (int i = 0; i < Cf::NPV; ++i) {
      const int x = tid + NTH * i;
      if (Cf::NVEC % NTH == 0 || x < Cf::NVEC) pf[i] = rv[x];
    }
    const int tn = ch * C;
    if (tid < C) pbe = gbeta[row0 + static_cast<size_t>(min(tn + tid, T - 1)) * H];
    if (comp) {
#pragma unroll
      for (int i = 0; i < Cf::NVL; ++i) {
        const int v = lane + kWave * i;
        if (Cf::NVV % kWave == 0 || v < Cf::NVV) {
          const int r = min(tn + v / Cf::VPR, T - 1);
          pv[i] = *reinterpret_cast<const u32x4*>(
              gv + (row0 + static_cast<size_t>(r) * H) * DV + jw + (v % Cf::VPR) * (16 / EB));
        }
      }
    }
  };

  if (NC > 0) fetch(0);
  for (int ch = 0; ch < NC; ++ch) {
    const int t0 = ch * C;
    const int nrows = min(C, T - t0);
    __syncthreads();   // every wave is done with the previous chunk's record
#pragma unroll
    for (int i = 0; i < Cf::NPV; ++i) {
      const int x = tid + NTH * i;
      if (Cf::NVEC % NTH == 0 || x < Cf::NVEC)
        *reinterpret_cast<u32x4*>(smem + rec_vec_lds<Cf>(x)) = pf[i];
    }
    if (tid < C) sBE[tid] = (tid < nrows) ? pbe : 0.f;
    __syncthreads();
    if (comp) {
      // (beta V)^T of this wave's columns, rows past T as zeros
#pragma unroll
      for (int i = 0; i < Cf::NVL; ++i) {
        const int v = lane + kWave * i;
        if (Cf::NVV % kWave == 0 || v < Cf::NVV) {
          const int r = v / Cf::VPR, c0 = (v % Cf::VPR) * (16 / EB);
          const float be = sBE[r];
#pragma unroll
          for (int q = 0; q < 16 / EB; ++q)
            VbT[(c0 + q) * LDC + r] = Ty<OpT>::from_f32(be * vec_elem<OpT>(pv[i], q));
        }
      }
    }
    if (ch + 1 < NC) fetch(ch + 1);
    if (comp) {
      const Lane ln = lane_now();
      // S^T of this wave's tile, as the B operand of the products over channels
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        E* dst = ST + ln.i * LDK + 16 * cb + 4 * ln.g;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) dst[rr] = Ty<OpT>::from_f32(S[cb][rr]);
      }
      wave_fence();
      // U = Y (beta V) - W S
#pragma unroll
      for (int R = 0; R < NB; ++R) {
        f32x4 u = mma_k<OpT>(0, 16 * (R + 1), Src<OpT>{Yb + 16 * R * LDC, LDC, ln},
                             Src<OpT>{VbT, LDC, ln});
        const f32x4 x = mma_k<OpT>(0, DK, Src<OpT>{Wm + 16 * R * LDK, LDK, ln},
                                   Src<OpT>{ST, LDK, ln});
        E* dst = UT + ln.i * LDC + 16 * R + 4 * ln.g;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) dst[rr] = Ty<OpT>::from_f32(u[rr] - x[rr]);
      }
      wave_fence();
      // O = (Q E) S + P U
      E* po = go + (row0 + static_cast<size_t>(t0) * H) * DV + jw;
      const int rsV = H * DV;
#pragma unroll
      for (int R = 0; R < NB; ++R) {
        f32x4 o = mma_k<OpT>(0, DK, Src<OpT>{Qg + 16 * R * LDK, LDK, ln}, Src<OpT>{ST, LDK, ln});
        add4(o, mma_k<OpT>(0, 16 * (R + 1), Src<OpT>{PP + 16 * R * LDC, LDC, ln},
                           Src<OpT>{UT, LDC, ln}));
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int rl = 16 * R + 4 * ln.g + rr;
          if (rl < nrows) po[rl * rsV + ln.i] = Ty<OpT>::from_f32(o[rr]);
        }
      }
      // S <- Diag(E_{C-1}) S + (K E')^T U
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const f32x4 acc = mma_k<OpT>(0, C, Src<OpT>{KgT + 16 * cb * LDC, LDC, ln},
                                     Src<OpT>{UT, LDC, ln});
        const float4 gc = *reinterpret_cast<const float4*>(sGC + 16 * cb + 4 * ln.g);
        S[cb][0] = gc.x * S[cb][0] + acc[0];
        S[cb][1] = gc.y * S[cb][1] + acc[1];
        S[cb][2] = gc.z * S[cb][2] + acc[2];
        S[cb][3] = gc.w * S[cb][3] + acc[3];
      }
    }
  }

  if (comp && gST != nullptr) {
    const Lane ln = lane_now();
    float* dst = gST + static_cast<size_t>(chain) * DK * DV + jw;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(16 * cb + 4 * ln.g + r) * DV + ln.i] = S[cb][r];
  }
}

// ----------------------------------------------------------------------------
// Split path: prep kernel over all chunks, then the scan.
// ----------------------------------------------------------------------------
template <typename OpT, int DK, int C, int NJ>
constexpr bool scan_fits() {
  return SCfg<OpT, DK, C, NJ>::kLds <= kMaxLds;
}

// Most computing waves (16 columns each) that divide dv and fit in LDS.
template <typename OpT, int DK, int C>
int pick_scan_nj(int dv) {
  int best = 0;
  if (dv % 16 == 0 && scan_fits<OpT, DK, C, 1>()) best = 1;
  if (dv % 32 == 0 && scan_fits<OpT, DK, C, 2>()) best = 2;
  if (dv % 64 == 0 && scan_fits<OpT, DK, C, 4>()) best = 4;
  if (dv % 128 == 0 && scan_fits<OpT, DK, C, 8>()) best = 8;
  return best;
}

template <typename OpT, int DK, int C>
size_t split_workspace_bytes(int B, int T, int H) {
  const size_t nc = static_cast<size_t>((T + C - 1) / C);
  return static_cast<size_t>(B) * H * nc * RecCfg<OpT, DK, C>::kBytes;
}

template <typename OpT, int DK, int C, int NJ>
hipError_t launch_scan(const PrefillArgs& a) {
  using E = typename Ty<OpT>::Elem;
  const long chains = static_cast<long>(a.B) * a.H;
  dim3 grid(static_cast<unsigned>(chains * (a.dv / (16 * NJ))));
  hipLaunchKernelGGL((kda_scan_kernel<OpT, DK, C, NJ>), grid, dim3(512), 0,
                     static_cast<hipStream_t>(a.stream), static_cast<const E*>(a.v), a.beta,
                     a.S0, static_cast<E*>(a.o), a.S_T, static_cast<const char*>(a.workspace),
                     a.B, a.T, a.H, a.dv);
  return hipGetLastError();
}

template <typename OpT, int DK, int C>
hipError_t launch_split(const PrefillArgs& a) {
  using E = typename Ty<OpT>::Elem;
  constexpr int kPrepDvt = 16;   // the prep kernel touches no value columns
  if constexpr (!fits<OpT, DK, C, kPrepDvt>()) return hipErrorInvalidValue;
  const long chains = static_cast<long>(a.B) * a.H;
  const int nc = (a.T + C - 1) / C;
  if constexpr (fits<OpT, DK, C, kPrepDvt>()) if (nc > 0) {
    dim3 grid(static_cast<unsigned>(chains * nc));
    hipLaunchKernelGGL((kda_prefill_kernel<OpT, DK, C, kPrepDvt, true>), grid, dim3(512), 0,
                       static_cast<hipStream_t>(a.stream), static_cast<const E*>(a.q),
                       static_cast<const E*>(a.k), static_cast<const E*>(a.v), a.alpha, a.beta,
                       a.S0, static_cast<E*>(a.o), a.S_T, a.B, a.T, a.H, a.dv,
                       static_cast<char*>(a.workspace));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  switch (pick_scan_nj<OpT, DK, C>(a.dv)) {
    case 1: if constexpr (scan_fits<OpT, DK, C, 1>()) return launch_scan<OpT, DK, C, 1>(a); break;
    case 2: if constexpr (scan_fits<OpT, DK, C, 2>()) return launch_scan<OpT, DK, C, 2>(a); break;
    case 4: if constexpr (scan_fits<OpT, DK, C, 4>()) return launch_scan<OpT, DK, C, 4>(a); break;
    case 8: if constexpr (scan_fits<OpT, DK, C, 8>()) return launch_scan<OpT, DK, C, 8>(a); break;
  }
  return hipErrorInvalidValue;
}

// ----------------------------------------------------------------------------
// Path choice and dispatch over C for one (element type, dk).
//   few chains  -> split: chunk-parallel prep kernel + scan kernel (workspace)
//   many chains -> fused kernel (no workspace)
// The fused kernel serialises the column-free chunk work on one workgroup
// per chain (and per slab); with few chains that leaves most of the chip
// idle, while the split path runs it for every chunk at once.
// ----------------------------------------------------------------------------
constexpr long kSplitMaxChains = 127;

template <typename OpT, int DK, int C>
bool use_split(long chains, int dv) {
  return chains <= kSplitMaxChains && fits<OpT, DK, C, 16>() &&
         pick_scan_nj<OpT, DK, C>(dv) > 0;
}

template <typename OpT, int DK, int C>
hipError_t launch_any(const PrefillArgs& a) {
  const long chains = static_cast<long>(a.B) * a.H;
  if (use_split<OpT, DK, C>(chains, a.dv)) return launch_split<OpT, DK, C>(a);
  return launch_c<OpT, DK, C>(a);
}

template <typename OpT, int DK>
hipError_t launch_dk(const PrefillArgs& a) {
  switch (a.C) {
    case 16: return launch_any<OpT, DK, 16>(a);
    case 32: return launch_any<OpT, DK, 32>(a);
    case 64: return launch_any<OpT, DK, 64>(a);
  }
  return hipErrorInvalidValue;
}

template <typename OpT, int DK, int C>
bool supported_c(int dv) {
  return pick_dvt<OpT, DK, C>(1 << 20, dv) > 0;
}

template <typename OpT, int DK>
bool supported_dk(int dv, int C) {
  switch (C) {
    case 16: return supported_c<OpT, DK, 16>(dv);
    case 32: return supported_c<OpT, DK, 32>(dv);
    case 64: return supported_c<OpT, DK, 64>(dv);
  }
  return false;
}

template <typename OpT, int DK, int C>
size_t workspace_c(int B, int T, int H, int dv) {
  if (!use_split<OpT, DK, C>(static_cast<long>(B) * H, dv)) return 0;
  return split_workspace_bytes<OpT, DK, C>(B, T, H);
}

template <typename OpT, int DK>
size_t workspace_dk(int B, int T, int H, int dv, int C) {
  switch (C) {
    case 16: return workspace_c<OpT, DK, 16>(B, T, H, dv);
    case 32: return workspace_c<OpT, DK, 32>(B, T, H, dv);
    case 64: return workspace_c<OpT, DK, 64>(B, T, H, dv);
  }
  return 0;
}

// One translation unit per (element type, dk) instantiates these.
#define KDA_PREFILL_INSTANCE(OPT, NAME, DK)                                           \
  hipError_t launch_prefill_##NAME##_##DK(const PrefillArgs& a) {                      \
    return launch_dk<OPT, DK>(a);                                                      \
  }                                                                                    \
  bool prefill_supported_##NAME##_##DK(int dv, int C) { return supported_dk<OPT, DK>(dv, C); } \
  size_t prefill_workspace_##NAME##_##DK(int B, int T, int H, int dv, int C) {         \
    return workspace_dk<OPT, DK>(B, T, H, dv, C);                                      \
  }

#define KDA_PREFILL_DECLARE(NAME, DK)                                                  \
  hipError_t launch_prefill_##NAME##_##DK(const PrefillArgs& a);                       \
  bool prefill_supported_##NAME##_##DK(int dv, int C);                                 \
  size_t prefill_workspace_##NAME##_##DK(int B, int T, int H, int dv, int C);

KDA_PREFILL_DECLARE(bf16, 16)
KDA_PREFILL_DECLARE(bf16, 32)
KDA_PREFILL_DECLARE(bf16, 64)
KDA_PREFILL_DECLARE(bf16, 128)
KDA_PREFILL_DECLARE(f32, 16)
KDA_PREFILL_DECLARE(f32, 32)
KDA_PREFILL_DECLARE(f32, 64)
KDA_PREFILL_DECLARE(f32, 128)

}  // namespace kda
