// KDA chunk scan: the sequential half of the split prefill.
//
// The prep kernel (kda_prefill_kernel<..., kPrep = true>) has already written,
// for every chunk of every chain, the state-free chunk quantities
//   W = Y Diag(beta)(K.E),  Q.E,  (K.E')^T,  P (gated Q K^T, lower),
//   the chunk decay E_{C-1},  U~ = Y Diag(beta) V
// to a workspace record (RecCfg), as matrix-core operand packets.  This
// kernel walks the chunks of one chain in order for one 16-column tile of the
// state:
//   U = U~ - W S,  O = (Q.E) S + P U,  S <- Diag(E_{C-1}) S + (K.E')^T U
// (the chunk algebra of "From GPT-2 to Kimi K3, Explained", section "DeltaNet
// (Parallelizing Linear Transformers with Delta Rule)", with the per-channel
// decay of section "KDA/Kimi Linear").
//
// A workgroup has one wave per 16-row block R of the chunk.  Wave R computes
// rows R of U and O and owns state row blocks R, R + C/16, ...; the state
// tile (S^T) and U^T are exchanged through LDS, two LDS-only barriers per
// chunk.  Every record operand goes straight from global memory into the
// registers of the wave that uses it, one chunk ahead, so the chain of
// dependent work per chunk is a handful of short MFMA chains.
#pragma once

#include <type_traits>

#include "prefill_kernel.hpp"

namespace kda {

template <typename OpT, int DK, int C>
struct SCfg {
  static constexpr int NB = C / 16, NCB = DK / 16;
  static constexpr int NTH = kWave * NB;
  static constexpr int CPW = (NCB + NB - 1) / NB;    // state row blocks per wave
  static constexpr int EB = Ty<OpT>::kBytes, PADE = 16 / EB;
  static constexpr int LDK = DK + PADE, LDC = C + PADE;
  using RC = RecCfg<OpT, DK, C>;
  static constexpr int KSD = RC::KSD, KSC = RC::KSC, NKD = RC::NKD, NKC = RC::NKC;
};

// One chunk's record operands for wave R.
template <typename OpT, int DK, int C>
struct ScanOps {
  using Cf = SCfg<OpT, DK, C>;
  using FD = typename Frag<OpT, Cf::KSD>::T;
  using FC = typename Frag<OpT, Cf::KSC>::T;
  FD w[Cf::NKD], q[Cf::NKD];
  FC p[Cf::NKC];
  FC kg[Cf::CPW][Cf::NKC];
  typename Acc4<OpT>::Raw ut;
  float4 gc[Cf::CPW];
};

template <typename OpT, int DK, int C>
__global__ void __launch_bounds__(kWave * (C / 16))
kda_scan_kernel(const float* gS0, typename Ty<OpT>::Elem* __restrict__ go, float* gST,
                const char* __restrict__ gws, int B, int T, int H, int DV) {
  using Cf = SCfg<OpT, DK, C>;
  using RC = typename Cf::RC;
  using E = typename Ty<OpT>::Elem;
  using Ops = ScanOps<OpT, DK, C>;
  constexpr int NB = Cf::NB, NCB = Cf::NCB, CPW = Cf::CPW, LDK = Cf::LDK, LDC = Cf::LDC;
  constexpr int KSD = Cf::KSD, KSC = Cf::KSC, NKD = Cf::NKD, NKC = Cf::NKC;
  constexpr int ND = KSD / 4, NCK = KSC / 4;   // elements per lane of one packet

  __shared__ __attribute__((aligned(16))) E ST[16 * LDK];   // S^T of the tile
  __shared__ __attribute__((aligned(16))) E UT[16 * LDC];   // U^T of the tile

  const int lane = threadIdx.x % kWave;
  const int R = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

  // Workgroup -> (chain, column tile); all tiles of a chain on one XCD so the
  // chain's records are read from HBM once and then hit that XCD's L2.
  const int NJV = DV / 16;
  const int total = gridDim.x;
  int L = blockIdx.x;
  if (NJV > 1 && (total % 8) == 0) L = (blockIdx.x % 8) * (total / 8) + blockIdx.x / 8;
  const int chain = L / NJV, jt = L % NJV;
  const int b = chain / H, h = chain % H;
  const int NC = (T + C - 1) / C;
  const size_t row0 = static_cast<size_t>(b) * T * H + h;
  const size_t rbytes = RC::bytes(DV);
  const char* rec0 = gws + static_cast<size_t>(chain) * NC * rbytes;

  // state row blocks cb = R + NB*m of the tile, in registers
  f32x4 S[CPW];
  {
    const Lane ln = lane_now();
#pragma unroll
    for (int m = 0; m < CPW; ++m) {
      const int cb = R + NB * m;
      S[m] = zero4();
      if (cb < NCB && gS0 != nullptr) {
        const float* src = gS0 + static_cast<size_t>(chain) * DK * DV + 16 * jt;
#pragma unroll
        for (int r = 0; r < 4; ++r) S[m][r] = src[(16 * cb + 4 * ln.g + r) * DV + ln.i];
      }
      // Land the loads here: a load still in flight at the loop entry makes
      // every chunk wait for all outstanding memory traffic.
      asm volatile("" : "+v"(S[m][0]), "+v"(S[m][1]), "+v"(S[m][2]), "+v"(S[m][3]));
    }
  }

  // The next chunk's operands, in four parts.  A CU's vector memory path
  // moves about 64 bytes per clock, so one wave issuing all of its ~17 KB at
  // once would stall on issue for most of a chunk; the parts are spread over
  // the phases of the chunk instead.
  auto fetch = [&](Ops& x, int ch, auto part) {
    constexpr int kPart = decltype(part)::value;
    const char* rc = rec0 + static_cast<size_t>(ch) * rbytes;
    const E* rw = reinterpret_cast<const E*>(rc);
    int l = lane;
    asm volatile("" : "+v"(l));
    if constexpr (kPart == 0 || kPart == 1) {
#pragma unroll
      for (int s = 0; s < NKD; ++s) {
        const size_t o = (static_cast<size_t>(R * NKD + s) * kWave + l) * ND;
        if constexpr (kPart == 0) x.w[s] = *reinterpret_cast<const typename Ops::FD*>(rw + RC::kW + o);
        else x.q[s] = *reinterpret_cast<const typename Ops::FD*>(rw + RC::kQ + o);
      }
    } else if constexpr (kPart == 2) {
#pragma unroll
      for (int s = 0; s < NKC; ++s)
        x.p[s] = *reinterpret_cast<const typename Ops::FC*>(
            rw + RC::kP + (static_cast<size_t>(R * NKC + s) * kWave + l) * NCK);
      x.ut = Acc4<OpT>::load(reinterpret_cast<const E*>(rc + RC::kUByte) +
                             (static_cast<size_t>(R * NJV + jt) * kWave + l) * 4);
    } else {
#pragma unroll
      for (int m = 0; m < CPW; ++m) {
        const int cb = min(R + NB * m, NCB - 1);   // blocks past dk: loaded, never used
#pragma unroll
        for (int s = 0; s < NKC; ++s)
          x.kg[m][s] = *reinterpret_cast<const typename Ops::FC*>(
              rw + RC::kKG + (static_cast<size_t>(cb * NKC + s) * kWave + l) * NCK);
        x.gc[m] = *reinterpret_cast<const float4*>(rc + RC::kGcByte + 4 * (16 * cb + 4 * (l / 16)));
      }
    }
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using P2 = std::integral_constant<int, 2>;
  using P3 = std::integral_constant<int, 3>;
  auto fetch_all = [&](Ops& x, int ch) {
    fetch(x, ch, P0{});
    fetch(x, ch, P1{});
    fetch(x, ch, P2{});
    fetch(x, ch, P3{});
  };


  E* po0 = go + row0 * DV + 16 * jt;
  const int rsV = H * DV;
  // One chunk: consumes `cur`, meanwhile the next chunk's operands load into
  // `nxt`.  Every chunk issues the same memory operations (the last one
  // re-fetches itself; only the partial last chunk masks its stores), so the
  // compiler's wait counts stay exact instead of draining all traffic.
  auto step = [&](const Ops& cur, Ops& nxt, int ch, auto tail) {
    const int chn = min(ch + 1, NC - 1);
    fetch(nxt, chn, P0{});
    __builtin_amdgcn_sched_barrier(0);
    const int t0 = ch * C;
    const int nrows = min(C, T - t0);
    const Lane ln = lane_now();

    // publish this wave's state rows as S^T (operand type)
#pragma unroll
    for (int m = 0; m < CPW; ++m) {
      const int cb = R + NB * m;
      if (cb < NCB) Acc4<OpT>::store(ST + ln.i * LDK + 16 * cb + 4 * ln.g, S[m]);
    }
    lds_barrier();
    typename Ops::FD stf[NKD];
#pragma unroll
    for (int s = 0; s < NKD; ++s) stf[s] = Src<OpT>{ST, LDK, ln}.template get<KSD>(s * KSD);
    // U_R = U~_R - W_R S  and the first half of O_R = (Q.E)_R S
    f32x4 x = zero4(), o = zero4();
#pragma unroll
    for (int s = 0; s < NKD; ++s) x = mfma<OpT, KSD>(cur.w[s], stf[s], x);
#pragma unroll
    for (int s = 0; s < NKD; ++s) o = mfma<OpT, KSD>(cur.q[s], stf[s], o);
    __builtin_amdgcn_sched_barrier(0);
    fetch(nxt, chn, P1{});
    __builtin_amdgcn_sched_barrier(0);
    f32x4 u = Acc4<OpT>::cvt(cur.ut);
#pragma unroll
    for (int r = 0; r < 4; ++r) u[r] -= x[r];
    // U^T[n][16R + 4g + r]
    Acc4<OpT>::store(UT + ln.i * LDC + 16 * R + 4 * ln.g, u);
    lds_barrier();
    typename Ops::FC utf[NKC];
#pragma unroll
    for (int s = 0; s < NKC; ++s) utf[s] = Src<OpT>{UT, LDC, ln}.template get<KSC>(s * KSC);
    // S <- Diag(E_{C-1}) S + (K.E')^T U for this wave's row blocks (first:
    // the next chunk waits on it), then O_R += P_R U (P is block-lower, its
    // upper blocks are zeros).
    f32x4 acc[CPW];
#pragma unroll
    for (int m = 0; m < CPW; ++m) {
      acc[m] = zero4();
      if (R + NB * m < NCB) {
#pragma unroll
        for (int s = 0; s < NKC; ++s) acc[m] = mfma<OpT, KSC>(cur.kg[m][s], utf[s], acc[m]);
      }
    }
    f32x4 pu = zero4();
#pragma unroll
    for (int s = 0; s < NKC; ++s) pu = mfma<OpT, KSC>(cur.p[s], utf[s], pu);
    __builtin_amdgcn_sched_barrier(0);
    fetch(nxt, chn, P2{});
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0; m < CPW; ++m) {
      if (R + NB * m < NCB) {
        const float4 gc = cur.gc[m];
        S[m][0] = gc.x * S[m][0] + acc[m][0];
        S[m][1] = gc.y * S[m][1] + acc[m][1];
        S[m][2] = gc.z * S[m][2] + acc[m][2];
        S[m][3] = gc.w * S[m][3] + acc[m][3];
      }
    }
    add4(o, pu);
    E* po = po0 + static_cast<size_t>(t0) * rsV;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rl = 16 * R + 4 * ln.g + r;
      if (!decltype(tail)::value || rl < nrows) po[rl * rsV + ln.i] = Ty<OpT>::from_f32(o[r]);
    }
    __builtin_amdgcn_sched_barrier(0);
    fetch(nxt, chn, P3{});
  };
  // Two operand sets in alternation (no register copies between chunks).
  using Full = std::integral_constant<bool, false>;
  using Tail = std::integral_constant<bool, true>;
  Ops opa, opb;
  if (NC > 0) fetch_all(opa, 0);
  const int nfull = T / C;
  int ch = 0;
  for (; ch + 2 <= nfull; ch += 2) {
    step(opa, opb, ch, Full{});
    step(opb, opa, ch + 1, Full{});
  }
  // at most two chunks left: one full and/or the partial last one
  if (ch < NC) {
    if (ch < nfull) step(opa, opb, ch, Full{});
    else step(opa, opb, ch, Tail{});
    if (ch + 1 < NC) step(opb, opa, ch + 1, Tail{});
  }

  if (gST != nullptr) {
    const Lane ln = lane_now();
    float* dst = gST + static_cast<size_t>(chain) * DK * DV + 16 * jt;
#pragma unroll
    for (int m = 0; m < CPW; ++m) {
      const int cb = R + NB * m;
      if (cb < NCB) {
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(16 * cb + 4 * ln.g + r) * DV + ln.i] = S[m][r];
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Split path: prep kernel over all chunks (one workgroup per chunk, all dv
// columns), then the scan.
// ----------------------------------------------------------------------------
template <typename OpT, int DK, int C>
bool split_fits(int dv) {
  switch (dv) {
    case 16: return fits<OpT, DK, C, 16>();
    case 32: return fits<OpT, DK, C, 32>();
    case 64: return fits<OpT, DK, C, 64>();
    case 128: return fits<OpT, DK, C, 128>();
  }
  return false;
}

template <typename OpT, int DK, int C>
size_t split_workspace_bytes(int B, int T, int H, int dv) {
  const size_t nc = static_cast<size_t>((T + C - 1) / C);
  return static_cast<size_t>(B) * H * nc * RecCfg<OpT, DK, C>::bytes(dv);
}

// Chunks per prep workgroup: about one workgroup per CU in total.
inline int prep_chunks_per_block(long chains, int nc) {
  constexpr long kCUs = 256;
  const long total = chains * nc;
  long cpb = (total + kCUs - 1) / kCUs;
  if (cpb < 1) cpb = 1;
  if (cpb > nc) cpb = nc;
  return static_cast<int>(cpb);
}

template <typename OpT, int DK, int C, int DVT>
hipError_t launch_prep(const PrefillArgs& a) {
  using E = typename Ty<OpT>::Elem;
  if constexpr (!fits<OpT, DK, C, DVT>()) {
    return hipErrorInvalidValue;
  } else {
    const long chains = static_cast<long>(a.B) * a.H;
    const int nc = (a.T + C - 1) / C;
    if (nc == 0) return hipSuccess;
    // One workgroup per CU at this LDS size: give each a run of chunks so that
    // all but the first chunk's loads hide behind compute.
    const int cpb = prep_chunks_per_block(chains, nc);
    const long blocks = chains * ((nc + cpb - 1) / cpb);
    hipLaunchKernelGGL((kda_prefill_kernel<OpT, DK, C, DVT, true>), dim3(static_cast<unsigned>(blocks)),
                       dim3(512), 0, static_cast<hipStream_t>(a.stream), static_cast<const E*>(a.q),
                       static_cast<const E*>(a.k), static_cast<const E*>(a.v), a.alpha, a.beta,
                       a.S0, static_cast<E*>(a.o), a.S_T, a.B, a.T, a.H, a.dv,
                       static_cast<char*>(a.workspace), cpb);
    return hipGetLastError();
  }
}

template <typename OpT, int DK, int C>
hipError_t launch_split(const PrefillArgs& a) {
  using E = typename Ty<OpT>::Elem;
  hipError_t e = hipErrorInvalidValue;
  switch (a.dv) {
    case 16: e = launch_prep<OpT, DK, C, 16>(a); break;
    case 32: e = launch_prep<OpT, DK, C, 32>(a); break;
    case 64: e = launch_prep<OpT, DK, C, 64>(a); break;
    case 128: e = launch_prep<OpT, DK, C, 128>(a); break;
  }
  if (e != hipSuccess) return e;
  const long chains = static_cast<long>(a.B) * a.H;
  dim3 grid(static_cast<unsigned>(chains * (a.dv / 16)));
  hipLaunchKernelGGL((kda_scan_kernel<OpT, DK, C>), grid, dim3(SCfg<OpT, DK, C>::NTH), 0,
                     static_cast<hipStream_t>(a.stream), a.S0, static_cast<E*>(a.o), a.S_T,
                     static_cast<const char*>(a.workspace), a.B, a.T, a.H, a.dv);
  return hipGetLastError();
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
  return chains <= kSplitMaxChains && split_fits<OpT, DK, C>(dv);
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
  return split_workspace_bytes<OpT, DK, C>(B, T, H, dv);
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
