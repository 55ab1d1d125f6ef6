// KDA chunk scan: the sequential half of the split prefill.
//
// The prep kernel (kda_prefill_kernel<..., kPrep = true>) has already written,
// for every chunk of the current segment of every chain, the state-free chunk
// quantities
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
// A workgroup has three waves per 16-row block R of the chunk.  The state
// wave of R computes rows R of U and owns state row blocks R, R + C/16, ...:
// it carries the recurrence (S -> U -> S) and touches only LDS and registers.
// The output wave of R computes rows R of O from the same S and U (its Q.E
// and P operands load into its registers three chunks ahead).  The loader wave
// of R streams the state wave's operands (W_R, the owned rows of (K.E')^T,
// U~_R of this tile, the decay) three chunks ahead from the record into one
// of four LDS buffers (two and three where four do not fit) with direct
// global-to-LDS loads.  A CU's vector memory
// path takes about 64 bytes per clock, so the ~60 KB a chunk needs occupy it
// for most of a chunk; the waves that wait on that path are never the ones
// the recurrence waits on.  S^T and U^T are exchanged through LDS; two
// barriers per chunk.
#pragma once

#include <algorithm>
#include <type_traits>

#include "prefill_kernel.hpp"

namespace kda {

template <typename OpT, int DK, int C>
struct SCfg {
  static constexpr int NB = C / 16, NCB = DK / 16;
  static constexpr int NTH = 3 * kWave * NB;         // state, output, loader waves
  static constexpr int CPW = (NCB + NB - 1) / NB;    // state row blocks per state wave
  static constexpr int EB = Ty<OpT>::kBytes, PADE = 16 / EB;
  static constexpr int LDK = DK + PADE, LDC = C + PADE, LDO = 16 + PADE;
  using RC = RecCfg<OpT, DK, C>;
  static constexpr int KSD = RC::KSD, KSC = RC::KSC, NKD = RC::NKD, NKC = RC::NKC;
  // one LDS operand buffer (byte offsets), laid out as in the record
  static constexpr int kWR = 16 * DK * EB;           // W rows of one block R
  static constexpr int kKR = 16 * C * EB;            // (K.E')^T rows of one block cb
  static constexpr int kUR = 256 * EB;               // one U~ accumulator packet
  static constexpr int oW = 0, oKG = oW + NB * kWR, oU = oKG + NCB * kKR, oGC = oU + NB * kUR;
  static constexpr int kBuf = align16(oGC + 4 * DK);
  // LDS: operand buffers, S^T, U^T, O staging (one tile per output wave), as
  // separate arrays so that the compiler can tell that LDS reads of the last
  // three never wait for the direct loads into the first.  Four buffers
  // (loads three chunks ahead) where they fit, else three (two ahead).
  static constexpr int kOS = align16(16 * LDO * EB);
  static constexpr int kRest = align16(16 * LDK * EB) + align16(16 * LDC * EB) + NB * kOS;
  static constexpr int kNBuf = (4 * kBuf + kRest <= kMaxLds) ? 4 : 3;
  static constexpr int kAhead = kNBuf - 1;
  static constexpr int kLds = kNBuf * kBuf + kRest;
};

// Register sets of record operands an output wave rotates through (opa..opd
// below): it loads chunk ch + kOutSets - 1 while computing chunk ch.
constexpr int kOutSets = 4;

// Workgroup barrier for a wave whose direct global-to-LDS loads must stay in
// flight across it (a release fence on LDS would wait for them): its own LDS
// operations complete, then the barrier; the asm also keeps the compiler from
// moving memory accesses across.  Pairs with lds_barrier() in other waves.
__device__ __forceinline__ void barrier_keep_fills() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

using lds_void = __attribute__((address_space(3))) void;
using gbl_void = const __attribute__((address_space(1))) void;

// BYTES contiguous bytes, global -> LDS, by one wave: 16-byte lanes when the
// size is a multiple of 1 KiB, else 4-byte lanes (the last pass masked, lane 0
// always active).  fill_insts: the number of load instructions it issues.
template <int BYTES>
__host__ __device__ constexpr int fill_insts() {
  return BYTES % 1024 == 0 ? BYTES / 1024 : (BYTES + 255) / 256;
}
template <int BYTES>
__device__ __forceinline__ void lds_fill(char* dst, const char* src, int lane) {
  static_assert(BYTES % 4 == 0, "4-byte granules");
  if constexpr (BYTES % 1024 == 0) {
#pragma unroll
    for (int i = 0; i < BYTES / 1024; ++i)
      __builtin_amdgcn_global_load_lds((gbl_void*)(src + 1024 * i + 16 * lane),
                                       (lds_void*)(dst + 1024 * i), 16, 0, 0);
  } else {
#pragma unroll
    for (int i = 0; i < (BYTES + 255) / 256; ++i)
      if ((BYTES % 256 == 0) || 256 * i + 4 * lane < BYTES)
        __builtin_amdgcn_global_load_lds((gbl_void*)(src + 256 * i + 4 * lane),
                                         (lds_void*)(dst + 256 * i), 4, 0, 0);
  }
}

template <typename OpT, int DK, int C>
struct OutOps {
  using Cf = SCfg<OpT, DK, C>;
  using FD = typename Frag<OpT, Cf::KSD>::T;
  using FC = typename Frag<OpT, Cf::KSC>::T;
  FD q[Cf::NKD];
  FC p[Cf::NKC];
};

template <typename OpT, int DK, int C>
__global__ void __launch_bounds__(3 * kWave * (C / 16))
kda_scan_kernel(const float* gS0, typename Ty<OpT>::Elem* __restrict__ go, float* gST,
                const char* __restrict__ gws, int B, int T, int H, int DV, int seg0, int segn,
                float* __restrict__ gSc) {
  using Cf = SCfg<OpT, DK, C>;
  using RC = typename Cf::RC;
  using E = typename Ty<OpT>::Elem;
  using OO = OutOps<OpT, DK, C>;
  using FD = typename OO::FD;
  using FC = typename OO::FC;
  constexpr int NB = Cf::NB, NCB = Cf::NCB, CPW = Cf::CPW, LDK = Cf::LDK, LDC = Cf::LDC;
  constexpr int KSD = Cf::KSD, KSC = Cf::KSC, NKD = Cf::NKD, NKC = Cf::NKC;
  constexpr int ND = KSD / 4, NCK = KSC / 4;   // elements per lane of one packet
  static_assert(Cf::kLds <= kMaxLds, "scan LDS plan exceeds 160 KiB");

  __shared__ __attribute__((aligned(16))) char opbuf[Cf::kNBuf * Cf::kBuf];
  __shared__ __attribute__((aligned(16))) E ST[16 * LDK];   // S^T of the tile
  __shared__ __attribute__((aligned(16))) E UT[16 * LDC];   // U^T of the tile
  __shared__ __attribute__((aligned(16))) E OSall[NB * Cf::kOS / Cf::EB];

  const int lane = threadIdx.x % kWave;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int R = wv % NB;
  const int role = wv / NB;   // 0 state, 1 output, 2 loader

  // Workgroup -> (chain, column tile); all tiles of a chain on one XCD so the
  // chain's records are read from HBM once and then hit that XCD's L2.
  const int NJV = DV / 16;
  const int total = gridDim.x;
  int L = blockIdx.x;
  if (NJV > 1 && (total % 8) == 0) L = (blockIdx.x % 8) * (total / 8) + blockIdx.x / 8;
  const int chain = L / NJV, jt = L % NJV;
  const int b = chain / H, h = chain % H;
  // This launch walks the segment of chunks [seg0, seg0 + segn): NC records
  // per chain, the first nfull of them full chunks; local chunk ch holds
  // tokens from (seg0 + ch) * C.
  const int NC = segn;
  const int nfull = max(0, min(segn, T / C - seg0));
  const size_t row0 = static_cast<size_t>(b) * T * H + h;
  const size_t rbytes = RC::bytes(DV);
  const char* rec0 = gws + static_cast<size_t>(chain) * NC * rbytes;
  auto buf = [&](int ch) { return opbuf + (ch % Cf::kNBuf) * Cf::kBuf; };

  if (role == 0) {
    // ---------------- state wave: S -> U -> S, LDS and registers only
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
      }
    }
    for (int ch = 0; ch < NC; ++ch) {
      const Lane ln = lane_now();
      const char* ob = buf(ch);
      if (gSc != nullptr) {
        // the state each chunk starts from, fp32, in fragment order:
        // [chain][chunk][column tile][row block][lane][4] (lane (g, i): rows
        // 4g .. 4g+3 of the block, column i), one 16-byte store per block
        const int nct = (T + C - 1) / C;
        float* dst = gSc + ((static_cast<size_t>(chain) * nct + seg0 + ch) * (DV / 16) + jt) * DK * 16;
#pragma unroll
        for (int m = 0; m < CPW; ++m) {
          const int cb = R + NB * m;
          if (cb < NCB)
            *reinterpret_cast<float4*>(dst + (cb * kWave + lane) * 4) =
                make_float4(S[m][0], S[m][1], S[m][2], S[m][3]);
        }
      }
      // publish this wave's state rows as S^T (operand type)
#pragma unroll
      for (int m = 0; m < CPW; ++m) {
        const int cb = R + NB * m;
        if (cb < NCB) Acc4<OpT>::store(ST + ln.i * LDK + 16 * cb + 4 * ln.g, S[m]);
      }
      lds_barrier();   // S^T published; this chunk's operand buffer is filled
      FD stf[NKD];
#pragma unroll
      for (int s = 0; s < NKD; ++s) stf[s] = Src<OpT>{ST, LDK, ln}.template get<KSD>(s * KSD);
      // U_R = U~_R - W_R S, published as U^T[n][16R + 4g + r]
      const E* wr = reinterpret_cast<const E*>(ob + Cf::oW + R * Cf::kWR);
      f32x4 x = zero4();
#pragma unroll
      for (int s = 0; s < NKD; ++s)
        x = mfma<OpT, KSD>(*reinterpret_cast<const FD*>(wr + (s * kWave + lane) * ND), stf[s], x);
      f32x4 u = Acc4<OpT>::cvt(
          Acc4<OpT>::load(reinterpret_cast<const E*>(ob + Cf::oU + R * Cf::kUR) + 4 * lane));
#pragma unroll
      for (int r = 0; r < 4; ++r) u[r] -= x[r];
      Acc4<OpT>::store(UT + ln.i * LDC + 16 * R + 4 * ln.g, u);
      lds_barrier();
      FC utf[NKC];
#pragma unroll
      for (int s = 0; s < NKC; ++s) utf[s] = Src<OpT>{UT, LDC, ln}.template get<KSC>(s * KSC);
      // S <- Diag(E_{C-1}) S + (K.E')^T U for this wave's row blocks
#pragma unroll
      for (int m = 0; m < CPW; ++m) {
        const int cb = R + NB * m;
        if (cb < NCB) {
          const E* kr = reinterpret_cast<const E*>(ob + Cf::oKG + cb * Cf::kKR);
          f32x4 acc = zero4();
#pragma unroll
          for (int s = 0; s < NKC; ++s)
            acc = mfma<OpT, KSC>(*reinterpret_cast<const FC*>(kr + (s * kWave + lane) * NCK), utf[s], acc);
          const float4 gc = *reinterpret_cast<const float4*>(ob + Cf::oGC + 4 * (16 * cb + 4 * ln.g));
          S[m][0] = gc.x * S[m][0] + acc[0];
          S[m][1] = gc.y * S[m][1] + acc[1];
          S[m][2] = gc.z * S[m][2] + acc[2];
          S[m][3] = gc.w * S[m][3] + acc[3];
        }
      }
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
  } else if (role == 1 && go == nullptr) {
    // ---------------- no output wanted (only the chunk states): the output
    // waves load nothing and keep the two barriers of every chunk
    for (int ch = 0; ch < NC; ++ch) {
      lds_barrier();
      lds_barrier();
    }
  } else if (role == 1) {
    // ---------------- output wave: O_R = (Q.E)_R S + P_R U
    auto fetch = [&](OO& x, int ch) {
      const E* rw = reinterpret_cast<const E*>(rec0 + static_cast<size_t>(ch) * rbytes);
      int l = lane;
      asm volatile("" : "+v"(l));
#pragma unroll
      for (int s = 0; s < NKD; ++s)
        x.q[s] = *reinterpret_cast<const FD*>(
            rw + RC::kQ + (static_cast<size_t>(R * NKD + s) * kWave + l) * ND);
#pragma unroll
      for (int s = 0; s < NKC; ++s)
        x.p[s] = *reinterpret_cast<const FC*>(
            rw + RC::kP + (static_cast<size_t>(R * NKC + s) * kWave + l) * NCK);
    };
    E* OS = OSall + R * (Cf::kOS / Cf::EB);
    E* po0 = go + row0 * DV + 16 * jt;
    const int rsV = H * DV;
    // Every chunk issues the same memory operations (the last one re-fetches
    // itself; only the partial last chunk masks its store), so the compiler's
    // wait counts stay exact instead of draining all outstanding traffic.
    auto step = [&](const OO& cur, OO& nxt, int ch, auto tail) {
      const int t0 = (seg0 + ch) * C;
      const int nrows = min(C, T - t0);
      const Lane ln = lane_now();
      lds_barrier();   // S^T of this chunk published
      fetch(nxt, min(ch + kOutSets - 1, NC - 1));
      FD stf[NKD];
#pragma unroll
      for (int s = 0; s < NKD; ++s) stf[s] = Src<OpT>{ST, LDK, ln}.template get<KSD>(s * KSD);
      f32x4 o = zero4();
#pragma unroll
      for (int s = 0; s < NKD; ++s) o = mfma<OpT, KSD>(cur.q[s], stf[s], o);
      lds_barrier();   // U^T published
      FC utf[NKC];
#pragma unroll
      for (int s = 0; s < NKC; ++s) utf[s] = Src<OpT>{UT, LDC, ln}.template get<KSC>(s * KSC);
      // P is block-lower; its upper blocks are zeros
      f32x4 pu = zero4();
#pragma unroll
      for (int s = 0; s < NKC; ++s) pu = mfma<OpT, KSC>(cur.p[s], utf[s], pu);
      add4(o, pu);
      // O tile through LDS: one 4-element row segment per lane, one store
#pragma unroll
      for (int r = 0; r < 4; ++r) OS[(4 * ln.g + r) * Cf::LDO + ln.i] = Ty<OpT>::from_f32(o[r]);
      wave_fence();
      const int orow = lane / 4, ocol = 4 * (lane % 4);
      const typename Quad<OpT>::T ov = *reinterpret_cast<const typename Quad<OpT>::T*>(OS + orow * Cf::LDO + ocol);
      const int rl = 16 * R + orow;
      if (!decltype(tail)::value || rl < nrows)
        *reinterpret_cast<typename Quad<OpT>::T*>(po0 + static_cast<size_t>(t0 + rl) * rsV + ocol) = ov;
    };
    using Full = std::integral_constant<bool, false>;
    using Tail = std::integral_constant<bool, true>;
    // Four register sets in rotation: the operands of chunk ch + 3 load while
    // chunk ch is computed, so the record reads have three chunks to land.
    static_assert(kOutSets == 4, "the rotation below has four register sets");
    OO opa, opb, opc, opd;
    if (NC > 0) {
      fetch(opa, 0);
      fetch(opb, min(1, NC - 1));
      fetch(opc, min(2, NC - 1));
    }
    int ch = 0;
    for (; ch + 4 <= nfull; ch += 4) {
      step(opa, opd, ch, Full{});
      step(opb, opa, ch + 1, Full{});
      step(opc, opb, ch + 2, Full{});
      step(opd, opc, ch + 3, Full{});
    }
    if (ch < NC) step(opa, opd, ch, Tail{});
    if (ch + 1 < NC) step(opb, opa, ch + 1, Tail{});
    if (ch + 2 < NC) step(opc, opb, ch + 2, Tail{});
    if (ch + 3 < NC) step(opd, opc, ch + 3, Tail{});
  } else {
    // ---------------- loader wave: state-wave operands, kAhead chunks ahead.
    // Operands of state wave R for chunk ch go into buffer ch % kNBuf.  Blocks
    // past dk are clamped (the same bytes written twice, never read).
    // Two halves, issued in the two halves of a chunk so that the issue
    // stalls of this wave never hold up a barrier for long.
    auto fill_a = [&](int ch) {
      const char* rc = rec0 + static_cast<size_t>(ch) * rbytes;
      char* ob = buf(ch);
      lds_fill<Cf::kWR>(ob + Cf::oW + R * Cf::kWR, rc + RC::kW * Cf::EB + R * Cf::kWR, lane);
      lds_fill<4 * DK / NB>(ob + Cf::oGC + R * (4 * DK / NB), rc + RC::kGcByte + R * (4 * DK / NB), lane);
    };
    auto fill_b = [&](int ch) {
      const char* rc = rec0 + static_cast<size_t>(ch) * rbytes;
      char* ob = buf(ch);
#pragma unroll
      for (int m = 0; m < CPW; ++m) {
        const int cb = min(R + NB * m, NCB - 1);
        lds_fill<Cf::kKR>(ob + Cf::oKG + cb * Cf::kKR, rc + RC::kKG * Cf::EB + cb * Cf::kKR, lane);
      }
      lds_fill<Cf::kUR>(ob + Cf::oU + R * Cf::kUR,
                        rc + RC::kUByte + static_cast<size_t>(R * NJV + jt) * Cf::kUR, lane);
    };
    // This wave issues nothing but fills, kFill instructions per chunk: at
    // the end of chunk ch, at most (kAhead - 1) * kFill in flight means the
    // fills for ch+1 (issued kAhead - 1 chunks earlier) have landed in LDS.
    constexpr int kAhead = Cf::kAhead;
    constexpr int kFill = fill_insts<Cf::kWR>() + CPW * fill_insts<Cf::kKR>() +
                          fill_insts<Cf::kUR>() + fill_insts<4 * DK / NB>();
    static_assert((kAhead - 1) * kFill < 63, "vmcnt range");
    if (NC > 0) {
#pragma unroll
      for (int i = 0; i < kAhead; ++i) {
        fill_a(min(i, NC - 1));
        fill_b(min(i, NC - 1));
      }
      __builtin_amdgcn_s_waitcnt(vmcnt_only((kAhead - 1) * kFill));   // buffer 0 ready
    }
    for (int ch = 0; ch < NC; ++ch) {
      const int chf = min(ch + kAhead, NC - 1);
      barrier_keep_fills();   // chunk ch starts; buffer (ch + kAhead) % kNBuf is free
      fill_a(chf);
      barrier_keep_fills();
      fill_b(chf);
      __builtin_amdgcn_s_waitcnt(vmcnt_only((kAhead - 1) * kFill));   // buffer ch + 1 ready
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));   // no fill left in flight
  }
}

// ----------------------------------------------------------------------------
// Split path: per segment of chunks, the prep kernel over all its chunks
// (runs of chunks per workgroup, all dv columns), then the scan.
// ----------------------------------------------------------------------------
template <typename OpT, int DK, int C>
constexpr bool scan_fits() {
  return SCfg<OpT, DK, C>::kLds <= kMaxLds;
}

template <typename OpT, int DK, int C>
bool split_fits(int dv) {
  if (!scan_fits<OpT, DK, C>()) return false;
  switch (dv) {
    case 16: return fits<OpT, DK, C, 16>();
    case 32: return fits<OpT, DK, C, 32>();
    case 64: return fits<OpT, DK, C, 64>();
    case 128: return fits<OpT, DK, C, 128>();
  }
  return false;
}

// The split path walks the sequence in segments of whole chunks: the prep
// kernel writes the records of one segment, the scan consumes them, and the
// next segment reuses the same records.  A segment's records are kept within
// kSegmentBudget bytes so that they stay in the chip's last-level cache
// (256 MiB of Infinity Cache on MI355X) between the two kernels, and the
// workspace does not grow with T.  Between segments the fp32 state goes
// through a carry region after the records.  Each prep launch pays ~16 us
// of fixed cost, so segments should be as large as the cache lets the scan
// find its records there.  With plain input loads that was 128 MiB (the scan
// read its records at 0.77 us per chunk up to 128 MiB, 0.92 / 1.11 us at 160
// / 192 MiB); with the inputs of a multi-segment call loaded non-temporally
// (launch_split) it is 192 MiB (32 chains x 2^20 tokens, dk = dv = 128,
// C = 64: 30.2 / 29.7 / 30.5 ms at 160 / 192 / 224 MiB).
constexpr size_t kSegmentBudget = size_t{192} << 20;

struct SplitPlan {
  int nc = 0;        // chunks per chain
  int nseg = 0;      // segments
  int segch = 0;     // chunks per segment (the last one may have fewer)
  size_t records = 0, carry = 0;   // workspace bytes: records, then carry
};

// budget: bytes of records one segment may hold (kSegmentBudget, or less
// when the workspace itself is bounded).
template <typename OpT, int DK, int C>
SplitPlan split_plan(int B, int T, int H, int dv, size_t budget = kSegmentBudget) {
  SplitPlan p;
  const size_t chains = static_cast<size_t>(B) * H;
  const size_t rec = RecCfg<OpT, DK, C>::bytes(dv);
  p.nc = (T + C - 1) / C;
  if (p.nc == 0) return p;
  const size_t per_chunk = chains * rec;   // one chunk of every chain
  size_t segmax = std::max<size_t>(1, budget / per_chunk);
  // The prep kernel splits a segment's chunks of each chain into
  // floor(256 / chains) equal runs (prep_chunks_per_block); a segment length
  // that is a multiple of that count leaves no run shorter than the others.
  const size_t runs = chains < 256 ? 256 / chains : 1;
  if (segmax > runs) segmax -= segmax % runs;
  p.nseg = static_cast<int>((static_cast<size_t>(p.nc) + segmax - 1) / segmax);
  size_t segch = (static_cast<size_t>(p.nc) + p.nseg - 1) / p.nseg;
  if (p.nseg > 1) segch = std::min(segmax, (segch + runs - 1) / runs * runs);
  p.segch = static_cast<int>(segch);
  p.records = chains * p.segch * rec;
  p.carry = p.nseg > 1 ? chains * DK * dv * sizeof(float) : 0;
  return p;
}

template <typename OpT, int DK, int C>
size_t split_workspace_bytes(int B, int T, int H, int dv, size_t budget) {
  const SplitPlan p = split_plan<OpT, DK, C>(B, T, H, dv, budget);
  return p.records + p.carry;
}

// Chunks per prep workgroup: each chain's nc chunks split into at most
// floor(256 / chains) equal runs (at least one), so that the grid is one
// round of at most one workgroup per CU whenever chains <= 256.
inline int prep_chunks_per_block(long chains, int nc) {
  constexpr long kCUs = 256;
  long runs = kCUs / (chains > 0 ? chains : 1);
  if (runs < 1) runs = 1;
  if (runs > nc) runs = nc;
  return static_cast<int>((nc + runs - 1) / runs);
}

template <typename OpT, int DK, int C, int DVT, int kIn>
hipError_t launch_prep(const PrefillArgs& a, int seg0, int segn, bool nt_in) {
  using E = typename Ty<OpT>::Elem;
  if constexpr (!fits<OpT, DK, C, DVT>()) {
    return hipErrorInvalidValue;
  } else {
    if (segn == 0) return hipSuccess;
    const long chains = static_cast<long>(a.B) * a.H;
    // One workgroup per CU at this LDS size: give each a run of chunks so that
    // all but the first chunk's loads hide behind compute.
    const int cpb = prep_chunks_per_block(chains, segn);
    const long blocks = chains * ((segn + cpb - 1) / cpb);
    hipLaunchKernelGGL((kda_prefill_kernel<OpT, DK, C, DVT, true, kIn>),
                       dim3(static_cast<unsigned>(blocks)), dim3(512), 0,
                       static_cast<hipStream_t>(a.stream), static_cast<const E*>(a.q),
                       static_cast<const E*>(a.k), static_cast<const E*>(a.v), a.gate, a.beta,
                       a.S0, static_cast<E*>(a.o), a.S_T, a.B, a.T, a.H, a.dv,
                       static_cast<char*>(a.workspace), cpb, seg0, segn, a.qk_map,
                       nt_in ? 1 : 0, nullptr);
    return hipGetLastError();
  }
}

template <typename OpT, int DK, int C, int kIn>
hipError_t launch_split(const PrefillArgs& a) {
  using E = typename Ty<OpT>::Elem;
  if constexpr (!scan_fits<OpT, DK, C>()) {
    return hipErrorInvalidValue;
  } else {
    const SplitPlan p = split_plan<OpT, DK, C>(a.B, a.T, a.H, a.dv,
                                               a.segment_budget ? a.segment_budget : kSegmentBudget);
    const long chains = static_cast<long>(a.B) * a.H;
    float* carry = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + p.records);
    // T = 0 still runs one (empty) scan: it copies S0, or zeros, to S_T.
    const int nlaunch = p.nseg > 0 ? p.nseg : 1;
    // Several segments: the inputs are streamed once and cannot stay in the
    // cache anyway, so the prep loads them with the non-temporal hint and the
    // records keep the cache (32 chains x 2^20 tokens: 32.1 -> 29.7 ms with
    // 192 MiB segments).  One segment: plain loads (inputs a caller has just
    // written, or re-reads, may still be cached).
    const bool nt_in = p.nseg > 1;
    for (int sgi = 0; sgi < nlaunch; ++sgi) {
      const int seg0 = sgi * p.segch;
      const int segn = p.nseg > 0 ? std::min(p.segch, p.nc - seg0) : 0;
      hipError_t e = hipErrorInvalidValue;
      switch (a.dv) {
        case 16: e = launch_prep<OpT, DK, C, 16, kIn>(a, seg0, segn, nt_in); break;
        case 32: e = launch_prep<OpT, DK, C, 32, kIn>(a, seg0, segn, nt_in); break;
        case 64: e = launch_prep<OpT, DK, C, 64, kIn>(a, seg0, segn, nt_in); break;
        case 128: e = launch_prep<OpT, DK, C, 128, kIn>(a, seg0, segn, nt_in); break;
      }
      if (e != hipSuccess) return e;
      const float* s_in = sgi == 0 ? a.S0 : carry;
      float* s_out = sgi == nlaunch - 1 ? a.S_T : carry;   // in place between segments
      dim3 grid(static_cast<unsigned>(chains * (a.dv / 16)));
      hipLaunchKernelGGL((kda_scan_kernel<OpT, DK, C>), grid, dim3(SCfg<OpT, DK, C>::NTH), 0,
                         static_cast<hipStream_t>(a.stream), s_in, static_cast<E*>(a.o), s_out,
                         static_cast<const char*>(a.workspace), a.B, a.T, a.H, a.dv, seg0, segn,
                         a.chunk_states);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
}

// ----------------------------------------------------------------------------
// Path choice and dispatch over C for one (element type, dk).
//   few chains  -> split: chunk-parallel prep kernel + scan kernel (workspace)
//   many chains -> fused kernel (no workspace)
// The fused kernel serialises the column-free chunk work on one workgroup
// per chain (and per slab); with few chains that leaves most of the chip
// idle, while the split path runs it for every chunk at once.  Measured at
// dk = dv = 128, C = 64, T = 8192: 128 chains take 1.22 ms split and 1.39 ms
// fused, 160 chains 1.97 ms split and 1.65 ms fused.
// ----------------------------------------------------------------------------
constexpr long kSplitMaxChains = 128;

template <typename OpT, int DK, int C>
bool use_split(long chains, int dv) {
  return chains <= kSplitMaxChains && split_fits<OpT, DK, C>(dv);
}

template <typename OpT, int DK, int C>
hipError_t launch_any(const PrefillArgs& a) {
  const long chains = static_cast<long>(a.B) * a.H;
  if (a.force_split && !split_fits<OpT, DK, C>(a.dv)) return hipErrorInvalidValue;
  const bool split = a.force_split || use_split<OpT, DK, C>(chains, a.dv);
  switch (a.gate_in) {
    case kGateAlpha:
      return split ? launch_split<OpT, DK, C, kGateAlpha>(a) : launch_c<OpT, DK, C, kGateAlpha>(a);
    case kGateLogit:
      return split ? launch_split<OpT, DK, C, kGateLogit>(a) : launch_c<OpT, DK, C, kGateLogit>(a);
    case kGateScalar:
      return split ? launch_split<OpT, DK, C, kGateScalar>(a)
                   : launch_c<OpT, DK, C, kGateScalar>(a);
  }
  return hipErrorInvalidValue;
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
size_t workspace_c(int B, int T, int H, int dv, size_t budget, bool force_split) {
  if (force_split ? !split_fits<OpT, DK, C>(dv) : !use_split<OpT, DK, C>(static_cast<long>(B) * H, dv))
    return 0;
  return split_workspace_bytes<OpT, DK, C>(B, T, H, dv, budget);
}

template <typename OpT, int DK>
size_t workspace_dk(int B, int T, int H, int dv, int C, size_t budget, bool force_split) {
  switch (C) {
    case 16: return workspace_c<OpT, DK, 16>(B, T, H, dv, budget, force_split);
    case 32: return workspace_c<OpT, DK, 32>(B, T, H, dv, budget, force_split);
    case 64: return workspace_c<OpT, DK, 64>(B, T, H, dv, budget, force_split);
  }
  return 0;
}

// One translation unit per (element type, dk) instantiates these.
#define KDA_PREFILL_INSTANCE(OPT, NAME, DK)                                           \
  hipError_t launch_prefill_##NAME##_##DK(const PrefillArgs& a) {                      \
    return launch_dk<OPT, DK>(a);                                                      \
  }                                                                                    \
  bool prefill_supported_##NAME##_##DK(int dv, int C) { return supported_dk<OPT, DK>(dv, C); } \
  size_t prefill_workspace_##NAME##_##DK(int B, int T, int H, int dv, int C,           \
                                         size_t budget, bool force_split) {           \
    return workspace_dk<OPT, DK>(B, T, H, dv, C, budget, force_split);                 \
  }

#define KDA_PREFILL_DECLARE(NAME, DK)                                                  \
  hipError_t launch_prefill_##NAME##_##DK(const PrefillArgs& a);                       \
  bool prefill_supported_##NAME##_##DK(int dv, int C);                                 \
  size_t prefill_workspace_##NAME##_##DK(int B, int T, int H, int dv, int C, size_t budget, \
                                         bool force_split);

KDA_PREFILL_DECLARE(bf16, 16)
KDA_PREFILL_DECLARE(bf16, 32)
KDA_PREFILL_DECLARE(bf16, 64)
KDA_PREFILL_DECLARE(bf16, 128)
KDA_PREFILL_DECLARE(f32, 16)
KDA_PREFILL_DECLARE(f32, 32)
KDA_PREFILL_DECLARE(f32, 64)
KDA_PREFILL_DECLARE(f32, 128)

}  // namespace kda
