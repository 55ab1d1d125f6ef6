// KDA prefill backward in chunk form, on the matrix cores (bf16 operands,
// fp32 accumulation), deterministic: every gradient element is written once
// by one lane, with no atomics.
//
// The forward is the chunk algebra of "From GPT-2 to Kimi K3, Explained",
// section "DeltaNet (Parallelizing Linear Transformers with Delta Rule)",
// with the per-channel decay of section "KDA/Kimi Linear".  Its adjoint, for
// a block of rows from state S with dL/dO and dS = dL/dS_new given:
//   dU = P^T dO + (K.E') dS          dZ = Y^T dU          dv = beta dZ
//   dP = tril(dO U^T)                dA = -Diag(beta) strict_tril(dZ U^T)
//   dbeta = rowsum(dZ . X) + rowsum(dA/beta . A),  X = V - (K.E) S
//   dq = E . (dO S^T) + G1           G1_r = sum_{i<=r} dP_ri k_i Gam_ri
//   dk = -beta E . (dZ S^T) + G2 + G3 + E' . (U dS^T)
//        G2_r = sum_{i<r} dA_ri k_i Gam_ri,  G3_i = sum_{r>=i} (dP_ri q_r + dA_ri k_r) Gam_ri
//   dS_prev = Diag(E_last) dS + (Q.E)^T dO - (K.E)^T Diag(beta) dZ
// (E_r the decay from the block start through r, E'_r the decay after r to
// the block end, Gam_ri = prod_{i<j<=r} alpha_j).  The state gradient runs
// backwards through the sequence; everything else is local to a block.
//
// Blocks are 16-row sub-chunks.  Within 16 rows every pairwise decay is taken
// exactly as a running product of alpha on the vector units, so the gate
// gradient needs neither a reciprocal nor a cumulative-sum difference: each
// term of dL/dalpha_t carries alpha_t as a factor, and the kernel forms the
// terms with that factor left out,
//   dalpha_t = F_{t-1} sum_{r>=t} rho_r Gam_rt + H_t sum_{i<t} sigma_i Gam_{t-1,i}
//            + F_{t-1} H_t fin + sum_{i<t} k_i Gam_{t-1,i} sum_{r>=t} x_ri Gam_rt
//   rho_r = q_r (dO S^T)_r - beta_r k_r (dZ S^T)_r,  sigma_i = k_i (U dS^T)_i,
//   fin = rowsum(dS . S),  x_ri = dP_ri q_r + dA_ri k_r,
// F_{t-1} = E_{t-1}, H_t = E'_t: exact at alpha_t = 0 as well.
//
// Launches (one stream):
//   1. the forward split path (prep + scan kernels of the prefill), which
//      also stores the state at the start of every 64-token chunk;
//   2. kda_cb_prep_kernel: per 64-token chunk, the four sub-chunks' gates,
//      A, P, Y = (I + Diag(beta) A)^-1, W = Y Diag(beta)(K.E), written as
//      matrix-core fragments (a "sub-chunk record");
//   3. kda_cb_scan_kernel: per (chain, 16-column tile of the state gradient),
//      the state gradient from the last sub-chunk to the first, storing it at
//      the end of every 64-token chunk, and dS0;
//   4. kda_cb_grad_kernel: per 64-token chunk, the states of its four
//      sub-chunks (forward from the stored chunk state), then the sub-chunks
//      from the last to the first: all gradients of their tokens.
#include <mutex>

#include "scan_kernel.hpp"

namespace kda {
namespace {

constexpr int kSB = 16;            // rows of a sub-chunk
constexpr int kCB = 64;            // tokens between stored states (forward chunk)
constexpr int kNSB = kCB / kSB;    // sub-chunks per chunk
constexpr int kCbThreads = 512;

// One sub-chunk record (bytes).  A "fragment" is one bf16 A operand of a
// matrix-core product in lane order.  16x16x16 (512 B): lane (g, i) holds
// row i, columns 4g .. 4g+3.  16x16x32 (1 KiB): lane (g, i) holds row i at
// eight contraction slots, numbered so that the B operand is a lane's own
// registers -- its four rows 4g .. 4g+3 of two 16-row blocks:
//   [(Q.E)^T | -W^T] for row block R of DK: slots (Q.E)[4g+x][16R+i],
//        then -W[4g+x][16R+i]   (contracts with [dO ; u] over the 16 rows)
//   K.E' for channels 32kk .. 32kk+31: slots (K.E')[i][32kk+4g+x], then
//        (K.E')[i][32kk+16+4g+x]  (contracts with state rows 2kk, 2kk+1)
template <int DK>
struct BRec {
  static constexpr int NM = DK / 16, NK = DK / 32;
  static constexpr int kFrag = 64 * 4 * 2, kFrag32 = 64 * 8 * 2;
  static constexpr int oQW = 0;                    // [(Q.E)^T | -W^T]: [NM] 16x16x32 fragments
  static constexpr int oK = oQW + NM * kFrag32;    // K.E': [NK] 16x16x32 fragments
  static constexpr int oP = oK + NK * kFrag32;     // P^T, one 16x16x16 fragment
  static constexpr int oG = oP + kFrag;          // decay of the sub-chunk, fp32 [DK]
  static constexpr int oY = oG + 4 * DK;         // Y, fp32 [16][16]
  static constexpr int oA = oY + 1024;           // A (before beta), fp32 [16][16]
  static constexpr int kBytes = oA + 1024;
  static_assert(kBytes % 256 == 0, "records stay 256-byte aligned");
};

__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
// A 16x16x32 contraction as two 16x16x16 products: lane (g, i) splits its
// eight contraction slots into the four of each half, which is the
// 16x16x16 operand layout.  (Single 16x16x32 bf16 products here were seen to
// read an accumulator that the compiler let following vector instructions
// overwrite a few cycles later: corrupted sums that varied from run to run.)
__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) {
  const uint4 ua = __builtin_bit_cast(uint4, a), ub = __builtin_bit_cast(uint4, b);
  const bf16x4 alo = __builtin_bit_cast(bf16x4, make_uint2(ua.x, ua.y));
  const bf16x4 ahi = __builtin_bit_cast(bf16x4, make_uint2(ua.z, ua.w));
  const bf16x4 blo = __builtin_bit_cast(bf16x4, make_uint2(ub.x, ub.y));
  const bf16x4 bhi = __builtin_bit_cast(bf16x4, make_uint2(ub.z, ub.w));
  return mma16(ahi, bhi, mma16(alo, blo, c));
}
__device__ __forceinline__ bf16x4 quad4(const f32x4& v) { return bf16_quad(v[0], v[1], v[2], v[3]); }
__device__ __forceinline__ bf16x4 ld4(const uint16_t* p) {
  return *reinterpret_cast<const bf16x4*>(p);
}
__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
// f(std::integral_constant<int, I>) for I = B .. E-1, as straight-line code.
template <int I, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < E) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, E>(f);
  }
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
  const uint2 x = __builtin_bit_cast(uint2, a), y = __builtin_bit_cast(uint2, b);
  return __builtin_bit_cast(bf16x8, make_uint4(x.x, x.y, y.x, y.y));
}
__device__ __forceinline__ bf16x4 bits4(uint16_t a, uint16_t b, uint16_t c, uint16_t d) {
  return __builtin_bit_cast(bf16x4, make_uint2(a | (static_cast<uint32_t>(b) << 16),
                                               c | (static_cast<uint32_t>(d) << 16)));
}
// Element x of a bf16x4, its bits.
__device__ __forceinline__ uint16_t half16(bf16x4 v, int x) {
  const uint2 u = __builtin_bit_cast(uint2, v);
  const uint32_t w = x < 2 ? u.x : u.y;
  return static_cast<uint16_t>((x & 1) ? (w >> 16) : w);
}
__device__ __forceinline__ float unbf(bf16x4 v, int x) {
  const uint2 u = __builtin_bit_cast(uint2, v);
  const uint32_t w = x < 2 ? u.x : u.y;
  return bf16_to_f32(static_cast<uint16_t>((x & 1) ? (w >> 16) : (w & 0xffffu)));
}
// Sum over the 16 lanes of a lane row (every lane gets it): rotations by 8,
// 4, 2, 1 within the row.
__device__ __forceinline__ float row16_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x124, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x122, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x121, 0xF, 0xF, false));
  return x;
}

// ---------------------------------------------------------------------------
// 2. Sub-chunk records.  One workgroup of two waves per (chain, sub-chunk):
// 15.5 KiB of LDS and ~100 registers, so that ten workgroups share a CU and
// one's loads overlap another's arithmetic (one workgroup of eight waves per
// 64-token chunk, one per CU by its LDS, took 88 us on H=16 T=4096).
// ---------------------------------------------------------------------------
constexpr int kPS = 1;   // sub-chunks per record workgroup (2 measured the same)
template <int DK>
__global__ void __launch_bounds__(DK * kPS) __attribute__((amdgpu_waves_per_eu(5)))
kda_cb_prep_kernel(const uint16_t* __restrict__ gq, const uint16_t* __restrict__ gk,
                   const float* __restrict__ galpha, const float* __restrict__ gbeta,
                   char* __restrict__ grec, int T, int H) {
  using RB = BRec<DK>;
  constexpr int NM = DK / 16, LDK = DK + 8, LDT = kSB + 8;
  constexpr int NTH = DK * kPS;
  // K.F and K / F (safe channels) feed only the A and P products; after
  // them the same bytes hold (beta K.F)^T, so that eight workgroups share a CU
  static_assert(kPS == 1, "one sub-chunk per workgroup");
  static_assert(DK * LDT <= 2 * kSB * LDK, "(beta K.F)^T fits where K.F and K / F were");
  __shared__ __attribute__((aligned(16))) uint16_t sKFI[2 * kSB * LDK];
  uint16_t (*sKF)[kSB * LDK] = reinterpret_cast<uint16_t (*)[kSB * LDK]>(sKFI);            // K.F
  uint16_t (*sKI)[kSB * LDK] = reinterpret_cast<uint16_t (*)[kSB * LDK]>(sKFI + kSB * LDK);  // K / F
  uint16_t (*sBK)[DK * LDT] = reinterpret_cast<uint16_t (*)[DK * LDT]>(sKFI);               // (beta K.F)^T
  // Q.F feeds only the P product; after it the same bytes hold K.H
  __shared__ __attribute__((aligned(16))) uint16_t sQF[kPS][kSB * LDK];   // Q.F
  uint16_t (*sKH)[kSB * LDK] = sQF;                                        // K.H
  __shared__ __attribute__((aligned(16))) uint16_t sY[kPS][kSB * LDT];    // Y
  __shared__ float sA[kPS][kSB * 17];
  __shared__ float sBT[kPS][DK];
  __shared__ float sBe[kPS * kSB];
  __shared__ int sFl[kPS];

  const int NS = (T + kSB - 1) / kSB, NP = (NS + kPS - 1) / kPS;
  const int chain = blockIdx.x / NP, cp = blockIdx.x % NP;
  const int b = chain / H, h = chain % H;
  const int t0 = cp * kPS * kSB;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const size_t row0 = static_cast<size_t>(b) * T * H + h;
  auto rec_of = [&](int J) { return grec + (static_cast<size_t>(chain) * NS + cp * kPS + J) * RB::kBytes; };
  auto live = [&](int J) { return t0 + kSB * J < T; };

  if (tid < kPS) sFl[tid] = 0;
  if (tid < kPS * kSB) sBe[tid] = (t0 + tid < T) ? gbeta[row0 + static_cast<size_t>(t0 + tid) * H] : 0.f;
  lds_barrier();

  // ---- gates and gated operands, item (channel c, sub-chunk J); rows past T
  // are identity steps (alpha 1, k = q = 0, beta 0).  The beta K.F row of
  // channel c waits in registers until the A and P products are done.
  static_assert(DK == NTH, "one channel per thread");
  uint32_t bkw[8], khw[8];
  {
    const int c = tid, J = 0;
    float a[kSB], kk[kSB], qq[kSB];
#pragma unroll
    for (int r = 0; r < kSB; ++r) {
      const int t = t0 + kSB * J + r;
      const bool ok = t < T;
      const size_t e = (row0 + static_cast<size_t>(ok ? t : 0) * H) * DK + c;
      // loads from a clamped row, then a select: no branch around a load
      const float av = galpha[e];
      const uint16_t kv = gk[e], qv = gq[e];
      a[r] = ok ? av : 1.f;
      kk[r] = ok ? bf16_to_f32(kv) : 0.f;
      qq[r] = ok ? bf16_to_f32(qv) : 0.f;
    }
    float F[kSB], Hs[kSB];
    F[0] = a[0];
#pragma unroll
    for (int r = 1; r < kSB; ++r) F[r] = F[r - 1] * a[r];
    Hs[kSB - 1] = 1.f;
#pragma unroll
    for (int r = kSB - 2; r >= 0; --r) Hs[r] = Hs[r + 1] * a[r + 1];
    const float bt = F[kSB - 1];
    // 1/F_r <= 1/bt: the reciprocal form is used while bt >= 2^-100
    const bool safe = bt >= kUnsafeBlockDecay;
    if (!safe) atomicOr(&sFl[J], 1);
    sBT[J][c] = bt;
    // 1/F_r = H_r / bt: one reciprocal per channel instead of a division per row
    const float rbt = safe ? 1.f / bt : 0.f;
#pragma unroll
    for (int r = 0; r < kSB; ++r) {
      sKF[J][r * LDK + c] = f32_to_bf16(kk[r] * F[r]);
      sKI[J][r * LDK + c] = f32_to_bf16(kk[r] * Hs[r] * rbt);
      sQF[J][r * LDK + c] = f32_to_bf16(qq[r] * F[r]);
    }
#pragma unroll
    for (int x = 0; x < 8; ++x) khw[x] = pack_bf16x2(kk[2 * x] * Hs[2 * x], kk[2 * x + 1] * Hs[2 * x + 1]);
#pragma unroll
    for (int x = 0; x < 8; ++x)
      bkw[x] = pack_bf16x2(sBe[kSB * J + 2 * x] * kk[2 * x] * F[2 * x],
                           sBe[kSB * J + 2 * x + 1] * kk[2 * x + 1] * F[2 * x + 1]);
    if (live(J)) {
      char* rec = rec_of(J);
      reinterpret_cast<float*>(rec + RB::oG)[c] = bt;
      // (Q.E)^T half of fragment c / 16, lane (g, c % 16): rows 4g .. 4g+3 of
      // Q.F, channel c
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<uint2*>(rec + RB::oQW + ((c / 16) * 64 + g * 16 + c % 16) * 16) =
            make_uint2(pack_bf16x2(qq[4 * g] * F[4 * g], qq[4 * g + 1] * F[4 * g + 1]),
                       pack_bf16x2(qq[4 * g + 2] * F[4 * g + 2], qq[4 * g + 3] * F[4 * g + 3]));
    }
  }
  lds_barrier();

  // ---- A and P of each sub-chunk: wave w -> sub-chunk w / 2, A (even) or P (odd)
  {
    const Lane ln = lane_now();
    const int J = wave >> 1;
    const bool isP = wave & 1;
    const uint16_t* am = isP ? sQF[J] : sKF[J];
    f32x4 acc = zero4();
#pragma unroll
    for (int k0 = 0; k0 < DK; k0 += 32)
      acc = mma32(ld8(am + ln.i * LDK + k0 + 8 * ln.g), ld8(sKI[J] + ln.i * LDK + k0 + 8 * ln.g), acc);
    if (sFl[J]) {
      // channels whose sub-chunk decay fell below 2^-100: exact running
      // products of alpha on the vector units
      const int tb = t0 + kSB * J;
      for (int c = 0; c < DK; ++c) {
        if (sBT[J][c] >= kUnsafeBlockDecay) continue;
        auto in = [&](const uint16_t* src, int row) {
          const int t = tb + row;
          return t < T ? bf16_to_f32(src[(row0 + static_cast<size_t>(t) * H) * DK + c]) : 0.f;
        };
        auto al = [&](int row) {
          const int t = tb + row;
          return t < T ? galpha[(row0 + static_cast<size_t>(t) * H) * DK + c] : 1.f;
        };
        const float ki = in(gk, ln.i);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int rl = 4 * ln.g + rr;
          if (ln.i > rl) continue;
          float ratio = 1.f;
          for (int j = ln.i + 1; j <= rl; ++j) ratio *= al(j);
          acc[rr] += (isP ? in(gq, rl) : in(gk, rl)) * ki * ratio;
        }
      }
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int rl = 4 * ln.g + rr;
      const bool keep = isP ? (ln.i <= rl) : (ln.i < rl);
      acc[rr] = keep ? acc[rr] : 0.f;
    }
    if (!isP) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) sA[J][(4 * ln.g + rr) * 17 + ln.i] = acc[rr];
    } else if (live(J)) {
      // lane (g, i) holds P[4g .. 4g+3][i] = row i of P^T: the P^T fragment
      *reinterpret_cast<bf16x4*>(rec_of(J) + RB::oP + lane * 8) = quad4(acc);
    }
  }
  lds_barrier();
  {
    // K.F and K / F are spent: (beta K.F)^T row c in their place; Q.F is
    // spent: K.H channel c in its place
    uint4* bk = reinterpret_cast<uint4*>(sBK[0] + tid * LDT);
    bk[0] = make_uint4(bkw[0], bkw[1], bkw[2], bkw[3]);
    bk[1] = make_uint4(bkw[4], bkw[5], bkw[6], bkw[7]);
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      sKH[0][(2 * x) * LDK + tid] = static_cast<uint16_t>(khw[x] & 0xffffu);
      sKH[0][(2 * x + 1) * LDK + tid] = static_cast<uint16_t>(khw[x] >> 16);
    }
  }

  // ---- Y = (I + Diag(beta) A)^-1 per sub-chunk by forward substitution:
  // wave J, lane j < 16 owns column j
  if (wave < kPS) {
    const int J = wave;
    if (lane < kSB) {
      const int j = lane;
      float y[kSB], acc[kSB];
#pragma unroll
      for (int r = 0; r < kSB; ++r) acc[r] = 0.f;
#pragma unroll
      for (int m = 0; m < kSB; ++m) {
        y[m] = (m < j) ? 0.f : ((m == j) ? 1.f : -acc[m]);
#pragma unroll
        for (int r = m + 1; r < kSB; ++r) acc[r] += sBe[kSB * J + r] * sA[J][r * 17 + m] * y[m];
      }
#pragma unroll
      for (int r = 0; r < kSB; ++r) sY[J][r * LDT + j] = f32_to_bf16(y[r]);
      if (live(J)) {
        float* yo = reinterpret_cast<float*>(rec_of(J) + RB::oY);
#pragma unroll
        for (int r = 0; r < kSB; ++r) yo[r * kSB + j] = y[r];
      }
    }
    if (live(J)) {
      float* ao = reinterpret_cast<float*>(rec_of(J) + RB::oA);
      for (int x = lane; x < kSB * kSB; x += kWave) ao[x] = sA[J][(x / kSB) * 17 + x % kSB];
    }
  }
  lds_barrier();

  // ---- W = Y (beta K.F): tile (J, channel block R) has lane (g, i) holding
  // W[4g .. 4g+3][16R + i], the -W^T half of fragment R
  for (int t = wave; t < kPS * NM; t += NTH / kWave) {
    const int J = t / NM, R = t % NM;
    if (!live(J)) continue;
    const Lane ln = lane_now();
    const f32x4 acc = mma16(ld4(sY[J] + ln.i * LDT + 4 * ln.g),
                            ld4(sBK[J] + (16 * R + ln.i) * LDT + 4 * ln.g), zero4());
    *reinterpret_cast<bf16x4*>(rec_of(J) + RB::oQW + (R * 64 + lane) * 16 + 8) =
        bf16_quad(-acc[0], -acc[1], -acc[2], -acc[3]);
  }
  // ---- K.E' fragments: lane (g, i) holds row i, channels 32kk + 4g .. +3
  // and 32kk + 16 + 4g .. +3
  constexpr int NK = DK / 32;
  for (int x = tid; x < kPS * NK * 64; x += NTH) {
    const int J = x / (NK * 64), kk = (x / 64) % NK, l = x % 64;
    if (!live(J)) continue;
    const uint16_t* row = sKH[J] + (l % 16) * LDK + 32 * kk + 4 * (l / 16);
    const uint2 lo = *reinterpret_cast<const uint2*>(row), hi = *reinterpret_cast<const uint2*>(row + 16);
    *reinterpret_cast<uint4*>(rec_of(J) + RB::oK + (kk * 64 + l) * 16) = make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
}

// ---------------------------------------------------------------------------
// 3. The state gradient, backwards over the sub-chunks.  One workgroup per
// (chain, NT 16-column tiles): two state waves hold the tiles in registers,
// state wave h the row blocks m of its half of the key channels, lane (g, i)
// holding rows 16m + 4g + r, column i (the product's output layout, which is
// also the layout of the next product's B operand),
//   dS <- Diag(E_last) dS + (Q.E)^T dO - W^T (P^T dO + (K.E') dS),
// each forming the part of P^T dO + (K.E') dS that its rows contribute and
// taking the other's through LDS (a step is bound by instruction issue, so
// halving each wave's products and conversions beats the extra exchange);
// and two loader waves stream each sub-chunk's record and dO tile into a ring
// of LDS slots with direct global-to-LDS loads, kAhead sub-chunks ahead (the
// walk is a chain of short matrix products: without the ring every step
// waited for its own loads; each loader issues half of every slot so that
// kAhead slots fit the 6-bit count of loads a wave can wait on).  One
// barrier per sub-chunk: the exchange of u, after which the next slot has
// landed (the loaders wait for it before they arrive) and the state waves
// read it together with u, so that its latency hides behind the update.
// ---------------------------------------------------------------------------
template <int DK, int NT>
struct ScanRing {
  using RB = BRec<DK>;
  static constexpr int kTiles = NT;                  // 16-column tiles per state wave
  static constexpr int kRec = RB::oG + 4 * DK;       // bytes of a record the walk reads
  static constexpr int kDO = kTiles * 16 * 16 * 2;   // dO tiles, 16 rows x 16 columns bf16 each
  static constexpr int kBuf = kRec + kDO;
  static constexpr int kAhead = NT == 1 ? 7 : 6, kNBuf = kAhead + 1;
  static constexpr int kInsts = kRec / 1024;                       // 16-byte-lane loads of a record
  static constexpr int kSplit = (kInsts + 1) / 2;                  // loader 1: [0, kSplit), loader 2: the rest
  static constexpr int kFill1 = kSplit, kFill2 = kInsts - kSplit + kDO / 256;   // loads per slot
  // every load of kAhead slots fits the wave's 6-bit count of loads in flight,
  // so waiting down to (kAhead - 1) slots means the oldest slot has landed
  static_assert(kRec % 1024 == 0 && kAhead * kFill1 <= 63 && kAhead * kFill2 <= 63, "fill plan");
};

template <int DK, int NT>
__global__ void __launch_bounds__(4 * kWave)
kda_cb_scan_kernel(const char* __restrict__ grec, const uint16_t* __restrict__ gdO,
                   const float* __restrict__ gdST, float* __restrict__ gdSc, float* gdS0, int T,
                   int H, int DV) {
  using RB = BRec<DK>;
  using RG = ScanRing<DK, NT>;
  constexpr int NM = DK / 16, NH = NM / 2;          // row blocks per state wave
  __shared__ __attribute__((aligned(16))) char ring[RG::kNBuf * RG::kBuf];
  __shared__ __attribute__((aligned(16))) float xu[2][2][NT][kWave * 4];   // [step parity][part] of u
  const int NJV = DV / (16 * NT);                    // workgroups per chain
  // Consecutive workgroup IDs are dealt round-robin to the 8 XCDs; the
  // workgroups of one chain read the same records, so they are gathered on
  // one XCD, where the records come from its L2 after the first read.
  int L = blockIdx.x;
  if (NJV > 1 && (gridDim.x % 8) == 0) L = (blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8;
  const int chain = L / NJV, jt0 = NT * (L % NJV);
  const int b = chain / H, h = chain % H;
  const int NS = (T + kSB - 1) / kSB, NC = (T + kCB - 1) / kCB;
  const int lane = threadIdx.x % kWave;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const size_t row0 = static_cast<size_t>(b) * T * H + h;
  auto slot = [&](int n) { return ring + (n % RG::kNBuf) * RG::kBuf; };

  if (wv >= 2) {
    // ---- loaders: order n (= sub-chunk NS - 1 - n) into slot n % kNBuf;
    // loader 1 the first kSplit KiB of the record, loader 2 the rest of it
    // and the dO tiles
    const bool first = wv == 2;
    auto fill = [&](int n) {
      const int s = NS - 1 - n;
      char* dst = slot(n);
      const char* src = grec + (static_cast<size_t>(chain) * NS + s) * RB::kBytes;
      if (first) {
#pragma unroll
        for (int i = 0; i < RG::kSplit; ++i)
          __builtin_amdgcn_global_load_lds((gbl_void*)(src + 1024 * i + 16 * lane),
                                           (lds_void*)(dst + 1024 * i), 16, 0, 0);
      } else {
#pragma unroll
        for (int i = RG::kSplit; i < RG::kInsts; ++i)
          __builtin_amdgcn_global_load_lds((gbl_void*)(src + 1024 * i + 16 * lane),
                                           (lds_void*)(dst + 1024 * i), 16, 0, 0);
#pragma unroll
        for (int p = 0; p < RG::kDO / 256; ++p) {
          const int d = 64 * p + lane;           // dword d: tile d / 128, row (d / 8) % 16, dword d % 8
          const int tt = d / 128;
          const int t = min(kSB * s + (d / 8) % 16, T - 1);
          __builtin_amdgcn_global_load_lds(
              (gbl_void*)(gdO + (row0 + static_cast<size_t>(t) * H) * DV + 16 * (jt0 + tt) + 2 * (d % 8)),
              (lds_void*)(dst + RG::kRec + 256 * p), 4, 0, 0);
        }
      }
    };
    auto wait_oldest = [&] {
      if (first) __builtin_amdgcn_s_waitcnt(vmcnt_only((RG::kAhead - 1) * RG::kFill1));
      else __builtin_amdgcn_s_waitcnt(vmcnt_only((RG::kAhead - 1) * RG::kFill2));
    };
    if (NS > 0) {
#pragma unroll
      for (int i = 0; i < RG::kAhead; ++i) fill(min(i, NS - 1));
      wait_oldest();          // order 0 landed
      barrier_keep_fills();   // slot 0 is ready
    }
    for (int n = 0; n < NS; ++n) {
      // into the slot of order n - 1, whose reads ended before the last barrier
      fill(min(n + RG::kAhead, NS - 1));
      wait_oldest();          // order n + 1 landed
      barrier_keep_fills();   // the exchange of step n; slot n + 1 is ready
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
    return;
  }

  const Lane ln = lane_now();
  const int hh = wv;                                 // this state wave's half
  f32x4 dS[NT][NH];                                  // row blocks m = NH hh + mm
#pragma unroll
  for (int tt = 0; tt < NT; ++tt)
#pragma unroll
    for (int mm = 0; mm < NH; ++mm)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        dS[tt][mm][r] = gdST ? gdST[(static_cast<size_t>(chain) * DK + 16 * (NH * hh + mm) + 4 * ln.g + r) * DV +
                                    16 * (jt0 + tt) + ln.i]
                             : 0.f;
  // a slot's operands, in registers: P^T (the first wave's; the other's is
  // zeroed at use), the dO tiles, this wave's K.E' fragments, rows of
  // [(Q.E)^T | -W^T] and decays
  struct Ops {
    uint2 pw;
    uint32_t d[NT][4];                               // dO halves, packed at use
    bf16x8 kf[NH / 2], qw[NH];
    float4 gc[NH];
  };
  auto read_slot = [&](const char* sb, Ops& o) {
    o.pw = *reinterpret_cast<const uint2*>(sb + RB::oP + lane * 8);
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      const uint16_t* dt = reinterpret_cast<const uint16_t*>(sb + RG::kRec) + 256 * tt;
#pragma unroll
      for (int r = 0; r < 4; ++r) o.d[tt][r] = dt[(4 * ln.g + r) * 16 + ln.i];
    }
#pragma unroll
    for (int k2 = 0; k2 < NH / 2; ++k2)
      o.kf[k2] = *reinterpret_cast<const bf16x8*>(sb + RB::oK + ((NH / 2 * hh + k2) * 64 + lane) * 16);
#pragma unroll
    for (int mm = 0; mm < NH; ++mm) {
      const int m = NH * hh + mm;
      o.qw[mm] = *reinterpret_cast<const bf16x8*>(sb + RB::oQW + (m * 64 + lane) * 16);
      o.gc[mm] = *reinterpret_cast<const float4*>(sb + RB::oG + 4 * (16 * m + 4 * ln.g));
    }
  };
  const uint32_t pmask = hh == 0 ? ~0u : 0u;
  // step n with the operands of slot n in cur; reads slot n + 1 into nxt
  auto step = [&](int n, const Ops& cur, Ops& nxt) {
    const int s = NS - 1 - n;
    if (s == NS - 1 || (s % kNSB) == kNSB - 1) {
      // the gradient at the end of chunk s / 4, for the gradient kernel, in
      // fragment order [chain][chunk][column tile][row block][lane][4]
      float* dst = gdSc + ((static_cast<size_t>(chain) * NC + s / kNSB) * (DV / 16) + jt0) * DK * 16 +
                   4 * lane;
#pragma unroll
      for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int mm = 0; mm < NH; ++mm)
          *reinterpret_cast<float4*>(dst + (tt * NM + NH * hh + mm) * kWave * 4) =
              make_float4(dS[tt][mm][0], dS[tt][mm][1], dS[tt][mm][2], dS[tt][mm][3]);
    }
    // this wave's part of u = P^T dO + (K.E') dS: its row blocks' share
    const bf16x4 pfr = __builtin_bit_cast(bf16x4, make_uint2(cur.pw.x & pmask, cur.pw.y & pmask));
    bf16x4 dob[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
      dob[tt] = __builtin_bit_cast(bf16x4, make_uint2(cur.d[tt][0] | (cur.d[tt][1] << 16),
                                                      cur.d[tt][2] | (cur.d[tt][3] << 16)));
    f32x4 t1[NT][2];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      t1[tt][0] = mma16(pfr, dob[tt], zero4());
      t1[tt][1] = zero4();
    }
#pragma unroll
    for (int k2 = 0; k2 < NH / 2; ++k2)
#pragma unroll
      for (int tt = 0; tt < NT; ++tt)
        t1[tt][k2 % 2] = mma32(cur.kf[k2], cat8(quad4(dS[tt][2 * k2]), quad4(dS[tt][2 * k2 + 1])),
                               t1[tt][k2 % 2]);
    float (*xs)[NT][kWave * 4] = xu[n & 1];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
      *reinterpret_cast<float4*>(&xs[hh][tt][4 * lane]) =
          make_float4(t1[tt][0][0] + t1[tt][1][0], t1[tt][0][1] + t1[tt][1][1],
                      t1[tt][0][2] + t1[tt][1][2], t1[tt][0][3] + t1[tt][1][3]);
    // the part of the update that u does not enter:
    // Diag(E_last) dS + (Q.E)^T dO, the dO half of each 16x16x32 row
#pragma unroll
    for (int mm = 0; mm < NH; ++mm) {
      const uint4 q = __builtin_bit_cast(uint4, cur.qw[mm]);
      const bf16x4 qlo = __builtin_bit_cast(bf16x4, make_uint2(q.x, q.y));
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        f32x4 e;
        e[0] = cur.gc[mm].x * dS[tt][mm][0];
        e[1] = cur.gc[mm].y * dS[tt][mm][1];
        e[2] = cur.gc[mm].z * dS[tt][mm][2];
        e[3] = cur.gc[mm].w * dS[tt][mm][3];
        dS[tt][mm] = mma16(qlo, dob[tt], e);
      }
    }
    bf16x4 qhi[NH];
#pragma unroll
    for (int mm = 0; mm < NH; ++mm) {
      const uint4 q = __builtin_bit_cast(uint4, cur.qw[mm]);
      qhi[mm] = __builtin_bit_cast(bf16x4, make_uint2(q.z, q.w));
    }
    lds_barrier();   // both parts of u written; slot n + 1 is ready; slot n is read
    // u (the two parts summed in the same order in both waves) and the next
    // slot's operands, all issued before the first use
    float4 ua[NT], uc[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      ua[tt] = *reinterpret_cast<const float4*>(&xs[0][tt][4 * lane]);
      uc[tt] = *reinterpret_cast<const float4*>(&xs[1][tt][4 * lane]);
    }
    read_slot(slot(min(n + 1, NS - 1)), nxt);
    asm volatile("" ::: "memory");       // the reads stay here, not sunk to their uses
    __builtin_amdgcn_sched_barrier(0);   // nor moved by the scheduler
    // dS <- (that) - W^T u
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      const bf16x4 uq = bf16_quad(ua[tt].x + uc[tt].x, ua[tt].y + uc[tt].y, ua[tt].z + uc[tt].z,
                                  ua[tt].w + uc[tt].w);
#pragma unroll
      for (int mm = 0; mm < NH; ++mm) dS[tt][mm] = mma16(qhi[mm], uq, dS[tt][mm]);
    }
  };
  Ops oa, ob;
  if (NS > 0) {
    lds_barrier();   // slot 0 is ready
    read_slot(slot(0), oa);
  }
  // two steps per pass, the operand sets alternating (no copies between steps)
  int n = 0;
  for (; n + 1 < NS; n += 2) {
    step(n, oa, ob);
    step(n + 1, ob, oa);
  }
  if (n < NS) step(n, oa, ob);
  if (gdS0) {
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
      for (int mm = 0; mm < NH; ++mm)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          gdS0[(static_cast<size_t>(chain) * DK + 16 * (NH * hh + mm) + 4 * ln.g + r) * DV +
               16 * (jt0 + tt) + ln.i] = dS[tt][mm][r];
  }
}

// ---------------------------------------------------------------------------
// 4. Gradients.  One workgroup of eight waves per (chain, 64-token chunk);
// wave w owns value columns 16w .. 16w+15 of the states (dv = 128).
// ---------------------------------------------------------------------------
template <int DK, int DV>
__global__ void __launch_bounds__(kCbThreads)
kda_cb_grad_kernel(const uint16_t* __restrict__ gq, const uint16_t* __restrict__ gk,
                   const uint16_t* __restrict__ gv, const float* __restrict__ galpha,
                   const float* __restrict__ gbeta, const uint16_t* __restrict__ gdO,
                   const float* __restrict__ gSc, const float* __restrict__ gdSc,
                   const char* __restrict__ grec, bf16x4* __restrict__ gSb,
                   float* __restrict__ gdq, float* __restrict__ gdk, float* __restrict__ gdv,
                   float* __restrict__ gda, float* __restrict__ gdb, float* __restrict__ gsink,
                   int T, int H) {
  using RB = BRec<DK>;
  constexpr int NM = DK / 16;
  constexpr int LDK = DK + 8, LDV = DV + 8, LDT = kSB + 8, LDF = DK + 4;
  static_assert(DV == 16 * (kCbThreads / kWave), "one 16-column tile per wave");
  static_assert(DK * 4 == kCbThreads, "four threads per key channel in the gate phase");
  __shared__ __attribute__((aligned(16))) uint16_t sS[DK * LDV];    // S of the sub-chunk
  __shared__ __attribute__((aligned(16))) uint16_t sdS[DK * LDV];   // dS at its end
  __shared__ __attribute__((aligned(16))) uint16_t sW[kSB * LDK];   // W
  __shared__ __attribute__((aligned(16))) uint16_t sKE[kSB * LDK];  // K.E
  __shared__ __attribute__((aligned(16))) uint16_t sKpT[DK * LDT];  // (K.E')^T
  __shared__ __attribute__((aligned(16))) uint16_t sY[kSB * LDT];
  __shared__ __attribute__((aligned(16))) uint16_t sYT[kSB * LDT];
  __shared__ __attribute__((aligned(16))) uint16_t sdO[kSB * LDV];
  __shared__ __attribute__((aligned(16))) uint16_t sU[kSB * LDV];
  __shared__ __attribute__((aligned(16))) uint16_t sdZ[kSB * LDV];
  __shared__ __attribute__((aligned(16))) uint16_t sQr[kSB * LDK];  // q, k raw
  __shared__ __attribute__((aligned(16))) uint16_t sKr[kSB * LDK];
  __shared__ float sAl[kSB * DK];                                    // alpha
  __shared__ float sOS[kSB * LDF];                                   // dO S^T
  __shared__ float sZS[kSB * LDF];                                   // dZ S^T
  __shared__ float sUS[kSB * LDF];                                   // U dS^T
  constexpr int LDP = kSB + 4;                                      // 16-byte rows
  __shared__ __attribute__((aligned(16))) float sdP[kSB * LDP];     // dP, dA and transposes
  __shared__ __attribute__((aligned(16))) float sdA[kSB * LDP];
  __shared__ __attribute__((aligned(16))) float sdPT[kSB * LDP];
  __shared__ __attribute__((aligned(16))) float sdAT[kSB * LDP];
  __shared__ float sPC[DK];
  // the whole sub-chunk record for the backward pass, [(Q.E)^T | -W^T],
  // K.E', P^T, decay, Y, A: loaded once per sub-chunk, read by every wave
  constexpr int kRecB = RB::kBytes - RB::oQW;
  static_assert(RB::oQW == 0 && kRecB % 1024 == 0, "record in 1 KiB pieces");
  __shared__ __attribute__((aligned(16))) char sRec[kRecB];
  __shared__ float sFin[DK];                                          // sum_j dS[c][j] S[c][j]
  __shared__ float sDb1[kCbThreads / kWave][kSB];
  __shared__ float sDb2[kSB];
  __shared__ float sBe[kCB];

  const int NC = (T + kCB - 1) / kCB, NS = (T + kSB - 1) / kSB;
  const int chain = blockIdx.x / NC, cc = blockIdx.x % NC;
  const int b = chain / H, h = chain % H;
  const int t0 = cc * kCB;
  const int ns = min(kNSB, (T - t0 + kSB - 1) / kSB);
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int jt = wave;
  const size_t row0 = static_cast<size_t>(b) * T * H + h;
  auto rec_of = [&](int J) {
    return grec + (static_cast<size_t>(chain) * NS + cc * kNSB + J) * RB::kBytes;
  };
  auto trow = [&](int t) { return row0 + static_cast<size_t>(t) * H; };

  if (tid < kCB) sBe[tid] = (t0 + tid < T) ? gbeta[trow(t0 + tid)] : 0.f;

  // state tile of this wave: rows 16m + 4g + r, column 16 jt + i
  // (chunk states and state gradients in fragment order: [chain][chunk]
  // [column tile][row block][lane][4], one 16-byte access per block)
  const size_t fbase = ((static_cast<size_t>(chain) * NC + cc) * (DV / 16) + jt) * DK * 16 + 4 * lane;
  f32x4 Sw[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const float4 v = *reinterpret_cast<const float4*>(gSc + fbase + m * kWave * 4);
    Sw[m][0] = v.x; Sw[m][1] = v.y; Sw[m][2] = v.z; Sw[m][3] = v.w;
  }
  // S of each sub-chunk (operand type) waits in the workspace between the
  // two passes (registers cannot hold them next to the gate phase), the
  // first one too, so that the backward pass loads every sub-chunk's S the
  // same way: [chain][chunk][sub-chunk][wave][m][lane]
  // (two row blocks m per 16-byte element: [..][wave][m / 2][lane])
  uint4* sbw = reinterpret_cast<uint4*>(gSb) +
               ((static_cast<size_t>(chain) * NC + cc) * kNSB * (kCbThreads / kWave) + wave) *
                   (NM / 2) * kWave + lane;
  auto sb_slot = [&](int J, int mp) {
    return sbw + (static_cast<size_t>(J) * (kCbThreads / kWave) * (NM / 2) + mp) * kWave;
  };
  // U of each sub-chunk (this wave's columns), after them: [chain][chunk][J][wave][lane]
  bf16x4* ubw = gSb + static_cast<size_t>(gridDim.x) * kNSB * (kCbThreads / kWave) * NM * kWave +
                ((static_cast<size_t>(chain) * NC + cc) * kNSB * (kCbThreads / kWave) + wave) * kWave + lane;
  auto ub_slot = [&](int J) { return ubw + static_cast<size_t>(J) * (kCbThreads / kWave) * kWave; };

  // ======== forward over the sub-chunks: S_J and U_J.  Each sub-chunk's
  // record pieces and value rows are loaded one sub-chunk ahead.
  static_assert(NM * 64 == kCbThreads && (DK / 32) * 64 <= kCbThreads, "one fragment lane per thread");
  struct FwdIn {
    uint2 wv;          // the -W^T half of one fragment lane
    uint4 kv;          // one K.E' fragment lane (threads below DK / 32 * 64)
    float y, pc;       // Y[tid], decay[tid]
    uint16_t v[4];     // V of this wave's column tile, rows 4g .. 4g+3
  };
  auto fetch_fwd = [&](int J, FwdIn& f) {
    const char* rec = rec_of(J);
    const int R = tid / 64, l = tid % 64;
    f.wv = *reinterpret_cast<const uint2*>(rec + RB::oQW + (R * 64 + l) * 16 + 8);
    // every load unconditional (indices wrap into range; the lanes past a
    // table's end load a repeat and never use it), and rows past T are
    // zeroed where they are used, so that nothing waits for these loads
    // before the next sub-chunk
    f.kv = *reinterpret_cast<const uint4*>(rec + RB::oK + (tid % ((DK / 32) * 64)) * 16);
    f.y = reinterpret_cast<const float*>(rec + RB::oY)[tid % (kSB * kSB)];
    f.pc = reinterpret_cast<const float*>(rec + RB::oG)[tid % DK];
    const Lane ln = lane_now();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + kSB * J + 4 * ln.g + r;
      f.v[r] = gv[trow(min(t, T - 1)) * DV + 16 * jt + ln.i];
    }
  };
  FwdIn fin_cur;
  fetch_fwd(0, fin_cur);
  // The backward pass's first loads (the state gradient at the chunk's end
  // and the last sub-chunk's rows) are issued here, next to the forward
  // pass's first ones, so that both wait for memory once.
  f32x4 dS[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const float4 v = *reinterpret_cast<const float4*>(gdSc + fbase + m * kWave * 4);
    dS[m][0] = v.x; dS[m][1] = v.y; dS[m][2] = v.z; dS[m][3] = v.w;
  }
  // gate phase: key channel, quarter of the rows (wave-uniform: DK is a
  // multiple of the wave size)
  const int c = tid % DK, part = __builtin_amdgcn_readfirstlane(tid / DK);
  // raw alpha, k, q of a sub-chunk, loaded one sub-chunk ahead: thread
  // (row rr, channel quad cq) holds channels 4cq .. 4cq+3 of row rr, so a row
  // piece is one 16-byte and two 8-byte loads
  static_assert(kSB * DK / 4 == kCbThreads, "one channel quad of one row per thread");
  const int rr = tid / (DK / 4), cq = 4 * (tid % (DK / 4));
  float4 na;
  uint2 nk, nq;
  auto fetch_rows = [&](int J) {
    // raw loads from a clamped row; a row past T is fixed up where it is
    // used (a select here would wait for the load)
    const int t = t0 + kSB * J + rr;
    const size_t e = trow(min(t, T - 1)) * DK + cq;
    na = *reinterpret_cast<const float4*>(galpha + e);
    nk = *reinterpret_cast<const uint2*>(gk + e);
    nq = *reinterpret_cast<const uint2*>(gq + e);
  };
  fetch_rows(ns - 1);
#pragma nounroll
  for (int J = 0; J < ns; ++J) {
    const FwdIn cur = fin_cur;
    if (J + 1 < ns) fetch_fwd(J + 1, fin_cur);
    // W (from its W^T fragments), (K.E')^T (from the K.E' fragments), Y
    {
      const int R = tid / 64, l = tid % 64;
      const int g = l / 16, i = l % 16;
      // -W, negated back (sign bit): W[4g+x][16R+i]
      const uint32_t wh[2] = {cur.wv.x ^ 0x80008000u, cur.wv.y ^ 0x80008000u};
      // K.E' lane (g, i) of fragment kk = R: row i, channels 32R+4g+x and 32R+16+4g+x
      const uint32_t kh[4] = {cur.kv.x, cur.kv.y, cur.kv.z, cur.kv.w};
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        sW[(4 * g + x) * LDK + 16 * R + i] = static_cast<uint16_t>(wh[x / 2] >> (16 * (x % 2)));
        if (R < DK / 32) {
          sKpT[(32 * R + 4 * g + x) * LDT + i] = static_cast<uint16_t>(kh[x / 2] >> (16 * (x % 2)));
          sKpT[(32 * R + 16 + 4 * g + x) * LDT + i] =
              static_cast<uint16_t>(kh[2 + x / 2] >> (16 * (x % 2)));
        }
      }
      if (tid < kSB * kSB) {
        sY[(tid / kSB) * LDT + tid % kSB] = f32_to_bf16(cur.y);
        sYT[(tid % kSB) * LDT + tid / kSB] = f32_to_bf16(cur.y);
      }
      if (tid < DK) sPC[tid] = cur.pc;
    }
    lds_barrier();
    {
      const Lane ln = lane_now();
      // U~ = Y (beta V)
      uint16_t vb[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // beta is zero past T, so is its product with the repeated row
        vb[r] = f32_to_bf16(sBe[kSB * J + 4 * ln.g + r] * bf16_to_f32(cur.v[r]));
      }
      f32x4 u = mma16(ld4(sY + ln.i * LDT + 4 * ln.g), bits4(vb[0], vb[1], vb[2], vb[3]), zero4());
      // U = U~ - W S
      f32x4 ws = zero4();
      uint2 sbp = make_uint2(0u, 0u);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const bf16x4 sb = quad4(Sw[m]);
        const uint2 sw = __builtin_bit_cast(uint2, sb);
        if (m % 2 == 0) sbp = sw;
        else *sb_slot(J, m / 2) = make_uint4(sbp.x, sbp.y, sw.x, sw.y);
        ws = mma16(ld4(sW + ln.i * LDK + 16 * m + 4 * ln.g), sb, ws);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) u[r] -= ws[r];
      const bf16x4 ub = quad4(u);
      *ub_slot(J) = ub;
      // S <- Diag(E_last) S + (K.E')^T U
      if (J + 1 < ns) {
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          const f32x4 x = mma16(ld4(sKpT + (16 * m + ln.i) * LDT + 4 * ln.g), ub, zero4());
          const float4 gc = *reinterpret_cast<const float4*>(sPC + 16 * m + 4 * ln.g);
          Sw[m][0] = gc.x * Sw[m][0] + x[0];
          Sw[m][1] = gc.y * Sw[m][1] + x[1];
          Sw[m][2] = gc.z * Sw[m][2] + x[2];
          Sw[m][3] = gc.w * Sw[m][3] + x[3];
        }
      }
    }
    lds_barrier();
  }

  // ======== backward over the sub-chunks
  // The gate phase leaves its results in LDS (the sS area, unused from the
  // contractions to the next column write): slot x of thread tid at
  // res[x * kCbThreads + tid], dalpha of rows 8 part + x (quarters 0, 1),
  // dq and dk of rows 8 (part - 2) + x in slots 2x, 2x + 1 (quarters 2, 3),
  // dbeta of row tid in slot 8 (threads below 16).  They go to memory at the
  // top of the next sub-chunk (after the barrier that ends this one), before
  // its row prefetch: thread (row rr, channel quad cq) stores 16 bytes of
  // each of dalpha, dq and dk of its row and one dbeta, the same four stores
  // in every thread and on every path (a row past T, and dbeta past the 16
  // rows, goes to a dump slot), so that the compiler knows how many stores
  // follow each load and never waits for a store to wait for a load.
  float* const res = reinterpret_cast<float*>(sS);
  static_assert(16 * kCbThreads * sizeof(float) <= sizeof(sS), "result slots");
  float* const dump = gsink + 4 * lane;
  auto flush = [&](int Jp, bool valid) {
    const int tbp = t0 + kSB * Jp, t = tbp + rr, x = rr % 8, hq = rr / 8;
    const bool ok = valid && t < T;
    const size_t e = trow(min(t, T - 1)) * DK + cq;
    const float4 va = *reinterpret_cast<const float4*>(res + x * kCbThreads + hq * DK + cq);
    const float4 vq = *reinterpret_cast<const float4*>(res + 2 * x * kCbThreads + (2 + hq) * DK + cq);
    const float4 vk = *reinterpret_cast<const float4*>(res + (2 * x + 1) * kCbThreads + (2 + hq) * DK + cq);
    const int rb = min(tid, kSB - 1);
    const float vb = res[8 * kCbThreads + rb];
    *reinterpret_cast<float4*>(ok ? gda + e : dump) = va;
    *reinterpret_cast<float4*>(ok ? gdq + e : dump) = vq;
    *reinterpret_cast<float4*>(ok ? gdk + e : dump) = vk;
    *(valid && tid < kSB && tbp + rb < T ? gdb + trow(min(tbp + rb, T - 1)) : dump) = vb;
  };
  // Per-wave loads of a sub-chunk (in the order they are needed): Y, the dO
  // and V rows of this wave's columns, U and S of the sub-chunk, and two
  // 16-byte pieces of the record's fragments and decay (every thread loads
  // pieces tid and kCbThreads + min(tid, ..), the threads past the end
  // repeating the last piece: the same bytes to the same place; stored to
  // LDS at the column write, one copy for every wave).  Issued at the end of
  // the sub-chunk before, after its gate phase, so that they land while it
  // finishes; rows past T load a repeat of row T - 1, zeroed at use.
  static_assert(kRecB / 16 > kCbThreads && kRecB / 16 <= 2 * kCbThreads, "two pieces per thread");
  const int rq1 = kCbThreads + min(tid, kRecB / 16 - kCbThreads - 1);
  struct WaveIn {
    float ypre;
    uint16_t dov[4], vv[4];
    bf16x4 uj;
    uint4 sb[NM / 2];
    uint4 rp0, rp1;
  };
  auto load_wave = [&](int J, WaveIn& w) {
    const char* rec = rec_of(J);
    const int tb = t0 + kSB * J;
    const Lane ln = lane_now();
    w.ypre = reinterpret_cast<const float*>(rec + RB::oY)[tid % (kSB * kSB)];
#pragma unroll
    for (int r = 0; r < 4; ++r) w.dov[r] = gdO[trow(min(tb + 4 * ln.g + r, T - 1)) * DV + 16 * jt + ln.i];
#pragma unroll
    for (int r = 0; r < 4; ++r) w.vv[r] = gv[trow(min(tb + 4 * ln.g + r, T - 1)) * DV + 16 * jt + ln.i];
    w.uj = *ub_slot(J);
#pragma unroll
    for (int mp = 0; mp < NM / 2; ++mp) w.sb[mp] = *sb_slot(J, mp);
    w.rp0 = *reinterpret_cast<const uint4*>(rec + RB::oQW + 16 * tid);
    w.rp1 = *reinterpret_cast<const uint4*>(rec + RB::oQW + 16 * rq1);
  };
  WaveIn wnext;
  load_wave(ns - 1, wnext);
#pragma nounroll
  for (int J = ns - 1; J >= 0; --J) {
    const char* rec = rec_of(J);
    const int tb = t0 + kSB * J;
    // this sub-chunk's per-wave loads, issued at the end of the last one
    const WaveIn win = wnext;
    const float ypre = win.ypre;
    uint16_t dov[4], vv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      dov[r] = win.dov[r];
      vv[r] = win.vv[r];
    }
    const bf16x4 uj = win.uj;
    bf16x4 Sj[NM];   // S of this sub-chunk, this wave's columns
#pragma unroll
    for (int mp = 0; mp < NM / 2; ++mp) {
      Sj[2 * mp] = __builtin_bit_cast(bf16x4, make_uint2(win.sb[mp].x, win.sb[mp].y));
      Sj[2 * mp + 1] = __builtin_bit_cast(bf16x4, make_uint2(win.sb[mp].z, win.sb[mp].w));
    }
    const uint4 rp0 = win.rp0, rp1 = win.rp1;
    // ---- stage: raw q, k, alpha of the sub-chunk; K.E and (K.E)^T; Y^T; decay
    {
      // this sub-chunk's rows, prefetched during the last one (read only
      // now, after this sub-chunk's loads have been issued); a row past T
      // is alpha = 1, k = q = 0
      {
        const bool ok = tb + rr < T;
        *reinterpret_cast<float4*>(sAl + rr * DK + cq) = ok ? na : make_float4(1.f, 1.f, 1.f, 1.f);
        *reinterpret_cast<uint2*>(sKr + rr * LDK + cq) = ok ? nk : make_uint2(0u, 0u);
        *reinterpret_cast<uint2*>(sQr + rr * LDK + cq) = ok ? nq : make_uint2(0u, 0u);
      }
      // the last sub-chunk's results (none yet before the first: the same
      // stores, to the dump), then the next prefetch
      flush(J + 1, J + 1 < ns);
      // unconditional (the last sub-chunk re-fetches its own rows) so that the
      // memory-operation count is the same on every path and later waits can
      // leave these loads in flight
      fetch_rows(J > 0 ? J - 1 : 0);
      lds_barrier();
      // F_r = prod of alpha through r within the sub-chunk
      float F = 1.f;
#pragma unroll
      for (int r = 0; r < 4 * part; ++r) F *= sAl[r * DK + c];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int r = 4 * part + x;
        F *= sAl[r * DK + c];
        sKE[r * LDK + c] = f32_to_bf16(bf16_to_f32(sKr[r * LDK + c]) * F);
      }
    }
    // ---- this wave's column tile: S, dS, dO, U into LDS (operand type);
    // Y^T and the decay (used from the column phase on, so the staging above
    // does not wait for this sub-chunk's loads)
    {
      if (tid < kSB * kSB) sYT[(tid % kSB) * LDT + tid / kSB] = f32_to_bf16(ypre);
      const Lane ln = lane_now();
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const bf16x4 dsb = quad4(dS[m]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * m + 4 * ln.g + r;
          sS[row * LDV + 16 * jt + ln.i] = half16(Sj[m], r);
          sdS[row * LDV + 16 * jt + ln.i] = half16(dsb, r);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = tb + 4 * ln.g + r;
        sdO[(4 * ln.g + r) * LDV + 16 * jt + ln.i] = t < T ? dov[r] : 0;
        sU[(4 * ln.g + r) * LDV + 16 * jt + ln.i] = half16(uj, r);
      }
    }
    // (the last pass's reads of sRec ended before the barrier that closed it)
    *reinterpret_cast<uint4*>(sRec + 16 * tid) = rp0;
    *reinterpret_cast<uint4*>(sRec + 16 * rq1) = rp1;
    lds_barrier();
    // dO of this wave's column tile as a B operand (rows 4g .. 4g+3, column i),
    // read back from LDS; sdO holds it until the next sub-chunk
    auto dO_operand = [&] {
      const Lane ln = lane_now();
      const uint16_t* col = sdO + 16 * jt + ln.i;
      return bits4(col[(4 * ln.g) * LDV], col[(4 * ln.g + 1) * LDV], col[(4 * ln.g + 2) * LDV],
                   col[(4 * ln.g + 3) * LDV]);
    };
    const bf16x4 dob = dO_operand();
    // ---- per column tile: dU, dZ, dv, X, the dbeta and fin partial sums
    f32x4 du;
    {
      const Lane ln = lane_now();
      du = mma16(*reinterpret_cast<const bf16x4*>(sRec + RB::oP + lane * 8), dob, zero4());
#pragma unroll
      for (int m = 0; m < NM / 2; ++m)
        du = mma32(*reinterpret_cast<const bf16x8*>(sRec + RB::oK + (m * 64 + lane) * 16),
                   cat8(quad4(dS[2 * m]), quad4(dS[2 * m + 1])), du);
      const f32x4 dZ = mma16(ld4(sYT + ln.i * LDT + 4 * ln.g), quad4(du), zero4());
      f32x4 ks = zero4();
#pragma unroll
      for (int m = 0; m < NM; ++m) ks = mma16(ld4(sKE + ln.i * LDK + 16 * m + 4 * ln.g), Sj[m], ks);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * ln.g + r, t = tb + row;
        const float v = t < T ? bf16_to_f32(vv[r]) : 0.f;
        const float x = v - ks[r];
        // unconditional (a row past T to the dump slot): a known store count
        *(t < T ? gdv + trow(min(t, T - 1)) * DV + 16 * jt + ln.i : dump) = sBe[kSB * J + row] * dZ[r];
        const float db = row16_sum(dZ[r] * x);
        if (ln.i == 0) sDb1[wave][row] = db;
        sdZ[row * LDV + 16 * jt + ln.i] = f32_to_bf16(dZ[r]);
      }
    }
    lds_barrier();
    // ---- contractions over the value columns: dO S^T, dZ S^T, U dS^T (tile
    // = channel block `wave`), dP and dA (waves 0 and 1)
    {
      const Lane ln = lane_now();
      f32x4 os = zero4(), zs = zero4(), us = zero4(), fd = zero4();
#pragma unroll
      for (int k0 = 0; k0 < DV; k0 += 32) {
        const bf16x8 sb = ld8(sS + (16 * wave + ln.i) * LDV + k0 + 8 * ln.g);
        const bf16x8 db = ld8(sdS + (16 * wave + ln.i) * LDV + k0 + 8 * ln.g);
        os = mma32(ld8(sdO + ln.i * LDV + k0 + 8 * ln.g), sb, os);
        zs = mma32(ld8(sdZ + ln.i * LDV + k0 + 8 * ln.g), sb, zs);
        us = mma32(ld8(sU + ln.i * LDV + k0 + 8 * ln.g), db, us);
        fd = mma32(db, sb, fd);   // dS S^T over the block's channels
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * ln.g + r;
        sOS[row * LDF + 16 * wave + ln.i] = os[r];
        sZS[row * LDF + 16 * wave + ln.i] = zs[r];
        sUS[row * LDF + 16 * wave + ln.i] = us[r];
        if (row == ln.i) sFin[16 * wave + ln.i] = fd[r];   // its diagonal
      }
      if (wave < 2) {
        f32x4 pp = zero4();
        const uint16_t* am = wave == 0 ? sdO : sdZ;
#pragma unroll
        for (int k0 = 0; k0 < DV; k0 += 32)
          pp = mma32(ld8(am + ln.i * LDV + k0 + 8 * ln.g), ld8(sU + ln.i * LDV + k0 + 8 * ln.g), pp);
        const float* Af = reinterpret_cast<const float*>(sRec + RB::oA);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 4 * ln.g + r;
          if (wave == 0) {
            const float dp = ln.i <= row ? pp[r] : 0.f;
            sdP[row * LDP + ln.i] = dp;
            sdPT[ln.i * LDP + row] = dp;
          } else {
            const float dl = ln.i < row ? -pp[r] : 0.f;
            sdA[row * LDP + ln.i] = sBe[kSB * J + row] * dl;
            sdAT[ln.i * LDP + row] = sBe[kSB * J + row] * dl;
            const float s2 = row16_sum(dl * Af[row * kSB + ln.i]);
            if (ln.i == 0) sDb2[row] = s2;
          }
        }
      }
    }
    lds_barrier();
    // ---- gate phase: thread (channel c, quarter `part`); exact running
    // products of alpha over the 16 rows of channel c (row values in
    // registers).  Quarters 0 and 1: dalpha for t < 8 and t >= 8; quarters 2
    // and 3: dq and dk for rows 0..7 and 8..15.
    {
      float a[kSB], kq[kSB], qq[kSB];
#pragma unroll
      for (int r = 0; r < kSB; ++r) {
        a[r] = sAl[r * DK + c];
        kq[r] = bf16_to_f32(sKr[r * LDK + c]);
        qq[r] = bf16_to_f32(sQr[r * LDK + c]);
      }
      if (part < 2) {
        // dalpha_t with alpha_t's own factor left out, t ascending:
        //   dalpha_t = F_{t-1} R_t + H_t colp_t + F_{t-1} H_t fin + pair_t,
        // R_t = sum_{r>=t} rho_r Gam(r, t), H_t = Gam(15, t) (backward
        // recurrences), colp_t = sum_{i<t} k_i (U dS^T)_i Gam(t-1, i), and
        //   pair_t = sum_{r>=t} Gam(r, t) v_r(t),
        //   v_r(t) = sum_{i<t} k_i (q_r dP_ri + k_r dA_ri) Gam(t-1, i),
        // v advanced with t (v_r(t+1) = alpha_t v_r(t) + k_t (q_r dP_rt + k_r dA_rt))
        // and pair_t summed by Horner's rule from r = 15 down
        const float fin = sFin[c];
        float R[kSB], Hh[kSB], v[kSB];
        {
          float rn = 0.f, hn = 1.f;
#pragma unroll
          for (int r = kSB - 1; r >= 0; --r) {
            const float rho = qq[r] * sOS[r * LDF + c] - sBe[kSB * J + r] * kq[r] * sZS[r * LDF + c];
            rn = r == kSB - 1 ? rho : fmaf(a[r + 1], rn, rho);
            if (r < kSB - 1) hn *= a[r + 1];
            R[r] = rn;
            Hh[r] = hn;
            v[r] = 0.f;
          }
        }
        // quarter 0: t = 0..7; quarter 1: t = 8..15, which needs v only for
        // rows r >= 8 (its recurrence still starts at t = 0)
        auto dalpha = [&](auto lo_c) {
          constexpr int tlo = decltype(lo_c)::value, thi = tlo + 8;
          float Fm = 1.f, colp = 0.f;     // F_{t-1}; colp_t
          static_for<0, thi>([&](auto t_c) {
            constexpr int t = decltype(t_c)::value;
            if constexpr (t >= tlo) {
              float pr = v[kSB - 1];
#pragma unroll
              for (int r = kSB - 2; r >= t; --r) pr = fmaf(a[r + 1], pr, v[r]);
              res[(t - tlo) * kCbThreads + tid] = Fm * R[t] + Hh[t] * colp + Fm * Hh[t] * fin + pr;
            }
            if constexpr (t + 1 < thi) {
              // column t of dP and dA, rows r > t (and r >= tlo)
              constexpr int rlo = (t + 1 > tlo ? t + 1 : tlo);
#pragma unroll
              for (int q4 = rlo / 4; q4 < kSB / 4; ++q4) {
                const float4 p4 = *reinterpret_cast<const float4*>(sdPT + t * LDP + 4 * q4);
                const float4 a4 = *reinterpret_cast<const float4*>(sdAT + t * LDP + 4 * q4);
                const float pv[4] = {p4.x, p4.y, p4.z, p4.w}, av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const int r = 4 * q4 + e;
                  if (r >= rlo) v[r] = fmaf(a[t], v[r], kq[t] * fmaf(qq[r], pv[e], kq[r] * av[e]));
                }
              }
              colp = a[t] * colp + kq[t] * sUS[t * LDF + c];
              Fm *= a[t];
            }
          });
        };
        if (part == 0) dalpha(std::integral_constant<int, 0>{});
        else dalpha(std::integral_constant<int, 8>{});
      } else {
        float F[kSB], Hs[kSB];
        F[0] = a[0];
#pragma unroll
        for (int r = 1; r < kSB; ++r) F[r] = F[r - 1] * a[r];
        Hs[kSB - 1] = 1.f;
#pragma unroll
        for (int r = kSB - 2; r >= 0; --r) Hs[r] = Hs[r + 1] * a[r + 1];
        const int xlo = 8 * (part - 2);
#pragma unroll
        for (int x = 0; x < kSB; ++x) {
          if (x < xlo || x >= xlo + 8) continue;
          // row x and column x of dP, dA (an offset the compiler cannot see
          // through keeps each row's loads next to their use; its low bits
          // are clear, so the loads stay 16 bytes wide)
          int z = 0;
          asm volatile("" : "+v"(z));
          z &= ~3;
          // G1, G2 over i <= x with Gam(x, i), from row x of dP and dA, by
          // Horner's rule from i = 0 up
          float g1 = 0.f, g2 = 0.f;
#pragma unroll
          for (int q4 = 0; q4 <= x / 4; ++q4) {
            const float4 p4 = *reinterpret_cast<const float4*>(sdP + z + x * LDP + 4 * q4);
            const float4 a4 = *reinterpret_cast<const float4*>(sdA + z + x * LDP + 4 * q4);
            const float pv[4] = {p4.x, p4.y, p4.z, p4.w}, av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int i = 4 * q4 + e;
              if (i <= x) {
                g1 = i == 0 ? pv[e] * kq[i] : fmaf(a[i], g1, pv[e] * kq[i]);
                g2 = i == 0 ? av[e] * kq[i] : fmaf(a[i], g2, av[e] * kq[i]);
              }
            }
          }
          // G3 over r >= x with Gam(r, x), from column x, by Horner's rule
          // from r = 15 down
          float g3 = 0.f;
#pragma unroll
          for (int q4 = kSB / 4 - 1; q4 >= x / 4; --q4) {
            const float4 p4 = *reinterpret_cast<const float4*>(sdPT + z + x * LDP + 4 * q4);
            const float4 a4 = *reinterpret_cast<const float4*>(sdAT + z + x * LDP + 4 * q4);
            const float pv[4] = {p4.x, p4.y, p4.z, p4.w}, av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
            for (int e = 3; e >= 0; --e) {
              const int r = 4 * q4 + e;
              if (r >= x) {
                const float y = fmaf(pv[e], qq[r], av[e] * kq[r]);
                g3 = r == kSB - 1 ? y : fmaf(a[r + 1], g3, y);
              }
            }
          }
          res[2 * (x % 8) * kCbThreads + tid] = F[x] * sOS[x * LDF + c] + g1;
          res[(2 * (x % 8) + 1) * kCbThreads + tid] =
              -sBe[kSB * J + x] * F[x] * sZS[x * LDF + c] + g2 + g3 + Hs[x] * sUS[x * LDF + c];
        }
      }
      if (tid < kSB) {
        float db = sDb2[tid];
#pragma unroll
        for (int w = 0; w < kCbThreads / kWave; ++w) db += sDb1[w][tid];
        res[8 * kCbThreads + tid] = db;
      }
    }
    // the next sub-chunk's per-wave loads (unconditional: the first
    // sub-chunk reloads its own)
    load_wave(J > 0 ? J - 1 : 0, wnext);
    // ---- dS <- Diag(E_last) dS + (Q.E)^T dO - W^T dU   (W^T dU = (K.E)^T Diag(beta) dZ)
    {
      const Lane ln = lane_now();
      const bf16x8 du8 = cat8(dO_operand(), quad4(du));
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const f32x4 aq = mma32(*reinterpret_cast<const bf16x8*>(sRec + RB::oQW + (m * 64 + lane) * 16), du8,
                               zero4());
        const float4 gc = *reinterpret_cast<const float4*>(sRec + RB::oG + 4 * (16 * m + 4 * ln.g));
        dS[m][0] = gc.x * dS[m][0] + aq[0];
        dS[m][1] = gc.y * dS[m][1] + aq[1];
        dS[m][2] = gc.z * dS[m][2] + aq[2];
        dS[m][3] = gc.w * dS[m][3] + aq[3];
      }
    }
    lds_barrier();
  }
  flush(0, true);
}

// A second stream per device, with the events of a fork and a join: the
// forward half (chunk states) and the record kernel's half (state gradients)
// of the backward share no data until the gradient kernel, and when the
// state-gradient scan fills at most half of the chip the forward runs beside
// it.  Created on first use with the device current and kept until the
// process ends; default priority.  The mutex makes each call's fork and join
// one unit against other host threads (the events are reused).
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxSideDevices = 64;
SideStream g_side[kMaxSideDevices];
std::mutex g_side_mu;

// The current device's side stream; the caller holds g_side_mu.
hipError_t side_stream(SideStream** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxSideDevices) return hipErrorInvalidDevice;
  SideStream& ss = g_side[dev];
  if (ss.s == nullptr) {
    hipStream_t st = nullptr;
    hipEvent_t a = nullptr, b = nullptr;
    if ((e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&a, hipEventDisableTiming)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&b, hipEventDisableTiming)) != hipSuccess) return e;
    ss.fork = a;
    ss.join = b;
    ss.s = st;
  }
  *out = &ss;
  return hipSuccess;
}

}  // namespace

size_t prefill_backward_chunked_workspace(int B, int T, int H, int dk, int dv) {
  if (dk != 128 || dv != 128) return 0;
  const size_t chains = static_cast<size_t>(B) * H;
  const size_t nc = (static_cast<size_t>(T) + kCB - 1) / kCB;
  const size_t ns = (static_cast<size_t>(T) + kSB - 1) / kSB;
  const size_t fwd = prefill_workspace(B, T, H, dk, dv, kCB, true, 0, true);
  const size_t states = chains * nc * dk * dv * sizeof(float);
  const size_t recs = chains * ns * BRec<128>::kBytes;
  const size_t sub_states = chains * nc * kNSB * dk * dv * 2;   // bf16
  const size_t sub_u = chains * nc * kNSB * kSB * dv * 2;            // bf16
  return fwd + 2 * states + recs + sub_states + sub_u;
}

hipError_t launch_prefill_backward_chunked(const PrefillBwdArgs& a) {
  if (!a.bf16 || a.dk != 128 || a.dv != 128 || a.gate_in != kGateAlpha) return hipErrorInvalidValue;
  const hipStream_t stream = static_cast<hipStream_t>(a.stream);
  const size_t chains = static_cast<size_t>(a.B) * a.H;
  const int NC = (a.T + kCB - 1) / kCB;
  const size_t fwd = prefill_workspace(a.B, a.T, a.H, a.dk, a.dv, kCB, true, 0, true);
  char* ws = static_cast<char*>(a.workspace);
  float* Sc = reinterpret_cast<float*>(ws + fwd);
  float* dSc = Sc + chains * NC * a.dk * a.dv;
  char* recs = reinterpret_cast<char*>(dSc + chains * NC * a.dk * a.dv);
  bf16x4* sbs = reinterpret_cast<bf16x4*>(recs + chains * ((a.T + kSB - 1) / kSB) * BRec<128>::kBytes);
  hipError_t e = hipSuccess;
  // the record kernel (sub-chunk records of the state-gradient scan)
  auto records = [&](hipStream_t st) {
    const unsigned pblocks =
        static_cast<unsigned>(chains * (((a.T + kSB - 1) / kSB + kPS - 1) / kPS));
    kda_cb_prep_kernel<128><<<pblocks, 128 * kPS, 0, st>>>(
        static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k), a.alpha, a.beta,
        recs, a.T, a.H);
    return hipGetLastError();
  };
  // the forward, chunk states only (no output): the split path for few
  // chains, the fused kernel for many (the prefill's own choice)
  auto forward = [&]() {
    PrefillArgs f{a.q, a.k, a.v, a.alpha, a.beta, a.S0, nullptr, nullptr, a.B, a.T, a.H, a.dk, a.dv,
                  kCB, true, a.stream, ws, fwd, kGateAlpha, kQkAsGiven};
    f.chunk_states = Sc;
    return launch_prefill(f);
  };
  // two column tiles per state wave once one tile per workgroup would fill
  // the chip (a state wave is issue-bound: two tiles share its fragment reads
  // but lengthen its step)
  const bool two = chains * (a.dv / 16) >= 256;
  auto state_grad = [&](hipStream_t st) {
    if (two)
      kda_cb_scan_kernel<128, 2><<<static_cast<unsigned>(chains * (a.dv / 32)), 4 * kWave, 0, st>>>(
          recs, static_cast<const uint16_t*>(a.dO), a.dS_T, dSc, a.g_S0, a.T, a.H, a.dv);
    else
      kda_cb_scan_kernel<128, 1><<<static_cast<unsigned>(chains * (a.dv / 16)), 4 * kWave, 0, st>>>(
          recs, static_cast<const uint16_t*>(a.dO), a.dS_T, dSc, a.g_S0, a.T, a.H, a.dv);
    return hipGetLastError();
  };
  if (a.T == 0) return state_grad(stream);   // dS0 = dS_T: no forward, no gradient kernel
  // With at most half of the chip taken by the state-gradient scan, it runs on
  // the side stream beside the forward, which takes the other CUs; the
  // gradient kernel waits for both.
  // A call on a stream that is being captured into a graph runs in order on
  // that stream alone, and so does one whose side stream cannot be made.
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if ((e = hipStreamIsCapturing(stream, &cap)) != hipSuccess) return e;
  std::unique_lock<std::mutex> lk(g_side_mu, std::defer_lock);
  SideStream* ss = nullptr;
  if (chains * (a.dv / 16) <= 128 && cap == hipStreamCaptureStatusNone) {
    lk.lock();
    if (side_stream(&ss) != hipSuccess) {
      ss = nullptr;
      lk.unlock();
      (void)hipGetLastError();   // clear the failed creation's error
    }
  }
  if (ss != nullptr) {
    if ((e = hipEventRecord(ss->fork, stream)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(ss->s, ss->fork, 0)) != hipSuccess) return e;
    if ((e = records(ss->s)) != hipSuccess) return e;
    if ((e = state_grad(ss->s)) != hipSuccess) return e;
    if ((e = hipEventRecord(ss->join, ss->s)) != hipSuccess) return e;
    e = forward();
    // the caller's stream waits for the side stream's work whatever happened
    // to the forward, so that nothing of this call outlives it there
    const hipError_t ej = hipStreamWaitEvent(stream, ss->join, 0);
    if (e != hipSuccess) return e;
    if (ej != hipSuccess) return ej;
  } else {
    if ((e = records(stream)) != hipSuccess) return e;
    if ((e = forward()) != hipSuccess) return e;
    if ((e = state_grad(stream)) != hipSuccess) return e;
  }
  kda_cb_grad_kernel<128, 128><<<static_cast<unsigned>(chains * NC), kCbThreads, 0, stream>>>(
      static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
      static_cast<const uint16_t*>(a.v), a.alpha, a.beta, static_cast<const uint16_t*>(a.dO), Sc,
      dSc, recs, sbs, a.g_q, a.g_k, a.g_v, a.g_alpha, a.g_beta, reinterpret_cast<float*>(ws), a.T,
      a.H);
  return hipGetLastError();
}

}  // namespace kda
