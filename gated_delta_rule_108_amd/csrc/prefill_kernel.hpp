// KDA chunked prefill: the chunk kernel, in two modes.
//
// Fused mode: a workgroup of eight waves owns one (batch, head) chain and a
// DVT-wide column slab of its dk x dv state, and walks the chunks of C tokens
// in order.  The fp32 state slab lives in registers for the whole sequence;
// every per-chunk intermediate lives in LDS; HBM sees each input once and
// each output once.  (Columns of the state evolve independently, so slabs of
// one chain run in parallel workgroups; they recompute the column-free
// chunk work and share its inputs through L2.)
//
// Prep mode (few chains): the same chunk work for a run of chunks per
// workgroup, all chunks of a segment in parallel across the chip, writing
// each chunk's state-free quantities to a workspace record for the scan
// kernel.
//
// Chunk algebra.  For a chunk with start state S, rows r = 0..C-1 and the
// per-channel cumulative decay E_r = prod_{j<=r} alpha_j (E'_r = prod_{j>r}):
//   A[r][i]  = sum_c k_r[c] k_i[c] E_r[c]/E_i[c]       (i <  r)  gated K K^T
//   P[r][i]  = sum_c q_r[c] k_i[c] E_r[c]/E_i[c]       (i <= r)  gated Q K^T
//   (I + L) Y = I,   L = strict_lower(Diag(beta) A)            UT transform
//   W = Y Diag(beta) (K . E),   U~ = Y Diag(beta) V             WY factors
//   U = U~ - W S
//   O = (Q . E) S + P U
//   S <- Diag(E_{C-1}) S + (K . E')^T U
// With alpha = 1 this is the chunkwise delta rule of "From GPT-2 to Kimi K3,
// Explained", section "DeltaNet (Parallelizing Linear Transformers with Delta
// Rule)" (T there is Y Diag(beta), built by forward substitution; the
// correction u = U - W S; o = q S + tril(q k^T) u; S += k^T u).  The ratio
// E_r/E_i is the cumulative decay of section "Gated Delta Net", one value per
// channel as in section "KDA/Kimi Linear".
//
// Overflow-free gates.  E_r/E_i is never formed as a quotient of chunk-level
// products (E_i underflows fp32 within one chunk for strong gates).  The
// chunk is cut into 16-row sub-blocks; within block J, F_r = prod of alpha
// from the block start through r and H_i = prod from i+1 through the block
// end.  For r in block R and i in block I < R
//     E_r/E_i = F_r * prod_{I<J<R} BT_J * H_i          (every factor <= 1)
// with BT_J the block's total decay, so the off-diagonal 16x16 tiles of A and
// P are products of pre-scaled operands on the matrix cores.  On diagonal
// tiles the ratio is F_r * (1/F_i), exact as long as the block total stays
// above 2^-100 per channel; a channel below that (a zero gate, or extreme
// decay) is masked out of the matrix product and added exactly on the vector
// units from running products of alpha.
#pragma once

#include <type_traits>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

constexpr float kUnsafeBlockDecay = 7.888609052210118e-31f;  // 2^-100

// ----------------------------------------------------------------------------
// MFMA fragment sources.  A source yields, for the calling lane, the operand
// fragment of rows row0 + (lane % 16) and contraction indices k0 + n*(lane/16)
// .. + n-1, n = 8 (bf16, K=32), 4 (bf16, K=16) or 1 (fp32, K=4).
//
// Lane coordinates come from `Lane`, re-derived once per phase through an
// opaque move so that the compiler computes fragment addresses where they are
// used instead of hoisting hundreds of them out of the chunk loop (which
// exhausts the register file).
// ----------------------------------------------------------------------------
template <typename OpT, int KS> struct Frag;
template <> struct Frag<bf16_t, 32> { using T = bf16x8; static constexpr int N = 8; };
template <> struct Frag<bf16_t, 16> { using T = bf16x4; static constexpr int N = 4; };
template <> struct Frag<float, 4> { using T = float; static constexpr int N = 1; };

struct Lane {
  int i, g;  // i = lane % 16, g = (lane % 64) / 16
};
__device__ __forceinline__ Lane lane_now() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return Lane{t & 15, (t & 63) >> 4};
}

// OpT rows, K-contiguous.
template <typename OpT> struct Src {
  using E = typename Ty<OpT>::Elem;
  const E* p;
  int ld;
  Lane l;
  template <int KS>
  __device__ __forceinline__ typename Frag<OpT, KS>::T get(int k0) const {
    using F = Frag<OpT, KS>;
    const E* a = p + l.i * ld + k0 + F::N * l.g;
    if constexpr (F::N == 1) return *a;
    else return *reinterpret_cast<const typename F::T*>(a);
  }
};

// OpT rows, element k multiplied by s[k] (an fp32 vector over K).
template <typename OpT> struct SrcScaled {
  using E = typename Ty<OpT>::Elem;
  const E* p;
  int ld;
  const float* s;
  Lane l;
  template <int KS>
  __device__ __forceinline__ typename Frag<OpT, KS>::T get(int k0) const {
    using F = Frag<OpT, KS>;
    const int kk = k0 + F::N * l.g;
    const E* a = p + l.i * ld + kk;
    if constexpr (F::N == 1) {
      return *a * s[kk];
    } else {
      typename F::T v = *reinterpret_cast<const typename F::T*>(a);
#pragma unroll
      for (int e = 0; e < F::N; ++e) v[e] = static_cast<__bf16>(static_cast<float>(v[e]) * s[kk + e]);
      return v;
    }
  }
};

// fp32 column source for the fp32 MFMA: B^T[n][k] = M[k][n] of a row-major M.
struct SrcColF32 {
  const float* p;
  int ld;
  Lane l;
  template <int KS>
  __device__ __forceinline__ float get(int k0) const {
    return p[(k0 + l.g) * ld + l.i];
  }
};

// Two adjacent elements loaded with one access (c even, so 4- or 8-byte aligned).
template <typename OpT> struct Pair;
template <> struct Pair<bf16_t> {
  using T = uint32_t;
  __device__ __forceinline__ static T load(const uint16_t* p) {
    return *reinterpret_cast<const uint32_t*>(p);
  }
  __device__ __forceinline__ static T zero() { return 0u; }
  __device__ __forceinline__ static float get(T v, int x) {
    return bf16_to_f32(static_cast<uint16_t>(x ? (v >> 16) : (v & 0xffffu)));
  }
  __device__ __forceinline__ static T pack(float lo, float hi) { return pack_bf16x2(lo, hi); }
};
template <> struct Pair<float> {
  using T = float2;
  __device__ __forceinline__ static T load(const float* p) {
    return *reinterpret_cast<const float2*>(p);
  }
  __device__ __forceinline__ static T zero() { return make_float2(0.f, 0.f); }
  __device__ __forceinline__ static float get(T v, int x) { return x ? v.y : v.x; }
  __device__ __forceinline__ static T pack(float lo, float hi) { return make_float2(lo, hi); }
};

// Four adjacent elements with one access (8 bytes bf16, 16 bytes fp32).
template <typename OpT> struct Quad;
template <> struct Quad<bf16_t> {
  using T = uint2;
  __device__ __forceinline__ static T load(const uint16_t* p) {
    return *reinterpret_cast<const uint2*>(p);
  }
  __device__ __forceinline__ static T zero() { return make_uint2(0u, 0u); }
  __device__ __forceinline__ static float get(T v, int x) {
    const uint32_t w = x < 2 ? v.x : v.y;
    return bf16_to_f32(static_cast<uint16_t>((x & 1) ? (w >> 16) : (w & 0xffffu)));
  }
  __device__ __forceinline__ static void store(uint16_t* p, float a, float b, float c, float d) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
  }
  __device__ __forceinline__ static T make(float a, float b, float c, float d) {
    return make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
  }
};
template <> struct Quad<float> {
  using T = float4;
  __device__ __forceinline__ static T load(const float* p) {
    return *reinterpret_cast<const float4*>(p);
  }
  __device__ __forceinline__ static T zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ __forceinline__ static float get(T v, int x) {
    return x == 0 ? v.x : x == 1 ? v.y : x == 2 ? v.z : v.w;
  }
  __device__ __forceinline__ static void store(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
  }
  __device__ __forceinline__ static T make(float a, float b, float c, float d) {
    return make_float4(a, b, c, d);
  }
};

// A 16-byte vector of 16 / sizeof(element) values.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Input loads with or without the non-temporal hint.  On a long sequence the
// split path streams every input once and keeps its chunk records in the
// last-level cache between the two kernels; hinting the input loads as
// streaming keeps them from evicting those records.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
template <bool NT>
__device__ __forceinline__ uint2 ld_in(const uint16_t* p) {
  if constexpr (NT) {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    return make_uint2(v.x, v.y);
  } else {
    return *reinterpret_cast<const uint2*>(p);
  }
}
template <bool NT>
__device__ __forceinline__ float4 ld_in(const float* p) {
  if constexpr (NT) {
    const f32x4v v = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
  } else {
    return *reinterpret_cast<const float4*>(p);
  }
}
template <bool NT>
__device__ __forceinline__ u32x4 ld_in16(const void* p) {
  if constexpr (NT) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  } else {
    return *reinterpret_cast<const u32x4*>(p);
  }
}
template <typename OpT>
__device__ __forceinline__ float vec_elem(const u32x4& v, int q) {
  if constexpr (Ty<OpT>::kBytes == 2)
    return bf16_to_f32(static_cast<uint16_t>((v[q >> 1] >> (16 * (q & 1))) & 0xffffu));
  else
    return __uint_as_float(v[q]);
}

// Lane layout of the per-chunk input items.  A gate item is (16-row block J,
// channel quad, row quarter h): four rows x four channels of alpha, k and q.
// The four lanes of each lane quad hold four consecutive channel quads of
// the same rows, so each 4-lane group of a load reads contiguous bytes of one
// row (a layout with the row quarter in the low lane bits made every lane
// quad touch four rows, and the loads of a chunk cost ~4k more cycles); the
// four row quarters of a channel quad sit 4 lanes apart in one 16-lane row.
// Value items (block J, 16-byte column vector, row quarter h) are laid out
// the same way.
struct ItemPos {
  int J, h, v;   // block, row quarter, channel quad (gate) or column vector (value)
};
template <int NV>   // channel quads or column vectors per row
__device__ __forceinline__ ItemPos item_pos(int item) {
  constexpr int L = NV < 4 ? NV : 4;   // consecutive vectors of one row per lane group
  const int local = item % (4 * NV);
  return ItemPos{item / (4 * NV), (local / L) % 4, local % L + L * (local / (4 * L))};
}

// The value of the lane holding row quarter (h - S) mod 4 of the same
// channel quad: a DPP rotation by 4 S lanes within the 16-lane row (row_ror,
// lane i reads lane i - 4 S), no LDS.
template <int S>
__device__ __forceinline__ float quarter_ror(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x120 + 4 * S, 0xF, 0xF, false));
}

// Orders this wave's LDS writes before its later LDS reads (no other wave
// takes part, so no barrier is needed).
__device__ __forceinline__ void wave_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}
// s_waitcnt immediate that waits until at most n vector memory operations of
// this wave are in flight (gfx9 encoding: vmcnt in bits 3:0 and 15:14; the
// export and LDS/scalar counters left at their maxima, i.e. not waited on).
__host__ __device__ constexpr int vmcnt_only(int n) {
  return (n & 0xf) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8);
}

// Workgroup barrier for LDS only: orders LDS accesses across the waves
// without waiting for outstanding global loads or stores (__syncthreads()
// would drain both, which throws away the prefetch of the next chunk and
// stalls on every output store).  No workgroup reads back global memory it
// wrote, so LDS is the only memory shared across waves.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
// Index of the off-diagonal block (R, I), I < R, in row-major lower order.
__host__ __device__ constexpr int yf_block(int R, int I) { return R * (R - 1) / 2 + I; }

template <typename OpT, int KS>
__device__ __forceinline__ f32x4 mfma(typename Frag<OpT, KS>::T a, typename Frag<OpT, KS>::T b,
                                      f32x4 c) {
  if constexpr (KS == 32) return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  else if constexpr (KS == 16) return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  else return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Four floats -> a bf16x4 matrix-core operand (round to nearest even), built
// from two packed pairs.  (Converting a float vector to a bf16 vector and then
// reading single elements back out of it was seen to compile every element
// to element 0; packed pairs and whole-register bit casts avoid that form.)
// Lane move inside each row of 16 lanes (CDNA data-parallel primitives:
// 0x100 + d = row_shl:d, lane l reads lane l + d; 0x110 + d = row_shr:d, lane
// l reads lane l - d); lanes whose source falls outside the row read 1.
template <int kCtrl>
__device__ __forceinline__ float dpp_or_one(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.f), __float_as_int(x), kCtrl,
                                                    0xF, 0xF, false));
}

__device__ __forceinline__ bf16x4 bf16_quad(float a, float b, float c, float d) {
  return __builtin_bit_cast(bf16x4, make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d)));
}

// Products on the matrix cores.  Each call returns A[.., kb..ke) * B[kb..ke, ..]
// (kb, ke multiples of 16) in fresh accumulators; callers combine partial
// products with vector adds.  A chain on one accumulator only ever uses one
// instruction kind: a 16-wide K tail after 32-wide steps is issued into its
// own zero accumulator.  (A 16x16x16 bf16 MFMA that reads, as its C operand,
// the result of the 16x16x32 MFMA issued just before it was seen to read
// stale values for two of the four accumulator registers, so the kernels
// never chain the two kinds.)
__device__ __forceinline__ void add4(f32x4& a, const f32x4& b) {
  a[0] += b[0]; a[1] += b[1]; a[2] += b[2]; a[3] += b[3];
}

template <typename OpT, class SA, class SB>
__device__ __forceinline__ f32x4 mma_k(int kb, int ke, const SA& sa, const SB& sb) {
  f32x4 acc = zero4();
  if constexpr (sizeof(typename Ty<OpT>::Elem) == 2) {
    int k = kb;
    for (; k + 32 <= ke; k += 32)
      acc = mfma<OpT, 32>(sa.template get<32>(k), sb.template get<32>(k), acc);
    if (k < ke) {
      if (k == kb) {
        acc = mfma<OpT, 16>(sa.template get<16>(k), sb.template get<16>(k), acc);
      } else {
        add4(acc, mfma<OpT, 16>(sa.template get<16>(k), sb.template get<16>(k), zero4()));
      }
    }
  } else {
    for (int k = kb; k < ke; k += 4)
      acc = mfma<OpT, 4>(sa.template get<4>(k), sb.template get<4>(k), acc);
  }
  return acc;
}

// Two products sharing the B operand: r1 = A1 B, r2 = A2 B.
template <typename OpT, class SA1, class SA2, class SB>
__device__ __forceinline__ void mma_k2(f32x4& r1, f32x4& r2, int kb, int ke, const SA1& a1,
                                       const SA2& a2, const SB& sb) {
  r1 = zero4();
  r2 = zero4();
  if constexpr (sizeof(typename Ty<OpT>::Elem) == 2) {
    int k = kb;
    for (; k + 32 <= ke; k += 32) {
      auto b = sb.template get<32>(k);
      r1 = mfma<OpT, 32>(a1.template get<32>(k), b, r1);
      r2 = mfma<OpT, 32>(a2.template get<32>(k), b, r2);
    }
    if (k < ke) {
      auto b = sb.template get<16>(k);
      if (k == kb) {
        r1 = mfma<OpT, 16>(a1.template get<16>(k), b, r1);
        r2 = mfma<OpT, 16>(a2.template get<16>(k), b, r2);
      } else {
        add4(r1, mfma<OpT, 16>(a1.template get<16>(k), b, zero4()));
        add4(r2, mfma<OpT, 16>(a2.template get<16>(k), b, zero4()));
      }
    }
  } else {
    for (int k = kb; k < ke; k += 4) {
      float b = sb.template get<4>(k);
      r1 = mfma<OpT, 4>(a1.template get<4>(k), b, r1);
      r2 = mfma<OpT, 4>(a2.template get<4>(k), b, r2);
    }
  }
}

// fp32 products used by the triangular solve, independent of OpT.
template <class SA, class SB>
__device__ __forceinline__ void mma_f32(f32x4& acc, int kb, int ke, const SA& sa, const SB& sb) {
  for (int k = kb; k < ke; k += 4)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sa.template get<4>(k), sb.template get<4>(k), acc,
                                               0, 0, 0);
}

// out[b] = A * B_b for a row of NBT tiles sharing the A operand; tile b's B
// source is `sb` moved by b * bstride elements.  Same chaining rule as mma_k.
template <typename OpT, int NBT, class SA, class SB>
__device__ __forceinline__ void mma_row(f32x4 (&out)[NBT], int kb, int ke, const SA& sa,
                                        const SB& sb, int bstride) {
#pragma unroll
  for (int b = 0; b < NBT; ++b) out[b] = zero4();
  if constexpr (sizeof(typename Ty<OpT>::Elem) == 2) {
    int k = kb;
    for (; k + 32 <= ke; k += 32) {
      const auto a = sa.template get<32>(k);
#pragma unroll
      for (int b = 0; b < NBT; ++b) {
        SB t = sb;
        t.p += b * bstride;
        out[b] = mfma<OpT, 32>(a, t.template get<32>(k), out[b]);
      }
    }
    if (k < ke) {
      const auto a = sa.template get<16>(k);
      const bool first = (k == kb);
#pragma unroll
      for (int b = 0; b < NBT; ++b) {
        SB t = sb;
        t.p += b * bstride;
        if (first) out[b] = mfma<OpT, 16>(a, t.template get<16>(k), out[b]);
        else add4(out[b], mfma<OpT, 16>(a, t.template get<16>(k), zero4()));
      }
    }
  } else {
    for (int k = kb; k < ke; k += 4) {
      const float a = sa.template get<4>(k);
#pragma unroll
      for (int b = 0; b < NBT; ++b) {
        SB t = sb;
        t.p += b * bstride;
        out[b] = mfma<OpT, 4>(a, t.template get<4>(k), out[b]);
      }
    }
  }
}

// Ownership of an NR x NCOL grid of 16x16 tiles by NW waves.  The waves form a
// WR x WC grid (WR divides NR, WC divides NCOL, WR * WC <= NW, as many active
// waves as possible); wave w < WR * WC owns the RA x CA block of tiles
// (row0(w) + a, col0(w) + b), a and b known at compile time, so one
// wave-dependent base addresses all of them.  Other waves own nothing.
__host__ __device__ constexpr int largest_divisor_le(int n, int cap) {
  int best = 1;
  for (int d = 1; d <= n && d <= cap; ++d)
    if (n % d == 0) best = d;
  return best;
}
__host__ __device__ constexpr int tile_wr(int NR, int NCOL, int NW) {
  int best_wr = 1, best_act = 0;
  for (int wr = 1; wr <= NR && wr <= NW; ++wr) {
    if (NR % wr) continue;
    const int wc = largest_divisor_le(NCOL, NW / wr);
    if (wr * wc > best_act) { best_act = wr * wc; best_wr = wr; }
  }
  return best_wr;
}
template <int NR, int NCOL, int NW>
struct TileMap {
  static constexpr int WR = tile_wr(NR, NCOL, NW);
  static constexpr int WC = largest_divisor_le(NCOL, NW / WR);
  static constexpr int RA = NR / WR;
  static constexpr int CA = NCOL / WC;
  __device__ __forceinline__ static bool active(int w) { return w < WR * WC; }
  __device__ __forceinline__ static int row0(int w) { return (w / WC) * RA; }
  __device__ __forceinline__ static int col0(int w) { return (w % WC) * CA; }
};

// ----------------------------------------------------------------------------
// Workspace record of one chunk, written by the prep kernel and read by the
// scan kernel.  Matrices are stored as matrix-core operand packets so that a
// wave loads each fragment with one contiguous access (64 lanes x n elements):
//   A packet (16-row block b, K step s of width KS): lane l holds row
//   16b + l%16, columns s*KS + (KS/4)*(l/16) .. + KS/4 - 1.
//   Accumulator packet (row block R, column tile j): lane l holds rows
//   16R + 4(l/16) .. + 3 of column 16j + l%16.
// Layout (elements of the operand type unless noted):
//   W [C x DK] A packets (KS = KSD) | Q.E [C x DK] (KSD) | (K.E')^T [DK x C] (KSC) |
//   P [C x C] (KSC) | decay E_{C-1} [DK] fp32 | U~ = Y Diag(beta) V [C x dv] accumulator packets
// KSD / KSC: the widest matrix-core K step that divides DK / C.
// ----------------------------------------------------------------------------
template <typename OpT, int K>
__host__ __device__ constexpr int kstep() {
  return Ty<OpT>::kBytes == 2 ? (K % 32 == 0 ? 32 : 16) : 4;
}

template <typename OpT, int DK, int C>
struct RecCfg {
  static constexpr int EB = Ty<OpT>::kBytes;
  static constexpr int KSD = kstep<OpT, DK>(), KSC = kstep<OpT, C>();
  static constexpr int NKD = DK / KSD, NKC = C / KSC;
  static constexpr size_t kW = 0;
  static constexpr size_t kQ = static_cast<size_t>(C) * DK;
  static constexpr size_t kKG = 2 * static_cast<size_t>(C) * DK;
  static constexpr size_t kP = 3 * static_cast<size_t>(C) * DK;
  static constexpr size_t kGcByte = (kP + static_cast<size_t>(C) * C) * EB;
  static constexpr size_t kUByte = kGcByte + 4 * DK;
  __host__ __device__ static constexpr size_t bytes(int dv) {
    return (kUByte + static_cast<size_t>(C) * dv * EB + 255) / 256 * 256;
  }
};

// Padded LDS matrix (row stride ld) -> A packets of width KS, 16-byte (or
// smaller) vectors; `blocks` 16-row blocks, `nks` K steps.
// When the packet count is a multiple of the thread count every thread
// issues the same, compile-time number of stores (no loop, no branch), so the
// compiler can count the memory operations in flight exactly.
template <typename OpT, int KS, int BLOCKS, int NKS, int NTH>
__device__ __forceinline__ void copy_packets(typename Ty<OpT>::Elem* dst,
                                             const typename Ty<OpT>::Elem* src, int ld, int tid) {
  using F = Frag<OpT, KS>;
  using V = typename F::T;
  constexpr int kTotal = BLOCKS * NKS * 64;
  auto one = [&](int x) {
    const int l = x % 64, bs = x / 64, blk = bs / NKS, s = bs % NKS;
    const typename Ty<OpT>::Elem* a = src + (16 * blk + l % 16) * ld + s * KS + F::N * (l / 16);
    *reinterpret_cast<V*>(dst + static_cast<size_t>(x) * F::N) = *reinterpret_cast<const V*>(a);
  };
  if constexpr (kTotal % NTH == 0) {
#pragma unroll
    for (int k = 0; k < kTotal / NTH; ++k) one(tid + NTH * k);
  } else {
    for (int x = tid; x < kTotal; x += NTH) one(x);
  }
}

// Four accumulator values of one lane in the operand type.
template <typename OpT> struct Acc4;
template <> struct Acc4<bf16_t> {
  using Raw = uint2;
  __device__ __forceinline__ static void store(uint16_t* p, const f32x4& v) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
  }
  __device__ __forceinline__ static Raw load(const uint16_t* p) {
    return *reinterpret_cast<const uint2*>(p);
  }
  __device__ __forceinline__ static f32x4 cvt(Raw r) {
    f32x4 v;
    v[0] = bf16_to_f32(static_cast<uint16_t>(r.x & 0xffffu));
    v[1] = bf16_to_f32(static_cast<uint16_t>(r.x >> 16));
    v[2] = bf16_to_f32(static_cast<uint16_t>(r.y & 0xffffu));
    v[3] = bf16_to_f32(static_cast<uint16_t>(r.y >> 16));
    return v;
  }
};
template <> struct Acc4<float> {
  using Raw = float4;
  __device__ __forceinline__ static void store(float* p, const f32x4& v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
  __device__ __forceinline__ static Raw load(const float* p) {
    return *reinterpret_cast<const float4*>(p);
  }
  __device__ __forceinline__ static f32x4 cvt(Raw r) {
    f32x4 v;
    v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
    return v;
  }
};

// ----------------------------------------------------------------------------
// LDS plan (element counts; every region 16-byte aligned).
// ----------------------------------------------------------------------------
__host__ __device__ constexpr int imax(int a, int b) { return a > b ? a : b; }
__host__ __device__ constexpr int align16(int bytes) { return (bytes + 15) & ~15; }

template <typename OpT, int DK, int C, int DVT>
struct PCfg {
  static constexpr int NTH = 512, NW = 8;
  static constexpr int NB = C / 16;            // 16-row sub-blocks per chunk
  static constexpr int NJ = DVT / 16;          // 16-column tiles of the slab
  static constexpr int NCB = DK / 16;          // 16-channel tiles
  static constexpr int EB = Ty<OpT>::kBytes;
  static constexpr int PADE = 16 / EB;         // one 16-byte pad per row
  static constexpr int LDK = DK + PADE;        // rows of length DK
  static constexpr int LDC = C + PADE;         // rows of length C
  static constexpr int LDT = C + 4;            // fp32 C x C
  static constexpr int LDZ = 20;               // fp32 16 x 16 scratch

  // region sizes in bytes
  static constexpr int kZ1 = align16(imax(imax(2 * C * LDK, DVT * LDC), DVT * LDK) * EB);
  static constexpr int kR1 = align16(C * LDK * EB);
  static constexpr int kR2 = align16(C * LDK * EB);
  static constexpr int kKT = align16(DK * LDC * EB);
  static constexpr int kKB = align16(imax(DK, DVT) * LDC * EB);
  static constexpr int kTT = align16(C * LDT * 4);
  static constexpr int kZB = align16(imax(NB, 1) * 16 * LDZ * 4);
  static constexpr int kYF = align16(imax(imax(NB * (NB - 1) / 2, 1) * 16 * LDZ * 4,
                                          (NB * (NB - 1) / 2 + NB) * 64 * 4 * 2));
  static constexpr int kPP = align16(C * LDC * EB);
  static constexpr int kBT = align16(NB * DK * 4);
  static constexpr int kMID = align16(imax(imax(NB * NB, 1) * DK * 4, C * LDC * EB));
  static constexpr int kGC = align16(DK * 4);
  static constexpr int kBE = align16(C * 4);
  static constexpr int kFL = align16(NB * 4);

  static constexpr int oZ1 = 0;
  static constexpr int oR1 = oZ1 + kZ1;
  static constexpr int oR2 = oR1 + kR1;
  static constexpr int oKB = oR2 + kR2;
  static constexpr int oKG = oKB + kKB;
  static constexpr int oTT = oKG + kKT;
  static constexpr int oZB = oTT + kTT;
  static constexpr int oYF = oZB + kZB;
  static constexpr int oPP = oYF + kYF;
  static constexpr int oBT = oPP + kPP;
  static constexpr int oPRE = oBT + kBT;
  static constexpr int oMID = oPRE + kBT;
  static constexpr int oGC = oMID + kMID;
  static constexpr int oBE = oGC + kGC;
  static constexpr int oFL = oBE + kBE;
  static constexpr int kLds = oFL + kFL;

  // work items
  // Gate items (block J, channel quad, row quarter): four rows x four
  // channels; the four quarters of a (block, quad) are adjacent lanes.
  static constexpr int NGI = NB * DK;
  static constexpr int NGT = (NGI + NTH - 1) / NTH;
  // Value items (block J, 16-byte column vector, row quarter).
  static constexpr int VEC = 16 / EB;                      // value columns per vector
  static constexpr int NVI = NB * (DVT / VEC) * 4;
  static constexpr int NVT = (NVI + NTH - 1) / NTH;
  static constexpr int NS = NCB * NJ;                      // state tiles
  static constexpr int NSW = (NS + NW - 1) / NW;
  static constexpr int NU = NB * NJ;                       // chunk-output tiles
  static constexpr int NUW = (NU + NW - 1) / NW;
  static constexpr int NAP = NB * (NB + 1) / 2;            // lower block pairs
};

constexpr int kMaxLds = 160 * 1024;

// kPrep = false: the fused prefill (all chunks of a chain, state in
// registers; cpb, seg0, segn unused).  kPrep = true: each workgroup (DVT =
// dv) takes a run of cpb consecutive chunks of one chain within the segment
// of chunks [seg0, seg0 + segn), computes their state-free quantities and
// writes them to the chunks' workspace records (W, Q.E, (K.E')^T, P, chunk
// decay, U~; segn records per chain) for the scan kernel; the next chunk's
// inputs load while the current one is processed.
//
// kIn (GateIn) says how the gate arrives.  kGateAlpha: ggate is alpha
// (fp32, one per key channel), gbeta is beta, q and k are used as given.
// kGateLogit: the input prologue runs on the fly: ggate holds gate logits g
// in the I/O type (alpha = 1 / (1 + e^g)), gbeta holds write-strength
// logits (beta = sigmoid), and q, k pass through qk_map (QkMap: as given,
// L2-normalised, or SiLU then L2-normalised per token); the row norms are
// sums of squares over the chunk's registers, reduced across the lanes of a
// wave and, at dk = 128, across two waves in LDS.  kGateScalar: ggate holds
// one alpha per token and head (Gated DeltaNet), broadcast over the
// channels as it is loaded, or is null for alpha = 1 (DeltaNet).
template <typename OpT, int DK, int C, int DVT, bool kPrep = false, int kIn = kGateAlpha,
          bool kStates = false>
__global__ void __launch_bounds__(512)
kda_prefill_kernel(const typename Ty<OpT>::Elem* __restrict__ gq,
                   const typename Ty<OpT>::Elem* __restrict__ gk,
                   const typename Ty<OpT>::Elem* __restrict__ gv,
                   const void* __restrict__ ggate, const float* __restrict__ gbeta,
                   const float* gS0, typename Ty<OpT>::Elem* __restrict__ go, float* gST,
                   int B, int T, int H, int DV, char* __restrict__ gws, int cpb, int seg0,
                   int segn, int qk_map, int nt_in, float* __restrict__ gSc) {
  using Cf = PCfg<OpT, DK, C, DVT>;
  using E = typename Ty<OpT>::Elem;
  using PT = typename Pair<OpT>::T;
  constexpr bool kLogit = kIn == kGateLogit;
  constexpr bool kScalar = kIn == kGateScalar;
  constexpr int NB = Cf::NB, NJ = Cf::NJ, NW = Cf::NW, NTH = Cf::NTH;
  constexpr int LDK = Cf::LDK, LDC = Cf::LDC, LDT = Cf::LDT, LDZ = Cf::LDZ;
  static_assert(Cf::kLds <= kMaxLds, "LDS plan exceeds 160 KiB");
  constexpr bool kBF = sizeof(E) == 2;
  // bf16 operands: W and U~ by blocked substitution (no off-diagonal Y).
  constexpr bool kSubst = kBF;
  constexpr int LDO = DVT + 16 / static_cast<int>(sizeof(E));
  constexpr bool kStageO = C * LDO * static_cast<int>(sizeof(E)) <= Cf::kR1;
  using SM = TileMap<Cf::NCB, NJ, NW>;   // state tiles (Cb, Jb)
  using UM = TileMap<NB, NJ, NW>;        // chunk-output tiles (R, Jb)

  __shared__ __attribute__((aligned(16))) char smem[Cf::kLds];
  E* Ki = reinterpret_cast<E*>(smem + Cf::oZ1);             // [C][LDK]
  E* Kinv = Ki + C * LDK;                                     // [C][LDK]
  E* VbT = reinterpret_cast<E*>(smem + Cf::oZ1);             // [DVT][LDC]  (after A/P)
  E* ST = reinterpret_cast<E*>(smem + Cf::oZ1);              // [DVT][LDK]  (scan)
  E* Kr = reinterpret_cast<E*>(smem + Cf::oR1);              // [C][LDK]
  E* Wm = reinterpret_cast<E*>(smem + Cf::oR1);              // [C][LDK]   (after A/P)
  E* Qr = reinterpret_cast<E*>(smem + Cf::oR2);              // [C][LDK]
  E* KbT = reinterpret_cast<E*>(smem + Cf::oKB);             // [DK][LDC]
  E* UT = reinterpret_cast<E*>(smem + Cf::oKB);              // [DVT][LDC] (scan)
  E* KgT = reinterpret_cast<E*>(smem + Cf::oKG);             // [DK][LDC]
  float* TT = reinterpret_cast<float*>(smem + Cf::oTT);      // [C][LDT]
  float* ZB = reinterpret_cast<float*>(smem + Cf::oZB);      // [NB-1][16][LDZ]
  float* YF = reinterpret_cast<float*>(smem + Cf::oYF);      // off-diagonal Y blocks, fp32
  // (bf16 operands) -L_RJ and Y_RR as matrix-core A fragments: fragment f,
  // lane l = 16 g + i holds elements [i][4g .. 4g + 3] of its 16x16 block
  E* LF = reinterpret_cast<E*>(smem + Cf::oYF);
  constexpr int kNLF = NB * (NB - 1) / 2;                    // first Y_RR fragment
  E* PP = reinterpret_cast<E*>(smem + Cf::oPP);              // [C][LDC]
  float* sBT = reinterpret_cast<float*>(smem + Cf::oBT);     // [NB][DK]
  float* sPRE = reinterpret_cast<float*>(smem + Cf::oPRE);   // [NB][DK]
  float* sMID = reinterpret_cast<float*>(smem + Cf::oMID);   // [NB][NB][DK]
  E* Yb = reinterpret_cast<E*>(smem + Cf::oMID);             // [C][LDC]  (after A/P)
  E* OS = reinterpret_cast<E*>(smem + Cf::oR1);              // [C][LDO]  (output staging)
  float* sGC = reinterpret_cast<float*>(smem + Cf::oGC);     // [DK]
  float* sBE = reinterpret_cast<float*>(smem + Cf::oBE);     // [C]
  int* sFL = reinterpret_cast<int*>(smem + Cf::oFL);         // [NB]
  // One gate per row: per-row decays in LDS the per-channel path uses for
  // its gated copies of K (idle here until beta V is staged after the A/P
  // products) and for its decay table before each block (idle up to Q E).
  // The gates, the within-block prefix / suffix products, the decays between
  // blocks and E' (decay to the chunk end) are read up to the A/P products,
  // E (decay from the chunk start) up to Q E.
  float* sRowA = reinterpret_cast<float*>(smem + Cf::oZ1);   // [C]
  float* sRowF = sRowA + C;          // [C]
  float* sRowH = sRowA + 2 * C;      // [C]
  float* sRowEp = sRowA + 3 * C;     // [C]
  float* sRowMID = sRowA + 4 * C;    // [NB][NB]
  float* sRowE = sPRE;               // [C]
  static_assert(!kScalar || ((4 * C + NB * NB) * 4 <= 2 * C * LDK * static_cast<int>(sizeof(E)) &&
                             C <= NB * DK && C <= kWave),
                "per-row gate tables");

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const float* galpha = static_cast<const float*>(ggate);   // kGateAlpha, kGateScalar
  const bool has_gate = galpha != nullptr;                   // kGateScalar: null is alpha = 1
  const E* glogit = static_cast<const E*>(ggate);           // kLogit = true
  // Per-row sums of squares of k and q, [part][k, q][C], part = which half of
  // the channels at dk = 128.  Lives in ZB, which is idle until phase SO.
  float* sNRM = ZB;
  const bool qk_norm = kLogit && qk_map != kQkAsGiven;
  const bool qk_silu = kLogit && qk_map == kQkSiluL2;

  // Workgroup -> (chain, slab).  Consecutive workgroups are dealt round-robin
  // to the 8 XCDs; keep all slabs of one chain on one XCD so they share L2.
  // Prep mode: workgroup -> (chain, run of cpb consecutive chunks of the
  // segment [seg0, seg0 + segn)); the segment's records are numbered from 0.
  const int NC = (T + C - 1) / C;
  const int ntiles = kPrep ? (segn + cpb - 1) / cpb : DV / DVT;
  const int total = gridDim.x;
  int L = blockIdx.x;
  if (!kPrep && ntiles > 1 && (total % 8) == 0) L = (blockIdx.x % 8) * (total / 8) + blockIdx.x / 8;
  const int chain = L / ntiles;
  const int j0 = kPrep ? 0 : (L % ntiles) * DVT;
  const int ch_begin = kPrep ? seg0 + (L % ntiles) * cpb : 0;
  const int ch_end = kPrep ? min(ch_begin + cpb, seg0 + segn) : NC;
  const int b = chain / H, h = chain % H;

  // Token t of this chain sits at row (b*T + t)*H + h of the [B*T*H, *]
  // arrays.  Within a chunk, rows are H apart: each chunk gets wave-uniform
  // 64-bit base pointers and 32-bit per-lane offsets.
  const size_t row0 = static_cast<size_t>(b) * T * H + h;
  const int rsK = H * DK, rsV = H * DV;

  // ---- state slab in registers, tiles (Cb, Jb) of the state map
  f32x4 Sreg[SM::RA][SM::CA];
  {
    const Lane ln = lane_now();
#pragma unroll
    for (int a = 0; a < SM::RA; ++a)
#pragma unroll
      for (int bb = 0; bb < SM::CA; ++bb) {
        Sreg[a][bb] = zero4();
        if (!kPrep && SM::active(wave) && gS0 != nullptr) {
          const int Cb = SM::row0(wave) + a, Jb = SM::col0(wave) + bb;
          const float* src = gS0 + static_cast<size_t>(chain) * DK * DV + j0 + 16 * Jb;
#pragma unroll
          for (int r = 0; r < 4; ++r) Sreg[a][bb][r] = src[(16 * Cb + 4 * ln.g + r) * DV + ln.i];
        }
      }
  }
  // Upper block triangles of TT and PP are never written again: zero once.
  for (int x = tid; x < C * C; x += NTH) {
    const int r = x / C, c = x % C;
    if (c / 16 > r / 16) {
      TT[r * LDT + c] = 0.f;
      PP[r * LDC + c] = Ty<OpT>::from_f32(0.f);
    }
  }

  // Raw chunk inputs live in registers and are fetched one chunk ahead: the
  // loads for chunk ch+1 are issued as soon as chunk ch is done with the
  // previous contents, so their latency hides behind chunk ch's compute.
  // Rows are clamped to the last token; rows past T are replaced by identity
  // padding (gate 1, key/query/value 0, strength 0) when consumed.
  using QT = typename Quad<OpT>::T;
  float ga[Cf::NGT][4][4];      // alpha [row][channel]
  QT gg[Cf::NGT][4];            // gate logits (kLogit), converted to ga in G1
  QT gkk[Cf::NGT][4], gqq[Cf::NGT][4];
  u32x4 gvv[Cf::NVT][4];
  float gbe = 0.f;
  float gsa = 1.f;              // scalar gate of row `lane` (wave 0, kScalar)
  auto fetch_gates_nt = [&](int tn, auto nt) {
    constexpr bool NT = decltype(nt)::value;
    const size_t base = (row0 + static_cast<size_t>(tn) * H) * DK;
    const float* pa = galpha + base;
    const E* pg = glogit + base;
    const E* pk = gk + base;
    const E* pq = gq + base;
    const int jmax = T - 1 - tn;
    int t_ = tid;
    asm volatile("" : "+v"(t_));
#pragma unroll
    for (int it = 0; it < Cf::NGT; ++it) {
      const int item = t_ + NTH * it;
      if (Cf::NGI % NTH == 0 || item < Cf::NGI) {
        const ItemPos ip = item_pos<DK / 4>(item);
        const int h = ip.h, J = ip.J, c = 4 * ip.v;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int off = min(16 * J + 4 * h + j, jmax) * rsK + c;
          if constexpr (kLogit) {
            gg[it][j] = Quad<OpT>::load(pg + off);
          } else if constexpr (kScalar) {
            // one gate per row: fetched below by wave 0, lane = row
          } else {
            const float4 a4 = ld_in<NT>(pa + off);
            ga[it][j][0] = a4.x;
            ga[it][j][1] = a4.y;
            ga[it][j][2] = a4.z;
            ga[it][j][3] = a4.w;
          }
          gkk[it][j] = ld_in<NT>(pk + off);
          gqq[it][j] = ld_in<NT>(pq + off);
        }
      }
    }
    if constexpr (kScalar) {
      if (wave == 0 && has_gate)
        gsa = galpha[row0 + static_cast<size_t>(tn + min(tid, jmax)) * H];
    }
  };
  auto fetch_gates = [&](int tn) {
    if constexpr (kPrep) {
      if (nt_in) fetch_gates_nt(tn, std::true_type{});
      else fetch_gates_nt(tn, std::false_type{});
    } else {
      fetch_gates_nt(tn, std::false_type{});
    }
  };
  auto fetch_values_nt = [&](int tn, auto nt) {
    constexpr bool NT = decltype(nt)::value;
    const E* pv = gv + (row0 + static_cast<size_t>(tn) * H) * DV + j0;
    const int jmax = T - 1 - tn;
    int t_ = tid;
    asm volatile("" : "+v"(t_));
#pragma unroll
    for (int it = 0; it < Cf::NVT; ++it) {
      const int item = t_ + NTH * it;
      if (Cf::NVI % NTH == 0 || item < Cf::NVI) {
        const ItemPos ip = item_pos<DVT / Cf::VEC>(item);
        const int h = ip.h, J = ip.J, cc = Cf::VEC * ip.v;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          gvv[it][j] = ld_in16<NT>(pv + min(16 * J + 4 * h + j, jmax) * rsV + cc);
      }
    }
  };
  auto fetch_values = [&](int tn) {
    if constexpr (kPrep) {
      if (nt_in) fetch_values_nt(tn, std::true_type{});
      else fetch_values_nt(tn, std::false_type{});
    } else {
      fetch_values_nt(tn, std::false_type{});
    }
  };
  auto fetch_beta = [&](int tn) {   // every thread loads (only tid < C keep it): no branch
    gbe = gbeta[row0 + static_cast<size_t>(min(tn + tid % C, T - 1)) * H];
  };

  if (ch_begin < ch_end) {
    fetch_gates(ch_begin * C);
    fetch_values(ch_begin * C);
    fetch_beta(ch_begin * C);
  }
  // Land every load issued so far (the first chunk needs them at once).  A
  // load still in flight at the loop entry would make the compiler assume, on
  // every chunk, that the registers it fills were loaded last, and wait for
  // all outstanding memory traffic (the previous chunk's stores included).
  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
  for (int ch = ch_begin; ch < ch_end; ++ch) {
    const int t0 = ch * C;
    const bool more = ch + 1 < ch_end;
    const bool full = t0 + C <= T;   // no padding rows in this chunk
    // ================= G1: pad the fetched chunk, within-block cumulative gates
    if (tid < C) sBE[tid] = (t0 + tid < T) ? (kLogit ? sigmoid_f(gbe) : gbe) : 0.f;
    fetch_beta(more ? t0 + C : t0);   // unconditional: uniform memory-op counts
    if (tid < NB) sFL[tid] = 0;
    // Per gate item: quarter products of alpha, combined across the four
    // quarters of the block (lanes of one group of four) into the block total
    // BT and this quarter's offsets: Foff = product over earlier quarters,
    // Hoff = product over later quarters.
    float foff[Cf::NGT][4], hoff[Cf::NGT][4], bt[Cf::NGT][4];
#pragma unroll
    for (int it = 0; it < Cf::NGT; ++it) {
      const int item = tid + NTH * it;
      if (Cf::NGI % NTH == 0 || item < Cf::NGI) {
        const ItemPos ip = item_pos<DK / 4>(item);
        const int h = ip.h, J = ip.J, c = 4 * ip.v;
        if constexpr (kLogit) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int x = 0; x < 4; ++x) ga[it][j][x] = gate_from_logit(Quad<OpT>::get(gg[it][j], x));
        }
        if (!full) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bool valid = t0 + 16 * J + 4 * h + j < T;
#pragma unroll
            for (int x = 0; x < 4; ++x) ga[it][j][x] = valid ? ga[it][j][x] : 1.f;
            gkk[it][j] = valid ? gkk[it][j] : Quad<OpT>::zero();
            gqq[it][j] = valid ? gqq[it][j] : Quad<OpT>::zero();
          }
        }
        if (qk_silu) {   // SiLU in place (rounded back to the I/O type)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const QT kq = gkk[it][j], qq = gqq[it][j];
            gkk[it][j] = Quad<OpT>::make(silu_f(Quad<OpT>::get(kq, 0)), silu_f(Quad<OpT>::get(kq, 1)),
                                         silu_f(Quad<OpT>::get(kq, 2)), silu_f(Quad<OpT>::get(kq, 3)));
            gqq[it][j] = Quad<OpT>::make(silu_f(Quad<OpT>::get(qq, 0)), silu_f(Quad<OpT>::get(qq, 1)),
                                         silu_f(Quad<OpT>::get(qq, 2)), silu_f(Quad<OpT>::get(qq, 3)));
          }
        }
#pragma unroll
        for (int x = 0; x < 4 && !kScalar; ++x) {
          // r_s = product of quarter (h - s) mod 4; the block total is the
          // same two pair products in every lane, (p_h p_h+2)(p_h+1 p_h+3).
          const float p = ga[it][0][x] * ga[it][1][x] * ga[it][2][x] * ga[it][3][x];
          const float r1 = quarter_ror<1>(p), r2 = quarter_ror<2>(p), r3 = quarter_ror<3>(p);
          foff[it][x] = h == 0 ? 1.f : h == 1 ? r1 : h == 2 ? r1 * r2 : (r1 * r2) * r3;
          hoff[it][x] = h == 3 ? 1.f : h == 2 ? r3 : h == 1 ? r3 * r2 : (r3 * r2) * r1;
          bt[it][x] = (p * r2) * (r1 * r3);
        }
        if (!kScalar && h == 0)
          *reinterpret_cast<float4*>(sBT + J * DK + c) =
              make_float4(bt[it][0], bt[it][1], bt[it][2], bt[it][3]);
      }
      if (qk_norm) {
        // Row sums of squares of k and q: this lane's four channels, then the
        // lanes of the wave that hold the same rows (lane bits 0-1 and 4.. pick
        // the channel quad), then, at dk = 128, the two waves of a block in LDS.
        const bool active = Cf::NGI % NTH == 0 || item < Cf::NGI;
        float nk[4], nq[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          nk[j] = 0.f;
          nq[j] = 0.f;
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const float kx = Quad<OpT>::get(gkk[it][j], x), qx = Quad<OpT>::get(gqq[it][j], x);
            nk[j] += kx * kx;
            nq[j] += qx * qx;
          }
          nk[j] = active ? nk[j] : 0.f;
          nq[j] = active ? nq[j] : 0.f;
        }
        constexpr int kSpan = DK < 64 ? DK : 64;   // lanes of a block within one wave
#pragma unroll
        for (int off = 1; off < kSpan; off <<= 1) {
          if (off == 4 || off == 8) continue;        // lane bits 2-3: the row quarter
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            nk[j] += __shfl_xor(nk[j], off);
            nq[j] += __shfl_xor(nq[j], off);
          }
        }
        const ItemPos ip = item_pos<DK / 4>(item);
        const int h = ip.h, J = ip.J, local = item % DK, part = local / 64;
        if (active && (local % kSpan) < 16 && (local & 3) == 0) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = 16 * J + 4 * h + j;
            sNRM[(2 * part) * C + r] = nk[j];
            sNRM[(2 * part + 1) * C + r] = nq[j];
          }
        }
      }
    }
#pragma unroll
    for (int it = 0; it < Cf::NVT; ++it) {
      const int item = tid + NTH * it;
      if (Cf::NVI % NTH == 0 || item < Cf::NVI) {
        const ItemPos ip = item_pos<DVT / Cf::VEC>(item);
        const int h = ip.h, J = ip.J;
        if (!full) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            gvv[it][j] = (t0 + 16 * J + 4 * h + j < T) ? gvv[it][j] : u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
    if constexpr (kScalar) {
      // One gate per row: wave 0, lane r = row r, makes every per-row decay
      // with lane products (DPP within each 16-row block, lane reads across
      // blocks).  Only products: an exact zero gate stays exact.
      //   F_r  = prod of a from the block start through r     (inclusive)
      //   H_r  = prod of a after r to the block end           (exclusive)
      //   BT_J = block total, E_r = prod_{J<R} BT_J F_r, E'_r = H_r prod_{J>R} BT_J
      //   MID(R, I) = prod_{I<J<R} BT_J, the chunk decay = prod_J BT_J
      if (wave == 0) {
        const int r = tid;
        const float a = (r < C && t0 + r < T) ? gsa : 1.f;
        float F = a, Hin = a;   // inclusive prefix / suffix products within the block
        F *= dpp_or_one<0x111>(F);
        Hin *= dpp_or_one<0x101>(Hin);
        F *= dpp_or_one<0x112>(F);
        Hin *= dpp_or_one<0x102>(Hin);
        F *= dpp_or_one<0x114>(F);
        Hin *= dpp_or_one<0x104>(Hin);
        F *= dpp_or_one<0x118>(F);
        Hin *= dpp_or_one<0x108>(Hin);
        const float Hx = dpp_or_one<0x101>(Hin);   // exclusive suffix
        float bt[4], all = 1.f;
#pragma unroll
        for (int J = 0; J < 4; ++J) {
          bt[J] = J < NB ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(F), 16 * J + 15)) : 1.f;
          all *= bt[J];
        }
        const int R = r / 16;
        float pre = 1.f, suf = 1.f;
#pragma unroll
        for (int J = 0; J < 4; ++J) {
          if (J < R) pre *= bt[J];
          if (J > R && J < NB) suf *= bt[J];
        }
        if (r < C) {
          sRowA[r] = a;
          sRowF[r] = F;
          sRowH[r] = Hx;
          sRowE[r] = pre * F;
          sRowEp[r] = Hx * suf;
        }
        if (r < NB * NB) {   // MID(R, I) at R * NB + I
          const int RR = r / NB, II = r % NB;
          float m = 1.f;
#pragma unroll
          for (int J = 0; J < 4; ++J)
            if (J > II && J < RR) m *= bt[J];
          sRowMID[r] = m;
        }
        for (int c = r; c < DK; c += kWave) sGC[c] = all;
      }
    }
    lds_barrier();

    // ================= G2: chunk-level gate products and MFMA operands
    if (!kScalar && tid < DK) {
      const int c = tid;
      float acc = 1.f;
      for (int J = 0; J < NB; ++J) {
        sPRE[J * DK + c] = acc;
        acc *= sBT[J * DK + c];
      }
      sGC[c] = acc;
      for (int R = 2; R < NB; ++R)
        for (int I = 0; I + 1 < R; ++I) {
          float m = 1.f;
          for (int J = I + 1; J < R; ++J) m *= sBT[J * DK + c];
          sMID[(R * NB + I) * DK + c] = m;
        }
    }
#pragma unroll
    for (int it = 0; it < Cf::NGT && kScalar; ++it) {
      // One gate per row: K and Q go to the A/P products unscaled (the decay
      // is a per-row-pair scalar applied to the product tiles), beta K E and
      // K E' are rows scaled by one value each.
      const int item = tid + NTH * it;
      if (Cf::NGI % NTH == 0 || item < Cf::NGI) {
        const ItemPos ip = item_pos<DK / 4>(item);
        const int h = ip.h, J = ip.J, c = 4 * ip.v;
        float kb[4][4], kg[4][4];   // [channel][row of the quarter]
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 16 * J + 4 * h + j;
          const float be = sBE[r] * sRowE[r], ep = sRowEp[r];
          float kk[4], qq[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            kk[x] = Quad<OpT>::get(gkk[it][j], x);
            qq[x] = Quad<OpT>::get(gqq[it][j], x);
            kb[x][j] = be * kk[x];
            kg[x][j] = ep * kk[x];
          }
          Quad<OpT>::store(Kr + r * LDK + c, kk[0], kk[1], kk[2], kk[3]);
          Quad<OpT>::store(Qr + r * LDK + c, qq[0], qq[1], qq[2], qq[3]);
        }
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          Quad<OpT>::store(KbT + (c + x) * LDC + 16 * J + 4 * h, kb[x][0], kb[x][1], kb[x][2], kb[x][3]);
          Quad<OpT>::store(KgT + (c + x) * LDC + 16 * J + 4 * h, kg[x][0], kg[x][1], kg[x][2], kg[x][3]);
        }
      }
    }
#pragma unroll
    for (int it = 0; it < Cf::NGT && !kScalar; ++it) {
      const int item = tid + NTH * it;
      if (Cf::NGI % NTH == 0 || item < Cf::NGI) {
        const ItemPos ip = item_pos<DK / 4>(item);
        const int h = ip.h, J = ip.J, c = 4 * ip.v;
        // decay of the blocks before / after J, and 1/BT_J (zero for an
        // unsafe block: its diagonal tile is then done exactly on the VALUs)
        float pre[4], suf[4], rbt[4];
        bool unsafe = false;
        // decay of the blocks before and after J for this channel quad.  With
        // dk >= 64 all items of a wave share J, so the loops run on the scalar
        // unit with no divergence and only the needed products on the VALUs.
        const int Ju = (DK >= 64 && Cf::NGI % NTH == 0) ? __builtin_amdgcn_readfirstlane(J) : J;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          pre[x] = 1.f;
          suf[x] = 1.f;
        }
        for (int JJ = 0; JJ < Ju; ++JJ) {
          const float4 b = *reinterpret_cast<const float4*>(sBT + JJ * DK + c);
          pre[0] *= b.x; pre[1] *= b.y; pre[2] *= b.z; pre[3] *= b.w;
        }
        for (int JJ = Ju + 1; JJ < NB; ++JJ) {
          const float4 b = *reinterpret_cast<const float4*>(sBT + JJ * DK + c);
          suf[0] *= b.x; suf[1] *= b.y; suf[2] *= b.z; suf[3] *= b.w;
        }
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const bool safe = bt[it][x] >= kUnsafeBlockDecay;
          unsafe |= !safe;
          // 1/F_i = H_i / BT_J: one reciprocal per channel instead of per row
          rbt[x] = safe ? __builtin_amdgcn_rcpf(bt[it][x]) : 0.f;
        }
        if (unsafe && h == 0) atomicOr(&sFL[J], 1);
        // H_r = product of alpha after row r within the block
        float hx[4][4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          hx[3][x] = hoff[it][x];
#pragma unroll
          for (int j = 2; j >= 0; --j) hx[j][x] = hx[j + 1][x] * ga[it][j + 1][x];
        }
        float f[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) f[x] = foff[it][x];
        float kb[4][4], kg[4][4];   // [channel][row of the quarter]
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 16 * J + 4 * h + j;
          const float be = sBE[r];
          float sk = 1.f, sq = 1.f;   // 1 / row norms (prologue)
          if (qk_norm) {
            float nk = sNRM[r], nq = sNRM[C + r];
            if constexpr (DK > 64) {
              nk += sNRM[2 * C + r];
              nq += sNRM[3 * C + r];
            }
            sk = inv_l2(nk);
            sq = inv_l2(nq);
          }
          float kr[4], qr[4], ki[4], kv[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            f[x] *= ga[it][j][x];
            const float kk = Quad<OpT>::get(gkk[it][j], x) * sk;
            const float qq = Quad<OpT>::get(gqq[it][j], x) * sq;
            kr[x] = kk * f[x];
            qr[x] = qq * f[x];
            ki[x] = kk * hx[j][x];
            kv[x] = ki[x] * rbt[x];
            kb[x][j] = be * kr[x] * pre[x];
            kg[x][j] = ki[x] * suf[x];
          }
          Quad<OpT>::store(Kr + r * LDK + c, kr[0], kr[1], kr[2], kr[3]);
          Quad<OpT>::store(Qr + r * LDK + c, qr[0], qr[1], qr[2], qr[3]);
          Quad<OpT>::store(Ki + r * LDK + c, ki[0], ki[1], ki[2], ki[3]);
          Quad<OpT>::store(Kinv + r * LDK + c, kv[0], kv[1], kv[2], kv[3]);
        }
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          Quad<OpT>::store(KbT + (c + x) * LDC + 16 * J + 4 * h, kb[x][0], kb[x][1], kb[x][2], kb[x][3]);
          Quad<OpT>::store(KgT + (c + x) * LDC + 16 * J + 4 * h, kg[x][0], kg[x][1], kg[x][2], kg[x][3]);
        }
      }
    }
    // The next chunk's gate loads.  With four blocks, waves 2.. issue theirs in
    // the second level of the off-diagonal solve below, where only waves 0
    // and 1 compute: issued here by all eight waves, the loads queue in the
    // CU's address unit and the last waves reach the barrier ~1.7k cycles
    // late.  (In the first level they would queue behind the value loads.)
    if (NB != 4 || wave < 2) fetch_gates(more ? t0 + C : t0);   // waves 2.. issue theirs later
    lds_barrier();

    // ================= AP + SD: gated K K^T (-> L in TT) and Q K^T (-> P) tiles.
    // Wave R < NB computes the diagonal pair (R, R) and inverts the 16x16
    // block I + L_RR straight away (its own LDS writes, no barrier); the
    // other waves compute the off-diagonal pairs meanwhile.
    {
      const Lane ln = lane_now();
      // which: 0 both tiles, 1 the A tile only, 2 the P tile only
      auto store_tiles = [&](int R, int I, const f32x4& accA, const f32x4& accP, int which = 0) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int rl = 4 * ln.g + rr, r = 16 * R + rl, i = 16 * I + ln.i;
          const bool diag = (I == R);
          const float a = (diag && ln.i >= rl) ? 0.f : accA[rr];
          const float pv = (diag && ln.i > rl) ? 0.f : accP[rr];
          if (which != 2) TT[r * LDT + i] = sBE[r] * a;
          if (which != 1) PP[r * LDC + i] = Ty<OpT>::from_f32(pv);
        }
      };
      if (wave < NB) {
        const int R = wave;
        f32x4 accA, accP;
        if constexpr (kScalar) {
          // decay from column i to row r inside block R: the gates of rows
          // i+1 .. r, multiplied out (no division, no underflow short of the
          // true value's)
          mma_k2<OpT>(accA, accP, 0, DK, Src<OpT>{Kr + 16 * R * LDK, LDK, ln},
                      Src<OpT>{Qr + 16 * R * LDK, LDK, ln}, Src<OpT>{Kr + 16 * R * LDK, LDK, ln});
          const float* ar = sRowA + 16 * R;
          float p = 1.f;
#pragma unroll
          for (int j = 1; j < 16; ++j)
            if (j > ln.i && j < 4 * ln.g) p *= ar[j];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int rl = 4 * ln.g + rr;
            if (rl > ln.i) p *= ar[rl];
            accA[rr] *= p;
            accP[rr] *= p;
          }
        } else {
          mma_k2<OpT>(accA, accP, 0, DK, Src<OpT>{Kr + 16 * R * LDK, LDK, ln},
                      Src<OpT>{Qr + 16 * R * LDK, LDK, ln}, Src<OpT>{Kinv + 16 * R * LDK, LDK, ln});
        }
        if (!kScalar && sFL[R]) {
          // Channels whose block decay fell below 2^-100: exact pairwise
          // products of alpha on the vector units.
          const size_t cb = (row0 + static_cast<size_t>(t0 + 16 * R) * H) * DK;
          const int jmax = T - 1 - (t0 + 16 * R);
          // prologue on single elements: feature map and 1 / row norm
          auto feat = [&](const E* src, int row, int kq) {
            float x = Ty<OpT>::to_f32(src[cb + row * rsK]);
            if (qk_silu) x = Ty<OpT>::to_f32(Ty<OpT>::from_f32(silu_f(x)));
            if (qk_norm) {
              const int r = 16 * R + row;
              float n = sNRM[kq * C + r];
              if constexpr (DK > 64) n += sNRM[(2 + kq) * C + r];
              x *= inv_l2(n);
            }
            return x;
          };
          auto gate = [&](int row, int c) {
            if constexpr (kLogit) {
              return gate_from_logit(Ty<OpT>::to_f32(glogit[cb + row * rsK + c]));
            } else if constexpr (kScalar) {
              const size_t tr = row0 + static_cast<size_t>(t0 + 16 * R + row) * H;
              return has_gate ? galpha[tr] : 1.f;
            } else {
              return galpha[cb + row * rsK + c];
            }
          };
          for (int c = 0; c < DK; ++c) {
            if (sBT[R * DK + c] >= kUnsafeBlockDecay) continue;
            const float ki = (ln.i <= jmax) ? feat(gk + c, ln.i, 0) : 0.f;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const int rl = 4 * ln.g + rr;
              if (ln.i > rl) continue;
              float ratio = 1.f;
              for (int j = ln.i + 1; j <= rl; ++j)
                ratio *= (j <= jmax) ? gate(j, c) : 1.f;
              const float kr = (rl <= jmax) ? feat(gk + c, rl, 0) : 0.f;
              const float qr = (rl <= jmax) ? feat(gq + c, rl, 1) : 0.f;
              accA[rr] += kr * ki * ratio;
              accP[rr] += qr * ki * ratio;
            }
          }
        }
        store_tiles(R, R, accA, accP);
        wave_fence();
        // Forward substitution for (I + L_RR) Y_RR = I, one column per lane of
        // the first lane group, column-oriented so the updates are independent.
        if (ln.g == 0) {
          const int j = ln.i;
          const float* Lb = TT + 16 * R * LDT + 16 * R;
          float y[16], acc[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
          for (int m = 0; m < 16; ++m) {
            y[m] = (m < j) ? 0.f : ((m == j) ? 1.f : -acc[m]);
#pragma unroll
            for (int r = m + 1; r < 16; ++r) acc[r] += Lb[r * LDT + m] * y[m];
          }
          wave_fence();
          // (Yb shares LDS with the MID scale table, which other waves may
          // still be reading in this phase: Yb is filled after the barrier.)
#pragma unroll
          for (int r = 0; r < 16; ++r) TT[(16 * R + r) * LDT + 16 * R + j] = y[r];

        }
      } else {
        // off-diagonal pair p -> (R, I), R > I; which as in store_tiles
        auto off_pair = [&](int p, auto which_c) {
          constexpr int which = decltype(which_c)::value;
          int R = 1, rem = p;
          while (rem >= R) { rem -= R; ++R; }
          const int I = rem;
          f32x4 accA = zero4(), accP = zero4();
          const Src<OpT> sKr{Kr + 16 * R * LDK, LDK, ln}, sQr{Qr + 16 * R * LDK, LDK, ln};
          auto run = [&](auto sb) {
            if constexpr (which == 0) mma_k2<OpT>(accA, accP, 0, DK, sKr, sQr, sb);
            else if constexpr (which == 1) accA = mma_k<OpT>(0, DK, sKr, sb);
            else accP = mma_k<OpT>(0, DK, sQr, sb);
          };
          if constexpr (kScalar) {
            // rows i+1 .. r = the rest of block I, the blocks between, and
            // block R through r
            run(Src<OpT>{Kr + 16 * I * LDK, LDK, ln});
            const float m = sRowMID[R * NB + I] * sRowH[16 * I + ln.i];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const float g = sRowF[16 * R + 4 * ln.g + rr] * m;
              accA[rr] *= g;
              accP[rr] *= g;
            }
          } else if (R == I + 1) {
            run(Src<OpT>{Ki + 16 * I * LDK, LDK, ln});
          } else {
            run(SrcScaled<OpT>{Ki + 16 * I * LDK, LDK, sMID + (R * NB + I) * DK, ln});
          }
          store_tiles(R, I, accA, accP, which);
        };
        if constexpr (NB == 4 && NW == 8 && !kPrep) {
          // six pairs, twelve products, on four waves: each wave one whole
          // pair and one product of pairs 4 and 5 (the A tiles on waves 4
          // and 5, the P tiles on waves 6 and 7), three products per wave
          // instead of four on two waves and two on the others.  (Fused
          // kernel only: B=8 H=32 T=8192 1142 -> 1116 us; the prep kernel,
          // which carries more registers here, measured 1-2% slower.)
          const int w = wave - NB;
          off_pair(w, std::integral_constant<int, 0>{});
          if (w < 2) off_pair(4 + w % 2, std::integral_constant<int, 1>{});
          else off_pair(4 + w % 2, std::integral_constant<int, 2>{});
        } else {
          for (int p = wave - NB; p < Cf::NAP - NB; p += NW - NB) {
            int R = 1, rem = p;
            while (rem >= R) { rem -= R; ++R; }
            const int I = rem;
            f32x4 accA, accP;
            const Src<OpT> sKr{Kr + 16 * R * LDK, LDK, ln}, sQr{Qr + 16 * R * LDK, LDK, ln};
            if constexpr (kScalar) {
              mma_k2<OpT>(accA, accP, 0, DK, sKr, sQr, Src<OpT>{Kr + 16 * I * LDK, LDK, ln});
              const float m = sRowMID[R * NB + I] * sRowH[16 * I + ln.i];
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) {
                const float g = sRowF[16 * R + 4 * ln.g + rr] * m;
                accA[rr] *= g;
                accP[rr] *= g;
              }
            } else if (R == I + 1) {
              mma_k2<OpT>(accA, accP, 0, DK, sKr, sQr, Src<OpT>{Ki + 16 * I * LDK, LDK, ln});
            } else {
              mma_k2<OpT>(accA, accP, 0, DK, sKr, sQr,
                          SrcScaled<OpT>{Ki + 16 * I * LDK, LDK, sMID + (R * NB + I) * DK, ln});
            }
            store_tiles(R, I, accA, accP);
          }
        }
      }
    }
    // With four blocks and the substitution below, waves 2, 3, 6 and 7 wait
    // here for waves 4 and 5 (two off-diagonal pairs each): they issue their
    // next-chunk gate loads now; waves 4 and 5 issue theirs in WU.
    if constexpr (kSubst) {
      if (NB == 4 && wave >= 2 && wave != 4 && wave != 5) fetch_gates(more ? t0 + C : t0);
    }
    lds_barrier();

    // ================= SO: stage beta V (transposed) for U~.  With fp32
    // operands, then the off-diagonal blocks of Y, one block row per barrier:
    //   Y_RI = -Y_RR * sum_{J=I}^{R-1} L_RJ Y_JI
    // (L stays in TT; off-diagonal Y goes to YF (fp32) and to Yb).  With bf16
    // operands Y is never formed off the diagonal: WU solves for W and U~ by
    // blocked substitution instead.
#pragma unroll
    for (int it = 0; it < Cf::NVT; ++it) {
      const int item = tid + NTH * it;
      if (Cf::NVI % NTH == 0 || item < Cf::NVI) {
        const ItemPos ip = item_pos<DVT / Cf::VEC>(item);
        const int h = ip.h, J = ip.J, cc = Cf::VEC * ip.v;
        const int r0 = 16 * J + 4 * h;
        const float b0 = sBE[r0], b1 = sBE[r0 + 1], b2 = sBE[r0 + 2], b3 = sBE[r0 + 3];
#pragma unroll
        for (int x = 0; x < Cf::VEC; ++x)
          Quad<OpT>::store(VbT + (cc + x) * LDC + r0, b0 * vec_elem<OpT>(gvv[it][0], x),
                           b1 * vec_elem<OpT>(gvv[it][1], x), b2 * vec_elem<OpT>(gvv[it][2], x),
                           b3 * vec_elem<OpT>(gvv[it][3], x));
      }
    }
    fetch_values(more ? t0 + C : t0);
    if constexpr (kSubst) {
      // -L_RJ and Y_RR from TT as bf16 A fragments (LF), one 16x16 block per
      // wave at a time: lane 16 g + i converts row i, columns 4g .. 4g + 3.
      {
        const int lane = tid % kWave;
        const int gi = lane % 16, gg = lane / 16;
        for (int f = wave; f < kNLF + NB; f += NW) {
          int R = f - kNLF, J = R;   // a Y_RR fragment ...
          if (f < kNLF) {            // ... or the off-diagonal block (R, J), f = yf_block(R, J)
            R = 1;
            int rem = f;
            while (rem >= R) { rem -= R; ++R; }
            J = rem;
          }
          const float4 v = *reinterpret_cast<const float4*>(TT + (16 * R + gi) * LDT + 16 * J + 4 * gg);
          const float sg = f < kNLF ? -1.f : 1.f;
          *reinterpret_cast<bf16x4*>(LF + f * 256 + 4 * lane) =
              bf16_quad(sg * v.x, sg * v.y, sg * v.z, sg * v.w);
        }
      }
      lds_barrier();   // beta V staged, the L and Y_RR fragments in LF
    } else {
    // diagonal blocks of Y into the operand-type copy
    for (int x = tid; x < NB * 256; x += NTH) {
      const int R = x / 256, r = (x % 256) / 16, j = x % 16;
      Yb[(16 * R + r) * LDC + 16 * R + j] = Ty<OpT>::from_f32(TT[(16 * R + r) * LDT + 16 * R + j]);
    }
    if constexpr (NB == 4) {
      // Four blocks: two levels instead of three.  Level 1: Y10 and Y32, the
      // off-diagonal blocks inside each half.  Level 2: the lower-left half
      // block  Y[23][01] = -Y[23][23] (L[23][01] Y[01][01]),  one wave per
      // block column c: M_Rc = L_R0 Y_0c + L_R1 Y_1c (R = 2, 3), then
      // Y_2c = -Y22 M_2c,  Y_3c = -(Y32 M_2c + Y33 M_3c).
      const Lane ln = lane_now();
      auto ydiag = [&](int J) { return SrcColF32{TT + 16 * J * LDT + 16 * J, LDT, ln}; };
      auto lsrc = [&](int R, int J) { return Src<float>{TT + 16 * R * LDT + 16 * J, LDT, ln}; };
      auto put_y = [&](int R, int I, const f32x4& y, bool keep_f32) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int rl = 4 * ln.g + rr;
          if (keep_f32) YF[yf_block(R, I) * 16 * LDZ + rl * LDZ + ln.i] = -y[rr];
          Yb[(16 * R + rl) * LDC + 16 * I + ln.i] = Ty<OpT>::from_f32(-y[rr]);
        }
      };
      if (wave < 2) {
        const int I = 2 * wave, R = I + 1;   // (1, 0) or (3, 2)
        f32x4 z = zero4();
        mma_f32(z, 0, 16, lsrc(R, I), ydiag(I));
        float* zb = ZB + wave * 16 * LDZ;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) zb[(4 * ln.g + rr) * LDZ + ln.i] = z[rr];
        wave_fence();
        f32x4 y = zero4();
        mma_f32(y, 0, 16, lsrc(R, R), SrcColF32{zb, LDZ, ln});
        put_y(R, I, y, true);
      }
      lds_barrier();
      if (wave >= 2) fetch_gates(more ? t0 + C : t0);   // idle waves (see G2)
      if (wave < 2) {
        const int c = wave;
        // Y_1c: Y10 (fp32 copy) for c = 0, Y11 (diagonal) for c = 1; Y_0c = 0 for c = 1
        const SrcColF32 y1c = (c == 0) ? SrcColF32{YF + yf_block(1, 0) * 16 * LDZ, LDZ, ln} : ydiag(1);
        float* m2 = ZB + (2 * c) * 16 * LDZ;
        float* m3 = ZB + (2 * c + 1) * 16 * LDZ;
        f32x4 a2 = zero4(), a3 = zero4();
        if (c == 0) {
          mma_f32(a2, 0, 16, lsrc(2, 0), ydiag(0));
          mma_f32(a3, 0, 16, lsrc(3, 0), ydiag(0));
        }
        mma_f32(a2, 0, 16, lsrc(2, 1), y1c);
        mma_f32(a3, 0, 16, lsrc(3, 1), y1c);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          m2[(4 * ln.g + rr) * LDZ + ln.i] = a2[rr];
          m3[(4 * ln.g + rr) * LDZ + ln.i] = a3[rr];
        }
        wave_fence();
        f32x4 y2 = zero4(), y3 = zero4();
        mma_f32(y2, 0, 16, lsrc(2, 2), SrcColF32{m2, LDZ, ln});
        // Y32 sits in YF (-Y32 stored as Y32 there: YF holds the blocks of Y)
        mma_f32(y3, 0, 16, Src<float>{YF + yf_block(3, 2) * 16 * LDZ, LDZ, ln}, SrcColF32{m2, LDZ, ln});
        mma_f32(y3, 0, 16, lsrc(3, 3), SrcColF32{m3, LDZ, ln});
        put_y(2, c, y2, false);
        put_y(3, c, y3, false);
      }
      lds_barrier();
    } else {
    for (int R = 1; R < NB; ++R) {
      const Lane ln = lane_now();
      for (int I = wave; I < R; I += NW) {
        f32x4 z = zero4();
        for (int J = I; J < R; ++J) {
          const float* yj = (J == I) ? TT + 16 * I * LDT + 16 * I : YF + yf_block(J, I) * 16 * LDZ;
          const int ldy = (J == I) ? LDT : LDZ;
          mma_f32(z, 0, 16, Src<float>{TT + 16 * R * LDT + 16 * J, LDT, ln},
                  SrcColF32{yj, ldy, ln});
        }
        float* zb = ZB + I * 16 * LDZ;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) zb[(4 * ln.g + rr) * LDZ + ln.i] = z[rr];
        wave_fence();
        f32x4 y = zero4();
        mma_f32(y, 0, 16, Src<float>{TT + 16 * R * LDT + 16 * R, LDT, ln}, SrcColF32{zb, LDZ, ln});
        float* yf = YF + yf_block(R, I) * 16 * LDZ;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int rl = 4 * ln.g + rr;
          yf[rl * LDZ + ln.i] = -y[rr];
          Yb[(16 * R + rl) * LDC + 16 * I + ln.i] = Ty<OpT>::from_f32(-y[rr]);
        }
      }
      lds_barrier();
    }
    if (NB == 1) lds_barrier();
    }
    }   // !kSubst

    // Y as a matrix-core operand (a copy in the operand type).
    auto ysrc = [&](int R, const Lane& ln) { return Src<OpT>{Yb + 16 * R * LDC, LDC, ln}; };

    // ================= WU: W = Y (beta K E) (stored row-major) and U~ = Y (beta V)
    f32x4 Ureg[UM::RA][UM::CA];
    if constexpr (kSubst) {
      // (I + L) [W | U~] = [beta K E | beta V], block row by block row:
      //   X_R = beta (K E | V)_R - sum_{J<R} L_RJ [W | U~]_J,  [W | U~]_R = Y_RR X_R
      // with L_RJ and Y_RR = (I + L_RR)^-1 from TT.  One wave owns whole
      // 16-column tiles of [U~ | W] over every block row, so the solve needs
      // no barrier: a 16x16x16 matrix-core result sits in exactly the lane
      // layout of the next product's B operand (lane (g, i) holds rows 4g..4g+3
      // of column i), and the solved blocks stay in registers as bf16 B
      // operands for the block rows below.  U~ tiles come first so that, with
      // a 128-column slab, wave w owns U~ column tile w: the tile the output
      // map UM gives it, so U~ stays in fp32 registers.  Otherwise U~ goes
      // back over beta V (bf16, in place) for the UM owners.
      constexpr int NCOL = NJ + Cf::NCB;
      constexpr int NCW = (NCOL + NW - 1) / NW;   // column tiles per wave
      constexpr bool kUdirect = NJ == NW && UM::RA == NB && UM::CA == 1 && UM::WC == NW;
      const Lane ln = lane_now();
      // -L_RJ and Y_RR as bf16 A operands, shared by this wave's columns, and
      // every column's right-hand side, all loaded before the first product so
      // that the products of the columns interleave without waiting on LDS.
      bf16x4 la[kNLF + 1], ya[NB];
      {
        const int lane = tid % kWave;
#pragma unroll
        for (int f = 0; f < kNLF; ++f) la[f] = *reinterpret_cast<const bf16x4*>(LF + f * 256 + 4 * lane);
#pragma unroll
        for (int R = 0; R < NB; ++R)
          ya[R] = *reinterpret_cast<const bf16x4*>(LF + (kNLF + R) * 256 + 4 * lane);
      }
      E* xs[NCW];
      bool isU[NCW], live[NCW];
      f32x4 rhs[NCW][NB];
#pragma unroll
      for (int ci = 0; ci < NCW; ++ci) {
        const int col = wave + NW * ci;
        live[ci] = NCOL % NW == 0 || col < NCOL;
        const int cc = live[ci] ? col : 0;   // a dead slot reads column 0 and stores nothing
        isU[ci] = cc < NJ;
        xs[ci] = (isU[ci] ? VbT + 16 * cc * LDC : KbT + 16 * (cc - NJ) * LDC) + ln.i * LDC +
                 4 * ln.g;
#pragma unroll
        for (int R = 0; R < NB; ++R) rhs[ci][R] = Acc4<OpT>::cvt(Acc4<OpT>::load(xs[ci] + 16 * R));
      }
      // Q E = Q F * (decay of the blocks before), in place (P is done with Q F);
      // independent LDS work that overlaps the products below.
      {
        constexpr int NQ = C * DK / 8;   // 16-byte units of 8 elements
        auto qe = [&](int x) {
          const int r = x / (DK / 8), c = 8 * (x % (DK / 8));
          u32x4* qp = reinterpret_cast<u32x4*>(Qr + r * LDK + c);
          float4 p0, p1;
          if constexpr (kScalar) {
            const float e = sRowE[r];
            p0 = p1 = make_float4(e, e, e, e);
          } else {
            const float4* pr = reinterpret_cast<const float4*>(sPRE + (r / 16) * DK + c);
            p0 = pr[0];
            p1 = pr[1];
          }
          const u32x4 v = *qp;
          *qp = u32x4{pack_bf16x2(vec_elem<OpT>(v, 0) * p0.x, vec_elem<OpT>(v, 1) * p0.y),
                      pack_bf16x2(vec_elem<OpT>(v, 2) * p0.z, vec_elem<OpT>(v, 3) * p0.w),
                      pack_bf16x2(vec_elem<OpT>(v, 4) * p1.x, vec_elem<OpT>(v, 5) * p1.y),
                      pack_bf16x2(vec_elem<OpT>(v, 6) * p1.z, vec_elem<OpT>(v, 7) * p1.w)};
        };
        if constexpr (NQ % NTH == 0) {
#pragma unroll
          for (int k = 0; k < NQ / NTH; ++k) qe(tid + NTH * k);
        } else {
          for (int x = tid; x < NQ; x += NTH) qe(x);
        }
      }
      bf16x4 ob[NCW][NB];
#pragma unroll
      for (int R = 0; R < NB; ++R) {
        f32x4 out[NCW];
#pragma unroll
        for (int ci = 0; ci < NCW; ++ci) {
          f32x4 x = rhs[ci][R];
#pragma unroll
          for (int J = 0; J < R; ++J) x = mfma<OpT, 16>(la[yf_block(R, J)], ob[ci][J], x);
          out[ci] = mfma<OpT, 16>(ya[R], bf16_quad(x[0], x[1], x[2], x[3]), zero4());
          ob[ci][R] = bf16_quad(out[ci][0], out[ci][1], out[ci][2], out[ci][3]);
        }
#pragma unroll
        for (int ci = 0; ci < NCW; ++ci) {
          if (!live[ci]) continue;
          if (isU[ci]) {
            if constexpr (kUdirect) {
              if (ci == 0) Ureg[R][0] = out[ci];   // col == wave == UM::col0(wave)
            } else {
              Acc4<OpT>::store(xs[ci] + 16 * R, out[ci]);
            }
          } else {
            // W[16R + 4g + r][16 (col - NJ) + i], row-major for the matrix-core A operand
            E* wd = Wm + (16 * R + 4 * ln.g) * LDK + 16 * (wave + NW * ci - NJ) + ln.i;
#pragma unroll
            for (int r = 0; r < 4; ++r) wd[r * LDK] = Ty<OpT>::from_f32(out[ci][r]);
          }
        }
      }
      // gate prefetch of waves 4 and 5, the slowest in the A/P phase (see there)
      if (NB == 4 && (wave == 4 || wave == 5)) fetch_gates(more ? t0 + C : t0);
      lds_barrier();
      if constexpr (!kUdirect) {
#pragma unroll
        for (int a = 0; a < UM::RA; ++a)
#pragma unroll
          for (int bb = 0; bb < UM::CA; ++bb) {
            Ureg[a][bb] = zero4();
            if (UM::active(wave)) {
              const int R = UM::row0(wave) + a, Jb = UM::col0(wave) + bb;
              Ureg[a][bb] = Acc4<OpT>::cvt(
                  Acc4<OpT>::load(VbT + (16 * Jb + ln.i) * LDC + 16 * R + 4 * ln.g));
            }
          }
        // the scan below writes S^T over beta V: every wave must have read U~
        if constexpr (!kPrep) lds_barrier();
      }
    } else {
    // Q E = Q F * (decay of the blocks before), in place: P is done with Q F.
    for (int x = tid; x < C * DK / 2; x += NTH) {
      const int r = x / (DK / 2), c = 2 * (x % (DK / 2));
      PT* qp = reinterpret_cast<PT*>(Qr + r * LDK + c);
      const float p0 = kScalar ? sRowE[r] : sPRE[(r / 16) * DK + c];
      const float p1 = kScalar ? sRowE[r] : sPRE[(r / 16) * DK + c + 1];
      const PT v = *qp;
      *qp = Pair<OpT>::pack(Pair<OpT>::get(v, 0) * p0, Pair<OpT>::get(v, 1) * p1);
    }
    {
      const Lane ln = lane_now();
      // W^T tiles (Cb, R) cost 16 (R + 1) of contraction: tile t = wave + NW i
      // is (t % NCB, t / NCB), so a wave takes every row block of its key
      // channels and the waves' totals match (one R per wave left the wave
      // pair of one SIMD with 4x the work of another).
      constexpr int NWT = Cf::NCB * NB;
#pragma unroll
      for (int i = 0; i < (NWT + NW - 1) / NW; ++i) {
        const int t = wave + NW * i;
        if (NWT % NW == 0 || t < NWT) {
          const int Cb = t % Cf::NCB, R = t / Cf::NCB;
          const f32x4 acc =
              mma_k<OpT>(0, 16 * (R + 1), Src<OpT>{KbT + 16 * Cb * LDC, LDC, ln}, ysrc(R, ln));
          // acc[rr] = W^T[c = 16Cb + 4g + rr][r = 16R + i]
          Quad<OpT>::store(Wm + (16 * R + ln.i) * LDK + 16 * Cb + 4 * ln.g, acc[0], acc[1], acc[2],
                           acc[3]);
        }
      }
#pragma unroll
      for (int a = 0; a < UM::RA; ++a) {
#pragma unroll
        for (int bb = 0; bb < UM::CA; ++bb) Ureg[a][bb] = zero4();
        if (UM::active(wave)) {
          const int R = UM::row0(wave) + a;
          mma_row<OpT, UM::CA>(Ureg[a], 0, 16 * (R + 1), ysrc(R, ln),
                               Src<OpT>{VbT + 16 * UM::col0(wave) * LDC, LDC, ln}, 16 * LDC);
        }
      }
    }
    lds_barrier();
    }   // !kSubst

    if constexpr (kPrep) {
      // chunk record -> workspace: operand packets, decay, U~ (this slab is all of dv)
      using RC = RecCfg<OpT, DK, C>;
      char* rec = gws + (static_cast<size_t>(chain) * segn + (ch - seg0)) * RC::bytes(DV);
      E* rw = reinterpret_cast<E*>(rec);
      copy_packets<OpT, RC::KSD, NB, RC::NKD, NTH>(rw + RC::kW, Wm, LDK, tid);
      copy_packets<OpT, RC::KSD, NB, RC::NKD, NTH>(rw + RC::kQ, Qr, LDK, tid);
      copy_packets<OpT, RC::KSC, Cf::NCB, RC::NKC, NTH>(rw + RC::kKG, KgT, LDC, tid);
      copy_packets<OpT, RC::KSC, NB, RC::NKC, NTH>(rw + RC::kP, PP, LDC, tid);
      {
        // every thread stores (threads past the decay vector repeat its last
        // 16 bytes): one store per thread, no branch
        const int v = min(tid, DK / 4 - 1);
        reinterpret_cast<float4*>(rec + RC::kGcByte)[v] = reinterpret_cast<const float4*>(sGC)[v];
      }
      if (UM::WR * UM::WC == NW || UM::active(wave)) {
        const int lane = tid % kWave;
        E* ru = reinterpret_cast<E*>(rec + RC::kUByte);
#pragma unroll
        for (int a = 0; a < UM::RA; ++a)
#pragma unroll
          for (int bb = 0; bb < UM::CA; ++bb) {
            const int R = UM::row0(wave) + a, Jb = UM::col0(wave) + bb;
            Acc4<OpT>::store(ru + (static_cast<size_t>(R * NJ + Jb) * kWave + lane) * 4, Ureg[a][bb]);
          }
      }
      continue;
    }

    // ================= scan: U = U~ - W S,  O = (Q E) S + P U,  S update
    if (SM::active(wave)) {
      const Lane ln = lane_now();
#pragma unroll
      for (int a = 0; a < SM::RA; ++a)
#pragma unroll
        for (int bb = 0; bb < SM::CA; ++bb) {
          const int Cb = SM::row0(wave) + a, Jb = SM::col0(wave) + bb;
          E* dst = ST + (16 * Jb + ln.i) * LDK + 16 * Cb + 4 * ln.g;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) dst[rr] = Ty<OpT>::from_f32(Sreg[a][bb][rr]);
        }
    }
    lds_barrier();
    // One column tile of S^T (and of U^T) per wave, the same tile for the
    // output and the state maps: its matrix-core B fragments load from LDS
    // once per chunk and serve every row block, instead of once per row
    // block (the state phases are bound by LDS bandwidth).
    constexpr bool kHoldB = kBF && UM::WR == 1 && SM::WR == 1 && UM::CA == 1 && SM::CA == 1 &&
                            UM::WC == SM::WC && DK % 32 == 0 && C % 32 == 0;
    using FB = typename Frag<OpT, kBF ? 32 : 4>::T;
    FB sB[kHoldB ? DK / 32 : 1];
    if constexpr (kHoldB) {
      if (UM::active(wave)) {
        const Lane ln = lane_now();
        const Src<OpT> sb{ST + 16 * UM::col0(wave) * LDK, LDK, ln};
#pragma unroll
        for (int k = 0; k < DK / 32; ++k) sB[k] = sb.template get<32>(32 * k);
      }
    }
    if (UM::active(wave)) {
      const Lane ln = lane_now();
#pragma unroll
      for (int a = 0; a < UM::RA; ++a) {
        const int R = UM::row0(wave) + a;
        f32x4 x[UM::CA];
        if constexpr (kHoldB) {
          const Src<OpT> wa{Wm + 16 * R * LDK, LDK, ln};
          x[0] = zero4();
#pragma unroll
          for (int k = 0; k < DK / 32; ++k) x[0] = mfma<OpT, 32>(wa.template get<32>(32 * k), sB[k], x[0]);
        } else {
          mma_row<OpT, UM::CA>(x, 0, DK, Src<OpT>{Wm + 16 * R * LDK, LDK, ln},
                               Src<OpT>{ST + 16 * UM::col0(wave) * LDK, LDK, ln}, 16 * LDK);
        }
        // U = U~ - W S, staged transposed for the products over tokens
#pragma unroll
        for (int bb = 0; bb < UM::CA; ++bb) {
          const int Jb = UM::col0(wave) + bb;
          E* dst = UT + (16 * Jb + ln.i) * LDC + 16 * R + 4 * ln.g;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) dst[rr] = Ty<OpT>::from_f32(Ureg[a][bb][rr] - x[bb][rr]);
        }
      }
    }
    lds_barrier();
    // kStates (the chunked backward's forward pass): the chunk states are
    // stored and the output products and stores are left out
    constexpr bool want_o = !kStates;
    E* po = want_o ? go + (row0 + static_cast<size_t>(t0) * H) * DV + j0 : nullptr;
    const int nrows = min(C, T - t0);
    {
      // O = (Q E) S + P U
      const Lane ln = lane_now();
      FB uB[kHoldB ? C / 32 : 1];
      if constexpr (kHoldB) {
        if (UM::active(wave)) {
          const Src<OpT> ub{UT + 16 * UM::col0(wave) * LDC, LDC, ln};
#pragma unroll
          for (int k = 0; k < C / 32; ++k) uB[k] = ub.template get<32>(32 * k);
        }
      }
      if (want_o && UM::active(wave)) {
#pragma unroll
        for (int a = 0; a < UM::RA; ++a) {
          const int R = UM::row0(wave) + a;
          f32x4 o[UM::CA], pu[UM::CA];
          if constexpr (kHoldB) {
            // P's blocks right of the diagonal are zeros in LDS, so the
            // product over tokens may run to the next multiple of 32
            const Src<OpT> qa{Qr + 16 * R * LDK, LDK, ln}, pa{PP + 16 * R * LDC, LDC, ln};
            o[0] = zero4();
            pu[0] = zero4();
#pragma unroll
            for (int k = 0; k < DK / 32; ++k) o[0] = mfma<OpT, 32>(qa.template get<32>(32 * k), sB[k], o[0]);
#pragma unroll
            for (int k = 0; k < C / 32; ++k)
              if (32 * k < 16 * (R + 1)) pu[0] = mfma<OpT, 32>(pa.template get<32>(32 * k), uB[k], pu[0]);
          } else {
            mma_row<OpT, UM::CA>(o, 0, DK, Src<OpT>{Qr + 16 * R * LDK, LDK, ln},
                                 Src<OpT>{ST + 16 * UM::col0(wave) * LDK, LDK, ln}, 16 * LDK);
            mma_row<OpT, UM::CA>(pu, 0, 16 * (R + 1), Src<OpT>{PP + 16 * R * LDC, LDC, ln},
                                 Src<OpT>{UT + 16 * UM::col0(wave) * LDC, LDC, ln}, 16 * LDC);
          }
#pragma unroll
          for (int bb = 0; bb < UM::CA; ++bb) add4(o[bb], pu[bb]);
#pragma unroll
          for (int bb = 0; bb < UM::CA; ++bb) {
            const int Jb = UM::col0(wave) + bb;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const int rl = 16 * R + 4 * ln.g + rr;
              if constexpr (kStageO) {
                OS[rl * LDO + 16 * Jb + ln.i] = Ty<OpT>::from_f32(o[bb][rr]);
              } else {
                if (full || rl < nrows) po[rl * rsV + 16 * Jb + ln.i] = Ty<OpT>::from_f32(o[bb][rr]);
              }
            }
          }
        }
      }
      // the state this chunk starts from, fp32, in fragment order:
      // [chain][chunk][column tile][row block][lane][4], one 16-byte store
      // per block (the layout of the scan kernel's chunk states)
      if (kStates && SM::active(wave)) {
#pragma unroll
        for (int a = 0; a < SM::RA; ++a)
#pragma unroll
          for (int bb = 0; bb < SM::CA; ++bb) {
            const int Cb = SM::row0(wave) + a, jt = (j0 >> 4) + SM::col0(wave) + bb;
            float* dst = gSc + ((static_cast<size_t>(chain) * NC + ch) * (DV / 16) + jt) * DK * 16;
            *reinterpret_cast<float4*>(dst + (Cb * kWave + (tid & 63)) * 4) =
                make_float4(Sreg[a][bb][0], Sreg[a][bb][1], Sreg[a][bb][2], Sreg[a][bb][3]);
          }
      }
      // S <- Diag(decay of the chunk) S + (K E')^T U
      if (SM::active(wave)) {
#pragma unroll
        for (int a = 0; a < SM::RA; ++a) {
          const int Cb = SM::row0(wave) + a;
          f32x4 acc[SM::CA];
          if constexpr (kHoldB) {
            const Src<OpT> ka{KgT + 16 * Cb * LDC, LDC, ln};
            acc[0] = zero4();
#pragma unroll
            for (int k = 0; k < C / 32; ++k) acc[0] = mfma<OpT, 32>(ka.template get<32>(32 * k), uB[k], acc[0]);
          } else {
            mma_row<OpT, SM::CA>(acc, 0, C, Src<OpT>{KgT + 16 * Cb * LDC, LDC, ln},
                                 Src<OpT>{UT + 16 * SM::col0(wave) * LDC, LDC, ln}, 16 * LDC);
          }
          const float4 gc = *reinterpret_cast<const float4*>(sGC + 16 * Cb + 4 * ln.g);
#pragma unroll
          for (int bb = 0; bb < SM::CA; ++bb) {
            Sreg[a][bb][0] = gc.x * Sreg[a][bb][0] + acc[bb][0];
            Sreg[a][bb][1] = gc.y * Sreg[a][bb][1] + acc[bb][1];
            Sreg[a][bb][2] = gc.z * Sreg[a][bb][2] + acc[bb][2];
            Sreg[a][bb][3] = gc.w * Sreg[a][bb][3] + acc[bb][3];
          }
        }
      }
    }
    lds_barrier();
    if constexpr (kStageO) {
      // staged output rows -> HBM with 16-byte stores
      constexpr int VPR = DVT * static_cast<int>(sizeof(E)) / 16;   // vectors per row
      constexpr int EPV = 16 / static_cast<int>(sizeof(E));          // elements per vector
      for (int x = want_o ? tid : C * VPR; x < C * VPR; x += NTH) {
        const int r = x / VPR, cv = x % VPR;
        if (full || r < nrows)
          *reinterpret_cast<uint4*>(po + r * rsV + cv * EPV) =
              *reinterpret_cast<const uint4*>(OS + r * LDO + cv * EPV);
      }
    }
  }

  if (!kPrep && gST != nullptr && SM::active(wave)) {
    const Lane ln = lane_now();
#pragma unroll
    for (int a = 0; a < SM::RA; ++a)
#pragma unroll
      for (int bb = 0; bb < SM::CA; ++bb) {
        const int Cb = SM::row0(wave) + a, Jb = SM::col0(wave) + bb;
        float* dst = gST + static_cast<size_t>(chain) * DK * DV + j0 + 16 * Jb;
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(16 * Cb + 4 * ln.g + r) * DV + ln.i] = Sreg[a][bb][r];
      }
  }
}

// ----------------------------------------------------------------------------
// Host dispatch
// ----------------------------------------------------------------------------
template <typename OpT, int DK, int C, int DVT, int kIn, bool kStates = false>
hipError_t launch_one(const PrefillArgs& a) {
  using E = typename Ty<OpT>::Elem;
  const long chains = static_cast<long>(a.B) * a.H;
  dim3 grid(static_cast<unsigned>(chains * (a.dv / DVT)));
  hipLaunchKernelGGL((kda_prefill_kernel<OpT, DK, C, DVT, false, kIn, kStates>), grid,
                     dim3(PCfg<OpT, DK, C, DVT>::NTH), 0, static_cast<hipStream_t>(a.stream),
                     static_cast<const E*>(a.q), static_cast<const E*>(a.k),
                     static_cast<const E*>(a.v), a.gate, a.beta, a.S0,
                     kStates ? nullptr : static_cast<E*>(a.o), a.S_T, a.B, a.T, a.H, a.dv,
                     nullptr, 0, 0, 0, a.qk_map, 0, kStates ? a.chunk_states : nullptr);
  return hipGetLastError();
}

template <typename OpT, int DK, int C, int DVT>
constexpr bool fits() {
  return DVT <= 128 && PCfg<OpT, DK, C, DVT>::kLds <= kMaxLds;
}

// Slab width for the fused kernel.  Every slab of a chain repeats the
// chain's column-free chunk work, so a slab costs about (1 + DVT/300) units
// per chunk (measured at dk = dv = 128, C = 64: 10.8 us per chunk at DVT =
// 64, 12.7 us at 128), and the grid runs in rounds of one workgroup per CU.
// Pick the width that fits with the fewest rounds x cost, the wider on a tie:
// narrow slabs fill the chip when chains are few, and a width that would
// spill a second, partly empty round is avoided.
template <typename OpT, int DK, int C>
int pick_dvt(long chains, int dv) {
  constexpr long kCUs = 256;
  int best = 0;
  double best_cost = 0.0;
  for (int d = 16; d <= dv; d *= 2) {
    bool ok = false;
    if (d == 16) ok = fits<OpT, DK, C, 16>();
    if (d == 32) ok = fits<OpT, DK, C, 32>();
    if (d == 64) ok = fits<OpT, DK, C, 64>();
    if (d == 128) ok = fits<OpT, DK, C, 128>();
    if (!ok) continue;
    const long rounds = (chains * (dv / d) + kCUs - 1) / kCUs;
    const double cost = static_cast<double>(rounds) * (1.0 + d / 300.0);
    if (best == 0 || cost <= best_cost) {
      best = d;
      best_cost = cost;
    }
  }
  return best;
}

template <typename OpT, int DK, int C, int kIn>
hipError_t launch_c(const PrefillArgs& a) {
  const int dvt = pick_dvt<OpT, DK, C>(static_cast<long>(a.B) * a.H, a.dv);
  if (a.chunk_states != nullptr) {
    // chunk states without output: built for the chunked backward's
    // configuration only (bf16, dk = 128, C = 64, per-channel gates)
    if constexpr (std::is_same<OpT, bf16_t>::value && DK == 128 && C == 64 && kIn == kGateAlpha) {
      switch (dvt) {
        case 64: return launch_one<OpT, DK, C, 64, kIn, true>(a);
        case 128: return launch_one<OpT, DK, C, 128, kIn, true>(a);
      }
    }
    return hipErrorInvalidValue;
  }
  switch (dvt) {
    case 16: if constexpr (fits<OpT, DK, C, 16>()) return launch_one<OpT, DK, C, 16, kIn>(a); break;
    case 32: if constexpr (fits<OpT, DK, C, 32>()) return launch_one<OpT, DK, C, 32, kIn>(a); break;
    case 64: if constexpr (fits<OpT, DK, C, 64>()) return launch_one<OpT, DK, C, 64, kIn>(a); break;
    case 128: if constexpr (fits<OpT, DK, C, 128>()) return launch_one<OpT, DK, C, 128, kIn>(a); break;
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
