// Host-side launch descriptors shared by the C ABI (kda_api.hip) and the
// kernel translation units.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace kda {

// How the gate reaches a kernel (a compile-time switch of the kernels):
//   kGateAlpha   one alpha per key channel, fp32 (Kimi Delta Attention)
//   kGateLogit   one gate logit per key channel in the I/O type, with the
//                whole input prologue of kda_device.hpp
//   kGateScalar  one alpha per token and head, fp32, the same on every
//                channel (Gated DeltaNet), or none at all: alpha = 1
//                (DeltaNet) when the pointer is null
enum GateIn : int { kGateAlpha = 0, kGateLogit = 1, kGateScalar = 2 };

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* gate;   // per gate_in (GateIn): alpha, gate logits, or a scalar gate
  const float* beta;  // beta, or its logit with kGateLogit
  const float* S_in;
  void* o;
  float* S_out;
  int N, H, dk, dv;
  bool bf16;
  void* stream;
  int gate_in;        // GateIn (kda_device.hpp)
  int qk_map;         // QkMap, used with kGateLogit
};

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* gate;   // per gate_in (GateIn): alpha, gate logits, or a scalar gate
  const float* beta;  // beta, or its logit with kGateLogit
  const float* S0;   // may be null (zeros)
  void* o;
  float* S_T;        // may be null (not written)
  int B, T, H, dk, dv, C;
  bool bf16;
  void* stream;
  void* workspace;          // split path only (see prefill_workspace)
  size_t workspace_bytes;
  int gate_in;              // GateIn (kda_device.hpp)
  int qk_map;               // QkMap, used with kGateLogit
  // Split path: bytes of records per segment (0: the default budget).  The
  // same value must size the workspace (prefill_workspace).
  size_t segment_budget = 0;
  // When set, the state every chunk of C tokens starts from, fp32 in
  // matrix-core fragment order [B*H][ceil(T/C)][dv/16][dk/16][64][4] (lane
  // 16g + i holds rows 4g .. 4g+3 of a 16 x 16 block, column i), for the
  // chunked backward; o may then be null (the states alone: the split scan
  // neither reads the output's record parts nor writes o, the fused kernel
  // skips its output products).  The fused kernel writes them only with
  // per-channel gates (kGateAlpha).
  float* chunk_states = nullptr;
  // Take the split path whatever the chain count.
  bool force_split = false;
};

// The adjoint of one decode step (decode_backward.hip).
struct DecodeBwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  const float* S_in;
  const void* dO;
  const float* dS_new;
  void* g_q;          // gradients written: dq, dk, dv (I/O type), dalpha, dbeta, dS
  void* g_k;
  void* g_v;
  float* g_alpha;
  float* g_beta;
  float* g_S;         // may equal dS_new
  int N, H, dk, dv;
  bool bf16;
  void* stream;
  int gate_in = kGateAlpha;   // kGateScalar: alpha, g_alpha [N,H] (or both null)
};

hipError_t launch_decode(const DecodeArgs& a);
hipError_t launch_decode_backward(const DecodeBwdArgs& a);

// Backward of a whole prefill.  Gradients are float32; g_S0 may be null.
struct PrefillBwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  const float* S0;     // may be null (zeros)
  const void* dO;
  const float* dS_T;   // may be null (zeros)
  float* g_q;          // [B,T,H,dk]
  float* g_k;
  float* g_v;          // [B,T,H,dv]
  float* g_alpha;      // [B,T,H,dk]
  float* g_beta;       // [B,T,H]
  float* g_S0;         // [B,H,dk,dv] or null
  void* workspace;     // prefill_backward_workspace bytes
  int B, T, H, dk, dv;
  bool bf16;
  void* stream;
  int gate_in = kGateAlpha;   // kGateScalar: alpha, g_alpha [B,T,H] (or both null)
};
hipError_t launch_prefill_backward(const PrefillBwdArgs& a);
// The chunked backward (chunk_backward.hip): bf16, dk = dv = 128, one alpha
// per channel; 0 / hipErrorInvalidValue for anything else.
size_t prefill_backward_chunked_workspace(int B, int T, int H, int dk, int dv);
hipError_t launch_prefill_backward_chunked(const PrefillBwdArgs& a);

// The input prologue alone over `rows` rows of dk channels: forward (raw q,
// k, g, b -> q_hat, k_hat in the I/O type, alpha, beta fp32) or its adjoint
// (-> d_q, d_k, d_g, d_b, fp32).
struct PrologueArgs {
  const void* q;
  const void* k;
  const void* g;
  const float* b;
  void* q_hat;            // forward outputs
  void* k_hat;
  float* alpha;
  float* beta;
  const float* dq_hat;    // adjoint inputs
  const float* dk_hat;
  const float* dalpha;
  const float* dbeta;
  float* d_q;             // adjoint outputs
  float* d_k;
  float* d_g;
  float* d_b;
  int rows, dk;
  bool bf16;
  int qk_map;
  bool backward;
  void* stream;
};
hipError_t launch_prologue(const PrologueArgs& a);
size_t prefill_backward_workspace(int B, int T, int H, int dk, int dv);

// Returns hipErrorInvalidValue when no compiled kernel covers (dk, C, dtype).
hipError_t launch_prefill(const PrefillArgs& a);
bool prefill_supported(int dk, int dv, int C, bool bf16);
// Bytes of the fixed device scratch array of kda_prefill_chunked_noalloc.
constexpr size_t kNoallocScratchBytes = size_t{64} << 20;

// Device workspace bytes the prefill needs for these sizes (0: none), with
// segments of at most `budget` bytes of records (0: the default budget).
size_t prefill_workspace(int B, int T, int H, int dk, int dv, int C, bool bf16,
                         size_t budget = 0, bool force_split = false);

}  // namespace kda
