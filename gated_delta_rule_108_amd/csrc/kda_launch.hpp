// Host-side launch descriptors shared by the C ABI (kda_api.hip) and the
// kernel translation units.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace kda {

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* gate;   // alpha (fp32), or gate logits g in the I/O type when logits
  const float* beta;  // beta, or its logit when logits
  const float* S_in;
  void* o;
  float* S_out;
  int N, H, dk, dv;
  bool bf16;
  void* stream;
  bool logits;        // run the input prologue (see kda_device.hpp)
  int qk_map;         // QkMap, used when logits
};

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* gate;   // alpha (fp32), or gate logits g in the I/O type when logits
  const float* beta;  // beta, or its logit when logits
  const float* S0;   // may be null (zeros)
  void* o;
  float* S_T;        // may be null (not written)
  int B, T, H, dk, dv, C;
  bool bf16;
  void* stream;
  void* workspace;          // split path only (see prefill_workspace)
  size_t workspace_bytes;
  bool logits;              // run the input prologue (see kda_device.hpp)
  int qk_map;               // QkMap, used when logits
};

hipError_t launch_decode(const DecodeArgs& a);

// Returns hipErrorInvalidValue when no compiled kernel covers (dk, C, dtype).
hipError_t launch_prefill(const PrefillArgs& a);
bool prefill_supported(int dk, int dv, int C, bool bf16);
// Device workspace bytes the prefill needs for these sizes (0: none).
size_t prefill_workspace(int B, int T, int H, int dk, int dv, int C, bool bf16);

}  // namespace kda
