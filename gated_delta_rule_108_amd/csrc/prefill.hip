// Dispatch of kda_prefill_chunked over (element type, dk); the kernels are
// instantiated in prefill_<type>_<dk>.hip so they compile in parallel.
#include "scan_kernel.hpp"

namespace kda {

bool prefill_supported(int dk, int dv, int C, bool bf16) {
  switch (dk) {
    case 16: return bf16 ? prefill_supported_bf16_16(dv, C) : prefill_supported_f32_16(dv, C);
    case 32: return bf16 ? prefill_supported_bf16_32(dv, C) : prefill_supported_f32_32(dv, C);
    case 64: return bf16 ? prefill_supported_bf16_64(dv, C) : prefill_supported_f32_64(dv, C);
    case 128: return bf16 ? prefill_supported_bf16_128(dv, C) : prefill_supported_f32_128(dv, C);
  }
  return false;
}

size_t prefill_workspace(int B, int T, int H, int dk, int dv, int C, bool bf16, size_t budget,
                         bool force_split) {
  if (budget == 0) budget = kSegmentBudget;
  switch (dk) {
    case 16: return bf16 ? prefill_workspace_bf16_16(B, T, H, dv, C, budget, force_split) : prefill_workspace_f32_16(B, T, H, dv, C, budget, force_split);
    case 32: return bf16 ? prefill_workspace_bf16_32(B, T, H, dv, C, budget, force_split) : prefill_workspace_f32_32(B, T, H, dv, C, budget, force_split);
    case 64: return bf16 ? prefill_workspace_bf16_64(B, T, H, dv, C, budget, force_split) : prefill_workspace_f32_64(B, T, H, dv, C, budget, force_split);
    case 128: return bf16 ? prefill_workspace_bf16_128(B, T, H, dv, C, budget, force_split) : prefill_workspace_f32_128(B, T, H, dv, C, budget, force_split);
  }
  return 0;
}

hipError_t launch_prefill(const PrefillArgs& a) {
  switch (a.dk) {
    case 16: return a.bf16 ? launch_prefill_bf16_16(a) : launch_prefill_f32_16(a);
    case 32: return a.bf16 ? launch_prefill_bf16_32(a) : launch_prefill_f32_32(a);
    case 64: return a.bf16 ? launch_prefill_bf16_64(a) : launch_prefill_f32_64(a);
    case 128: return a.bf16 ? launch_prefill_bf16_128(a) : launch_prefill_f32_128(a);
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
