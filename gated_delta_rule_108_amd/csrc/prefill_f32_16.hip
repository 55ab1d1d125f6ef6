// Chunked-prefill kernels for f32 q/k/v/o and dk = 16.
#include "scan_kernel.hpp"

namespace kda {
KDA_PREFILL_INSTANCE(float, f32, 16)
}  // namespace kda
