// Chunked-prefill kernels for f32 q/k/v/o and dk = 128.
#include "scan_kernel.hpp"

namespace kda {
KDA_PREFILL_INSTANCE(float, f32, 128)
}  // namespace kda
