// Chunked-prefill kernels for bf16 q/k/v/o and dk = 32.
#include "scan_kernel.hpp"

namespace kda {
KDA_PREFILL_INSTANCE(bf16_t, bf16, 32)
}  // namespace kda
