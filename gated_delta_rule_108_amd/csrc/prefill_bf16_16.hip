// Chunked-prefill kernels for bf16 q/k/v/o and dk = 16.
#include "scan_kernel.hpp"

namespace kda {
KDA_PREFILL_INSTANCE(bf16_t, bf16, 16)
}  // namespace kda
