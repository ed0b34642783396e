// Prefill projection kernel instantiations: bf16 weights.
#include "fp_prefill.hpp"

namespace fp {

hipError_t launch_prefill_bf16(const ProjArgs &a, unsigned grid, hipStream_t s) {
    return launch_prefill_t<ACT_BF16, 0>(a, grid, s);
}

}  // namespace fp
