// Prefill projection kernel instantiations: MXFP4 weights (bf16 activations).
#include "fp_prefill.hpp"

namespace fp {

hipError_t launch_prefill_mx(const ProjArgs &a, unsigned grid, hipStream_t s) {
    return launch_prefill_t<ACT_BF16, 3>(a, grid, s);
}

}  // namespace fp
