// Prefill projection kernel instantiations: bf16 weights, row-major or tile-packed.
#include "fp_prefill.hpp"

namespace fp {

hipError_t launch_prefill_bf16(const ProjArgs &a, unsigned grid, hipStream_t s) {
    // tile-packed weights: the packed-order B tile (WQ 5)
    return a.w_layout ? launch_prefill_t<ACT_BF16, 5>(a, grid, s) : launch_prefill_t<ACT_BF16, 0>(a, grid, s);
}

}  // namespace fp
