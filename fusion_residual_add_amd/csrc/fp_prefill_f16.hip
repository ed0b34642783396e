// Prefill projection kernel instantiations: f16 weights, row-major or tile-packed.
#include "fp_prefill.hpp"

namespace fp {

hipError_t launch_prefill_f16(const ProjArgs &a, unsigned grid, hipStream_t s) {
    // tile-packed weights: the packed-order B tile (WQ 5)
    return a.w_layout ? launch_prefill_t<ACT_F16, 5>(a, grid, s) : launch_prefill_t<ACT_F16, 0>(a, grid, s);
}

}  // namespace fp
