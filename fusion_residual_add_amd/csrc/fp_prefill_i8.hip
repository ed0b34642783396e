// Prefill projection kernel instantiations: i8 weights.
#include "fp_prefill.hpp"

namespace fp {

hipError_t launch_prefill_i8(const ProjArgs &a, unsigned grid, hipStream_t s) {
    return launch_prefill_t<ACT_BF16, 1>(a, grid, s);
}

}  // namespace fp
