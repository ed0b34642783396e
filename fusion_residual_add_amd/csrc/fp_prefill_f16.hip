// Prefill projection kernel instantiations: f16 weights.
#include "fp_prefill.hpp"

namespace fp {

void launch_prefill_f16(const ProjArgs &a, unsigned grid, hipStream_t s) {
    launch_prefill_t<ACT_F16, 0>(a, grid, s);
}

}  // namespace fp
