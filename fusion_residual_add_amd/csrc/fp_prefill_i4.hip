// 128 x 512 projection kernel instantiations: int4 weights (one scale per
// row and group of 128 k).
#include "fp_prefill.hpp"

namespace fp {

hipError_t launch_prefill_i4(const ProjArgs &a, unsigned grid, hipStream_t s) {
    return launch_prefill_t<ACT_BF16, 2>(a, grid, s);
}

}  // namespace fp
