// Weight-streaming projection kernel instantiations: int4 weights (one scale
// per row and group of 128 k).
#include "fp_stream.hpp"

namespace fp {

hipError_t launch_stream_i4(const StreamCfg &c, const ProjArgs &a, unsigned grid, hipStream_t s) {
    return launch_stream_t<ACT_BF16, 2>(c, a, grid, s);
}

}  // namespace fp
