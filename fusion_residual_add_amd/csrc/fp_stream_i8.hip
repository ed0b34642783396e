// Weight-streaming projection kernel instantiations: i8 weights.
#include "fp_stream.hpp"

namespace fp {

hipError_t launch_stream_i8(const StreamCfg &c, const ProjArgs &a, unsigned grid, hipStream_t s) {
    return launch_stream_t<ACT_BF16, 1>(c, a, grid, s);
}

}  // namespace fp
