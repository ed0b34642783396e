// Weight-streaming projection kernel instantiations: f16 weights.
#include "fp_stream.hpp"

namespace fp {

hipError_t launch_stream_f16(const StreamCfg &c, const ProjArgs &a, unsigned grid, hipStream_t s) {
    return launch_stream_t<ACT_F16, 0>(c, a, grid, s);
}

}  // namespace fp
