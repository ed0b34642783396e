// Weight-streaming projection kernel instantiations: bf16 weights.
#include "fp_stream.hpp"

namespace fp {

hipError_t launch_stream_bf16(const StreamCfg &c, const ProjArgs &a, unsigned grid, hipStream_t s) {
    return launch_stream_t<ACT_BF16, 0>(c, a, grid, s);
}

}  // namespace fp
