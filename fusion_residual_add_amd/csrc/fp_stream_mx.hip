// Weight-streaming projection kernel instantiations: MXFP4 weights (bf16 activations).
#include "fp_stream.hpp"

namespace fp {

hipError_t launch_stream_mx(const StreamCfg &c, const ProjArgs &a, unsigned grid, hipStream_t s) {
    return launch_stream_t<ACT_BF16, 3>(c, a, grid, s);
}

}  // namespace fp
