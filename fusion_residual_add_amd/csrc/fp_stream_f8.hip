// Weight-streaming projection kernel instantiations: E4M3 weights with one
// scale per row and E4M3 per-token activation codes (the FP8 W8A8 call at
// decode token counts), bf16 or f16 outputs.
#include "fp_stream.hpp"

namespace fp {

hipError_t launch_stream_f8(int act, const StreamCfg &c, const ProjArgs &a, unsigned grid, hipStream_t s) {
    if (act == ACT_F16) return launch_stream_t<ACT_F16, 4>(c, a, grid, s);
    return launch_stream_t<ACT_BF16, 4>(c, a, grid, s);
}

}  // namespace fp
