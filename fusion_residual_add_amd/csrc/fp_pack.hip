// Tile-packed weight layout: the pack and unpack kernels behind
// fused_pack_weight / fused_unpack_weight, and the unpacking the library does
// itself before a kernel that reads row-major weights only.  The pages'
// deployment flow converts the checkpoint once, re-laying the weights out for
// the target GPU ("TensorRT-LLM 深度工程实践…", the build workflow, step 1:
// weight preparation and conversion); here the layout is the one that lets a
// workgroup stream 128 weight rows as contiguous runs (packed_row_off).
#include "fp_device.hpp"

namespace fp {

// One thread per 16-byte vector of the packed weight, grid-stride: packed
// vector q sits in 1 KB block slice q / 64 (group t, K slice s, block i) at
// (g, i') = ((q / 16) % 4, q % 16), which holds row-major bytes
// 64 s + 16 g .. + 15 of the block's row i'.
__global__ __launch_bounds__(256) void pack_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                  int64_t n_vec, int64_t row_bytes, int64_t F, int layout,
                                                  int unpack) {
    const int64_t S = row_bytes >> 6;   // 64-byte slices per row
    for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < n_vec; q += (int64_t)gridDim.x * 256) {
        const int64_t blk = q >> 6;
        const int g = (int)((q >> 4) & 3), ii = (int)(q & 15);
        const int64_t t = blk / (8 * S), rem = blk - t * 8 * S;
        const int64_t s = rem >> 3;
        const int i = (int)(rem & 7);
        int64_t r;
        if (layout == WL_PACKED_GATE_UP) {
            const int64_t j = 64 * t + 16 * (i & 3) + ii;
            r = i < 4 ? j : F + j;
        } else {
            r = 128 * t + 16 * i + ii;
        }
        const int64_t v = (r * row_bytes + 64 * s + 16 * g) >> 4;
        if (unpack) dst[v] = src[q];
        else dst[q] = src[v];
    }
}

hipError_t launch_pack(const void *src, void *dst, int64_t n_rows, int64_t row_bytes, int64_t F, int layout,
                       bool unpack, hipStream_t s) {
    const int64_t n_vec = n_rows * row_bytes / 16;
    if (n_vec <= 0) return hipSuccess;
    int64_t grid = (n_vec + 255) / 256;
    if (grid > 8192) grid = 8192;
    return launch_k(pack_kernel, (unsigned)grid, s, (const u32x4 *)src, (u32x4 *)dst, n_vec, row_bytes, F, layout,
                    (int)unpack);
}

const char *pack_kernel_name(bool unpack) { return unpack ? "unpack_kernel" : "pack_kernel"; }

}  // namespace fp
