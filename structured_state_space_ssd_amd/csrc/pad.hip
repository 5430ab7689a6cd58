// Zero-padding of the state dimension N. The kernels run with N in
// {16, 32, 64, 128, 256}; any other multiple of 16 runs with the next of
// these, its B and C columns (and the initial state's) past N set to zero.
// The padded columns then contribute exact zeros to every sum over n (C_i.B_j,
// H C_i) and the padded state columns stay zero (no input reaches them), so
// the result is the one at N up to summation order; the state and gradient
// outputs are cut back to N.
#include <algorithm>

#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

// dst[r][0 .. dst_bytes) = src[r][0 .. src_bytes) followed by zeros (or cut
// to dst_bytes when src_bytes is larger), in 16-byte pieces (both row sizes
// are multiples of 16 bytes).
__global__ __launch_bounds__(256) void pad_rows_kernel(const uint4 *__restrict__ src,
                                                       uint4 *__restrict__ dst, size_t rows,
                                                       int src_pieces, int dst_pieces) {
    const size_t total = rows * (size_t)dst_pieces;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < total;
         i += (size_t)gridDim.x * 256) {
        const size_t r = i / dst_pieces;
        const int q = (int)(i - r * dst_pieces);
        dst[i] = q < src_pieces ? src[r * src_pieces + q] : make_uint4(0, 0, 0, 0);
    }
}

}  // namespace

int kernel_dstate(int dstate) {
    for (int n : {16, 32, 64, 128, 256})
        if (dstate <= n) return n;
    return 0;
}

hipError_t launch_pad_rows(const void *src, void *dst, size_t rows, int src_cols, int dst_cols,
                           int elem_bytes, hipStream_t stream) {
    const int sp = src_cols * elem_bytes / 16, dp = dst_cols * elem_bytes / 16;
    const size_t total = rows * (size_t)dp;
    if (total == 0) return hipSuccess;
    const size_t blocks = std::min<size_t>((total + 255) / 256, 8192);
    pad_rows_kernel<<<(unsigned)blocks, 256, 0, stream>>>(static_cast<const uint4 *>(src),
                                                          static_cast<uint4 *>(dst), rows, sp, dp);
    return hipGetLastError();
}

}  // namespace ssd
