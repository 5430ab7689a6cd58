// Stage 1 of the SSD block decomposition: within-chunk inclusive prefix sums
// of a_t = dt_t * A_h ("Mamba 模型", section 4.1: the decay between tokens j <= i
// of one chunk is exp(s_i - s_j), the segment sum of a over (j, i]).
//
// One workgroup per (chunk, batch, block of 32 heads). The Q x 32 tile of a is
// read with row-contiguous (head-fastest) loads into LDS, then each wavefront
// scans one head at a time: every lane sums Q/64 consecutive tokens, a
// wavefront-wide inclusive scan of the lane totals gives each lane its
// offset, and the chunk row s[b][h][cQ .. cQ+Q) is written contiguously.
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

constexpr int kCumsumHeads = 32;

template <typename T>
__global__ __launch_bounds__(256) void chunk_cumsum_kernel(const T *__restrict__ dt,
                                                           const float *__restrict__ A, int L,
                                                           int H, int Q, int nC,
                                                           float *__restrict__ out) {
    __shared__ float tile[256][kCumsumHeads + 1];
    const int c = blockIdx.x, b = blockIdx.y, h0 = blockIdx.z * kCumsumHeads;
    const int t0 = c * Q;
    const int len = min(Q, L - t0);
    for (int idx = threadIdx.x; idx < Q * kCumsumHeads; idx += blockDim.x) {
        const int t = idx / kCumsumHeads, hh = idx % kCumsumHeads, h = h0 + hh;
        float a = 0.0f;
        if (t < len && h < H) a = to_f32(dt[((size_t)b * L + t0 + t) * H + h]) * A[h];
        tile[t][hh] = a;
    }
    __syncthreads();
    const int w = wave_id(), l = lane_id();
    const int per = Q >> 6;  // tokens per lane: 1, 2 or 4
    for (int hh = w; hh < kCumsumHeads; hh += 4) {
        const int h = h0 + hh;
        if (h >= H) break;  // uniform across the wavefront
        float v[4];
        float run = 0.0f;
        for (int k = 0; k < per; ++k) {
            run += tile[l * per + k][hh];
            v[k] = run;
        }
        float incl = run;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float o = __shfl_up(incl, off);
            if (l >= off) incl += o;
        }
        const float excl = incl - run;
        float *dst = out + ((size_t)b * H + h) * ((size_t)nC * Q) + t0 + l * per;
        for (int k = 0; k < per; ++k) dst[k] = excl + v[k];
    }
}

hipError_t launch_chunk_cumsum(const void *dt, const float *A, int batch, int seqlen, int nheads,
                               int chunk, bool bf16, float *dA_cumsum, hipStream_t stream) {
    const int nC = (seqlen + chunk - 1) / chunk;
    dim3 grid(nC, batch, (nheads + kCumsumHeads - 1) / kCumsumHeads);
    if (bf16)
        chunk_cumsum_kernel<bf16_t><<<grid, 256, 0, stream>>>(
            static_cast<const bf16_t *>(dt), A, seqlen, nheads, chunk, nC, dA_cumsum);
    else
        chunk_cumsum_kernel<float><<<grid, 256, 0, stream>>>(
            static_cast<const float *>(dt), A, seqlen, nheads, chunk, nC, dA_cumsum);
    return hipGetLastError();
}

}  // namespace ssd
