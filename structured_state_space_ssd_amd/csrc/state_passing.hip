// Stage 3 of the SSD block decomposition: carry the hidden state across chunks
// ("Mamba 模型", section 4.1: the off-diagonal blocks act through the SSM's
// hidden state). With alpha_c = exp(s_end(c)) the total decay of chunk c and
// S_c its own contribution (stage 2):
//   H_0 = init,  H_{c+1} = alpha_c * H_c + S_c,  chunk_init[c] = H_c.
//
// Sequential over chunks, parallel over (batch, head, P*N/4): each thread owns
// one float4 of a head's P x N state. The chunk loop is unrolled by 8 so that
// the loads of 8 chunks' S are in flight before the dependent updates run; a
// wavefront reads and writes 1 KiB contiguous per chunk. Pure HBM streaming.
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

__global__ __launch_bounds__(256) void state_passing_kernel(
    const float *__restrict__ states, const float *__restrict__ dA_cumsum,
    const float *__restrict__ init, int L, int H, int PN, int Q, int nC,
    float *__restrict__ chunk_init, float *__restrict__ final_state) {
    const int h = blockIdx.y, b = blockIdx.z;
    const int e4 = blockIdx.x * 256 + threadIdx.x;
    if (e4 * 4 >= PN) return;
    const float *s = dA_cumsum + ((size_t)b * H + h) * (size_t)nC * Q;
    const size_t head = (size_t)b * H + h;
    floatx4 hc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (init) hc = reinterpret_cast<const floatx4 *>(init + head * PN)[e4];
    const size_t cstride = (size_t)H * PN;
    const float *sp = states + ((size_t)b * nC * H + h) * PN + (size_t)e4 * 4;
    float *cp = chunk_init + ((size_t)b * nC * H + h) * PN + (size_t)e4 * 4;
    constexpr int U = 8;
    for (int c0 = 0; c0 < nC; c0 += U) {
        floatx4 sv[U];
        float dec[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u;
            if (c < nC) {
                sv[u] = *reinterpret_cast<const floatx4 *>(sp + c * cstride);
                const int lenc = min(Q, L - c * Q);
                dec[u] = exp2f(s[(size_t)c * Q + lenc - 1] * kLog2e);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u;
            if (c < nC) {
                *reinterpret_cast<floatx4 *>(cp + c * cstride) = hc;
                hc = dec[u] * hc + sv[u];
            }
        }
    }
    if (final_state) reinterpret_cast<floatx4 *>(final_state + head * PN)[e4] = hc;
}

hipError_t launch_state_passing(const float *states, const float *dA_cumsum, const float *init,
                                int batch, int seqlen, int nheads, int dstate, int chunk,
                                float *chunk_init, float *final_state, hipStream_t stream) {
    const int nC = (seqlen + chunk - 1) / chunk;
    const int PN = 64 * dstate;
    dim3 grid((PN / 4 + 255) / 256, nheads, batch);
    state_passing_kernel<<<grid, 256, 0, stream>>>(states, dA_cumsum, init, seqlen, nheads, PN,
                                                   chunk, nC, chunk_init, final_state);
    return hipGetLastError();
}

}  // namespace ssd
