// Stage 3 of the SSD block decomposition: carry the hidden state across chunks
// ("Mamba 模型", section 4.1: the off-diagonal blocks act through the SSM's
// hidden state). With alpha_c = exp(s_end(c)) the total decay of chunk c and
// S_c its own contribution (stage 2):
//   H_0 = init,  H_{c+1} = alpha_c * H_c + S_c,  chunk_init[c] = H_c.
// Packed sequences (seg given): alpha_c = 0 where the sequence of chunk c's
// last token begins inside chunk c (S_c then holds that sequence's tokens only).
// REV (backward): the adjoint pass over the chunks in reverse, G_nC = dfinal,
// G_c = alpha_c G_{c+1} + dS_c, writing out[c] = G_{c+1} (the gradient of the
// state leaving chunk c) and G_0 (the initial state's gradient) as "final".
//
// Sequential over chunks, parallel over (batch, head, P*N/4): each thread owns
// one float4 of a head's P x N state. The chunk loop is unrolled by 8 so that
// the loads of 8 chunks' S are in flight before the dependent updates run; a
// wavefront reads 1 KiB contiguous per chunk. chunk_init is written in the
// operand type chunk_scan multiplies it in (bf16 for bf16 inputs: the same
// rounding chunk_scan would apply), which halves its bytes. Pure HBM streaming.
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

__device__ __forceinline__ void store4(float *p, const floatx4 &v) {
    *reinterpret_cast<floatx4 *>(p) = v;
}
__device__ __forceinline__ void store4(__bf16 *p, const floatx4 &v) {
    *reinterpret_cast<bf16x4 *>(p) = bf16x4{static_cast<__bf16>(v[0]), static_cast<__bf16>(v[1]),
                                            static_cast<__bf16>(v[2]), static_cast<__bf16>(v[3])};
}

// OutT: element type of chunk_init (float, or __bf16 = the bf16 MFMA operand
// type chunk_scan reads; the recurrence itself always runs in float32).
template <typename OutT, bool REV>
__global__ __launch_bounds__(256) void state_passing_kernel(
    const float *__restrict__ states, const float *__restrict__ dA_cumsum,
    const float *__restrict__ init, const int *__restrict__ seg, int L, int H, int PN, int Q,
    int nC, OutT *__restrict__ chunk_init, float *__restrict__ final_state) {
    const int h = blockIdx.y, b = blockIdx.z;
    const int e4 = blockIdx.x * 256 + threadIdx.x;
    if (e4 * 4 >= PN) return;
    const float *s = dA_cumsum + ((size_t)b * H + h) * (size_t)nC * Q;
    const size_t head = (size_t)b * H + h;
    floatx4 hc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (init) hc = reinterpret_cast<const floatx4 *>(init + head * PN)[e4];
    const size_t cstride = (size_t)H * PN;
    const float *sp = states + ((size_t)b * nC * H + h) * PN + (size_t)e4 * 4;
    OutT *cp = chunk_init + ((size_t)b * nC * H + h) * PN + (size_t)e4 * 4;
    constexpr int U = 8;
    for (int c0 = 0; c0 < nC; c0 += U) {
        floatx4 sv[U];
        float dec[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = REV ? nC - 1 - (c0 + u) : c0 + u;
            if (c0 + u < nC) {
                sv[u] = *reinterpret_cast<const floatx4 *>(sp + c * cstride);
                const int lenc = min(Q, L - c * Q);
                dec[u] = exp2f(s[(size_t)c * Q + lenc - 1] * kLog2e);
                if (seg && seg[((size_t)b * nC + c) * Q + lenc - 1] >= 0) dec[u] = 0.0f;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = REV ? nC - 1 - (c0 + u) : c0 + u;
            if (c0 + u < nC) {
                store4(cp + c * cstride, hc);
                hc = dec[u] * hc + sv[u];
            }
        }
    }
    if (final_state) reinterpret_cast<floatx4 *>(final_state + head * PN)[e4] = hc;
}

template <bool REV>
static hipError_t launch_sp(const float *states, const float *dA_cumsum, const float *init,
                            const int *seg, int batch, int seqlen, int nheads, int dstate,
                            int chunk, bool bf16, void *chunk_init, float *final_state,
                            hipStream_t stream) {
    const int nC = (seqlen + chunk - 1) / chunk;
    const int PN = 64 * dstate;
    const dim3 grid((PN / 4 + 255) / 256, nheads, batch);
    if (bf16)
        state_passing_kernel<__bf16, REV><<<grid, 256, 0, stream>>>(
            states, dA_cumsum, init, seg, seqlen, nheads, PN, chunk, nC,
            static_cast<__bf16 *>(chunk_init), final_state);
    else
        state_passing_kernel<float, REV><<<grid, 256, 0, stream>>>(
            states, dA_cumsum, init, seg, seqlen, nheads, PN, chunk, nC,
            static_cast<float *>(chunk_init), final_state);
    return hipGetLastError();
}

hipError_t launch_state_passing(const float *states, const float *dA_cumsum, const float *init,
                                const int *seg, int batch, int seqlen, int nheads, int dstate,
                                int chunk, bool bf16, void *chunk_init, float *final_state,
                                hipStream_t stream, bool reverse) {
    if (reverse)
        return launch_sp<true>(states, dA_cumsum, init, seg, batch, seqlen, nheads, dstate, chunk,
                               bf16, chunk_init, final_state, stream);
    return launch_sp<false>(states, dA_cumsum, init, seg, batch, seqlen, nheads, dstate, chunk,
                            bf16, chunk_init, final_state, stream);
}

}  // namespace ssd
