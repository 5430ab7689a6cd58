// Packed variable-length sequences: several sequences concatenated along the
// token axis of a batch-1 input, sequence k being tokens cu[k] .. cu[k+1]-1,
// each with its own recurrence from the zero state (the dynamic packing of
// variable-length sequences listed on the "Mamba-2架构深度解析" page, section 5).
//
// The chunked stages stay as they are, with one int per token position, seg:
// the first token of the token's sequence relative to the first token of its
// chunk, or -1 if that sequence began in an earlier chunk. Since sequences are
// contiguous, two tokens i >= j of one chunk share a sequence exactly when
// j >= seg[i]; the stages use it as a mask (chunk_state: only the last
// sequence's tokens make the chunk's state; state_passing: no carry into a
// chunk's last sequence if it begins inside the chunk; chunk_scan: pairs and
// the state-to-output term of other sequences are zero). The within-chunk
// prefix sums of dt*A run across boundaries: every difference the stages take
// is then between tokens of one sequence.
//
// Each sequence's final state (the state after its last token te, in chunk
// c) is H = [seg[te] < 0] exp(s_te) H_c + sum_{j = max(seg[te], 0)}^{te}
// exp(s_te - s_j) w_j x_j B_j^T, from the chunk_init of the state passing and
// the chunk's own tokens: for bf16 by the chunk state kernel on MFMA (its
// final-state variant), for float32 by varlen_final_state_kernel below.
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

// seg for every token position t < nC*Q (positions past the last token take
// the last sequence). Any cu_seqlens contents give in-range values.
__global__ __launch_bounds__(256) void varlen_seg_kernel(const int *__restrict__ cu, int nseq,
                                                         int Q, int ntok, int *__restrict__ seg) {
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= ntok) return;
    // the largest k in [0, nseq - 1] with cu[k] <= t (empty sequences are passed over)
    int lo = 0, hi = nseq - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= t) lo = mid;
        else hi = mid - 1;
    }
    const int c0 = t - t % Q;
    seg[t] = max(cu[lo] - c0, -1);
}

hipError_t launch_varlen_seg(const int *cu_seqlens, int nseq, int seqlen, int chunk, int *seg,
                             hipStream_t stream) {
    const int ntok = (seqlen + chunk - 1) / chunk * chunk;
    varlen_seg_kernel<<<(ntok + 255) / 256, 256, 0, stream>>>(cu_seqlens, nseq, chunk, ntok, seg);
    return hipGetLastError();
}

// One workgroup per (sequence, head); thread t owns the state entries
// t + 256 i (row p = (t + 256 i) / N, column n = t % N), accumulated in
// float32 over 32-token blocks staged in LDS.
template <typename T, typename HT, int N>
__global__ __launch_bounds__(256) void varlen_final_state_kernel(
    const T *__restrict__ x, const T *__restrict__ B, const float *__restrict__ delta,
    const float *__restrict__ dA_cumsum, const int *__restrict__ cu, const int *__restrict__ seg,
    const HT *__restrict__ chunk_init, int L, int H, int G, int Q, int nC,
    float *__restrict__ seq_states) {
    constexpr int P = 64, PN = P * N, PER = PN / 256, TB = 32;
    __shared__ float xs[TB][P];
    __shared__ float bs[TB][N];
    __shared__ float wv[TB];
    const int k = blockIdx.x, h = blockIdx.y, g = h / (H / G);
    const int tid = threadIdx.x, n = tid % N, p0 = tid / N;
    float *out = seq_states + ((size_t)k * H + h) * PN;
    const int a = min(max(cu[k], 0), L), e = min(max(cu[k + 1], a), L);
    float acc[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = 0.0f;
    if (e > a) {  // uniform: an empty sequence's state is zero
        const int te = e - 1, c = te / Q, t0 = c * Q, el = te - t0;
        const int fs = min(seg[te], el);
        const float *s = dA_cumsum + (size_t)h * nC * Q + t0;
        const float *dl = delta + (size_t)h * nC * Q + t0;
        const float se = s[el];
        if (fs < 0) {  // the sequence began before chunk c: H_c is its state there
            const float dec = exp2f(se * kLog2e);
            const HT *hc = chunk_init + ((size_t)c * H + h) * PN;
#pragma unroll
            for (int i = 0; i < PER; ++i) acc[i] = dec * static_cast<float>(hc[tid + 256 * i]);
        }
        for (int jb = max(fs, 0); jb <= el; jb += TB) {
            __syncthreads();  // the previous block's values are consumed
            for (int idx = tid; idx < TB * P; idx += 256) {
                const int jj = idx / P, pp = idx % P, j = jb + jj;
                xs[jj][pp] = j <= el ? to_f32(x[((size_t)(t0 + j) * H + h) * P + pp]) : 0.0f;
            }
            for (int idx = tid; idx < TB * N; idx += 256) {
                const int jj = idx / N, nn = idx % N, j = jb + jj;
                bs[jj][nn] = j <= el ? to_f32(B[((size_t)(t0 + j) * G + g) * N + nn]) : 0.0f;
            }
            if (tid < TB) {
                const int j = jb + tid;
                wv[tid] = j <= el ? exp2f((se - s[j]) * kLog2e) * dl[j] : 0.0f;
            }
            __syncthreads();
            for (int jj = 0; jj < TB; ++jj) {
                const float bw = bs[jj][n] * wv[jj];
#pragma unroll
                for (int i = 0; i < PER; ++i) acc[i] += xs[jj][p0 + i * (256 / N)] * bw;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) out[tid + 256 * i] = acc[i];
}

template <typename T, typename HT>
static hipError_t final_states_n(int N, dim3 grid, const void *x, const void *B,
                                 const float *delta, const float *dA, const int *cu,
                                 const int *seg, const void *ci, int L, int H, int G, int Q,
                                 int nC, float *out, hipStream_t stream) {
    const T *xx = static_cast<const T *>(x), *bb = static_cast<const T *>(B);
    const HT *hc = static_cast<const HT *>(ci);
#define SSD_FINAL(NN)                                                                          \
    varlen_final_state_kernel<T, HT, NN><<<grid, 256, 0, stream>>>(xx, bb, delta, dA, cu, seg, \
                                                                   hc, L, H, G, Q, nC, out)
    switch (N) {
        case 16: SSD_FINAL(16); break;
        case 32: SSD_FINAL(32); break;
        case 64: SSD_FINAL(64); break;
        case 128: SSD_FINAL(128); break;
        case 256: SSD_FINAL(256); break;
        default: return hipErrorInvalidValue;
    }
#undef SSD_FINAL
    return hipGetLastError();
}

hipError_t launch_varlen_final_states_bf16(const void *x, const void *B, const float *delta,
                                           const float *dA_cumsum, const int *cu_seqlens,
                                           const int *seg, const void *chunk_init, int nseq,
                                           int seqlen, int nheads, int ngroups, int dstate,
                                           int chunk, float *seq_states, hipStream_t stream);

hipError_t launch_varlen_final_states(const void *x, const void *B, const float *delta,
                                      const float *dA_cumsum, const int *cu_seqlens,
                                      const int *seg, const void *chunk_init, int nseq,
                                      int seqlen, int nheads, int ngroups, int dstate, int chunk,
                                      bool bf16, float *seq_states, hipStream_t stream) {
    const int nC = (seqlen + chunk - 1) / chunk;
    const dim3 grid(nseq, nheads);
    if (bf16)  // on MFMA, by the chunk state kernel (chunk_state.hip)
        return launch_varlen_final_states_bf16(x, B, delta, dA_cumsum, cu_seqlens, seg,
                                               chunk_init, nseq, seqlen, nheads, ngroups, dstate,
                                               chunk, seq_states, stream);
    return final_states_n<float, float>(dstate, grid, x, B, delta, dA_cumsum, cu_seqlens, seg,
                                        chunk_init, seqlen, nheads, ngroups, chunk, nC,
                                        seq_states, stream);
}

}  // namespace ssd
