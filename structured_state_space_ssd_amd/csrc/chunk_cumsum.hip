// Stage 1 of the SSD block decomposition: within-chunk inclusive prefix sums
// of a_t = dt_t * A_h ("Mamba 模型", section 4.1: the decay between tokens j <= i
// of one chunk is exp(s_i - s_j), the segment sum of a over (j, i]).
//
// Two-level scan with an LDS transpose. A workgroup of 1024 threads covers one
// (chunk, batch, block of 64 heads). Thread (k, hh) owns the k-th of 16 runs of
// Q/16 consecutive tokens of head hh. Its loads are unconditional (the token
// and head indices are clamped into range and out-of-range values replaced by
// zero with a select), so all of them are in flight together; one load
// instruction reads 64 consecutive heads of one token (128 contiguous bytes of
// bf16 dt). Each thread forms its run's prefix sums in registers and writes
// them, and the run total, to LDS; one wavefront per head then turns the 16
// run totals into run offsets. The outputs are written token-fastest: lanes
// take consecutive tokens of one head, so each store instruction writes 256
// contiguous bytes of s[b][h][.]. The raw dt is first turned into the step
// size (bias, softplus, clamp as DtOpts asks) and s sums step * A. If
// requested, each token's input weight (the step size, or its zero-order-hold
// weight) is also written, as float32 in the same chunk-padded [b][h][token]
// layout (zero past the end), straight from each thread's run (Q/16
// consecutive tokens of one head): the later stages read it contiguously per
// head instead of dt.
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

constexpr int kCumsumHeads = 64;
constexpr int kCumsumRuns = 16;

template <typename T, int Q>
__global__ __launch_bounds__(1024) void chunk_cumsum_kernel(const T *__restrict__ dt,
                                                            const float *__restrict__ A, int L,
                                                            int H, int nC,
                                                            float *__restrict__ out,
                                                            float *__restrict__ delta,
                                                            DtOpts o) {
    constexpr int R = Q / kCumsumRuns;  // tokens per run: 4, 8 or 16
    __shared__ float tile[Q][kCumsumHeads + 1];
    __shared__ float off[kCumsumRuns][kCumsumHeads];
    const int c = blockIdx.x, b = blockIdx.y, h0 = blockIdx.z * kCumsumHeads;
    const int tid = threadIdx.x;
    const int hh = tid & 63, k = tid >> 6, h = h0 + hh;
    const int hc = min(h, H - 1);
    const int t0 = c * Q;
    const float a = h < H ? A[hc] : 0.0f;
    const float bias = o.bias ? o.bias[hc] : 0.0f;
    // all loads first (they stay in flight together), then the options, each
    // a uniform branch around the whole run
    float d[R], v[R], dv[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        d[r] = to_f32(dt[((size_t)b * L + min(t0 + k * R + r, L - 1)) * H + hc]);
#pragma unroll
    for (int r = 0; r < R; ++r) d[r] += bias;
    if (o.softplus) {
#pragma unroll
        for (int r = 0; r < R; ++r) d[r] = fmaxf(d[r], 0.0f) + log1pf(expf(-fabsf(d[r])));
    }
    if (o.clamp) {
#pragma unroll
        for (int r = 0; r < R; ++r) d[r] = fminf(fmaxf(d[r], o.lo), o.hi);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const bool in = h < H && t0 + k * R + r < L;
        v[r] = in ? d[r] * a : 0.0f;
        dv[r] = in ? d[r] : 0.0f;
    }
    if (o.zoh) {  // input weight (exp(d a) - 1) / a; d itself where a == 0
#pragma unroll
        for (int r = 0; r < R; ++r) dv[r] = a != 0.0f ? expm1f(v[r]) / a : dv[r];
    }
    if (delta && h < H) {
        float *dd = delta + ((size_t)b * H + h) * ((size_t)nC * Q) + t0 + k * R;
#pragma unroll
        for (int r = 0; r < R; r += 4)
            *reinterpret_cast<float4 *>(dd + r) = make_float4(dv[r], dv[r + 1], dv[r + 2], dv[r + 3]);
    }
#pragma unroll
    for (int r = 1; r < R; ++r) v[r] += v[r - 1];
#pragma unroll
    for (int r = 0; r < R; ++r) tile[k * R + r][hh] = v[r];
    off[k][hh] = v[R - 1];
    __syncthreads();
    if (tid < kCumsumHeads) {  // exclusive prefix of the run totals, one head per thread
        float run = 0.0f;
#pragma unroll
        for (int kk = 0; kk < kCumsumRuns; ++kk) {
            const float t = off[kk][tid];
            off[kk][tid] = run;
            run += t;
        }
    }
    __syncthreads();
    const int tt = tid & 63, hq = tid >> 6;
    for (int hl = hq; hl < kCumsumHeads; hl += 16) {
        const int hg = h0 + hl;
        if (hg >= H) break;  // uniform across the wavefront
        float *dst = out + ((size_t)b * H + hg) * ((size_t)nC * Q) + t0;
#pragma unroll
        for (int tb = 0; tb < Q; tb += 64) {
            const int t = tb + tt;
            dst[t] = tile[t][hl] + off[t / R][hl];
        }
    }
}

hipError_t launch_chunk_cumsum(const void *dt, const float *A, int batch, int seqlen, int nheads,
                               int chunk, bool bf16, const DtOpts &opts, float *dA_cumsum,
                               float *delta, hipStream_t stream) {
    const int nC = (seqlen + chunk - 1) / chunk;
    const dim3 grid(nC, batch, (nheads + kCumsumHeads - 1) / kCumsumHeads);
#define SSD_CUMSUM(T, Q)                                                                       \
    chunk_cumsum_kernel<T, Q><<<grid, 1024, 0, stream>>>(static_cast<const T *>(dt), A, seqlen, \
                                                        nheads, nC, dA_cumsum, delta, opts)
    if (bf16) {
        if (chunk == 64) SSD_CUMSUM(bf16_t, 64);
        else if (chunk == 128) SSD_CUMSUM(bf16_t, 128);
        else if (chunk == 256) SSD_CUMSUM(bf16_t, 256);
        else return hipErrorInvalidValue;
    } else {
        if (chunk == 64) SSD_CUMSUM(float, 64);
        else if (chunk == 128) SSD_CUMSUM(float, 128);
        else if (chunk == 256) SSD_CUMSUM(float, 256);
        else return hipErrorInvalidValue;
    }
#undef SSD_CUMSUM
    return hipGetLastError();
}

}  // namespace ssd
