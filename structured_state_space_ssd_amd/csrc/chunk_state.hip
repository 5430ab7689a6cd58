// Stage 2 of the SSD block decomposition: the state each chunk contributes at
// its right edge, from a zero state ("Mamba 模型", section 4.1: the low-rank
// factor through which the off-diagonal blocks act):
//   S_c[p][n] = sum_{j in c} w_j * x_j[p] * B_j[n],  w_j = exp(s_end - s_j) * dt_j.
//
// One workgroup (4 wavefronts) per (chunk, head, batch). S_c = X^T (w o B) is a
// [P x Q] x [Q x N] product whose contraction index is the token, which is the
// slow (row) index of both x and B in memory, so both operands are staged
// through LDS transposed: XT[p][j] and BT[n][j] (w folded into B in fp32
// before rounding to the operand type). Tokens go through LDS 64 at a time:
// global loads are 16-byte row segments; each thread packs two tokens into
// 4-byte LDS writes. The MFMA phase reads 16-byte fragments (8 consecutive
// tokens) for both operands. Wavefront w owns output column tiles w, w+4, ...
// over all four 16-row tiles of P = 64.
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

template <typename E>
__device__ __forceinline__ void lds_store2(E *dst, float a, float b);
template <>
__device__ __forceinline__ void lds_store2<__bf16>(__bf16 *dst, float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v;
    v[0] = static_cast<__bf16>(a);
    v[1] = static_cast<__bf16>(b);
    *reinterpret_cast<bf16x2 *>(dst) = v;
}
template <>
__device__ __forceinline__ void lds_store2<float>(float *dst, float a, float b) {
    *reinterpret_cast<float2 *>(dst) = make_float2(a, b);
}

template <typename T, int N>
__global__ __launch_bounds__(256) void chunk_state_kernel(
    const T *__restrict__ x, const T *__restrict__ B, const T *__restrict__ dt,
    const float *__restrict__ dA_cumsum, int L, int H, int G, int Q, int nC,
    float *__restrict__ states) {
    using E = typename LdsT<T>::type;
    constexpr int P = 64, JB = 64, LD = JB + 8;
    constexpr int NT = N / 16;              // 16-wide column tiles of S
    constexpr int NTW = (NT + 3) / 4;       // tiles per wavefront
    __shared__ __attribute__((aligned(16))) E xt[P * LD];
    __shared__ __attribute__((aligned(16))) E bt[N * LD];
    __shared__ float wj[256];

    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int g = h / (H / G);
    const int t0 = c * Q, len = min(Q, L - t0);
    const float *s = dA_cumsum + ((size_t)b * H + h) * (size_t)nC * Q + (size_t)c * Q;
    const float s_end = s[len - 1];
    for (int j = threadIdx.x; j < Q; j += 256) {
        float wv = 0.0f;
        if (j < len)
            wv = exp2f((s_end - s[j]) * kLog2e) * to_f32(dt[((size_t)b * L + t0 + j) * H + h]);
        wj[j] = wv;
    }

    const int w = wave_id(), l = lane_id(), g4 = l >> 4, r16 = l & 15;
    floatx4 acc[4][NTW];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
        for (int i = 0; i < NTW; ++i) acc[pt][i] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

    const T *xh = x + (((size_t)b * L + t0) * H + h) * P;     // token stride H*P
    const T *bg = B + (((size_t)b * L + t0) * G + g) * N;     // token stride G*N
    const size_t xs = (size_t)H * P, bs = (size_t)G * N;

    for (int jb = 0; jb < len; jb += JB) {
        __syncthreads();  // previous block consumed (first pass: wj written)
        {   // x block -> XT[p][j]; thread = (8-wide p slice, token pair)
            const int pb = threadIdx.x >> 5, jp = threadIdx.x & 31;
            const int j0 = jb + 2 * jp;
            float v0[8], v1[8];
            if (j0 < len) load8(xh + (size_t)j0 * xs + pb * 8, v0);
            else for (int e = 0; e < 8; ++e) v0[e] = 0.0f;
            if (j0 + 1 < len) load8(xh + (size_t)(j0 + 1) * xs + pb * 8, v1);
            else for (int e = 0; e < 8; ++e) v1[e] = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) lds_store2<E>(xt + (pb * 8 + e) * LD + 2 * jp, v0[e], v1[e]);
        }
        // B block scaled by w -> BT[n][j]
        for (int idx = threadIdx.x; idx < 32 * (N / 8); idx += 256) {
            const int nb = idx >> 5, jp = idx & 31;
            const int j0 = jb + 2 * jp;
            float v0[8], v1[8];
            if (j0 < len) {
                load8(bg + (size_t)j0 * bs + nb * 8, v0);
                const float w0 = wj[j0];
                for (int e = 0; e < 8; ++e) v0[e] *= w0;
            } else {
                for (int e = 0; e < 8; ++e) v0[e] = 0.0f;
            }
            if (j0 + 1 < len) {
                load8(bg + (size_t)(j0 + 1) * bs + nb * 8, v1);
                const float w1 = wj[j0 + 1];
                for (int e = 0; e < 8; ++e) v1[e] *= w1;
            } else {
                for (int e = 0; e < 8; ++e) v1[e] = 0.0f;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) lds_store2<E>(bt + (nb * 8 + e) * LD + 2 * jp, v0[e], v1[e]);
        }
        __syncthreads();
        const int kend = min(JB, len - jb);
        for (int kk = 0; kk < kend; kk += 32) {
            Frag<T> a[4];
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) lds_frag8(a[pt], xt + (pt * 16 + r16) * LD + kk + 8 * g4);
#pragma unroll
            for (int i = 0; i < NTW; ++i) {
                const int nt = w + 4 * i;
                if (nt < NT) {
                    Frag<T> bf;
                    lds_frag8(bf, bt + (nt * 16 + r16) * LD + kk + 8 * g4);
#pragma unroll
                    for (int pt = 0; pt < 4; ++pt) mma(acc[pt][i], a[pt], bf);
                }
            }
        }
    }

    float *dst = states + (((size_t)b * nC + c) * H + h) * (size_t)P * N;
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
        const int nt = w + 4 * i;
        if (nt < NT) {
#pragma unroll
            for (int pt = 0; pt < 4; ++pt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dst[(size_t)(pt * 16 + 4 * g4 + r) * N + nt * 16 + r16] = acc[pt][i][r];
        }
    }
}

template <typename T, int N>
static void launch_cs(const void *x, const void *B, const void *dt, const float *dA, int batch,
                      int L, int H, int G, int Q, float *states, hipStream_t stream) {
    const int nC = (L + Q - 1) / Q;
    dim3 grid(nC, H, batch);
    chunk_state_kernel<T, N><<<grid, 256, 0, stream>>>(
        static_cast<const T *>(x), static_cast<const T *>(B), static_cast<const T *>(dt), dA, L, H,
        G, Q, nC, states);
}

template <typename T>
static hipError_t dispatch_cs(const void *x, const void *B, const void *dt, const float *dA,
                              int batch, int L, int H, int G, int N, int Q, float *states,
                              hipStream_t stream) {
    switch (N) {
        case 16: launch_cs<T, 16>(x, B, dt, dA, batch, L, H, G, Q, states, stream); break;
        case 32: launch_cs<T, 32>(x, B, dt, dA, batch, L, H, G, Q, states, stream); break;
        case 64: launch_cs<T, 64>(x, B, dt, dA, batch, L, H, G, Q, states, stream); break;
        case 128: launch_cs<T, 128>(x, B, dt, dA, batch, L, H, G, Q, states, stream); break;
        case 256: launch_cs<T, 256>(x, B, dt, dA, batch, L, H, G, Q, states, stream); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_chunk_state(const void *x, const void *B, const void *dt, const float *dA_cumsum,
                              int batch, int seqlen, int nheads, int ngroups, int dstate, int chunk,
                              bool bf16, float *states, hipStream_t stream) {
    if (bf16)
        return dispatch_cs<bf16_t>(x, B, dt, dA_cumsum, batch, seqlen, nheads, ngroups, dstate,
                                   chunk, states, stream);
    return dispatch_cs<float>(x, B, dt, dA_cumsum, batch, seqlen, nheads, ngroups, dstate, chunk,
                              states, stream);
}

}  // namespace ssd
