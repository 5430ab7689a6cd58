// Recurrent (linear-mode) decode: one token for every (batch, head)
// ("从Transformer到Mamba" tutorial, section 2.2; the linear mode of the
// "Mamba-2架构深度解析" page, section 2.2 table):
//   h <- exp(dt A_h) h + w x B^T,   y = h C + D_h x   (output after the update),
// with dt the step size after DtOpts' preprocessing and w its input weight
// (dt itself, or the zero-order hold's (exp(dt A) - 1) / A).
//
// Bandwidth-bound: the float32 P x N state is read once and written once.
// One workgroup (4 wavefronts) per (batch, head); wavefront w owns state rows
// 16w .. 16w+15, a contiguous 16*N*4-byte span that it streams with 16-byte
// non-temporal loads and stores, each instruction covering 1 KiB contiguous.
// Lane l's float4 always has the same state columns n = 4l mod N, so its
// B and C values are loaded once. Row sums for y are reduced with xor
// shuffles among the N/4 lanes that share a row.
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

template <typename T, int N>
__global__ __launch_bounds__(256) void decode_step_kernel(
    float *__restrict__ state, const T *__restrict__ x, const T *__restrict__ dt,
    const float *__restrict__ A, const T *__restrict__ B, const T *__restrict__ C,
    const float *__restrict__ D, int H, int G, T *__restrict__ y, DtOpts o) {
    constexpr int P = 64;
    constexpr int ITER = N / 16;  // float4 per lane: 16 rows * N / (64 lanes * 4)
    constexpr int LPR = N / 4;    // lanes sharing one state row within an instruction
    const int bh = blockIdx.x;
    const int b = bh / H, h = bh % H, g = h / (H / G);
    const int w = wave_id(), l = lane_id();
    const float Ah = A[h];
    const float d = step_size(o, to_f32(dt[bh]), o.bias ? o.bias[h] : 0.0f);
    const float a = exp2f(d * Ah * kLog2e);
    const float wt = input_weight(o, d, Ah);
    const float Dh = D ? D[h] : 0.0f;

    floatx4 *st = reinterpret_cast<floatx4 *>(state + ((size_t)bh * P + w * 16) * N);
    floatx4 hv[ITER];
#pragma unroll
    for (int m = 0; m < ITER; ++m) hv[m] = __builtin_nontemporal_load(st + m * 64 + l);

    const int n = (4 * l) % N;
    const T *bp = B + ((size_t)b * G + g) * N + n;
    const T *cp = C + ((size_t)b * G + g) * N + n;
    float bv[4], cv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        bv[k] = to_f32(bp[k]);
        cv[k] = to_f32(cp[k]);
    }
    const T *xp = x + (size_t)bh * P;
    float part[ITER], xr[ITER];
#pragma unroll
    for (int m = 0; m < ITER; ++m) {
        const int p = w * 16 + (m * 256 + 4 * l) / N;
        xr[m] = to_f32(xp[p]);
        const float dx = wt * xr[m];
        floatx4 v = hv[m];
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[k] = a * v[k] + dx * bv[k];
            acc += cv[k] * v[k];
        }
        part[m] = acc;
        __builtin_nontemporal_store(v, st + m * 64 + l);
    }
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1)
#pragma unroll
        for (int m = 0; m < ITER; ++m) part[m] += __shfl_xor(part[m], off);
    if ((l % LPR) == 0) {
#pragma unroll
        for (int m = 0; m < ITER; ++m) {
            const int p = w * 16 + (m * 256 + 4 * l) / N;
            y[(size_t)bh * P + p] = from_f32<T>(part[m] + Dh * xr[m]);
        }
    }
}

// State sizes that are not powers of two (48, 80, ..., 240): a row's N/4
// float4s do not line up with lane groups of a power of two, so each lane's
// four-term products go to LDS and lane r of the wavefront then sums row r's
// N/4 of them in order. Same layout and streaming as above; B and C of the
// group are staged in LDS first.
template <typename T, int N>
__global__ __launch_bounds__(256) void decode_step_rows_kernel(
    float *__restrict__ state, const T *__restrict__ x, const T *__restrict__ dt,
    const float *__restrict__ A, const T *__restrict__ B, const T *__restrict__ C,
    const float *__restrict__ D, int H, int G, T *__restrict__ y, DtOpts o) {
    constexpr int P = 64;
    constexpr int F = 4 * N;      // float4s per wavefront: 16 rows x N/4
    constexpr int ITER = N / 16;  // float4s per lane
    constexpr int FPR = N / 4;    // float4s per state row
    __shared__ float part[4][F];
    __shared__ float bs[N], cs[N];
    const int bh = blockIdx.x;
    const int b = bh / H, h = bh % H, g = h / (H / G);
    const int w = wave_id(), l = lane_id();
    const float Ah = A[h];
    const float d = step_size(o, to_f32(dt[bh]), o.bias ? o.bias[h] : 0.0f);
    const float a = exp2f(d * Ah * kLog2e);
    const float wt = input_weight(o, d, Ah);
    const float Dh = D ? D[h] : 0.0f;
    for (int i = threadIdx.x; i < N; i += 256) {
        bs[i] = to_f32(B[((size_t)b * G + g) * N + i]);
        cs[i] = to_f32(C[((size_t)b * G + g) * N + i]);
    }

    floatx4 *st = reinterpret_cast<floatx4 *>(state + ((size_t)bh * P + w * 16) * N);
    floatx4 hv[ITER];
#pragma unroll
    for (int m = 0; m < ITER; ++m) hv[m] = __builtin_nontemporal_load(st + m * 64 + l);
    __syncthreads();
    const T *xp = x + (size_t)bh * P + w * 16;
#pragma unroll
    for (int m = 0; m < ITER; ++m) {
        const int f = m * 64 + l, r = f / FPR, n = 4 * (f - r * FPR);
        const float dx = wt * to_f32(xp[r]);
        floatx4 v = hv[m];
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[k] = a * v[k] + dx * bs[n + k];
            acc += cs[n + k] * v[k];
        }
        part[w][f] = acc;
        __builtin_nontemporal_store(v, st + m * 64 + l);
    }
    __syncthreads();
    if (l < 16) {
        float sum = 0.0f;
        for (int q = 0; q < FPR; ++q) sum += part[w][l * FPR + q];
        y[(size_t)bh * P + w * 16 + l] = from_f32<T>(sum + Dh * to_f32(xp[l]));
    }
}

template <typename T>
static hipError_t dispatch_decode(int N, float *state, const void *x, const void *dt,
                                  const float *A, const void *B, const void *C, const float *D,
                                  int batch, int H, int G, void *y, const DtOpts &o,
                                  hipStream_t stream) {
    const dim3 grid(batch * H);
    const T *xx = static_cast<const T *>(x), *dd = static_cast<const T *>(dt);
    const T *bb = static_cast<const T *>(B), *cc = static_cast<const T *>(C);
    T *yy = static_cast<T *>(y);
    switch (N) {
        case 16: decode_step_kernel<T, 16><<<grid, 256, 0, stream>>>(state, xx, dd, A, bb, cc, D, H, G, yy, o); break;
        case 32: decode_step_kernel<T, 32><<<grid, 256, 0, stream>>>(state, xx, dd, A, bb, cc, D, H, G, yy, o); break;
        case 64: decode_step_kernel<T, 64><<<grid, 256, 0, stream>>>(state, xx, dd, A, bb, cc, D, H, G, yy, o); break;
        case 128: decode_step_kernel<T, 128><<<grid, 256, 0, stream>>>(state, xx, dd, A, bb, cc, D, H, G, yy, o); break;
        case 256: decode_step_kernel<T, 256><<<grid, 256, 0, stream>>>(state, xx, dd, A, bb, cc, D, H, G, yy, o); break;
#define SSD_DECODE_ROWS(NN) \
        case NN: decode_step_rows_kernel<T, NN><<<grid, 256, 0, stream>>>(state, xx, dd, A, bb, cc, D, H, G, yy, o); break;
        SSD_DECODE_ROWS(48) SSD_DECODE_ROWS(80) SSD_DECODE_ROWS(96) SSD_DECODE_ROWS(112)
        SSD_DECODE_ROWS(144) SSD_DECODE_ROWS(160) SSD_DECODE_ROWS(176) SSD_DECODE_ROWS(192)
        SSD_DECODE_ROWS(208) SSD_DECODE_ROWS(224) SSD_DECODE_ROWS(240)
#undef SSD_DECODE_ROWS
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_decode_step(float *state, const void *x, const void *dt, const float *A,
                              const void *B, const void *C, const float *D, int batch, int nheads,
                              int ngroups, int dstate, bool bf16, const DtOpts &opts, void *y,
                              hipStream_t stream) {
    if (bf16)
        return dispatch_decode<bf16_t>(dstate, state, x, dt, A, B, C, D, batch, nheads, ngroups, y,
                                       opts, stream);
    return dispatch_decode<float>(dstate, state, x, dt, A, B, C, D, batch, nheads, ngroups, y,
                                  opts, stream);
}

}  // namespace ssd
