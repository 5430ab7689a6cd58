// Stage 4 of the SSD block decomposition: every chunk's outputs
// ("Mamba 模型", section 4.1 and "Draft:Mamba2", SSD section):
//   y_i = sum_{j<=i in chunk} (C_i . B_j) exp(s_i - s_j) dt_j x_j     diagonal block
//       + exp(s_i) H_c C_i                                            off-diagonal blocks
//       + D_h x_i.
// The diagonal block is the masked "attention-like" product (L o C B^T)(dt o x)
// (quadratic mode of the "Mamba-2架构深度解析" page, section 2.2 table); the
// off-diagonal part reads the state H_c carried into the chunk (stage 3).
//
// One workgroup per (chunk, head, batch) with Q/32 wavefronts. Wavefront w
// owns the 16-row output tiles w and Q/16-1-w, which balances the causal work
// (each pair covers Q/16+1 column tiles). Per wavefront:
//   1. state-to-output: acc = (exp(s_i) C_i) H_c^T on MFMA (K = N), H_c staged
//      in LDS in the operand type;
//   2. tokens stream through LDS 64 at a time: B block in natural layout
//      [j][n] and x block transposed [p][j]. For each 32-token slice at or
//      below the diagonal, two MFMA tiles give (B C^T)[j][i] (K = N); each
//      lane holds 4 consecutive j of one column i, exactly the A-operand
//      fragment of the next product after the decay exp2(s_i - s_j) * dt_j
//      and the causal mask are applied in fp32 (rounded to the operand type),
//      so acc += M X runs on MFMA with no shuffles;
//   3. D_h x_i is added from the staged x block holding row i;
//   4. the Q x 64 output tile is staged through LDS and stored as 16-byte row
//      segments.
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

template <typename E, int N, int Q>
struct ScanSmem {
    static constexpr int P = 64, JB = 64;
    static constexpr int LDB = N + 8, LDH = N + 8, LDX = JB + 8, LDY = P + 8;
    float sl[Q];   // s * log2(e)
    float dtl[Q];  // dt (0 past the sequence end)
    union {
        struct {
            E hb[P * LDH];   // H_c [p][n]
            E bb[JB * LDB];  // B block [j][n]
            E xt[P * LDX];   // x block [p][j]
        } s;
        E yt[Q * LDY];       // output tile [i][p]
    } u;
};

template <typename T, int N, int Q>
__global__ __launch_bounds__(Q * 2) void chunk_scan_kernel(
    const T *__restrict__ x, const T *__restrict__ dt, const float *__restrict__ dA_cumsum,
    const T *__restrict__ B, const T *__restrict__ C, const float *__restrict__ D,
    const float *__restrict__ chunk_init, int L, int H, int G, int nC, T *__restrict__ y) {
    using E = typename LdsT<T>::type;
    using S = ScanSmem<E, N, Q>;
    constexpr int P = 64, JB = 64, NTHR = Q * 2;
    constexpr int NK = (N + 31) / 32;  // 32-wide slices of the state index
    __shared__ __attribute__((aligned(16))) S sm;

    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int g = h / (H / G);
    const int t0 = c * Q, len = min(Q, L - t0);
    const int tid = threadIdx.x;

    const float *s = dA_cumsum + ((size_t)b * H + h) * (size_t)nC * Q + (size_t)c * Q;
    for (int i = tid; i < Q; i += NTHR) {
        sm.sl[i] = s[i] * kLog2e;
        sm.dtl[i] = i < len ? to_f32(dt[((size_t)b * L + t0 + i) * H + h]) : 0.0f;
    }
    {   // H_c -> LDS
        const float *Hc = chunk_init + (((size_t)b * nC + c) * H + h) * (size_t)P * N;
        for (int idx = tid; idx < P * N / 4; idx += NTHR) {
            const floatx4 v = reinterpret_cast<const floatx4 *>(Hc)[idx];
            const int p = (idx * 4) / N, n = (idx * 4) % N;
            E *d = sm.u.s.hb + p * S::LDH + n;
            d[0] = to_lds(v[0], d); d[1] = to_lds(v[1], d);
            d[2] = to_lds(v[2], d); d[3] = to_lds(v[3], d);
        }
    }

    const int w = wave_id(), l = lane_id(), g4 = l >> 4, r16 = l & 15;
    const int tiles[2] = {w, Q / 16 - 1 - w};
    const size_t xs = (size_t)H * P, bs = (size_t)G * N;
    const T *xh = x + (((size_t)b * L + t0) * H + h) * P;
    const T *bg = B + (((size_t)b * L + t0) * G + g) * N;
    const T *cg = C + (((size_t)b * L + t0) * G + g) * N;
    const float Dh = D ? D[h] : 0.0f;

    // C rows of this wavefront's two tiles, unscaled (operand fragments).
    Frag<T> cf[2][NK];
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
        const int i = tiles[ti] * 16 + r16;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            const int n0 = kk * 32 + 8 * g4;
            if (i < len && n0 < N) {
                float v[8];
                load8(cg + (size_t)i * bs + n0, v);
                for (int e = 0; e < 8; ++e) cf[ti][kk].set(e, v[e]);
            } else {
                cf[ti][kk].zero();
            }
        }
    }
    __syncthreads();  // sl, dtl, hb ready

    floatx4 acc[2][4];
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
        // state-to-output: (exp(s_i) C_i) . H_c[p]
        const int i = tiles[ti] * 16 + r16;
        const float sc = exp2f(sm.sl[i]);
        Frag<T> cs[NK];
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
            for (int e = 0; e < 8; ++e) cs[kk].set(e, cf[ti][kk].get(e) * sc);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
            acc[ti][pt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
                const int n0 = kk * 32 + 8 * g4;
                Frag<T> hf;
                if (n0 < N) lds_frag8(hf, sm.u.s.hb + (pt * 16 + r16) * S::LDH + n0);
                else hf.zero();
                mma(acc[ti][pt], cs[kk], hf);
            }
        }
    }

    for (int jb = 0; jb < len; jb += JB) {
        __syncthreads();  // previous block (or H_c) consumed
        // B block, natural layout: 16-byte segments
        for (int idx = tid; idx < JB * (N / 8); idx += NTHR) {
            const int j = idx / (N / 8), nb = idx % (N / 8);
            float v[8];
            if (jb + j < len) load8(bg + (size_t)(jb + j) * bs + nb * 8, v);
            else for (int e = 0; e < 8; ++e) v[e] = 0.0f;
            E *d = sm.u.s.bb + j * S::LDB + nb * 8;
            for (int e = 0; e < 8; ++e) d[e] = to_lds(v[e], d);
        }
        // x block transposed: thread = (8-wide p slice, token pair)
        for (int idx = tid; idx < 8 * 32; idx += NTHR) {
            const int pb = idx >> 5, jp = idx & 31;
            const int j0 = jb + 2 * jp;
            float v0[8], v1[8];
            if (j0 < len) load8(xh + (size_t)j0 * xs + pb * 8, v0);
            else for (int e = 0; e < 8; ++e) v0[e] = 0.0f;
            if (j0 + 1 < len) load8(xh + (size_t)(j0 + 1) * xs + pb * 8, v1);
            else for (int e = 0; e < 8; ++e) v1[e] = 0.0f;
            for (int e = 0; e < 8; ++e) {
                E *d = sm.u.s.xt + (pb * 8 + e) * S::LDX + 2 * jp;
                d[0] = to_lds(v0[e], d);
                d[1] = to_lds(v1[e], d);
            }
        }
        __syncthreads();

#pragma unroll
        for (int ti = 0; ti < 2; ++ti) {
            const int i0 = tiles[ti] * 16;
            if (i0 + 15 < jb || i0 >= len) continue;  // tile entirely before this block, or padding
            const int il = i0 + r16;                   // this lane's column i of (B C^T)
            const float si = sm.sl[il];
            for (int jp = 0; jp < 2; ++jp) {
                const int j0 = jb + 32 * jp;
                if (j0 > i0 + 15 || j0 >= len) break;  // slice strictly above the diagonal
                floatx4 m[2];
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    m[half] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
                    const int jl = 32 * jp + 16 * half + r16;  // B row within the block
#pragma unroll
                    for (int kk = 0; kk < NK; ++kk) {
                        const int n0 = kk * 32 + 8 * g4;
                        Frag<T> bf;
                        if (n0 < N) lds_frag8(bf, sm.u.s.bb + jl * S::LDB + n0);
                        else bf.zero();
                        mma(m[half], bf, cf[ti][kk]);
                    }
                }
                Frag<T> mf;
#pragma unroll
                for (int half = 0; half < 2; ++half)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = j0 + 16 * half + 4 * g4 + r;  // chunk-local token
                        float v = 0.0f;
                        if (j <= il) v = m[half][r] * exp2f(si - sm.sl[j]) * sm.dtl[j];
                        mf.set(half * 4 + r, v);
                    }
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    const E *xr = sm.u.s.xt + (pt * 16 + r16) * S::LDX + 32 * jp + 4 * g4;
                    Frag<T> xf;
                    lds_frag4x2(xf, xr, xr + 16);
                    mma(acc[ti][pt], mf, xf);
                }
            }
            if (i0 >= jb && i0 < jb + JB) {  // D x from the staged block holding rows i0..i0+15
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    const E *xr = sm.u.s.xt + (pt * 16 + r16) * S::LDX + (i0 - jb) + 4 * g4;
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[ti][pt][r] += Dh * static_cast<float>(xr[r]);
                }
            }
        }
    }

    __syncthreads();  // all blocks consumed; reuse LDS for the output tile
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
        const int i0 = tiles[ti] * 16;
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                E *d = sm.u.yt + (i0 + 4 * g4 + r) * S::LDY + pt * 16 + r16;
                *d = to_lds(acc[ti][pt][r], d);
            }
    }
    __syncthreads();
    T *yh = y + (((size_t)b * L + t0) * H + h) * P;
    constexpr int SEG = 16 / sizeof(T);  // elements per 16-byte store
    for (int idx = tid; idx < len * (P / SEG); idx += NTHR) {
        const int i = idx / (P / SEG), k = (idx % (P / SEG)) * SEG;
        *reinterpret_cast<uint4 *>(yh + (size_t)i * xs + k) =
            *reinterpret_cast<const uint4 *>(sm.u.yt + i * S::LDY + k);
    }
}

template <typename T, int N, int Q>
static void launch_scan(const void *x, const void *dt, const float *dA, const void *B,
                        const void *C, const float *D, const float *Hc, int batch, int L, int H,
                        int G, void *y, hipStream_t stream) {
    const int nC = (L + Q - 1) / Q;
    dim3 grid(nC, H, batch);
    chunk_scan_kernel<T, N, Q><<<grid, Q * 2, 0, stream>>>(
        static_cast<const T *>(x), static_cast<const T *>(dt), dA, static_cast<const T *>(B),
        static_cast<const T *>(C), D, Hc, L, H, G, nC, static_cast<T *>(y));
}

template <typename T, int N>
static bool dispatch_q(int Q, const void *x, const void *dt, const float *dA, const void *B,
                       const void *C, const float *D, const float *Hc, int batch, int L, int H,
                       int G, void *y, hipStream_t stream) {
    switch (Q) {
        case 64: launch_scan<T, N, 64>(x, dt, dA, B, C, D, Hc, batch, L, H, G, y, stream); return true;
        case 128: launch_scan<T, N, 128>(x, dt, dA, B, C, D, Hc, batch, L, H, G, y, stream); return true;
        case 256: launch_scan<T, N, 256>(x, dt, dA, B, C, D, Hc, batch, L, H, G, y, stream); return true;
        default: return false;
    }
}

template <typename T>
static hipError_t dispatch_scan(int N, int Q, const void *x, const void *dt, const float *dA,
                                const void *B, const void *C, const float *D, const float *Hc,
                                int batch, int L, int H, int G, void *y, hipStream_t stream) {
    bool ok = false;
    switch (N) {
        case 16: ok = dispatch_q<T, 16>(Q, x, dt, dA, B, C, D, Hc, batch, L, H, G, y, stream); break;
        case 32: ok = dispatch_q<T, 32>(Q, x, dt, dA, B, C, D, Hc, batch, L, H, G, y, stream); break;
        case 64: ok = dispatch_q<T, 64>(Q, x, dt, dA, B, C, D, Hc, batch, L, H, G, y, stream); break;
        case 128: ok = dispatch_q<T, 128>(Q, x, dt, dA, B, C, D, Hc, batch, L, H, G, y, stream); break;
        case 256: ok = dispatch_q<T, 256>(Q, x, dt, dA, B, C, D, Hc, batch, L, H, G, y, stream); break;
        default: break;
    }
    if (!ok) return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_chunk_scan(const void *x, const void *dt, const float *dA_cumsum, const void *B,
                             const void *C, const float *D, const float *chunk_init, int batch,
                             int seqlen, int nheads, int ngroups, int dstate, int chunk, bool bf16,
                             void *y, hipStream_t stream) {
    if (bf16)
        return dispatch_scan<bf16_t>(dstate, chunk, x, dt, dA_cumsum, B, C, D, chunk_init, batch,
                                     seqlen, nheads, ngroups, y, stream);
    return dispatch_scan<float>(dstate, chunk, x, dt, dA_cumsum, B, C, D, chunk_init, batch,
                                seqlen, nheads, ngroups, y, stream);
}

}  // namespace ssd
