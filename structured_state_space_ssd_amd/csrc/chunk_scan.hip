// Stage 4 of the SSD block decomposition: every chunk's outputs
// ("Mamba 模型", section 4.1 and "Draft:Mamba2", SSD section):
//   y_i = sum_{j<=i in chunk} (C_i . B_j) exp(s_i - s_j) dt_j x_j     diagonal block
//       + exp(s_i) H_c C_i                                            off-diagonal blocks
//       + D_h x_i.
// The diagonal block is the masked "attention-like" product (L o C B^T)(dt o x)
// (quadratic mode of the "Mamba-2架构深度解析" page, section 2.2 table); the
// off-diagonal part reads the state H_c carried into the chunk (stage 3).
//
// C B^T comes precomputed per B/C group (chunk_cb.hip) in MFMA fragment
// order. One workgroup per (chunk, head, batch) with Q/32 wavefronts; the
// output is accumulated transposed, Y^T[p][i], so each lane ends up with 4
// consecutive head-dim values of one token.
//   prologue (the only global-load phase): the chunk's x rows (128 bytes per
//     token) are loaded with 8 lanes per row and copied to LDS as they are;
//     H_c (stored by stage 3 in the operand type) is copied to LDS; s*log2(e)
//     and dt go to LDS. Wavefront w owns output tiles w and Q/16-1-w (equal
//     causal work: Q/32+1 slices of 32 tokens) and loads, in this same phase,
//     its C rows and all its C B^T fragments into registers.
//   then, with no further global load, each wavefront computes
//     - state to output: Y^T += H_c (exp(s_i) C_i)^T on MFMA (K = N);
//     - D_h x_i;
//     - per 32-token slice at or below the diagonal: the C B^T fragment times
//       the decay exp2(s_i - s_j) dt_j in fp32, rounded to the operand type.
//       Below the diagonal it factors as exp2(s_i - s_end(slice)) times a
//       per-token table exp2(s_end(slice) - s_j) dt_j (both factors <= 1):
//       one exp per lane per slice. The slice holding the diagonal takes the
//       exp per element (bf16: exp2(s_i - (s_j - log2 dt_j))) and the causal
//       mask as a select. The x operand (token index = contraction index)
//       is read with the transposing LDS read, then Y^T += X^T M^T on MFMA;
//   epilogue: Y^T tiles go to LDS as 4-element row pieces and leave as full
//     token rows.
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

template <typename E, int N, int Q>
struct ScanSmem {
    static constexpr int P = 64;
    static constexpr int LDX = colfrag_stride(P, sizeof(E));  // x rows [j][p]
    static constexpr int LDH = colfrag_stride(N, sizeof(E));  // H_c rows [p][n]
    static constexpr int LDY = P + 4;                         // output rows [i][p]
    float sl[Q];    // s * log2(e)
    float dtl[Q];   // bf16: s * log2(e) - log2(dt) (+inf past the end); float: dt (0 past the end)
    float colf[Q];  // exp2(s_end(slice of j) - s_j) * dt_j: column factor below the diagonal
    union {
        struct {
            E xs[Q * LDX];
            E hb[P * LDH];
        } s;
        E yt[Q * LDY];
    } u;
};

__device__ __forceinline__ void store4_lds(__bf16 *p, const floatx4 &v) {
    *reinterpret_cast<bf16x4 *>(p) = bf16x4{static_cast<__bf16>(v[0]), static_cast<__bf16>(v[1]),
                                            static_cast<__bf16>(v[2]), static_cast<__bf16>(v[3])};
}
__device__ __forceinline__ void store4_lds(float *p, const floatx4 &v) {
    *reinterpret_cast<floatx4 *>(p) = v;
}

template <typename T, int N, int Q>
__global__ __launch_bounds__(Q * 2, 4) void chunk_scan_kernel(
    const T *__restrict__ x, const T *__restrict__ dt, const float *__restrict__ dA_cumsum,
    const T *__restrict__ C, const typename LdsT<T>::type *__restrict__ cb,
    const float *__restrict__ D, const typename LdsT<T>::type *__restrict__ chunk_init, int L,
    int H, int G, int nC, T *__restrict__ y) {
    using E = typename LdsT<T>::type;
    using S = ScanSmem<E, N, Q>;
    constexpr int P = 64, NTHR = Q * 2, NT = Q / 16;
    constexpr int NK = (N + 31) / 32;
    constexpr int ENTRIES = (NT / 2) * (NT / 2 + 1);
    constexpr int NJP = NT / 2 + 1;              // 32-token slices per wavefront (both tiles)
    constexpr int SEG = 16 / sizeof(T);          // elements per 16-byte piece
    constexpr int XPIECES = Q * P / SEG / NTHR;  // x pieces per thread
    __shared__ __attribute__((aligned(16))) S sm;

    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int g = h / (H / G);
    const int t0 = c * Q, len = min(Q, L - t0);
    const int tid = threadIdx.x;
    const int w = wave_id(), l = lane_id(), g4 = l >> 4, r16 = l & 15;
    const int tiles[2] = {w, NT - 1 - w};
    const int njp0 = tiles[0] / 2 + 1;  // slices of tile 0; tile 1 has the rest
    const size_t xs = (size_t)H * P;
    const T *xh = x + (((size_t)b * L + t0) * H + h) * P;

    // ---- prologue: every global load of the workgroup issued up front
    uint4 xv[XPIECES];
#pragma unroll
    for (int k = 0; k < XPIECES; ++k) {
        const int idx = tid + k * NTHR;
        const int j = idx / (P / SEG), q = idx % (P / SEG);
        if (j < len) xv[k] = *reinterpret_cast<const uint4 *>(xh + (size_t)j * xs + q * SEG);
        else xv[k] = make_uint4(0, 0, 0, 0);
    }
    constexpr int HSEG = 16 / sizeof(E);
    constexpr int HITEMS = (P * N / HSEG + NTHR - 1) / NTHR;
    const E *Hc = chunk_init + (((size_t)b * nC + c) * H + h) * (size_t)P * N;
    uint4 hv[HITEMS];
#pragma unroll
    for (int it = 0; it < HITEMS; ++it) {
        const int idx = tid + it * NTHR;
        if (idx < P * N / HSEG) hv[it] = reinterpret_cast<const uint4 *>(Hc)[idx];
    }
    // this wavefront's C rows (state to output; loaded here when small) ...
    const T *cg = C + (((size_t)b * L + t0) * G + g) * N;
    const size_t cstride = (size_t)G * N;
    constexpr bool kEarlyC = NK <= 2;
    Raw8<T> cv[2][NK];
    if (kEarlyC) {
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) {
            const int il = tiles[ti] * 16 + r16;
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
                const int n0 = kk * 32 + 8 * g4;
                if (il < len && n0 < N) cv[ti][kk].load(cg + (size_t)il * cstride + n0);
                else cv[ti][kk].zero();
            }
        }
    }
    // ... and all its C B^T fragments: tile 0's slices, then tile 1's
    const E *cbc = cb + (((size_t)b * nC + c) * G + g) * (size_t)ENTRIES * 512 + l * 8;
    Frag<T> cbf[NJP];
#pragma unroll
    for (int k = 0; k < NJP; ++k) {
        const int ti = k < njp0 ? 0 : 1;
        const int it = tiles[ti], jp = ti ? k - njp0 : k;
        const int m0 = it / 2;
        const int start = (it % 2 == 0) ? m0 * (m0 + 1) : (m0 + 1) * (m0 + 1);
        load_frag8(cbf[k], cbc + (size_t)(start + jp) * 512);
    }
    // bf16: the decay-and-dt factor exp2(s_i - s_j) * dt_j is formed as one
    // exp2(s_i - (s_j - log2 dt_j)); float keeps the product (tighter rounding)
    constexpr bool kFoldDt = sizeof(T) == 2;
    const float *s = dA_cumsum + ((size_t)b * H + h) * (size_t)nC * Q + (size_t)c * Q;
    for (int i = tid; i < Q; i += NTHR) {
        const float si_ = s[i] * kLog2e;
        const float se_ = s[i | 31] * kLog2e;  // last token of i's 32-token slice
        const float draw = to_f32(dt[((size_t)b * L + t0 + min(i, len - 1)) * H + h]);
        const float d = i < len ? draw : 0.0f;
        sm.sl[i] = si_;
        sm.dtl[i] = kFoldDt ? si_ - __log2f(d) : d;
        sm.colf[i] = __builtin_amdgcn_exp2f(se_ - si_) * d;
    }
#pragma unroll
    for (int k = 0; k < XPIECES; ++k) {
        const int idx = tid + k * NTHR;
        const int j = idx / (P / SEG), q = idx % (P / SEG);
        *reinterpret_cast<uint4 *>(sm.u.s.xs + j * S::LDX + q * SEG) = xv[k];
    }
#pragma unroll
    for (int it = 0; it < HITEMS; ++it) {
        const int idx = tid + it * NTHR;
        if (idx < P * N / HSEG) {
            const int p = (idx * HSEG) / N, n = (idx * HSEG) % N;
            *reinterpret_cast<uint4 *>(sm.u.s.hb + p * S::LDH + n) = hv[it];
        }
    }
    __syncthreads();

    const float Dh = D ? D[h] : 0.0f;
    floatx4 acc[2][4];  // Y^T tiles: lane 16*g4 + i holds p = 16*pt + 4*g4 + 0..3 of token i
    float si[2];
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
        const int i0 = tiles[ti] * 16;
        si[ti] = sm.sl[i0 + r16];
        // ---- state to output: Y^T[p][i] += sum_n H_c[p][n] exp(s_i) C_i[n]
        if (!kEarlyC) {
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
                const int n0 = kk * 32 + 8 * g4;
                if (i0 + r16 < len && n0 < N) cv[ti][kk].load(cg + (size_t)(i0 + r16) * cstride + n0);
                else cv[ti][kk].zero();
            }
        }
        const float sc = __builtin_amdgcn_exp2f(si[ti]);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) acc[ti][pt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            const int n0 = kk * 32 + 8 * g4;
            Frag<T> cf;
#pragma unroll
            for (int e = 0; e < 8; ++e) cf.set(e, cv[ti][kk].get(e) * sc);
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                Frag<T> hf;
                if (n0 < N) lds_frag8(hf, sm.u.s.hb + (pt * 16 + r16) * S::LDH + n0);
                else hf.zero();
                mma(acc[ti][pt], hf, cf);
            }
        }
        // ---- D_h x_i: token i0 + r16, head-dim 16*pt + 4*g4 + 0..3
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
            const E *xr = sm.u.s.xs + (i0 + r16) * S::LDX + pt * 16 + 4 * g4;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[ti][pt][r] += Dh * static_cast<float>(xr[r]);
        }
    }
    // ---- diagonal blocks: NJP slices of 32 tokens, tile 0's first
#pragma unroll
    for (int k = 0; k < NJP; ++k) {
        const int ti = k < njp0 ? 0 : 1;  // uniform across the wavefront
        const int jp = ti ? k - njp0 : k;
        const int il = tiles[ti] * 16 + r16;
        const float s_i = ti ? si[1] : si[0];
        const int jb = jp * 32 + 4 * g4;  // this lane's first token (elements 0..3)
        Frag<T> mf;
        if (jp != tiles[ti] / 2) {
            // strictly below the diagonal: exp2(s_i - s_j) dt_j =
            // exp2(s_i - s_end(slice)) * colf[j], both factors <= 1; no mask
            const float rowf = __builtin_amdgcn_exp2f(s_i - sm.sl[jp * 32 + 31]);
            const floatx4 c0 = *reinterpret_cast<const floatx4 *>(sm.colf + jb);
            const floatx4 c1 = *reinterpret_cast<const floatx4 *>(sm.colf + jb + 16);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                mf.set(r, cbf[k].get(r) * c0[r] * rowf);
                mf.set(4 + r, cbf[k].get(4 + r) * c1[r] * rowf);
            }
        } else {
            // the slice holding the diagonal: per-element decay and causal mask
            const floatx4 d0 = *reinterpret_cast<const floatx4 *>(sm.dtl + jb);
            const floatx4 d1 = *reinterpret_cast<const floatx4 *>(sm.dtl + jb + 16);
            float v[8];
            if (kFoldDt) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    v[r] = cbf[k].get(r) * __builtin_amdgcn_exp2f(s_i - d0[r]);
                    v[4 + r] = cbf[k].get(4 + r) * __builtin_amdgcn_exp2f(s_i - d1[r]);
                }
            } else {
                const floatx4 s0 = *reinterpret_cast<const floatx4 *>(sm.sl + jb);
                const floatx4 s1 = *reinterpret_cast<const floatx4 *>(sm.sl + jb + 16);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    v[r] = cbf[k].get(r) * __builtin_amdgcn_exp2f(s_i - s0[r]) * d0[r];
                    v[4 + r] = cbf[k].get(4 + r) * __builtin_amdgcn_exp2f(s_i - s1[r]) * d1[r];
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                mf.set(r, jb + r <= il ? v[r] : 0.0f);
                mf.set(4 + r, jb + 16 + r <= il ? v[4 + r] : 0.0f);
            }
        }
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
            Frag<T> xf;  // x^T rows p = 16*pt + r16 at tokens jb + 0..3 and jb + 16 + 0..3
            lds_colfrag(xf, sm.u.s.xs, S::LDX, jb, jb + 16, pt * 16);
            if (ti == 0) mma(acc[0][pt], xf, mf);
            else mma(acc[1][pt], xf, mf);
        }
    }

    __syncthreads();  // x and H no longer read; reuse LDS for the output tile
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
        const int i = tiles[ti] * 16 + r16;
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) store4_lds(sm.u.yt + i * S::LDY + pt * 16 + 4 * g4, acc[ti][pt]);
    }
    __syncthreads();
    T *yh = y + (((size_t)b * L + t0) * H + h) * P;
    constexpr int QSEG = 8 / sizeof(T);  // elements per 8-byte piece
    for (int idx = tid; idx < len * (P / QSEG); idx += NTHR) {
        const int i = idx / (P / QSEG), k = (idx % (P / QSEG)) * QSEG;
        *reinterpret_cast<uint2 *>(yh + (size_t)i * xs + k) =
            *reinterpret_cast<const uint2 *>(sm.u.yt + i * S::LDY + k);
    }
}

template <typename T, int N, int Q>
static void launch_scan(const void *x, const void *dt, const float *dA, const void *C,
                        const void *cb, const float *D, const void *Hc, int batch, int L, int H,
                        int G, void *y, hipStream_t stream) {
    using E = typename LdsT<T>::type;
    const int nC = (L + Q - 1) / Q;
    const dim3 grid(nC, H, batch);
    chunk_scan_kernel<T, N, Q><<<grid, Q * 2, 0, stream>>>(
        static_cast<const T *>(x), static_cast<const T *>(dt), dA, static_cast<const T *>(C),
        static_cast<const E *>(cb), D, static_cast<const E *>(Hc), L, H, G, nC,
        static_cast<T *>(y));
}

template <typename T, int N>
static bool scan_q(int Q, const void *x, const void *dt, const float *dA, const void *C,
                   const void *cb, const float *D, const void *Hc, int batch, int L, int H, int G,
                   void *y, hipStream_t s) {
    switch (Q) {
        case 64: launch_scan<T, N, 64>(x, dt, dA, C, cb, D, Hc, batch, L, H, G, y, s); return true;
        case 128: launch_scan<T, N, 128>(x, dt, dA, C, cb, D, Hc, batch, L, H, G, y, s); return true;
        case 256: launch_scan<T, N, 256>(x, dt, dA, C, cb, D, Hc, batch, L, H, G, y, s); return true;
        default: return false;
    }
}

template <typename T>
static hipError_t scan_dispatch(int N, int Q, const void *x, const void *dt, const float *dA,
                                const void *C, const void *cb, const float *D, const void *Hc,
                                int batch, int L, int H, int G, void *y, hipStream_t s) {
    bool ok = false;
    switch (N) {
        case 16: ok = scan_q<T, 16>(Q, x, dt, dA, C, cb, D, Hc, batch, L, H, G, y, s); break;
        case 32: ok = scan_q<T, 32>(Q, x, dt, dA, C, cb, D, Hc, batch, L, H, G, y, s); break;
        case 64: ok = scan_q<T, 64>(Q, x, dt, dA, C, cb, D, Hc, batch, L, H, G, y, s); break;
        case 128: ok = scan_q<T, 128>(Q, x, dt, dA, C, cb, D, Hc, batch, L, H, G, y, s); break;
        case 256: ok = scan_q<T, 256>(Q, x, dt, dA, C, cb, D, Hc, batch, L, H, G, y, s); break;
        default: break;
    }
    if (!ok) return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_chunk_scan(const void *x, const void *dt, const float *dA_cumsum, const void *C,
                             const void *cb, const float *D, const void *chunk_init, int batch,
                             int seqlen, int nheads, int ngroups, int dstate, int chunk, bool bf16,
                             void *y, hipStream_t stream) {
    if (bf16)
        return scan_dispatch<bf16_t>(dstate, chunk, x, dt, dA_cumsum, C, cb, D, chunk_init, batch,
                                     seqlen, nheads, ngroups, y, stream);
    return scan_dispatch<float>(dstate, chunk, x, dt, dA_cumsum, C, cb, D, chunk_init, batch,
                                seqlen, nheads, ngroups, y, stream);
}

}  // namespace ssd
