// Backward pass of the chunked SSD layer: the gradients of
//   loss = sum_t dy_t . y_t + <dfinal, h_L>
// with respect to x, dt, A, B, C, D, the initial state and the dt bias.
//
// The adjoint of the state, g_t = dloss/dh_t, runs backward in time:
// g_t = dy_t C_t^T + a_{t+1} g_{t+1}. Chunked like the forward ("Mamba 模型",
// section 4.1: the same semiseparable matrix, transposed), with s the
// within-chunk prefix sums of step*A, w the input weights, H_c the state
// entering chunk c (forward recompute) and G_{c+1} the adjoint of the state
// leaving chunk c (the reverse state passing over dS_c = sum_i e^{s_i} dy_i C_i^T),
// one chunk's gradients are, for tokens i >= j of the chunk,
//   dx_j  = w_j sum_i e^{s_i-s_j} (C_i.B_j) dy_i + w_j e^{s_end-s_j} G B_j + D dy_j
//   dw_j  = sum_i e^{s_i-s_j} (C_i.B_j)(dy_i.x_j) + e^{s_end-s_j} x_j.(G B_j)
//   dB_j += w_j sum_i e^{s_i-s_j} (dy_i.x_j) C_i + w_j e^{s_end-s_j} G^T x_j
//   dC_i += sum_j e^{s_i-s_j} w_j (dy_i.x_j) B_j + e^{s_i} H^T dy_i
//   ds_i  = sum_{j<i} T_ij - sum_{k>i} T_ki + e^{s_i} dy_i.(H C_i)
//           - w_i e^{s_end-s_i} x_i.(G B_i),   T_ij = e^{s_i-s_j}(C_i.B_j) w_j (dy_i.x_j),
// and the chunk's last token also takes d/ds_end = sum_j w_j e^{s_end-s_j}
// x_j.(G B_j) + e^{s_end} <G, H>. The stage-1 backward then turns ds into
// dstep = A * (suffix sums of ds) and adds the weight's dw.
//
// chunk_bwd_kernel: one workgroup per (batch, chunk, B/C group) and block of
// heads of that group, Q/16 wavefronts; wavefront w owns tokens 16w..16w+15
// both as the column index j (first pass: the products over the tokens
// i >= j of every 32-token slice, dx, dB, dw and the column sums of T) and as
// the row index i (second pass: slices j <= i, dC and the row sums of T), so
// the causal work is the same for every wavefront. Every 16x16 block of
// dy.x is formed on MFMA in the orientation the next product needs (its rows
// the contraction index, split over the two halves of a slice); the C.B
// blocks, the same for every head of the workgroup, are formed once and kept
// in LDS in float32 (read in either orientation) where LDS allows. Blocks
// are decayed and masked in fp32, rounded to the operand type and multiplied.
// dB and dC accumulate over the block's heads in registers and leave as
// float32 partial sums per head block (reduced by bwd_reduce_kernel).
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

__device__ __forceinline__ float xor_sum_groups(float v) {  // over the 4 lane groups of 16
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

__device__ __forceinline__ float xor_sum_16(float v) {  // over the 16 lanes of a group
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o);
    return v;
}

template <typename T>
__device__ __forceinline__ void store4_global(T *p, const floatx4 &v);
template <>
__device__ __forceinline__ void store4_global<bf16_t>(bf16_t *p, const floatx4 &v) {
    *reinterpret_cast<bf16x4 *>(p) = bf16x4{static_cast<__bf16>(v[0]), static_cast<__bf16>(v[1]),
                                            static_cast<__bf16>(v[2]), static_cast<__bf16>(v[3])};
}
template <>
__device__ __forceinline__ void store4_global<float>(float *p, const floatx4 &v) {
    *reinterpret_cast<floatx4 *>(p) = v;
}

// Four consecutive LDS elements as floats (8- or 16-byte aligned).
__device__ __forceinline__ void read4(float (&v)[4], const __bf16 *p) {
    const bf16x4 b = *reinterpret_cast<const bf16x4 *>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = static_cast<float>(b[e]);
}
__device__ __forceinline__ void read4(float (&v)[4], const float *p) {
    const floatx4 b = *reinterpret_cast<const floatx4 *>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = b[e];
}

}  // namespace

template <typename T, int N, int Q>
struct BwdLds {
    using E = typename LdsT<T>::type;
    static constexpr int P = 64;
    static constexpr int LDX = colfrag_stride(P, sizeof(E));
    static constexpr int LDB = colfrag_stride(N, sizeof(E));
    static constexpr size_t kBytes =
        sizeof(E) * ((size_t)2 * Q * LDX + (size_t)2 * Q * LDB + (size_t)2 * P * LDB) +
        4 * Q * sizeof(float) + 16;
    // The chunk's C_i . B_j in 16x16 blocks (row block bi of tokens i, column
    // block bj of tokens j), float32, kept for all heads of the workgroup where
    // LDS allows: the blocks with bi >= 2 floor(bj / 2), those the first pass
    // of wavefront bj reads (the second pass reads the same blocks transposed).
    static constexpr int QB = Q / 16;
    static constexpr int kCbBlocks = [] {
        int n = 0;
        for (int bj = 0; bj < QB; ++bj) n += QB - 2 * (bj / 2);
        return n;
    }();
    static constexpr bool kCbCache = kBytes + (size_t)kCbBlocks * 1024 <= 160 * 1024;
};

// Index of block (bi, bj) in the C . B^T cache (bi >= 2 floor(bj / 2)).
template <int QB>
__device__ __forceinline__ int cb_block(int bi, int bj) {
    const int pj = bj >> 1;
    return pj * (2 * QB - 2 * pj + 2) + (bj & 1) * (QB - 2 * pj) + bi - 2 * pj;
}
// Lane l's 16-byte slot within a cached block: swizzled so that both the
// first pass's 16-byte reads (lane l, its own slot) and the second pass's
// 4-byte transposed reads hit distinct banks.
__device__ __forceinline__ int cb_slot(int l) { return l ^ ((l >> 4) & 3); }

template <typename T, int N, int Q>
__global__ __launch_bounds__(Q * 4) void chunk_bwd_kernel(
    const T *__restrict__ x, const T *__restrict__ dy, const float *__restrict__ dA_cumsum,
    const float *__restrict__ delta, const T *__restrict__ B, const T *__restrict__ C,
    const float *__restrict__ D, const typename LdsT<T>::type *__restrict__ chunk_init,
    const typename LdsT<T>::type *__restrict__ grad_next, int batch, int L, int H, int G, int nC,
    int nblk,
    T *__restrict__ dx, float *__restrict__ ds_out, float *__restrict__ dw_out,
    float *__restrict__ dB_part, float *__restrict__ dC_part, float *__restrict__ dD_part) {
    using E = typename LdsT<T>::type;
    using S = BwdLds<T, N, Q>;
    constexpr int P = 64, NTHR = Q * 4, NT = N / 16, NK = (N + 31) / 32;
    constexpr int LDX = S::LDX, LDB = S::LDB;
    constexpr int XPR = P * (int)sizeof(T) / 16;  // 16-byte pieces per x / dy row
    constexpr int BPR = N * (int)sizeof(T) / 16;  // ... per B / C / H / G row
    constexpr int EPP = 16 / (int)sizeof(T);      // elements per piece
    __shared__ __attribute__((aligned(32))) E xs[Q * LDX];
    __shared__ __attribute__((aligned(32))) E dys[Q * LDX];
    __shared__ __attribute__((aligned(32))) E bs[Q * LDB];
    __shared__ __attribute__((aligned(32))) E cs[Q * LDB];
    __shared__ __attribute__((aligned(32))) E hs[P * LDB];
    __shared__ __attribute__((aligned(32))) E gs[P * LDB];
    __shared__ __attribute__((aligned(16))) float slt[Q];  // s * log2(e)
    __shared__ __attribute__((aligned(16))) float wt[Q];   // input weights (0 past the end)
    // per token t, within its 32-token slice [r, e]: exp(s_t - s_r) and
    // exp(s_e - s_t) w_t (both <= 1), the column and row factors of the decay
    // between tokens of different slices
    __shared__ __attribute__((aligned(16))) float p1t[Q];
    __shared__ __attribute__((aligned(16))) float p2t[Q];
    __shared__ float red[4];
    __shared__ __attribute__((aligned(16))) floatx4 cbc[S::kCbCache ? S::kCbBlocks * 64 : 1];

    const int kb = blockIdx.x % nblk, u = blockIdx.x / nblk;
    const int hpg = H / G;
    const int c = u % nC, g = (u / nC) % G, b = u / (nC * G);
    const int nh = (hpg - kb + nblk - 1) / nblk;
    const int t0 = c * Q, len = min(Q, L - t0);
    // (the wavefront index as a scalar: the slice loops below run per wavefront)
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = lane_id(), g4 = l >> 4, c16 = l & 15;
    const int tok = 16 * w + c16;  // this lane's token: column j of pass 1, row i of pass 2
    const size_t xrow = (size_t)H * P, brow = (size_t)G * N;

    // ---- B and C rows of the chunk (zero past the end), for every head
    for (int idx = tid; idx < Q * BPR; idx += NTHR) {
        const int j = idx / BPR, q = idx % BPR;
        uint4 vb = make_uint4(0, 0, 0, 0), vc = make_uint4(0, 0, 0, 0);
        if (j < len) {
            const size_t o = ((size_t)b * L + t0 + j) * brow + (size_t)g * N + q * EPP;
            vb = *reinterpret_cast<const uint4 *>(B + o);
            vc = *reinterpret_cast<const uint4 *>(C + o);
        }
        *reinterpret_cast<uint4 *>(bs + j * LDB + q * EPP) = vb;
        *reinterpret_cast<uint4 *>(cs + j * LDB + q * EPP) = vc;
    }
    if constexpr (S::kCbCache) {
        // wavefront w forms blocks (bi, w), bi >= 2 floor(w / 2): rows i = 16 bi +
        // 4 g4 + e, column j = tok (its first pass's C . B blocks), once for every
        // head of the workgroup; the head loop's first barrier publishes them
        __syncthreads();  // B and C rows in LDS
        Frag<T> ob[NK];
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            const int n0 = kk * 32 + 8 * g4;
            if (n0 < N) lds_frag8(ob[kk], bs + tok * LDB + n0);
            else ob[kk].zero();
        }
        for (int bi = 2 * (w / 2); bi < Q / 16; ++bi) {  // wave-uniform trip count
            const int ir = 16 * bi + c16;  // A-operand row (token i)
            floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
                const int n0 = kk * 32 + 8 * g4;
                Frag<T> fa;
                if (n0 < N) lds_frag8(fa, cs + ir * LDB + n0);
                else fa.zero();
                mma(acc, fa, ob[kk]);
            }
            cbc[cb_block<Q / 16>(bi, w) * 64 + cb_slot(l)] = acc;
        }
    }

    floatx4 dBT[NT], dCT[NT];  // lane (g4, c16): rows n = 16nt + 4g4 + e, column token tok
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) dBT[nt] = dCT[nt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

    // Per head, x, dy, H_c, G and the tables travel through registers: the next
    // head's loads are issued right after this head's values reach LDS and
    // complete while this head computes (nothing in between waits on a global
    // load: the head's barrier below is an LDS-only one).
    constexpr int XI = (Q * XPR + NTHR - 1) / NTHR, HI = (P * BPR + NTHR - 1) / NTHR;
    uint4 px[XI], pd[XI], ph[HI], pg[HI];
    float ps = 0.0f, pw = 0.0f, pD = 0.0f;
    auto fetch = [&](int h) {
        const T *xh = x + ((size_t)b * L + t0) * xrow + (size_t)h * P;
        const T *dyh = dy + ((size_t)b * L + t0) * xrow + (size_t)h * P;
#pragma unroll
        for (int i = 0; i < XI; ++i) {
            const int idx = tid + i * NTHR, j = idx / XPR, q = idx % XPR;
            px[i] = pd[i] = make_uint4(0, 0, 0, 0);
            if (idx < Q * XPR && j < len) {
                px[i] = *reinterpret_cast<const uint4 *>(xh + (size_t)j * xrow + q * EPP);
                pd[i] = *reinterpret_cast<const uint4 *>(dyh + (size_t)j * xrow + q * EPP);
            }
        }
        const size_t st = (((size_t)b * nC + c) * H + h) * (size_t)P * N;
#pragma unroll
        for (int i = 0; i < HI; ++i) {
            const int idx = tid + i * NTHR, p = idx / BPR, q = idx % BPR;
            if (idx < P * BPR) {
                ph[i] = *reinterpret_cast<const uint4 *>(chunk_init + st + (size_t)p * N + q * EPP);
                pg[i] = *reinterpret_cast<const uint4 *>(grad_next + st + (size_t)p * N + q * EPP);
            }
        }
        if (tid < Q) {
            const size_t srow = ((size_t)b * H + h) * (size_t)nC * Q + (size_t)c * Q;
            ps = dA_cumsum[srow + tid];
            pw = delta[srow + tid];
        }
        pD = D ? D[h] : 0.0f;
    };
    fetch(g * hpg + kb);

    for (int k = 0; k < nh; ++k) {
        const int h = g * hpg + kb + k * nblk;
        __syncthreads();  // the previous head is done with LDS; this head's loads are in
        if (tid < 4) red[tid] = 0.0f;
#pragma unroll
        for (int i = 0; i < XI; ++i) {
            const int idx = tid + i * NTHR, j = idx / XPR, q = idx % XPR;
            if (idx < Q * XPR) {
                *reinterpret_cast<uint4 *>(xs + j * LDX + q * EPP) = px[i];
                *reinterpret_cast<uint4 *>(dys + j * LDX + q * EPP) = pd[i];
            }
        }
#pragma unroll
        for (int i = 0; i < HI; ++i) {
            const int idx = tid + i * NTHR, p = idx / BPR, q = idx % BPR;
            if (idx < P * BPR) {
                *reinterpret_cast<uint4 *>(hs + p * LDB + q * EPP) = ph[i];
                *reinterpret_cast<uint4 *>(gs + p * LDB + q * EPP) = pg[i];
            }
        }
        if (tid < Q) {  // whole wavefronts; a slice's tokens share one
            const float sl = ps * kLog2e;
            slt[tid] = sl;
            wt[tid] = pw;
            const float sr = __shfl(sl, l & ~31), se = __shfl(sl, l | 31);
            p1t[tid] = __builtin_amdgcn_exp2f(sl - sr);
            p2t[tid] = __builtin_amdgcn_exp2f(se - sl) * pw;
        }
        const float Dh = pD;
        const size_t srow = ((size_t)b * H + h) * (size_t)nC * Q + (size_t)c * Q;
        barrier_lds();
        if (k + 1 < nh) fetch(h + nblk);

        const float sl_t = slt[tok], w_t = wt[tok];
        const float sl_end = slt[len - 1];
        const float f_t = __builtin_amdgcn_exp2f(sl_end - sl_t);  // exp(s_end - s_tok)
        const float e_t = __builtin_amdgcn_exp2f(sl_t);           // exp(s_tok)

        // the lane's own token rows as MFMA B operands, for every slice of both
        // passes (B and C rows kept in registers for N <= 64, else re-read)
        constexpr bool kKeepBC = NK <= 2;
        Frag<T> tx[P / 32], tdy[P / 32], tb[kKeepBC ? NK : 1], tc[kKeepBC ? NK : 1];
#pragma unroll
        for (int kk = 0; kk < P / 32; ++kk) {
            lds_frag8(tx[kk], xs + tok * LDX + kk * 32 + 8 * g4);
            lds_frag8(tdy[kk], dys + tok * LDX + kk * 32 + 8 * g4);
        }
        auto own = [&](const E *m, int kk, Frag<T> &f) {  // row tok of B or C at k-step kk
            const int n0 = kk * 32 + 8 * g4;
            if (n0 < N) lds_frag8(f, m + tok * LDB + n0);
            else f.zero();
        };
        if constexpr (kKeepBC) {
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
                own(bs, kk, tb[kk]);
                own(cs, kk, tc[kk]);
            }
        }
        auto own_b = [&](int kk) -> Frag<T> {
            if constexpr (kKeepBC) return tb[kk];
            Frag<T> f;
            own(bs, kk, f);
            return f;
        };
        auto own_c = [&](int kk) -> Frag<T> {
            if constexpr (kKeepBC) return tc[kk];
            Frag<T> f;
            own(cs, kk, f);
            return f;
        };

        // ================= pass 1: tok as column j, slices of rows i >= j
        floatx4 dxT[4];  // lane (g4, c16): dx[tok][16pt + 4g4 + e]
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) dxT[pt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
        float cin = 0.0f, cex = 0.0f;  // column sums of e^{s_i-s_j} CB DX (with / without i = j)
        float cfar = 0.0f;             // the part of both from slices after tok's
        // a slice's dy_i.x_j and C_i.B_j blocks, rows i of the slice, column tok
        auto p1_blocks = [&](int sl, floatx4 (&dxo)[2], floatx4 (&cbo)[2]) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int ir = 32 * sl + 16 * half + c16;  // A-operand row (token i)
                dxo[half] = cbo[half] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int kk = 0; kk < P / 32; ++kk) {
                    Frag<T> fa;
                    lds_frag8(fa, dys + ir * LDX + kk * 32 + 8 * g4);
                    mma(dxo[half], fa, tx[kk]);
                }
                if constexpr (S::kCbCache) {
                    cbo[half] = cbc[cb_block<Q / 16>(2 * sl + half, w) * 64 + cb_slot(l)];
                } else {
#pragma unroll
                    for (int kk = 0; kk < NK; ++kk) {
                        const int n0 = kk * 32 + 8 * g4;
                        Frag<T> fa;
                        if (n0 < N) lds_frag8(fa, cs + ir * LDB + n0);
                        else fa.zero();
                        mma(cbo[half], fa, own_b(kk));
                    }
                }
            }
        };
        auto p1_products = [&](int sl, const Frag<T> &mf, const Frag<T> &ef) {
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                Frag<T> fa;  // dy^T: rows p = 16pt + c16, contraction over the slice's tokens
                lds_colfrag(fa, dys, LDX, 32 * sl + 4 * g4, 32 * sl + 16 + 4 * g4, pt * 16);
                mma(dxT[pt], fa, mf);
            }
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                Frag<T> fa;  // C^T: rows n = 16nt + c16
                lds_colfrag(fa, cs, LDB, 32 * sl + 4 * g4, 32 * sl + 16 + 4 * g4, nt * 16);
                mma(dBT[nt], fa, ef);
            }
        };
        {  // the slice holding tok: exp per element, mask i >= tok
            const int sl = w / 2;
            floatx4 dxo[2], cbo[2];
            p1_blocks(sl, dxo, cbo);
            // element (half, e): token i = 32 sl + 16 half + 4 g4 + e, column j = tok
            Frag<T> mf, ef;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int i0 = 32 * sl + 16 * half + 4 * g4;
                const floatx4 si4 = *reinterpret_cast<const floatx4 *>(slt + i0);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = i0 + e;
                    const float lij = i >= tok ? __builtin_amdgcn_exp2f(si4[e] - sl_t) : 0.0f;
                    const float lcb = lij * cbo[half][e];
                    const float t = lcb * dxo[half][e];
                    cin += t;
                    cex += i != tok ? t : 0.0f;
                    mf.set(4 * half + e, lcb * w_t);
                    ef.set(4 * half + e, lij * dxo[half][e] * w_t);
                }
            }
            p1_products(sl, mf, ef);
        }
        for (int sl = w / 2 + 1; sl < Q / 32; ++sl) {
            // every i > tok: e^{s_i - s_tok} = e^{s_i - s_r} e^{s_r - s_tok}, r = 32 sl,
            // both factors <= 1
            floatx4 dxo[2], cbo[2];
            p1_blocks(sl, dxo, cbo);
            const float fr = __builtin_amdgcn_exp2f(slt[32 * sl] - sl_t);
            Frag<T> mf, ef;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int i0 = 32 * sl + 16 * half + 4 * g4;
                const floatx4 c4 = *reinterpret_cast<const floatx4 *>(p1t + i0);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float lij = c4[e] * fr;
                    const float lcb = lij * cbo[half][e];
                    cfar = __builtin_fmaf(lcb, dxo[half][e], cfar);
                    mf.set(4 * half + e, lcb * w_t);
                    ef.set(4 * half + e, (lij * w_t) * dxo[half][e]);
                }
            }
            p1_products(sl, mf, ef);
        }
        // ---- the state leaving the chunk: U = G B_j^T, V = G^T x_j
        float xu = 0.0f;  // x_j . (G B_j), partial over this lane's p
        const float wf = w_t * f_t;
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
            floatx4 uo = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
                const int n0 = kk * 32 + 8 * g4;
                Frag<T> fa;
                if (n0 < N) lds_frag8(fa, gs + (pt * 16 + c16) * LDB + n0);
                else fa.zero();
                mma(uo, fa, own_b(kk));
            }
            float xv[4], dv[4];
            read4(xv, xs + tok * LDX + pt * 16 + 4 * g4);
            read4(dv, dys + tok * LDX + pt * 16 + 4 * g4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xu += xv[e] * uo[e];
                dxT[pt][e] += wf * uo[e] + Dh * dv[e];
            }
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            floatx4 vo = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < P / 32; ++kk) {
                Frag<T> fa, fb;  // contraction over p
                lds_colfrag(fa, gs, LDB, kk * 32 + 4 * g4, kk * 32 + 16 + 4 * g4, nt * 16);
                lds_frag4x2(fb, xs + tok * LDX + kk * 32 + 4 * g4, xs + tok * LDX + kk * 32 + 16 + 4 * g4);
                mma(vo, fa, fb);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) dBT[nt][e] += wf * vo[e];
        }
        // ordinary stores: each instruction writes a quarter of every row, and
        // the four quarters meet in L2 as whole lines before they go to memory
        // (as non-temporal stores they reached memory as partial lines, which
        // cost half as many bytes again as dx itself)
        if (tok < len) {
            T *dxr = dx + ((size_t)b * L + t0 + tok) * xrow + (size_t)h * P;
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) store4_global<T>(dxr + pt * 16 + 4 * g4, dxT[pt]);
        }
        cin = xor_sum_groups(cin + cfar);
        cex = xor_sum_groups(cex + cfar);
        xu = xor_sum_groups(xu);
        const float dw_t = cin + f_t * xu;
        float ds_t = -w_t * cex - wf * xu;
        {  // d/ds_end: sum_j w_j f_j x_j.(G B_j), one wavefront partial
            const float part = xor_sum_16(g4 == 0 ? wf * xu : 0.0f);
            if (l == 0) atomicAdd(&red[0], part);
        }

        // ================= pass 2: tok as row i, slices of columns j <= i
        float rs = 0.0f;  // row sum of T over j < i
        // a slice's x_j.dy_i and B_j.C_i blocks, rows j of the slice, column tok
        auto p2_blocks = [&](int sl, floatx4 (&dxo)[2], floatx4 (&cbo)[2]) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int jr = 32 * sl + 16 * half + c16;  // A-operand row (token j)
                dxo[half] = cbo[half] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int kk = 0; kk < P / 32; ++kk) {
                    Frag<T> fa;
                    lds_frag8(fa, xs + jr * LDX + kk * 32 + 8 * g4);
                    mma(dxo[half], fa, tdy[kk]);
                }
                if constexpr (S::kCbCache) {
                    // element e: C_tok . B_j, j = 16 bj + 4 g4 + e, held in block
                    // (w, bj) by lane 16 (c16 / 4) + 4 g4 + e as its element c16 % 4
                    const float *blk = reinterpret_cast<const float *>(
                        cbc + cb_block<Q / 16>(w, 2 * sl + half) * 64);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        cbo[half][e] = blk[cb_slot(16 * (c16 >> 2) + 4 * g4 + e) * 4 + (c16 & 3)];
                } else {
#pragma unroll
                    for (int kk = 0; kk < NK; ++kk) {
                        const int n0 = kk * 32 + 8 * g4;
                        Frag<T> fa;
                        if (n0 < N) lds_frag8(fa, bs + jr * LDB + n0);
                        else fa.zero();
                        mma(cbo[half], fa, own_c(kk));
                    }
                }
            }
        };
        auto p2_products = [&](int sl, const Frag<T> &wfr) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                Frag<T> fa;  // B^T: rows n = 16nt + c16, contraction over the slice's tokens
                lds_colfrag(fa, bs, LDB, 32 * sl + 4 * g4, 32 * sl + 16 + 4 * g4, nt * 16);
                mma(dCT[nt], fa, wfr);
            }
        };
        for (int sl = 0; sl < w / 2; ++sl) {
            // every j < tok: e^{s_tok - s_j} w_j = e^{s_tok - s_e} (e^{s_e - s_j} w_j),
            // e = 32 sl + 31, both factors <= 1
            floatx4 dxo[2], cbo[2];
            p2_blocks(sl, dxo, cbo);
            const float fe = __builtin_amdgcn_exp2f(sl_t - slt[32 * sl + 31]);
            Frag<T> wfr;  // e^{s_i-s_j} w_j (dy_i.x_j), rows j of the slice
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int j0 = 32 * sl + 16 * half + 4 * g4;
                const floatx4 c4 = *reinterpret_cast<const floatx4 *>(p2t + j0);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float v = (c4[e] * fe) * dxo[half][e];
                    wfr.set(4 * half + e, v);
                    rs = __builtin_fmaf(v, cbo[half][e], rs);
                }
            }
            p2_products(sl, wfr);
        }
        {  // the slice holding tok: exp per element, mask j <= tok
            const int sl = w / 2;
            floatx4 dxo[2], cbo[2];
            p2_blocks(sl, dxo, cbo);
            Frag<T> wfr;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int j0 = 32 * sl + 16 * half + 4 * g4;
                const floatx4 sj4 = *reinterpret_cast<const floatx4 *>(slt + j0);
                const floatx4 wj4 = *reinterpret_cast<const floatx4 *>(wt + j0);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = j0 + e;
                    const float lw = j <= tok ? __builtin_amdgcn_exp2f(sl_t - sj4[e]) * wj4[e] : 0.0f;
                    const float v = lw * dxo[half][e];
                    wfr.set(4 * half + e, v);
                    rs += j < tok ? v * cbo[half][e] : 0.0f;
                }
            }
            p2_products(sl, wfr);
        }
        // ---- the state entering the chunk: H^T dy_i and H C_i
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            floatx4 vo = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < P / 32; ++kk) {
                Frag<T> fa, fb;
                lds_colfrag(fa, hs, LDB, kk * 32 + 4 * g4, kk * 32 + 16 + 4 * g4, nt * 16);
                lds_frag4x2(fb, dys + tok * LDX + kk * 32 + 4 * g4, dys + tok * LDX + kk * 32 + 16 + 4 * g4);
                mma(vo, fa, fb);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) dCT[nt][e] += e_t * vo[e];
        }
        float dych = 0.0f, dd = 0.0f;
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
            floatx4 co = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
                const int n0 = kk * 32 + 8 * g4;
                Frag<T> fa;
                if (n0 < N) lds_frag8(fa, hs + (pt * 16 + c16) * LDB + n0);
                else fa.zero();
                mma(co, fa, own_c(kk));
            }
            float xv[4], dv[4];
            read4(xv, xs + tok * LDX + pt * 16 + 4 * g4);
            read4(dv, dys + tok * LDX + pt * 16 + 4 * g4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dych += dv[e] * co[e];
                dd += dv[e] * xv[e];
            }
        }
        rs = xor_sum_groups(rs);
        dych = xor_sum_groups(dych);
        dd = xor_sum_groups(dd);
        ds_t += rs + e_t * dych;
        {
            const float part = xor_sum_16(g4 == 0 ? dd : 0.0f);
            if (l == 0) atomicAdd(&red[2], part);
        }
        {  // <G, H>, spread over the workgroup: eight consecutive n per thread
            float gh = 0.0f;
            for (int idx = tid; idx < P * N / 8; idx += NTHR) {
                const int o = idx / (N / 8) * LDB + idx % (N / 8) * 8;
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    float gv[4], hv[4];
                    read4(gv, gs + o + 4 * hf);
                    read4(hv, hs + o + 4 * hf);
#pragma unroll
                    for (int e = 0; e < 4; ++e) gh = __builtin_fmaf(gv[e], hv[e], gh);
                }
            }
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) gh += __shfl_xor(gh, o);
            if (l == 0) atomicAdd(&red[1], gh);
        }
        barrier_lds();  // red[] complete
        if (tok == len - 1) ds_t += red[0] + __builtin_amdgcn_exp2f(sl_end) * red[1];
        if (g4 == 0) {
            ds_out[srow + tok] = ds_t;
            dw_out[srow + tok] = dw_t;
        }
        if (tid == 0) dD_part[((size_t)b * nC + c) * H + h] = red[2];
    }

    // ---- this head block's share of dB and dC: dB_part[kb][b][t][g][n]
    if (tok < len) {
        const size_t o = ((size_t)kb * batch + b) * L * brow + (size_t)(t0 + tok) * brow + (size_t)g * N;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            *reinterpret_cast<floatx4 *>(dB_part + o + nt * 16 + 4 * g4) = dBT[nt];
            *reinterpret_cast<floatx4 *>(dC_part + o + nt * 16 + 4 * g4) = dCT[nt];
        }
    }
}

// dB, dC (input dtype) = the sums of the head blocks' float32 partial sums,
// both in one launch: blockIdx.y picks the array.
template <typename T>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const float *__restrict__ part0,
                                                         const float *__restrict__ part1, int nblk,
                                                         size_t n4, T *__restrict__ out0,
                                                         T *__restrict__ out1) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    const float *part = blockIdx.y ? part1 : part0;
    T *out = blockIdx.y ? out1 : out0;
    floatx4 acc = reinterpret_cast<const floatx4 *>(part)[i];
    for (int k = 1; k < nblk; ++k) {
        const floatx4 v = reinterpret_cast<const floatx4 *>(part)[(size_t)k * n4 + i];
        acc += v;
    }
    store4_global<T>(out + 4 * i, acc);
}

// Stage-1 backward: per (chunk, batch, block of 64 heads), thread (run k,
// head hh) owns Q/16 consecutive tokens (the layout of chunk_cumsum). With da
// the suffix sums of ds within the chunk (s_i sums step_k A over k <= i):
//   dstep = A da + dw dw/dstep,   dA += step da + dw dw/dA,
//   d(raw dt) = dstep d(step)/d(raw)  (softplus: sigmoid; clamp: 0 outside),
// written as ddt (input dtype); the per-(batch, chunk, head) sums of the dA
// and dt-bias terms go to dA_part, dbias_part.
template <typename T, int Q>
__global__ __launch_bounds__(1024) void bwd_dt_kernel(
    const T *__restrict__ dt, const float *__restrict__ A, const float *__restrict__ ds,
    const float *__restrict__ dw, int L, int H, int nC, DtOpts o, T *__restrict__ ddt,
    float *__restrict__ dA_part, float *__restrict__ dbias_part) {
    constexpr int R = Q / 16, HB = 64, RUNS = 16;
    __shared__ float tot[RUNS][HB];
    __shared__ float pa[RUNS][HB], pb[RUNS][HB];
    const int c = blockIdx.x, b = blockIdx.y, h0 = blockIdx.z * HB;
    const int tid = threadIdx.x, hh = tid & 63, k = tid >> 6, h = h0 + hh;
    const int hc = min(h, H - 1);
    const int t0 = c * Q + k * R;
    const size_t row = ((size_t)b * H + hc) * (size_t)nC * Q + t0;
    static_assert(R % 4 == 0, "runs of whole float4s");
    float dsv[R], dwv[R], raw[R];
    // (a lane's R tokens are consecutive in its ds / dw row: 16-byte loads)
#pragma unroll
    for (int r = 0; r < R; r += 4) {
        const float4 s4 = *reinterpret_cast<const float4 *>(ds + row + r);
        const float4 w4 = *reinterpret_cast<const float4 *>(dw + row + r);
        const bool on = h < H;
        dsv[r] = on ? s4.x : 0.0f;
        dsv[r + 1] = on ? s4.y : 0.0f;
        dsv[r + 2] = on ? s4.z : 0.0f;
        dsv[r + 3] = on ? s4.w : 0.0f;
        dwv[r] = on ? w4.x : 0.0f;
        dwv[r + 1] = on ? w4.y : 0.0f;
        dwv[r + 2] = on ? w4.z : 0.0f;
        dwv[r + 3] = on ? w4.w : 0.0f;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) raw[r] = to_f32(dt[((size_t)b * L + min(t0 + r, L - 1)) * H + hc]);
    // suffix sums within the run, then across runs
#pragma unroll
    for (int r = R - 2; r >= 0; --r) dsv[r] += dsv[r + 1];
    tot[k][hh] = dsv[0];
    __syncthreads();
    float after = 0.0f;  // sum of the later runs of this chunk
    for (int kk = k + 1; kk < RUNS; ++kk) after += tot[kk][hh];
    const float a = h < H ? A[hc] : 0.0f;
    const float bias = o.bias ? o.bias[hc] : 0.0f;
    float sa = 0.0f, sb = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int t = t0 + r;
        const float da = dsv[r] + after;
        float v = raw[r] + bias, slope = 1.0f;
        if (o.softplus) {
            slope = 1.0f / (1.0f + expf(-v));
            v = fmaxf(v, 0.0f) + log1pf(expf(-fabsf(v)));
        }
        if (o.clamp) {
            if (v < o.lo || v > o.hi) slope = 0.0f;
            v = fminf(fmaxf(v, o.lo), o.hi);
        }
        float wd = 1.0f, wa = 0.0f;  // dw/dstep, dw/dA
        if (o.zoh) {
            const float z = v * a;
            wd = expf(z);
            if (fabsf(z) < 0.5f) {  // step^2 sum_{m>=2} (m-1)/m! z^(m-2)
                wa = v * v * (0.5f + z * (1.0f / 3 + z * (1.0f / 8 + z * (1.0f / 30 + z * (1.0f / 144 +
                     z * (1.0f / 840 + z * (1.0f / 5760 + z * (1.0f / 45360))))))));
            } else {
                wa = (z * expf(z) - expm1f(z)) / (a * a);
            }
        }
        const float dstep = a * da + dwv[r] * wd;
        const float draw = dstep * slope;
        if (h < H && t < L) {
            ddt[((size_t)b * L + t) * H + h] = from_f32<T>(draw);
            sa += v * da + dwv[r] * wa;
            sb += draw;
        }
    }
    pa[k][hh] = sa;
    pb[k][hh] = sb;
    __syncthreads();
    if (k == 0 && h < H) {
        float ta = 0.0f, tb = 0.0f;
        for (int kk = 0; kk < RUNS; ++kk) {
            ta += pa[kk][hh];
            tb += pb[kk][hh];
        }
        dA_part[((size_t)b * nC + c) * H + h] = ta;
        dbias_part[((size_t)b * nC + c) * H + h] = tb;
    }
}

// Per-head totals of the (batch, chunk) partial sums: one workgroup per head
// and array (blockIdx.y; up to three arrays in one launch).
struct HeadSums {
    const float *part[3];
    float *out[3];
};
__global__ __launch_bounds__(256) void bwd_head_sum_kernel(HeadSums hs, int nbc, int H) {
    __shared__ float red[4];
    const int h = blockIdx.x;
    const float *part = hs.part[blockIdx.y];
    float *out = hs.out[blockIdx.y];
    float v = 0.0f;
    for (int i = threadIdx.x; i < nbc; i += 256) v += part[(size_t)i * H + h];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
    if (lane_id() == 0) red[wave_id()] = v;
    __syncthreads();
    if (threadIdx.x == 0) out[h] = red[0] + red[1] + red[2] + red[3];
}

// ---- launchers

// Chunk length of the backward for a state size (its LDS holds a chunk's x,
// dy, B, C and two P x N states): the largest of 256, 128, 64 that fits.
int bwd_chunk(int dstate, bool bf16) {
    // 512 threads (Q = 128) keep the accumulators of N <= 64 in registers;
    // larger states take Q = 64 (256 threads, twice the registers per thread)
    const int q = dstate <= 64 ? 128 : 64;
    size_t bytes = 0;
#define SSD_BWD_BYTES(TT, NN, QQ) \
    if (dstate == NN && q == QQ) bytes = BwdLds<TT, NN, QQ>::kBytes;
#define SSD_BWD_BYTES_Q(TT, NN) SSD_BWD_BYTES(TT, NN, 64) SSD_BWD_BYTES(TT, NN, 128)
    if (bf16) {
        SSD_BWD_BYTES_Q(bf16_t, 16) SSD_BWD_BYTES_Q(bf16_t, 32) SSD_BWD_BYTES_Q(bf16_t, 64)
        SSD_BWD_BYTES_Q(bf16_t, 128) SSD_BWD_BYTES_Q(bf16_t, 256)
    } else {
        SSD_BWD_BYTES_Q(float, 16) SSD_BWD_BYTES_Q(float, 32) SSD_BWD_BYTES_Q(float, 64)
        SSD_BWD_BYTES_Q(float, 128) SSD_BWD_BYTES_Q(float, 256)
    }
#undef SSD_BWD_BYTES_Q
#undef SSD_BWD_BYTES
    if (bytes && bytes <= 160 * 1024) return q;
    if (q == 128) {  // float32 N = 64: half the chunk
        if (!bf16 && dstate == 64 && BwdLds<float, 64, 64>::kBytes <= 160 * 1024) return 64;
    }
    return 0;
}

int bwd_head_blocks(int batch, int seqlen, int nheads, int ngroups, int chunk) {
    // the chunk kernel runs one workgroup per compute unit (its LDS): split the
    // heads of each (batch, chunk, group) unit so that one round of about 256
    // workgroups covers them (fewer rounds, fewer dB / dC partial sums)
    const int nC = (seqlen + chunk - 1) / chunk;
    const int nU = batch * nC * ngroups;
    int nblk = (256 + nU - 1) / nU;
    const int hpg = nheads / ngroups;
    return nblk < 1 ? 1 : (nblk > hpg ? hpg : nblk);
}

template <typename T, int N, int Q>
static void launch_bwd_q(const BwdArgs &a, hipStream_t s) {
    using E = typename LdsT<T>::type;
    const int nC = (a.seqlen + Q - 1) / Q;
    const int nU = a.batch * nC * a.ngroups;
    chunk_bwd_kernel<T, N, Q><<<nU * a.nblk, Q * 4, 0, s>>>(
        static_cast<const T *>(a.x), static_cast<const T *>(a.dy), a.dA_cumsum, a.delta,
        static_cast<const T *>(a.B), static_cast<const T *>(a.C), a.D,
        static_cast<const E *>(a.chunk_init), static_cast<const E *>(a.grad_next), a.batch,
        a.seqlen, a.nheads, a.ngroups, nC, a.nblk, static_cast<T *>(a.dx), a.ds, a.dw, a.dB_part,
        a.dC_part, a.dD_part);
}

template <typename T, int N>
static bool launch_bwd_n(int Q, const BwdArgs &a, hipStream_t s) {
    switch (Q) {
        case 64: launch_bwd_q<T, N, 64>(a, s); return true;
        case 128:
            if constexpr (BwdLds<T, N, 128>::kBytes <= 160 * 1024) {
                launch_bwd_q<T, N, 128>(a, s);
                return true;
            }
            return false;
        default: return false;
    }
}

template <typename T>
static bool launch_bwd_t(const BwdArgs &a, hipStream_t s) {
    switch (a.dstate) {
        case 16: return launch_bwd_n<T, 16>(a.chunk, a, s);
        case 32: return launch_bwd_n<T, 32>(a.chunk, a, s);
        case 64: return launch_bwd_n<T, 64>(a.chunk, a, s);
        case 128:
            if constexpr (BwdLds<T, 128, 64>::kBytes <= 160 * 1024) return launch_bwd_n<T, 128>(a.chunk, a, s);
            return false;
        case 256:
            if constexpr (BwdLds<T, 256, 64>::kBytes <= 160 * 1024) return launch_bwd_n<T, 256>(a.chunk, a, s);
            return false;
        default: return false;
    }
}

hipError_t launch_chunk_bwd(const BwdArgs &a, hipStream_t stream) {
    const bool ok = a.bf16 ? launch_bwd_t<bf16_t>(a, stream) : launch_bwd_t<float>(a, stream);
    return ok ? hipGetLastError() : hipErrorInvalidValue;
}

hipError_t launch_bwd_reduce(const float *part0, const float *part1, int nblk, size_t count,
                             bool bf16, void *out0, void *out1, hipStream_t stream) {
    const size_t n4 = count / 4;
    const dim3 grid((unsigned)((n4 + 255) / 256), 2);
    if (n4 == 0) return hipSuccess;
    if (bf16)
        bwd_reduce_kernel<bf16_t><<<grid, 256, 0, stream>>>(part0, part1, nblk, n4,
                                                            static_cast<bf16_t *>(out0),
                                                            static_cast<bf16_t *>(out1));
    else
        bwd_reduce_kernel<float><<<grid, 256, 0, stream>>>(part0, part1, nblk, n4,
                                                           static_cast<float *>(out0),
                                                           static_cast<float *>(out1));
    return hipGetLastError();
}

hipError_t launch_bwd_dt(const void *dt, const float *A, const float *ds, const float *dw,
                         int batch, int seqlen, int nheads, int chunk, bool bf16,
                         const DtOpts &opts, void *ddt, float *dA_part, float *dbias_part,
                         hipStream_t stream) {
    const int nC = (seqlen + chunk - 1) / chunk;
    const dim3 grid(nC, batch, (nheads + 63) / 64);
#define SSD_BWD_DT(TT, QQ)                                                                    \
    bwd_dt_kernel<TT, QQ><<<grid, 1024, 0, stream>>>(static_cast<const TT *>(dt), A, ds, dw,  \
                                                     seqlen, nheads, nC, opts,                \
                                                     static_cast<TT *>(ddt), dA_part, dbias_part)
    if (bf16) {
        if (chunk == 64) SSD_BWD_DT(bf16_t, 64);
        else if (chunk == 128) SSD_BWD_DT(bf16_t, 128);
        else if (chunk == 256) SSD_BWD_DT(bf16_t, 256);
        else return hipErrorInvalidValue;
    } else {
        if (chunk == 64) SSD_BWD_DT(float, 64);
        else if (chunk == 128) SSD_BWD_DT(float, 128);
        else if (chunk == 256) SSD_BWD_DT(float, 256);
        else return hipErrorInvalidValue;
    }
#undef SSD_BWD_DT
    return hipGetLastError();
}

hipError_t launch_bwd_head_sum(const float *const *part, float *const *out, int n, int nbc,
                               int nheads, hipStream_t stream) {
    HeadSums hs{};
    int k = 0;
    for (int i = 0; i < n; ++i)
        if (out[i]) {
            hs.part[k] = part[i];
            hs.out[k] = out[i];
            ++k;
        }
    if (k == 0) return hipSuccess;
    bwd_head_sum_kernel<<<dim3(nheads, k), 256, 0, stream>>>(hs, nbc, nheads);
    return hipGetLastError();
}

}  // namespace ssd
