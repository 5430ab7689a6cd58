// Stage 2 of the SSD block decomposition: the state each chunk contributes at
// its right edge, from a zero state ("Mamba 模型", section 4.1: the low-rank
// factor through which the off-diagonal blocks act):
//   S_c[p][n] = sum_{j in c} w_j * x_j[p] * B_j[n],  w_j = exp(s_end - s_j) * delta_j,
// with delta_j token j's input weight (stage 1 writes it: the step size, or its
// zero-order-hold weight).
//
// One workgroup (8 wavefronts) per (chunk, head, batch). S_c = X^T (w o B) is a
// [P x Q] x [Q x N] product whose contraction index, the token, is the row of
// both x and B in memory. Both are kept in LDS in their natural row layout:
// every global load is a piece of 8 elements of a token row (16 bytes for
// bf16) with consecutive lanes on consecutive pieces, and every LDS write is
// that same piece (w folded
// into B in fp32 before rounding to the operand type). The MFMA operands, which
// need 4 consecutive tokens per lane, come from the transposing LDS read
// (lds_colfrag). All global loads of the chunk are issued at the start; LDS
// holds half of the chunk at a time (two phases; four for the largest float
// tiles). Wavefront w owns the output
// tiles of P-rows 16*(w%4) .. +15 and N-column tiles w/4, w/4+2, ...
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

template <typename T, int N, int Q>
__global__ __launch_bounds__(512) void chunk_state_kernel(
    const T *__restrict__ x, const T *__restrict__ B, const float *__restrict__ delta,
    const float *__restrict__ dA_cumsum, const int *__restrict__ seg, int dout, int L, int H,
    int G, int nC, float *__restrict__ states) {
    using E = typename LdsT<T>::type;
    constexpr int P = 64, NTHR = 512;
    constexpr int LDX = colfrag_stride(P, sizeof(E));
    constexpr int LDB = colfrag_stride(N, sizeof(E));
    // LDS holds Q / NPH tokens at a time: two phases, or four if that is too big
    constexpr int NPH = (Q / 2) * (LDX + LDB) * (int)sizeof(E) > 96 * 1024 ? 4 : 2;
    constexpr int QH = Q / NPH;
    constexpr int SEG = 8;                            // elements per piece (one Raw8)
    constexpr int XPR = P / SEG, BPR = N / SEG;       // pieces per token row
    constexpr int XP = Q * XPR / NTHR;                // x pieces per thread (whole chunk)
    constexpr int BP = (Q * BPR + NTHR - 1) / NTHR;   // B pieces per thread
    constexpr int NTW = (N / 16 + 1) / 2;             // N-column tiles per wavefront
    __shared__ __attribute__((aligned(16))) E xs[QH * LDX];
    __shared__ __attribute__((aligned(16))) E bs[QH * LDB];
    __shared__ float wj[Q];

    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int g = h / (H / G);
    const int t0 = c * Q, len = min(Q, L - t0);
    const int tid = threadIdx.x;
    const T *xh = x + (((size_t)b * L + t0) * H + h) * P;
    const T *bg = B + (((size_t)b * L + t0) * G + g) * N;
    const size_t xstride = (size_t)H * P, bstride = (size_t)G * N;

    // ---- all global loads of the chunk, issued up front
    Raw8<T> xv[XP], bv[BP];
#pragma unroll
    for (int k = 0; k < XP; ++k) {
        const int idx = tid + k * NTHR, j = idx / XPR, q = idx % XPR;
        if (j < len) xv[k].load(xh + (size_t)j * xstride + q * SEG);
        else xv[k].zero();
    }
#pragma unroll
    for (int k = 0; k < BP; ++k) {
        const int idx = tid + k * NTHR, j = idx / BPR, q = idx % BPR;
        if (idx < Q * BPR && j < len) bv[k].load(bg + (size_t)j * bstride + q * SEG);
        else bv[k].zero();
    }
    const size_t row = ((size_t)b * H + h) * (size_t)nC * Q + (size_t)c * Q;
    const float *s = dA_cumsum + row, *dl = delta + row;
    const float s_end = s[len - 1];
    // packed sequences: only the tokens of the last token's sequence count
    const int j0 = seg ? seg[(size_t)(b * nC + c) * Q + len - 1] : -1;
    for (int j = tid; j < Q; j += NTHR) {
        float wv = 0.0f;
        if (j < len && j >= j0)
            wv = dout ? __builtin_amdgcn_exp2f(s[j] * kLog2e)
                      : __builtin_amdgcn_exp2f((s_end - s[j]) * kLog2e) * dl[j];
        wj[j] = wv;
    }

    const int w = wave_id(), l = lane_id(), g4 = l >> 4;
    const int pt = w % 4;
    floatx4 acc[NTW];
#pragma unroll
    for (int i = 0; i < NTW; ++i) acc[i] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

#pragma unroll
    for (int ph = 0; ph < NPH; ++ph) {
        __syncthreads();  // wj ready (phase 0) / previous phase consumed (phase 1)
#pragma unroll
        for (int k = 0; k < XP; ++k) {
            const int idx = tid + k * NTHR, j = idx / XPR, q = idx % XPR;
            if (j / QH == ph) {
                E *d = xs + (j - ph * QH) * LDX + q * SEG;
                Frag<T> f;
#pragma unroll
                for (int e = 0; e < 8; ++e) f.set(e, xv[k].get(e));
                store_frag8(d, f);
            }
        }
#pragma unroll
        for (int k = 0; k < BP; ++k) {
            const int idx = tid + k * NTHR, j = idx / BPR, q = idx % BPR;
            if (idx < Q * BPR && j / QH == ph) {
                const float wv = wj[j];
                E *d = bs + (j - ph * QH) * LDB + q * SEG;
                Frag<T> f;
#pragma unroll
                for (int e = 0; e < 8; ++e) f.set(e, bv[k].get(e) * wv);
                store_frag8(d, f);
            }
        }
        __syncthreads();
        const int kend = min(QH, len - ph * QH);  // tokens of this phase (<= 0: none)
        for (int kb = 0; kb < kend; kb += 32) {
            const int jb = kb + 4 * g4;
            Frag<T> xf;
            lds_colfrag(xf, xs, LDX, jb, jb + 16, pt * 16);
#pragma unroll
            for (int i = 0; i < NTW; ++i) {
                const int nt = w / 4 + 2 * i;
                if (nt < N / 16) {
                    Frag<T> bf;
                    lds_colfrag(bf, bs, LDB, jb, jb + 16, nt * 16);
                    mma(acc[i], xf, bf);
                }
            }
        }
    }

    float *dst = states + (((size_t)b * nC + c) * H + h) * (size_t)P * N;
    const int cc = l & 15;
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
        const int nt = w / 4 + 2 * i;
        if (nt < N / 16) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dst[(size_t)(pt * 16 + 4 * g4 + r) * N + nt * 16 + cc] = acc[i][r];
        }
    }
}

// ---- bf16: a pipeline of global-to-LDS loads over phases of TP tokens ------
//
// The same product, S_c = (w o X)^T B over the chunk's tokens, with the chunk
// streamed through LDS in phases of TP tokens (64, or 32 for N >= 128): while
// phase k is multiplied, phase k+1's x and B rows are already on their way by
// direct global-to-LDS loads, so a workgroup keeps memory busy instead of
// loading everything and then computing. The token weights w_j are applied to
// the x^T operand fragments (8 multiplies per fragment, shared by the
// wavefront's N tiles), so x and B land in LDS exactly as stored. Both tiles
// are read with the transposing LDS read (colfrag_swz; contraction index =
// token = row).
//
// FIN (packed sequences): one workgroup per (sequence k, head) forms the
// sequence's final state instead: the chunk c holding its last token te is
// cut after te (len = te - cQ + 1, so s_end = s_te), its tokens before the
// sequence's first are masked by seg as usual, and exp(s_te) H_c (chunk_init,
// the state entering chunk c) is added when the sequence began before chunk c.
// states is then seq_states [nseq][H][P][N].
template <int N, int Q, bool FIN>
__global__ __launch_bounds__(512) void chunk_state_bf16_kernel(
    const bf16_t *__restrict__ x, const bf16_t *__restrict__ B, const float *__restrict__ delta,
    const float *__restrict__ dA_cumsum, const int *__restrict__ seg, const int *__restrict__ cu,
    const __bf16 *__restrict__ chunk_init, int dout, int L, int H, int G, int nC,
    float *__restrict__ states) {
    constexpr int P = 64, NW = 8;
    constexpr int TP = N >= 128 ? 32 : 64;  // tokens per phase
    constexpr int NPH = Q / TP;
    constexpr int PPR = N / 8;               // 16-byte pieces per B row
    constexpr int XSL = TP * 8 / 64;         // x loads per phase (64 pieces each)
    constexpr int BSL = TP * PPR / 64;       // B loads per phase
    constexpr int NTW = (N / 16 + 1) / 2;    // N tiles per wavefront
    __shared__ __attribute__((aligned(16))) __bf16 xs0[TP * P];
    __shared__ __attribute__((aligned(16))) __bf16 xs1[TP * P];
    __shared__ __attribute__((aligned(16))) __bf16 bs0[TP * N];
    __shared__ __attribute__((aligned(16))) __bf16 bs1[TP * N];
    __shared__ __attribute__((aligned(16))) float wj[Q];

    const int h = blockIdx.y;
    const int tid = threadIdx.x, w = wave_id(), l = lane_id(), g4 = l >> 4;
    int c, b, len;
    float *dst;
    if constexpr (FIN) {
        const int k = blockIdx.x;
        const int a = min(max(cu[k], 0), L), e = min(max(cu[k + 1], a), L);
        dst = states + ((size_t)k * H + h) * (size_t)P * N;
        if (e <= a) {  // an empty sequence: zero state (uniform across the workgroup)
            for (int i = tid; i < P * N; i += 512) dst[i] = 0.0f;
            return;
        }
        b = 0;
        c = (e - 1) / Q;
        len = e - c * Q;
    } else {
        c = blockIdx.x;
        b = blockIdx.z;
        len = min(Q, L - c * Q);
        dst = states + (((size_t)b * nC + c) * H + h) * (size_t)P * N;
    }
    const int g = h / (H / G);
    const int t0 = c * Q;
    const size_t xrow = (size_t)H * P, brow = (size_t)G * N;
    const bf16_t *xh = x + ((size_t)b * L + t0) * xrow + (size_t)h * P;
    const bf16_t *bg = B + ((size_t)b * L + t0) * brow + (size_t)g * N;

    // one phase's x and B rows into buffer pair `ph & 1`: slot s of a load is
    // row s / PPR (resp. s / 8) at the piece that its swizzle maps there; rows
    // past the end repeat the last row (their weight w_j is zero)
    auto issue = [&](int ph) {
        __bf16 *xd = (ph & 1) ? xs1 : xs0;
        __bf16 *bd = (ph & 1) ? bs1 : bs0;
        for (int i = w; i < XSL; i += NW) {
            const int s = i * 64 + l, r = s >> 3, q = (s & 7) ^ tr_swz<8>(r);
            dma16(xh + (size_t)min(ph * TP + r, len - 1) * xrow + q * 8, xd + i * 512);
        }
        for (int i = w; i < BSL; i += NW) {
            const int s = i * 64 + l, r = s / PPR, q = (s % PPR) ^ tr_swz<PPR>(r);
            dma16(bg + (size_t)min(ph * TP + r, len - 1) * brow + q * 8, bd + i * 512);
        }
    };
    issue(0);
    // token weights w_j = exp(s_end - s_j) delta_j (zero past the end)
    const size_t row = ((size_t)b * H + h) * (size_t)nC * Q + (size_t)c * Q;
    const float *s = dA_cumsum + row, *dl = delta + row;
    const float s_end = s[len - 1];
    // packed sequences: only the tokens of the last token's sequence count
    const int j0 = seg ? seg[(size_t)(b * nC + c) * Q + len - 1] : -1;
    for (int j = tid; j < Q; j += 512) {
        float wv = 0.0f;
        if (j < len && j >= j0)
            wv = dout ? __builtin_amdgcn_exp2f(s[j] * kLog2e)
                      : __builtin_amdgcn_exp2f((s_end - s[j]) * kLog2e) * dl[j];
        wj[j] = wv;
    }

    const int pt = w % 4;
    floatx4 acc[NTW];
#pragma unroll
    for (int i = 0; i < NTW; ++i) acc[i] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ph = 0; ph < NPH; ++ph) {
        wait_barrier<0>();  // phase ph in LDS; phase ph-1's buffers free
        if (ph + 1 < NPH && (ph + 1) * TP < len) issue(ph + 1);  // uniform
        const __bf16 *xsp = (ph & 1) ? xs1 : xs0;
        const __bf16 *bsp = (ph & 1) ? bs1 : bs0;
        const int kend = min(TP, len - ph * TP);  // tokens of this phase (<= 0: none)
#pragma unroll
        for (int kb = 0; kb < TP; kb += 32) {
            if (kb < kend) {  // uniform
                const int jb = kb + 4 * g4;
                Frag<bf16_t> xf;
                colfrag_swz<8>(xf, xsp, jb, jb + 16, pt * 16);
                const floatx4 w0 = *reinterpret_cast<const floatx4 *>(wj + ph * TP + jb);
                const floatx4 w1 = *reinterpret_cast<const floatx4 *>(wj + ph * TP + jb + 16);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    xf.set(r, xf.get(r) * w0[r]);
                    xf.set(4 + r, xf.get(4 + r) * w1[r]);
                }
#pragma unroll
                for (int i = 0; i < NTW; ++i) {
                    const int nt = w / 4 + 2 * i;
                    if (nt < N / 16) {
                        Frag<bf16_t> bf;
                        colfrag_swz<PPR>(bf, bsp, jb, jb + 16, nt * 16);
                        mma(acc[i], xf, bf);
                    }
                }
            }
        }
    }

    const int cc = l & 15;
    // FIN: the state the sequence entered chunk c with, decayed to its last token
    const bool carry = FIN && j0 < 0;
    const float dec = carry ? __builtin_amdgcn_exp2f(s_end * kLog2e) : 0.0f;
    const __bf16 *hc = FIN ? chunk_init + ((size_t)c * H + h) * (size_t)P * N : nullptr;
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
        const int nt = w / 4 + 2 * i;
        if (nt < N / 16) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const size_t o = (size_t)(pt * 16 + 4 * g4 + r) * N + nt * 16 + cc;
                float v = acc[i][r];
                if (carry) v += dec * static_cast<float>(hc[o]);
                dst[o] = v;
            }
        }
    }
}

// ---- bf16, stages 2 and 3 together: one workgroup per (batch, head) -------
//
// The workgroup walks the chunks of its sequence in order. Chunk c's state
// contribution S_c is formed as above (phases of TP tokens streamed through
// LDS, the next phase always in flight, across chunk boundaries too), and the
// running state H_c of stage 3 stays in registers, in float32, in the layout
// of the MFMA accumulators: H_{c+1} = exp(s_end(c)) H_c + S_c. The state
// entering each chunk goes out once (in bf16, the operand type of the chunk
// scan) and the final state in float32; the per-chunk float32 states of the
// separate stages never exist. The chunk's prefix sums s and input weights
// delta (stage 1's float32 outputs) arrive by direct loads too, so nothing inside the loop
// waits on a global load. Products are formed transposed, S^T[n][p] (B rows as
// the A operand, weighted x as the B operand): a lane then holds 4
// consecutive n of one p, which is how the [P][N] state is stored.
//
// REV (backward): the adjoint of the state, the same recurrence run over the
// chunks in reverse, G_nC = dfinal (`init`), G_c = exp(s_end(c)) G_{c+1} + dS_c
// with dS_c = sum_i exp(s_i) dy_i C_i^T: `x` is dy, `B` is C, the token
// weights are exp(s_i) (zero past the end; delta is not read), chunk_init[c]
// receives G_{c+1} (the gradient of the state leaving chunk c) and
// final_state G_0 (the initial state's gradient).
template <int N, int Q, bool REV>
__global__ __launch_bounds__(512, 4) void chunk_state_passing_bf16_kernel(
    const bf16_t *__restrict__ x, const bf16_t *__restrict__ B,
    const float *__restrict__ dA_cumsum, const float *__restrict__ delta,
    const float *__restrict__ init, int L, int H, int G, int nC, __bf16 *__restrict__ chunk_init,
    float *__restrict__ final_state) {
    constexpr int P = 64, NW = 8;
    constexpr int TP = N >= 128 ? 32 : 64;  // tokens per phase
    constexpr int NPH = Q / TP;              // phases per chunk
    constexpr int PPR = N / 8;
    constexpr int XSL = TP * 8 / 64;         // x loads per phase
    constexpr int BSL = TP * PPR / 64;       // B loads per phase
    constexpr int SQ = Q < 256 ? 256 : Q;    // s / delta buffers hold whole 1 KB loads
    constexpr int SL = SQ * 4 / 1024;        // loads of one chunk's s (or delta) row
    constexpr int NTW = (N / 16 + 1) / 2;    // N tiles per wavefront
    __shared__ __attribute__((aligned(16))) __bf16 xs0[TP * P];
    __shared__ __attribute__((aligned(16))) __bf16 xs1[TP * P];
    __shared__ __attribute__((aligned(16))) __bf16 bs0[TP * N];
    __shared__ __attribute__((aligned(16))) __bf16 bs1[TP * N];
    __shared__ __attribute__((aligned(16))) float sv0[SQ], sv1[SQ], dv0[SQ], dv1[SQ];
    __shared__ __attribute__((aligned(16))) float wj[Q];
    // a chunk state on its way out, bf16 rows of N (padded to shift the rows'
    // banks; 16-byte aligned)
    constexpr int HRS = N + 8;
    __shared__ __attribute__((aligned(16))) __bf16 hst[P * HRS];

    const int h = blockIdx.x, b = blockIdx.y;
    const int g = h / (H / G);
    const int tid = threadIdx.x, w = wave_id(), l = lane_id(), g4 = l >> 4, cc = l & 15;
    const size_t xrow = (size_t)H * P, brow = (size_t)G * N;
    const bf16_t *xh = x + (size_t)b * L * xrow + (size_t)h * P;
    const bf16_t *bg = B + (size_t)b * L * brow + (size_t)g * N;
    const size_t srow = ((size_t)b * H + h) * (size_t)nC * Q;  // this head's s / delta rows
    const int nph = nC * NPH;

    // chunk of phase k (the chunks run in reverse for REV)
    auto chunk_of = [&](int k) { return REV ? nC - 1 - k / NPH : k / NPH; };
    // phase k (chunk chunk_of(k), tokens from (k % NPH) * TP) into buffer pair
    // k & 1; a chunk's first phase also brings its s and delta rows (buffer
    // pair c & 1; REV reads no delta)
    auto issue = [&](int k) {
        const int c = chunk_of(k), t0 = c * Q + (k % NPH) * TP;
        __bf16 *xd = (k & 1) ? xs1 : xs0;
        __bf16 *bd = (k & 1) ? bs1 : bs0;
        for (int i = w; i < XSL; i += NW) {
            const int s = i * 64 + l, r = s >> 3, q = (s & 7) ^ tr_swz<8>(r);
            dma16(xh + (size_t)min(t0 + r, L - 1) * xrow + q * 8, xd + i * 512);
        }
        for (int i = w; i < BSL; i += NW) {
            const int s = i * 64 + l, r = s / PPR, q = (s % PPR) ^ tr_swz<PPR>(r);
            dma16(bg + (size_t)min(t0 + r, L - 1) * brow + q * 8, bd + i * 512);
        }
        if (k % NPH == 0 && w < (REV ? SL : 2 * SL)) {
            const int i = w % SL;  // waves 0..SL-1: s, SL..2SL-1: delta
            // (for Q < 256 the lanes past the row re-read its last 16 bytes)
            const float *src = (w < SL ? dA_cumsum : delta) + srow + (size_t)c * Q +
                               min(i * 256 + l * 4, Q - 4);
            float *dst = w < SL ? ((c & 1) ? sv1 : sv0) : ((c & 1) ? dv1 : dv0);
            dma16(src, dst + i * 256);
        }
    };

    const int pt = w % 4;
    floatx4 acc[NTW], hreg[NTW];  // S^T and H^T tiles: lane (g4, cc) rows n = 16nt + 4g4 + r, column p = 16pt + cc
    issue(0);
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
        const int nt = w / 4 + 2 * i;
        acc[i] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
        hreg[i] = acc[i];
        if (init && nt < N / 16) {
            const float4 v = *reinterpret_cast<const float4 *>(
                init + (((size_t)b * H + h) * P + pt * 16 + cc) * N + nt * 16 + 4 * g4);
            hreg[i] = floatx4{v.x, v.y, v.z, v.w};
        }
    }
    // H_c -> chunk_init[b][c][h]: through LDS, so that each store is a 16-byte
    // piece of a row and consecutive lanes write whole 128-byte lines (the
    // accumulator layout would write 8 bytes per lane, 32-byte pieces of
    // sixteen rows per instruction: partial lines that cost the memory more
    // than the whole stream of x and B). Every wavefront takes part.
    auto put_init = [&](int c) {
#pragma unroll
        for (int i = 0; i < NTW; ++i) {
            const int nt = w / 4 + 2 * i;
            if (nt < N / 16) {
                const bf16x4 v{static_cast<__bf16>(hreg[i][0]), static_cast<__bf16>(hreg[i][1]),
                               static_cast<__bf16>(hreg[i][2]), static_cast<__bf16>(hreg[i][3])};
                *reinterpret_cast<bf16x4 *>(hst + (pt * 16 + cc) * HRS + nt * 16 + 4 * g4) = v;
            }
        }
        barrier_lds();
        __bf16 *dst = chunk_init + (((size_t)b * nC + c) * H + h) * (size_t)(P * N);
        for (int idx = tid; idx < P * N / 8; idx += 512) {
            const int p = idx / (N / 8), q = idx % (N / 8);
            *reinterpret_cast<uint4 *>(dst + (size_t)p * N + q * 8) =
                *reinterpret_cast<const uint4 *>(hst + p * HRS + q * 8);
        }
    };
    put_init(REV ? nC - 1 : 0);

    for (int k = 0; k < nph; ++k) {
        const int c = chunk_of(k), kq = k % NPH;
        wait_barrier<0>();  // phase k (and, at a chunk start, its s and delta) in LDS
        if (k + 1 < nph) issue(k + 1);
        if (kq == 0) {
            // token weights of chunk c: w_j = exp(s_end - s_j) delta_j (zero past the end)
            const float *svc = (c & 1) ? sv1 : sv0;
            const float *dvc = (c & 1) ? dv1 : dv0;
            const float se = svc[Q - 1];  // s is constant past the end
            const int lenc = min(Q, L - c * Q);
            for (int j = tid; j < Q; j += 512) {
                if (REV) wj[j] = j < lenc ? __builtin_amdgcn_exp2f(svc[j] * kLog2e) : 0.0f;
                else wj[j] = __builtin_amdgcn_exp2f((se - svc[j]) * kLog2e) * dvc[j];
            }
            barrier_lds();
        }
        const __bf16 *xsp = (k & 1) ? xs1 : xs0;
        const __bf16 *bsp = (k & 1) ? bs1 : bs0;
        const int kend = min(TP, L - (c * Q + kq * TP));  // tokens of this phase
#pragma unroll
        for (int kb = 0; kb < TP; kb += 32) {
            if (kb < kend) {  // uniform
                const int jb = kb + 4 * g4;
                Frag<bf16_t> xf;
                colfrag_swz<8>(xf, xsp, jb, jb + 16, pt * 16);
                const floatx4 w0 = *reinterpret_cast<const floatx4 *>(wj + kq * TP + jb);
                const floatx4 w1 = *reinterpret_cast<const floatx4 *>(wj + kq * TP + jb + 16);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    xf.set(r, xf.get(r) * w0[r]);
                    xf.set(4 + r, xf.get(4 + r) * w1[r]);
                }
#pragma unroll
                for (int i = 0; i < NTW; ++i) {
                    const int nt = w / 4 + 2 * i;
                    if (nt < N / 16) {
                        Frag<bf16_t> bf;
                        colfrag_swz<PPR>(bf, bsp, jb, jb + 16, nt * 16);
                        mma(acc[i], bf, xf);
                    }
                }
            }
        }
        if (kq == NPH - 1) {
            // end of chunk c: H_{c+1} = exp(s_end(c)) H_c + S_c
            const float dec = __builtin_amdgcn_exp2f(((c & 1) ? sv1 : sv0)[Q - 1] * kLog2e);
#pragma unroll
            for (int i = 0; i < NTW; ++i) {
#pragma unroll
                for (int r = 0; r < 4; ++r) hreg[i][r] = dec * hreg[i][r] + acc[i][r];
                acc[i] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
            }
            if (REV ? c > 0 : c + 1 < nC) put_init(REV ? c - 1 : c + 1);
        }
    }
    if (final_state) {
#pragma unroll
        for (int i = 0; i < NTW; ++i) {
            const int nt = w / 4 + 2 * i;
            if (nt < N / 16)
                *reinterpret_cast<float4 *>(final_state + (((size_t)b * H + h) * P + pt * 16 + cc) * N +
                                            nt * 16 + 4 * g4) =
                    make_float4(hreg[i][0], hreg[i][1], hreg[i][2], hreg[i][3]);
        }
    }
}

template <int N, int Q>
static void launch_fused(const void *x, const void *B, const float *dA, const float *delta,
                         const float *init, int batch, int L, int H, int G, void *chunk_init,
                         float *final_state, bool rev, hipStream_t stream) {
    const int nC = (L + Q - 1) / Q;
    if (rev)
        chunk_state_passing_bf16_kernel<N, Q, true><<<dim3(H, batch), 512, 0, stream>>>(
            static_cast<const bf16_t *>(x), static_cast<const bf16_t *>(B), dA, delta, init, L,
            H, G, nC, static_cast<__bf16 *>(chunk_init), final_state);
    else
        chunk_state_passing_bf16_kernel<N, Q, false><<<dim3(H, batch), 512, 0, stream>>>(
            static_cast<const bf16_t *>(x), static_cast<const bf16_t *>(B), dA, delta, init, L,
            H, G, nC, static_cast<__bf16 *>(chunk_init), final_state);
}

template <int N>
static bool fused_q(int Q, const void *x, const void *B, const float *dA, const float *delta,
                    const float *init, int batch, int L, int H, int G, void *ci, float *fs,
                    bool rev, hipStream_t s) {
    switch (Q) {
        case 64: launch_fused<N, 64>(x, B, dA, delta, init, batch, L, H, G, ci, fs, rev, s); return true;
        case 128: launch_fused<N, 128>(x, B, dA, delta, init, batch, L, H, G, ci, fs, rev, s); return true;
        case 256: launch_fused<N, 256>(x, B, dA, delta, init, batch, L, H, G, ci, fs, rev, s); return true;
        default: return false;
    }
}

bool state_passing_fused(int batch, int nheads, bool bf16) {
    // one workgroup per (batch, head): worth it once that fills the GPU (two
    // per compute unit at least); otherwise the separate stages parallelise
    // over chunks as well
    return bf16 && batch * nheads >= 512;
}

hipError_t launch_chunk_state_passing(const void *x, const void *B, const float *dA_cumsum,
                                      const float *delta, const float *init, int batch,
                                      int seqlen, int nheads, int ngroups, int dstate, int chunk,
                                      void *chunk_init, float *final_state, hipStream_t stream,
                                      bool reverse) {
    bool ok = false;
    switch (dstate) {
        case 16: ok = fused_q<16>(chunk, x, B, dA_cumsum, delta, init, batch, seqlen, nheads, ngroups, chunk_init, final_state, reverse, stream); break;
        case 32: ok = fused_q<32>(chunk, x, B, dA_cumsum, delta, init, batch, seqlen, nheads, ngroups, chunk_init, final_state, reverse, stream); break;
        case 64: ok = fused_q<64>(chunk, x, B, dA_cumsum, delta, init, batch, seqlen, nheads, ngroups, chunk_init, final_state, reverse, stream); break;
        case 128: ok = fused_q<128>(chunk, x, B, dA_cumsum, delta, init, batch, seqlen, nheads, ngroups, chunk_init, final_state, reverse, stream); break;
        case 256: ok = fused_q<256>(chunk, x, B, dA_cumsum, delta, init, batch, seqlen, nheads, ngroups, chunk_init, final_state, reverse, stream); break;
        default: break;
    }
    if (!ok) return hipErrorInvalidValue;
    return hipGetLastError();
}

template <typename T, int N, int Q>
static void launch_cs(const void *x, const void *B, const float *dl, const float *dA,
                      const int *seg, int dout, int batch, int L, int H, int G, float *states,
                      hipStream_t stream) {
    const int nC = (L + Q - 1) / Q;
    const dim3 grid(nC, H, batch);
    if constexpr (sizeof(T) == 2) {
        chunk_state_bf16_kernel<N, Q, false><<<grid, 512, 0, stream>>>(
            static_cast<const bf16_t *>(x), static_cast<const bf16_t *>(B),
            dl, dA, seg, nullptr, nullptr, dout, L, H, G, nC, states);
    } else {
        chunk_state_kernel<T, N, Q><<<grid, 512, 0, stream>>>(
            static_cast<const T *>(x), static_cast<const T *>(B), dl, dA, seg, dout, L,
            H, G, nC, states);
    }
}

template <typename T, int N>
static bool cs_q(int Q, const void *x, const void *B, const float *dl, const float *dA,
                 const int *seg, int dout, int batch, int L, int H, int G, float *states, hipStream_t s) {
    switch (Q) {
        case 64: launch_cs<T, N, 64>(x, B, dl, dA, seg, dout, batch, L, H, G, states, s); return true;
        case 128: launch_cs<T, N, 128>(x, B, dl, dA, seg, dout, batch, L, H, G, states, s); return true;
        case 256: launch_cs<T, N, 256>(x, B, dl, dA, seg, dout, batch, L, H, G, states, s); return true;
        default: return false;
    }
}

template <typename T>
static hipError_t dispatch_cs(const void *x, const void *B, const float *dl, const float *dA,
                              const int *seg, int dout, int batch, int L, int H, int G, int N, int Q,
                              float *states, hipStream_t s) {
    bool ok = false;
    switch (N) {
        case 16: ok = cs_q<T, 16>(Q, x, B, dl, dA, seg, dout, batch, L, H, G, states, s); break;
        case 32: ok = cs_q<T, 32>(Q, x, B, dl, dA, seg, dout, batch, L, H, G, states, s); break;
        case 64: ok = cs_q<T, 64>(Q, x, B, dl, dA, seg, dout, batch, L, H, G, states, s); break;
        case 128: ok = cs_q<T, 128>(Q, x, B, dl, dA, seg, dout, batch, L, H, G, states, s); break;
        case 256: ok = cs_q<T, 256>(Q, x, B, dl, dA, seg, dout, batch, L, H, G, states, s); break;
        default: break;
    }
    if (!ok) return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_chunk_state(const void *x, const void *B, const float *delta,
                              const float *dA_cumsum, const int *seg, int batch, int seqlen,
                              int nheads, int ngroups, int dstate, int chunk, bool bf16,
                              float *states, hipStream_t stream, bool dout) {
    if (bf16)
        return dispatch_cs<bf16_t>(x, B, delta, dA_cumsum, seg, dout, batch, seqlen, nheads,
                                   ngroups, dstate, chunk, states, stream);
    return dispatch_cs<float>(x, B, delta, dA_cumsum, seg, dout, batch, seqlen, nheads, ngroups,
                              dstate, chunk, states, stream);
}

}  // namespace ssd

namespace ssd {

// Packed sequences, bf16: each sequence's final state by the chunk state
// kernel's FIN variant (MFMA over the sequence's tokens in its last chunk).
hipError_t launch_varlen_final_states_bf16(const void *x, const void *B, const float *delta,
                                           const float *dA_cumsum, const int *cu_seqlens,
                                           const int *seg, const void *chunk_init, int nseq,
                                           int seqlen, int nheads, int ngroups, int dstate,
                                           int chunk, float *seq_states, hipStream_t stream) {
    const int nC = (seqlen + chunk - 1) / chunk;
    const dim3 grid(nseq, nheads);
    const bf16_t *xx = static_cast<const bf16_t *>(x), *bb = static_cast<const bf16_t *>(B);
    const __bf16 *hc = static_cast<const __bf16 *>(chunk_init);
#define SSD_FIN(NN, QQ)                                                                         \
    chunk_state_bf16_kernel<NN, QQ, true><<<grid, 512, 0, stream>>>(                            \
        xx, bb, delta, dA_cumsum, seg, cu_seqlens, hc, 0, seqlen, nheads, ngroups, nC, seq_states)
#define SSD_FIN_Q(NN)                                                                           \
    switch (chunk) {                                                                            \
        case 64: SSD_FIN(NN, 64); break;                                                        \
        case 128: SSD_FIN(NN, 128); break;                                                      \
        case 256: SSD_FIN(NN, 256); break;                                                      \
        default: return hipErrorInvalidValue;                                                   \
    }
    switch (dstate) {
        case 16: SSD_FIN_Q(16); break;
        case 32: SSD_FIN_Q(32); break;
        case 64: SSD_FIN_Q(64); break;
        case 128: SSD_FIN_Q(128); break;
        case 256: SSD_FIN_Q(256); break;
        default: return hipErrorInvalidValue;
    }
#undef SSD_FIN_Q
#undef SSD_FIN
    return hipGetLastError();
}

}  // namespace ssd
