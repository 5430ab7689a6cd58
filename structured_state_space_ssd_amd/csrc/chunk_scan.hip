// Stage 4 of the SSD block decomposition: every chunk's outputs
// ("Mamba 模型", section 4.1 and "Draft:Mamba2", SSD section):
//   y_i = sum_{j<=i in chunk} (C_i . B_j) exp(s_i - s_j) delta_j x_j  diagonal block
//       + exp(s_i) H_c C_i                                            off-diagonal blocks
//       + D_h x_i,
// with delta_j token j's input weight (written by stage 1: the step size, or
// its zero-order-hold weight). The diagonal block is the masked
// "attention-like" product (L o C B^T)(delta o x)
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
//     and delta go to LDS. Wavefront w owns output tiles w and Q/16-1-w (equal
//     causal work: Q/32+1 slices of 32 tokens) and loads, in this same phase,
//     its C rows and all its C B^T fragments into registers.
//   then, with no further global load, each wavefront computes
//     - state to output: Y^T += H_c (exp(s_i) C_i)^T on MFMA (K = N);
//     - D_h x_i;
//     - per 32-token slice at or below the diagonal: the C B^T fragment times
//       the decay exp2(s_i - s_j) delta_j in fp32, rounded to the operand type.
//       Below the diagonal it factors as exp2(s_i - s_end(slice)) times a
//       per-token table exp2(s_end(slice) - s_j) delta_j (both factors <= 1):
//       one exp per lane per slice. The slice holding the diagonal takes the
//       exp per element (bf16: exp2(s_i - (s_j - log2 delta_j))) and the causal
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
    float dtl[Q];   // bf16: s * log2(e) - log2(delta) (+inf past the end); float: delta (0 past the end)
    float colf[Q];  // exp2(s_end(slice of j) - s_j) * delta_j: column factor below the diagonal
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

template <typename T, int N, int Q, bool VL>
__global__ __launch_bounds__(Q * 2, 4) void chunk_scan_kernel(
    const T *__restrict__ x, const float *__restrict__ delta, const float *__restrict__ dA_cumsum,
    const T *__restrict__ C, const typename LdsT<T>::type *__restrict__ cb,
    const float *__restrict__ D, const typename LdsT<T>::type *__restrict__ chunk_init,
    const int *__restrict__ seg, int L, int H, int G, int nC, T *__restrict__ y) {
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
    // bf16: the decay-and-weight factor exp2(s_i - s_j) * delta_j is formed as
    // one exp2(s_i - (s_j - log2 delta_j)); float keeps the product (tighter rounding)
    constexpr bool kFoldDt = sizeof(T) == 2;
    const size_t srow = ((size_t)b * H + h) * (size_t)nC * Q + (size_t)c * Q;
    const float *s = dA_cumsum + srow;
    const int *sg = seg + (size_t)(b * nC + c) * Q;  // packed sequences only (VL)
    for (int i = tid; i < Q; i += NTHR) {
        const float si_ = s[i] * kLog2e;
        const float se_ = s[i | 31] * kLog2e;  // last token of i's 32-token slice
        const float d = delta[srow + i];        // zero past the end
        sm.sl[i] = si_;
        sm.dtl[i] = kFoldDt ? si_ - __log2f(d) : d;
        float cf = __builtin_amdgcn_exp2f(se_ - si_) * d;
        if constexpr (VL) cf = sg[i | 31] <= i ? cf : 0.0f;  // slice end in i's sequence
        sm.colf[i] = cf;
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
    int fs[2];  // first token (within the chunk) of row i's sequence, -1: earlier chunk
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
        const int i0 = tiles[ti] * 16;
        si[ti] = sm.sl[i0 + r16];
        fs[ti] = VL ? sg[i0 + r16] : -1;
        // ---- state to output: Y^T[p][i] += sum_n H_c[p][n] exp(s_i) C_i[n]
        if (!kEarlyC) {
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
                const int n0 = kk * 32 + 8 * g4;
                if (i0 + r16 < len && n0 < N) cv[ti][kk].load(cg + (size_t)(i0 + r16) * cstride + n0);
                else cv[ti][kk].zero();
            }
        }
        float sc = __builtin_amdgcn_exp2f(si[ti]);
        if constexpr (VL) sc = fs[ti] < 0 ? sc : 0.0f;  // H_c belongs to row i's sequence
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
        const int f_i = ti ? fs[1] : fs[0];
        const int jb = jp * 32 + 4 * g4;  // this lane's first token (elements 0..3)
        Frag<T> mf;
        if (jp != tiles[ti] / 2) {
            // strictly below the diagonal: exp2(s_i - s_j) delta_j =
            // exp2(s_i - s_end(slice)) * colf[j], both factors <= 1; no causal
            // mask (packed sequences: zero unless i, the slice end and j share
            // a sequence; colf holds the j side)
            float rowf = __builtin_amdgcn_exp2f(s_i - sm.sl[jp * 32 + 31]);
            if constexpr (VL) rowf = f_i <= jp * 32 + 31 ? rowf : 0.0f;
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
            for (int r = 0; r < 4; ++r) {  // causal, and (packed) j in i's sequence
                mf.set(r, jb + r <= il && (!VL || jb + r >= f_i) ? v[r] : 0.0f);
                mf.set(4 + r, jb + 16 + r <= il && (!VL || jb + 16 + r >= f_i) ? v[4 + r] : 0.0f);
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

// ============================================================================
// bf16 inputs: persistent head blocks fed by global-to-LDS loads
// ============================================================================
//
// A workgroup owns one (batch, chunk, B/C group) and a run of consecutive heads
// of that group, which it processes one after another; in the main
// configurations it fills a compute unit's LDS, one workgroup per compute unit.
//   - Head-independent data is prepared once: the causal C B^T tiles of the
//     chunk are computed on MFMA straight into LDS (in the fragment layout of
//     chunk_cb.hip, which this path therefore does not need), and the C rows of
//     the wavefront's two tiles stay in registers.
//   - Per head, x and H_c reach LDS through direct global-to-LDS loads (16
//     bytes per lane, no registers involved). x has two buffers: the next
//     head's x streams in during the whole of this head. H_c, read only by the
//     state-to-output product at the start of a head, is refilled right after
//     that product. The next head's decay tables are formed meanwhile.
//   - Inside a head no value is waited for from global memory: every operand
//     comes from LDS or registers. (Memory operations complete in issue order
//     for the wait counter, so a wait on any global load issued after the
//     prefetch would also wait for the prefetch.)
//   - Outputs are staged through the head's x buffer and leave as whole
//     128-byte token rows, with non-temporal stores (y is not read again on
//     the GPU; ordinary stores would displace the x, H_c and B rows other
//     workgroups are about to read); the next head's first wait leaves those
//     stores in flight.
// The products are those of the float kernel above, except that the
// state-to-output product takes raw C rows and scales its result by exp(s_i)
// per token, and every wavefront's slice sequence is fixed at compile time
// (one code path per tile pair). LDS rows are 128 bytes (x) or 2N bytes (H_c)
// with their 16-byte pieces XOR-swizzled so that the transposing reads of x
// and the row reads of H_c touch distinct banks.

namespace {

// H_c rows of N bf16 (N/8 pieces); piece q of row p is stored at q ^ f(p), f
// chosen so that one fragment read (16 consecutive rows, one piece) touches
// distinct bank groups.
template <int N>
__device__ __forceinline__ int h_swz(int p) {
    constexpr int PPR = N / 8;
    constexpr int RPW = PPR >= 16 ? 1 : 16 / PPR;  // rows per 256-byte bank window
    constexpr int MSK = (PPR >= 16 ? 16 : PPR) - 1;
    return (p / RPW) & MSK;
}


// Per-head decay tables (as in the float kernel).
template <int Q>
struct ScanTables {
    float sl[Q];    // s * log2(e)
    float dtl[Q];   // s * log2(e) - log2(delta) (+inf past the end)
    float colf[Q];  // exp2(s_end(slice of j) - s_j) * delta_j
};

// Entry of causal tile (it, jp) in a unit's C B^T tile list: tiles are stored
// row-tile-major, row tile it holding jp = 0..it/2.
__device__ __forceinline__ int cb_tile_start(int it) {
    const int m0 = it / 2;
    return (it % 2 == 0) ? m0 * (m0 + 1) : (m0 + 1) * (m0 + 1);
}

// Slice JP (0..JMAX) of this wavefront's row tile it (JMAX = it/2; slice
// JMAX holds the diagonal). cbl: this lane's C B^T fragment of slice 0 of the
// tile in LDS (the slices of a tile are consecutive entries).
template <int Q, int JMAX, int JP, bool VL>
__device__ __forceinline__ void scan_slice(floatx4 (&acc)[4], const __bf16 *cbl,
                                           const __bf16 *xs, const int (&xo)[4],
                                           const ScanTables<Q> &tb, float s_i, int il, int fs,
                                           int g4) {
    constexpr bool DIAG = JP == JMAX;
    const int jb = JP * 32 + 4 * g4;
    Frag<bf16_t> cbk, mf;
    cbk.v = *reinterpret_cast<const bf16x8 *>(cbl + JP * 512);
    if constexpr (!DIAG) {
        // strictly below the diagonal: exp2(s_i - s_j) delta_j =
        // exp2(s_i - s_end(slice)) * colf[j], both factors <= 1; no causal mask
        // (packed sequences: fs, the first token of row i's sequence, masks the row side)
        float rowf = __builtin_amdgcn_exp2f(s_i - tb.sl[JP * 32 + 31]);
        if constexpr (VL) rowf = fs <= JP * 32 + 31 ? rowf : 0.0f;
        const floatx4 c0 = *reinterpret_cast<const floatx4 *>(tb.colf + jb);
        const floatx4 c1 = *reinterpret_cast<const floatx4 *>(tb.colf + jb + 16);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            mf.set(r, cbk.get(r) * (c0[r] * rowf));
            mf.set(4 + r, cbk.get(4 + r) * (c1[r] * rowf));
        }
    } else {
        // the slice holding the diagonal: exp2(s_i - (s_j - log2 delta_j)) and the causal mask
        const floatx4 d0 = *reinterpret_cast<const floatx4 *>(tb.dtl + jb);
        const floatx4 d1 = *reinterpret_cast<const floatx4 *>(tb.dtl + jb + 16);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float v0 = cbk.get(r) * __builtin_amdgcn_exp2f(s_i - d0[r]);
            const float v1 = cbk.get(4 + r) * __builtin_amdgcn_exp2f(s_i - d1[r]);
            mf.set(r, jb + r <= il && (!VL || jb + r >= fs) ? v0 : 0.0f);
            mf.set(4 + r, jb + 16 + r <= il && (!VL || jb + 16 + r >= fs) ? v1 : 0.0f);
        }
    }
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
        Frag<bf16_t> xf;
        x_colfrag<JP>(xf, xs, xo[pt]);
        mma(acc[pt], xf, mf);
    }
}

template <int Q, int JMAX, int JP, bool VL>
__device__ __forceinline__ void scan_slices(floatx4 (&acc)[4], const __bf16 *cbl,
                                            const __bf16 *xs, const int (&xo)[4],
                                            const ScanTables<Q> &tb, float s_i, int il, int fs,
                                            int g4) {
    if constexpr (JP <= JMAX) {
        scan_slice<Q, JMAX, JP, VL>(acc, cbl, xs, xo, tb, s_i, il, fs, g4);
        scan_slices<Q, JMAX, JP + 1, VL>(acc, cbl, xs, xo, tb, s_i, il, fs, g4);
    }
}

// Dispatch on the (wavefront-uniform) tile's last slice index jmax.
template <int Q, int JMAX, bool VL>
__device__ __forceinline__ void scan_tile(int jmax, floatx4 (&acc)[4], const __bf16 *cbl,
                                          const __bf16 *xs, const int (&xo)[4],
                                          const ScanTables<Q> &tb, float s_i, int il, int fs,
                                          int g4) {
    if constexpr (JMAX < Q / 32) {
        if (jmax == JMAX) scan_slices<Q, JMAX, 0, VL>(acc, cbl, xs, xo, tb, s_i, il, fs, g4);
        else scan_tile<Q, JMAX + 1, VL>(jmax, acc, cbl, xs, xo, tb, s_i, il, fs, g4);
    }
}

// Row tile of wavefront w (one per wavefront). Wavefronts w and w + 4k share a
// SIMD; the assignment gives every SIMD the same number of 32-token slices:
// SIMD s takes tiles s, 7-s, 8+s, 15-s (Q = 256), s, 7-s (Q = 128), s (Q = 64).
__device__ __forceinline__ int scan_tile_of(int w) {
    const int s = w & 3, k = w >> 2;
    return (k >> 1) * 8 + ((k & 1) ? 7 - s : s);
}

// LDS of the bf16 kernel and whether x is double-buffered.
template <int N, int Q>
struct ScanBf16Lds {
    static constexpr int ENTRIES = (Q / 32) * (Q / 32 + 1);
    static constexpr size_t kSingle = (size_t)Q * 64 * 2 + 64 * N * 2 + 2 * sizeof(ScanTables<Q>) +
                                      (size_t)ENTRIES * 1024;
    static constexpr bool kDbuf = kSingle + (size_t)Q * 64 * 2 <= 160 * 1024;
    static constexpr size_t kBytes = kSingle + (kDbuf ? (size_t)Q * 64 * 2 : 0);
};

}  // namespace

template <int N, int Q, bool VL>
__global__ __launch_bounds__(Q * 4) void chunk_scan_bf16_kernel(
    const bf16_t *__restrict__ x, const float *__restrict__ delta,
    const float *__restrict__ dA_cumsum, const bf16_t *__restrict__ B,
    const bf16_t *__restrict__ C, const float *__restrict__ D,
    const __bf16 *__restrict__ chunk_init, const int *__restrict__ seg, int L, int H, int G,
    int nC, int nU, int nblk, bf16_t *__restrict__ y) {
    constexpr int P = 64, NW = Q / 16;  // one wavefront per 16-row tile
    constexpr int NK = (N + 31) / 32;
    constexpr int ENTRIES = ScanBf16Lds<N, Q>::ENTRIES;
    constexpr bool DBUF = ScanBf16Lds<N, Q>::kDbuf;
    constexpr int PPR = N / 8;           // 16-byte pieces per H_c row
    constexpr int XI = Q * 8 / 64 / NW;  // x loads (and y stores) per wavefront per head
    __shared__ __attribute__((aligned(16))) __bf16 xb0[Q * P];
    __shared__ __attribute__((aligned(16))) __bf16 xb1[DBUF ? Q * P : 8];
    __shared__ __attribute__((aligned(16))) __bf16 hbuf[P * N];
    __shared__ __attribute__((aligned(16))) __bf16 cbs[ENTRIES * 512];
    __shared__ __attribute__((aligned(16))) ScanTables<Q> tab0;
    __shared__ __attribute__((aligned(16))) ScanTables<Q> tab1;

    // workgroup -> (unit u = c + nC*(g + G*b), head block kb); the nblk blocks
    // of one unit get ids with the same id % 8, i.e. the same XCD, which then
    // reads that unit's B and C once
    const int id = blockIdx.x;
    const int q8 = id / (8 * nblk), rem = id - q8 * 8 * nblk;
    const int kb = rem / 8, u = q8 * 8 + rem % 8;
    if (u >= nU) return;  // whole workgroup
    const int hpg = H / G;
    const int c = u % nC, g = (u / nC) % G, b = u / (nC * G);
    // the block's heads are g*hpg + kb + k*nblk, k = 0..nh-1: the nblk blocks
    // of a unit work on adjacent heads at the same time, so their x and y
    // rows are neighbouring 128-byte pieces of the same token rows
    const int hfirst = g * hpg + kb;
    const int nh = (hpg - kb + nblk - 1) / nblk;
    if (nh <= 0) return;  // whole workgroup

    const int t0 = c * Q, len = min(Q, L - t0);
    const bool full = len == Q;
    const int tid = threadIdx.x, w = wave_id(), l = lane_id(), g4 = l >> 4, r16 = l & 15;
    const int tile = scan_tile_of(w), jmax = tile / 2;
    const int il = tile * 16 + r16;
    const size_t xrow = (size_t)H * P;  // token stride of x and y
    const bf16_t *xbase = x + ((size_t)b * L + t0) * xrow;
    bf16_t *ybase = y + ((size_t)b * L + t0) * xrow;
    const __bf16 *hbase = chunk_init + ((size_t)b * nC + c) * H * (size_t)(P * N);
    const float *sbase = dA_cumsum + (size_t)b * H * nC * Q + (size_t)c * Q;
    const float *dbase = delta + (size_t)b * H * nC * Q + (size_t)c * Q;
    const size_t bcrow = (size_t)G * N;  // token stride of B and C
    const bf16_t *Bc = B + ((size_t)b * L + t0) * bcrow + (size_t)g * N;
    const bf16_t *Cc = C + ((size_t)b * L + t0) * bcrow + (size_t)g * N;

    // Per-head address arithmetic takes the lane index from opaque_tid(),
    // which the compiler cannot see through: otherwise it keeps the
    // loop-invariant 64-bit addresses of every load and store alive across the
    // head loop, runs out of registers and spills them, and every reload of a
    // spill waits for all outstanding memory operations, the prefetch
    // included.
    auto opaque_tid = []() {
        int t = threadIdx.x;
        asm volatile("" : "+v"(t));
        return t;
    };
    auto issue_x = [&](int h, const __bf16 *buf, int ln) {
        const bf16_t *xh = xbase + (size_t)h * P;
#pragma unroll
        for (int k = 0; k < XI; ++k) {
            const int i = k * NW + w;  // 8 token rows per load
            const int s = i * 64 + ln;
            const int r = s >> 3, q = (s & 7) ^ (r & 7);
            dma16(xh + (size_t)min(r, len - 1) * xrow + q * 8, buf + i * 512);
        }
    };
    auto issue_h = [&](int h, int ln) {
        const __bf16 *hc = hbase + (size_t)h * (P * N);
#pragma unroll
        for (int i = w; i < PPR; i += NW) {  // 64 pieces per load, PPR loads in all
            const int s = i * 64 + ln;
            const int p = s / PPR, q = (s % PPR) ^ h_swz<N>(p);
            dma16(hc + (size_t)p * N + q * 8, hbuf + i * 512);
        }
    };
    // table inputs are loaded raw (s, s at the slice end, delta) and only
    // turned into table entries by tab_store
    auto tab_load = [&](int h, int td, float &sv, float &se, float &d) {
        if (td < Q) {
            const float *s = sbase + (size_t)h * nC * Q;
            sv = s[td];
            se = s[td | 31];
            d = dbase[(size_t)h * nC * Q + td];
        }
    };
    // packed sequences: the rows' first tokens of their sequences, and whether
    // this thread's table token shares a sequence with its slice end
    const int *sg = seg + (size_t)(b * nC + c) * Q;
    const float cmask = VL && tid < Q ? (sg[tid | 31] <= tid ? 1.0f : 0.0f) : 1.0f;
    auto tab_store = [&](ScanTables<Q> &t, int td, float sv, float se, float d) {
        if (td < Q) {  // d = delta_j, zero past the end
            const float si_ = sv * kLog2e;
            t.sl[td] = si_;
            t.dtl[td] = si_ - __log2f(d);
            t.colf[td] = __builtin_amdgcn_exp2f(se * kLog2e - si_) * (VL ? d * cmask : d);
        }
    };

    // ---- prologue. The first head's x and H_c on their way ...
    issue_x(hfirst, xb0, l);
    issue_h(hfirst, l);
    // ... the unit's causal C B^T tiles into LDS: tile e = (it, jp) by
    // wavefront e % NW, two 16x16 products of B rows against C rows over N
    // (fragment layout: lane 16*g + r holds row 16*it + r at tokens
    // 32*jp + 4*g + 0..3 and 32*jp + 16 + 4*g + 0..3; past the end: zero)
#pragma unroll 3
    for (int e = w; e < ENTRIES; e += NW) {
        int it = 0;
        while (cb_tile_start(it + 1) <= e) ++it;
        const int jp = e - cb_tile_start(it);
        const int i = it * 16 + r16;
        floatx4 m[2] = {floatx4{0.0f, 0.0f, 0.0f, 0.0f}, floatx4{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            const int n0 = kk * 32 + 8 * g4;
            const bool kin = n0 < N;
            uint4 cr = *reinterpret_cast<const uint4 *>(Cc + (size_t)min(i, len - 1) * bcrow +
                                                        min(n0, N - 8));
            if (!(kin && i < len)) cr = make_uint4(0, 0, 0, 0);
            Frag<bf16_t> cf;
            cf.v = __builtin_bit_cast(bf16x8, cr);
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int j = jp * 32 + half * 16 + r16;
                uint4 br = *reinterpret_cast<const uint4 *>(Bc + (size_t)min(j, len - 1) * bcrow +
                                                            min(n0, N - 8));
                if (!(kin && j < len)) br = make_uint4(0, 0, 0, 0);
                Frag<bf16_t> bf;
                bf.v = __builtin_bit_cast(bf16x8, br);
                mma(m[half], bf, cf);
            }
        }
        Frag<bf16_t> out;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            out.set(r, m[0][r]);
            out.set(4 + r, m[1][r]);
        }
        *reinterpret_cast<bf16x8 *>(cbs + e * 512 + l * 8) = out.v;
    }
    // ... the first head's tables, and the C rows of the wavefront's tile
    // (state-to-output B operand), kept in registers for all heads
    {
        float sv = 0.0f, se = 0.0f, d = 0.0f;
        tab_load(hfirst, tid, sv, se, d);
        tab_store(tab0, tid, sv, se, d);
    }
    Frag<bf16_t> cf[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
        const int n0 = kk * 32 + 8 * g4;
        uint4 raw = *reinterpret_cast<const uint4 *>(Cc + (size_t)min(il, len - 1) * bcrow +
                                                     min(n0, N - 8));
        if (!(il < len && n0 < N)) raw = make_uint4(0, 0, 0, 0);
        cf[kk].v = __builtin_bit_cast(bf16x8, raw);
    }
    const __bf16 *cbl = cbs + cb_tile_start(tile) * 512 + l * 8;
    int xo[4];
    x_colfrag_offsets(xo, l);
    const int fs = VL ? sg[il] : -1;  // first token (within the chunk) of row il's sequence

    for (int k = 0; k < nh; ++k) {
        const int h = hfirst + k * nblk, hn = h + nblk;
        const bool more = k + 1 < nh;
        const bool odd = DBUF && (k & 1);
        __bf16 *xs = odd ? xb1 : xb0;
        const ScanTables<Q> &tb = (k & 1) ? tab1 : tab0;
        // x(h), H_c(h) and tables(h) are in LDS, head h-1 is done with its
        // buffers; head h-1's XI output stores (the most recent global
        // operations, full chunks only) may stay in flight
        if (DBUF && full && k > 0) wait_barrier<XI>();
        else wait_barrier<0>();
        const int td = opaque_tid(), ln = td & 63;
        float nsv = 0.0f, nse = 0.0f, nd = 0.0f;
        if (more) tab_load(hn, td, nsv, nse, nd);  // before the prefetch: waited for at the end
        if (DBUF && more) issue_x(hn, odd ? xb0 : xb1, ln);

        // ---- state to output: Y^T[p][i] = sum_n H_c[p][n] C_i[n], scaled by exp(s_i) below
        floatx4 acc[4];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) acc[pt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            const int n0 = kk * 32 + 8 * g4;
            const int q = min(n0, N - 8) >> 3;
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                const int p = pt * 16 + r16;
                Frag<bf16_t> hf;
                hf.v = *reinterpret_cast<const bf16x8 *>(hbuf + p * N + ((q ^ h_swz<N>(p)) << 3));
                if (n0 >= N) hf.zero();  // only N = 16
                mma(acc[pt], hf, cf[kk]);
            }
        }
        barrier_lds();  // every wavefront has read H_c(h)
        if (more) issue_h(hn, ln);

        const float Dh = D ? D[h] : 0.0f;
        const float si = tb.sl[il];
        {
            float sc = __builtin_amdgcn_exp2f(si);
            if constexpr (VL) sc = fs < 0 ? sc : 0.0f;  // H_c belongs to row il's sequence
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                const bf16x4 xv = *reinterpret_cast<const bf16x4 *>(xs + x_at(il, pt * 16 + 4 * g4));
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[pt][r] = acc[pt][r] * sc + Dh * static_cast<float>(xv[r]);
            }
        }
        // ---- diagonal blocks
        scan_tile<Q, 0, VL>(jmax, acc, cbl, xs, xo, tb, si, il, fs, g4);

        // ---- next head's tables. Their inputs are consumed only here: the
        // empty asm keeps the compiler from waiting for their loads early
        // (which, memory operations completing in issue order, would also
        // wait for the prefetch issued after them); here that wait costs
        // nothing, and it precedes this head's output stores.
        asm volatile("" : "+v"(nsv), "+v"(nse), "+v"(nd));
        if (more) tab_store((k & 1) ? tab0 : tab1, td, nsv, nse, nd);

        // ---- outputs, staged in this head's x buffer and stored as whole rows
        barrier_lds();  // every wavefront is done reading x(h)
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
            const bf16x4 v{static_cast<__bf16>(acc[pt][0]), static_cast<__bf16>(acc[pt][1]),
                           static_cast<__bf16>(acc[pt][2]), static_cast<__bf16>(acc[pt][3])};
            *reinterpret_cast<bf16x4 *>(xs + x_at(il, pt * 16 + 4 * g4)) = v;
        }
        barrier_lds();
        bf16_t *yh = ybase + (size_t)h * P;
#pragma unroll
        for (int kq = 0; kq < XI; ++kq) {
            const int i = kq * NW + w;
            const int s = i * 64 + ln;
            const int r = s >> 3, q = (s & 7) ^ (r & 7);
            const uint4 v = *reinterpret_cast<const uint4 *>(xs + s * 8);
            if (r < len) store_nt16(yh + (size_t)r * xrow + q * 8, v);
        }
        if (!DBUF && more) {
            barrier_lds();  // every wavefront has read its outputs out of x(h)
            issue_x(hn, xb0, ln);
        }
    }
}

// ---- small states (N <= 64 at chunk 256): two workgroups per compute unit
//
// For small N the chunk's B rows fit in LDS next to x and H_c, so the C B^T
// values of a slice are formed right where they are needed (two 16x16 MFMA
// products of B rows from LDS against the wavefront's C rows in registers),
// in float32, and the decay multiplies them before the single rounding to
// bf16. A workgroup then needs under half of the LDS, two of them share a
// compute unit, and each wavefront owns a pair of row tiles with equal
// causal work (tiles 2*MM + (w&1) and NT-1-2*MM-(w&1): NT/2 + 1 slices of 32
// tokens). x is single-buffered: the next head's x is loaded once this head's
// outputs have left its buffer, while the other workgroup computes.

namespace {

// Slice K of wavefront pair index MM (see scan_slice for the decay).
template <int N, int Q, int MM, int K, bool VL>
__device__ __forceinline__ void pair_slice(floatx4 (&acc)[2][4], const Frag<bf16_t> (&cf)[2][(N + 31) / 32],
                                           const __bf16 *bsm, const int (&bo)[(N + 31) / 32],
                                           const __bf16 *xs, const int (&xo)[4],
                                           const ScanTables<Q> &tb, const float (&si)[2], int il0,
                                           int il1, const int (&fs)[2], int g4, int r16) {
    constexpr int NT = Q / 16, NK = (N + 31) / 32;
    constexpr int TI = K <= MM ? 0 : 1;
    constexpr int JP = TI ? K - MM - 1 : K;
    constexpr bool DIAG = TI ? (JP == NT / 2 - 1 - MM) : (JP == MM);
    const int il = TI ? il1 : il0;
    const float s_i = si[TI];
    const int jb = JP * 32 + 4 * g4;
    // the slice's x^T fragments first: their LDS latency overlaps the C B^T
    // products and the decay arithmetic below
    Frag<bf16_t> xf[4];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) x_colfrag<JP>(xf[pt], xs, xo[pt]);
    // C B^T of the slice: lane 16*g + r gets rows (tokens) i = 16*tile + r at
    // tokens jb + 0..3 (m[0]) and jb + 16 + 0..3 (m[1])
    floatx4 m[2] = {floatx4{0.0f, 0.0f, 0.0f, 0.0f}, floatx4{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            Frag<bf16_t> bfr;
            bfr.v = *reinterpret_cast<const bf16x8 *>(bsm + bo[kk] + (JP * 32 + half * 16) * N);
            if (kk * 32 + 8 * g4 >= N) bfr.zero();  // only N = 16
            mma(m[half], bfr, cf[TI][kk]);
        }
    }
    Frag<bf16_t> mf;
    const int f_i = fs[TI];  // packed sequences: first token of row il's sequence
    if constexpr (!DIAG) {
        float rowf = __builtin_amdgcn_exp2f(s_i - tb.sl[JP * 32 + 31]);
        if constexpr (VL) rowf = f_i <= JP * 32 + 31 ? rowf : 0.0f;
        const floatx4 c0 = *reinterpret_cast<const floatx4 *>(tb.colf + jb);
        const floatx4 c1 = *reinterpret_cast<const floatx4 *>(tb.colf + jb + 16);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            mf.set(r, m[0][r] * (c0[r] * rowf));
            mf.set(4 + r, m[1][r] * (c1[r] * rowf));
        }
    } else {
        const floatx4 d0 = *reinterpret_cast<const floatx4 *>(tb.dtl + jb);
        const floatx4 d1 = *reinterpret_cast<const floatx4 *>(tb.dtl + jb + 16);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float v0 = m[0][r] * __builtin_amdgcn_exp2f(s_i - d0[r]);
            const float v1 = m[1][r] * __builtin_amdgcn_exp2f(s_i - d1[r]);
            mf.set(r, jb + r <= il && (!VL || jb + r >= f_i) ? v0 : 0.0f);
            mf.set(4 + r, jb + 16 + r <= il && (!VL || jb + 16 + r >= f_i) ? v1 : 0.0f);
        }
    }
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) mma(acc[TI][pt], xf[pt], mf);
}

template <int N, int Q, int MM, int K, bool VL>
__device__ __forceinline__ void pair_slices(floatx4 (&acc)[2][4], const Frag<bf16_t> (&cf)[2][(N + 31) / 32],
                                            const __bf16 *bsm, const int (&bo)[(N + 31) / 32],
                                            const __bf16 *xs, const int (&xo)[4],
                                            const ScanTables<Q> &tb, const float (&si)[2], int il0,
                                            int il1, const int (&fs)[2], int g4, int r16) {
    if constexpr (K < Q / 32 + 1) {
        pair_slice<N, Q, MM, K, VL>(acc, cf, bsm, bo, xs, xo, tb, si, il0, il1, fs, g4, r16);
        __builtin_amdgcn_sched_barrier(0);  // keep slices apart: bounded register use
        pair_slices<N, Q, MM, K + 1, VL>(acc, cf, bsm, bo, xs, xo, tb, si, il0, il1, fs, g4, r16);
    }
}

template <int N, int Q, int MM, bool VL>
__device__ __forceinline__ void pair_slices_of(int M, floatx4 (&acc)[2][4],
                                               const Frag<bf16_t> (&cf)[2][(N + 31) / 32],
                                               const __bf16 *bsm, const int (&bo)[(N + 31) / 32],
                                               const __bf16 *xs, const int (&xo)[4],
                                               const ScanTables<Q> &tb, const float (&si)[2],
                                               int il0, int il1, const int (&fs)[2], int g4,
                                               int r16) {
    if constexpr (MM < Q / 64) {
        if (M == MM)
            pair_slices<N, Q, MM, 0, VL>(acc, cf, bsm, bo, xs, xo, tb, si, il0, il1, fs, g4, r16);
        else
            pair_slices_of<N, Q, MM + 1, VL>(M, acc, cf, bsm, bo, xs, xo, tb, si, il0, il1, fs, g4,
                                             r16);
    }
}

// Element offset, within a row-major LDS matrix of N-element rows stored with
// the h_swz piece swizzle, of the 8 elements one lane reads for an MFMA
// operand: row r16 (+ any multiple of 16 rows, which leaves the swizzle
// unchanged) at columns 32*kk + 8*g (clamped into the row for N = 16).
template <int N>
__device__ __forceinline__ void swz_row_offsets(int (&o)[(N + 31) / 32], int l) {
    const int g4 = l >> 4, r16 = l & 15;
#pragma unroll
    for (int kk = 0; kk < (N + 31) / 32; ++kk) {
        const int q = min(kk * 32 + 8 * g4, N - 8) >> 3;
        o[kk] = r16 * N + ((q ^ h_swz<N>(r16)) << 3);
    }
}

template <int N, int Q>
struct PairLds {
    static constexpr size_t kBytes = (size_t)Q * 64 * 2 + 64 * N * 2 + (size_t)Q * N * 2 +
                                     2 * sizeof(ScanTables<Q>);
    static constexpr bool kFits = kBytes <= 80 * 1024;  // two per compute unit
};

}  // namespace

template <int N, int Q, bool VL>
__global__ __launch_bounds__(Q * 2, 4) void chunk_scan_bf16_pair_kernel(
    const bf16_t *__restrict__ x, const float *__restrict__ delta,
    const float *__restrict__ dA_cumsum, const bf16_t *__restrict__ B,
    const bf16_t *__restrict__ C, const float *__restrict__ D,
    const __bf16 *__restrict__ chunk_init, const int *__restrict__ seg, int L, int H, int G,
    int nC, int nU, int nblk, bf16_t *__restrict__ y) {
    constexpr int P = 64, NW = Q / 32, NT = Q / 16;
    constexpr int NK = (N + 31) / 32;
    constexpr int PPR = N / 8;            // 16-byte pieces per H_c / B row
    constexpr int XI = Q * 8 / 64 / NW;   // x loads (and y stores) per wavefront per head
    constexpr int BI = Q * PPR / 64;      // B loads per workgroup
    __shared__ __attribute__((aligned(16))) __bf16 xs[Q * P];
    __shared__ __attribute__((aligned(16))) __bf16 hbuf[P * N];
    __shared__ __attribute__((aligned(16))) __bf16 bsm[Q * N];
    __shared__ __attribute__((aligned(16))) ScanTables<Q> tab0;
    __shared__ __attribute__((aligned(16))) ScanTables<Q> tab1;

    // workgroup -> (unit u = c + nC*(g + G*b), head block kb), XCD-aware as above
    const int id = blockIdx.x;
    const int q8 = id / (8 * nblk), rem = id - q8 * 8 * nblk;
    const int kb = rem / 8, u = q8 * 8 + rem % 8;
    if (u >= nU) return;  // whole workgroup
    const int hpg = H / G;
    const int c = u % nC, g = (u / nC) % G, b = u / (nC * G);
    // the block's heads are g*hpg + kb + k*nblk, k = 0..nh-1: the nblk blocks
    // of a unit work on adjacent heads at the same time, so their x and y
    // rows are neighbouring 128-byte pieces of the same token rows
    const int hfirst = g * hpg + kb;
    const int nh = (hpg - kb + nblk - 1) / nblk;
    if (nh <= 0) return;  // whole workgroup

    const int t0 = c * Q, len = min(Q, L - t0);
    const int tid = threadIdx.x, w = wave_id(), l = lane_id(), g4 = l >> 4, r16 = l & 15;
    const int M = w >> 1;
    const int tile0 = 2 * M + (w & 1), tile1 = NT - 1 - tile0;
    const int il0 = tile0 * 16 + r16, il1 = tile1 * 16 + r16;
    const size_t xrow = (size_t)H * P;
    const bf16_t *xbase = x + ((size_t)b * L + t0) * xrow;
    bf16_t *ybase = y + ((size_t)b * L + t0) * xrow;
    const __bf16 *hbase = chunk_init + ((size_t)b * nC + c) * H * (size_t)(P * N);
    const float *sbase = dA_cumsum + (size_t)b * H * nC * Q + (size_t)c * Q;
    const float *dbase = delta + (size_t)b * H * nC * Q + (size_t)c * Q;
    const size_t bcrow = (size_t)G * N;
    const bf16_t *Bc = B + ((size_t)b * L + t0) * bcrow + (size_t)g * N;
    const bf16_t *Cc = C + ((size_t)b * L + t0) * bcrow + (size_t)g * N;

    auto opaque_tid = []() {  // see chunk_scan_bf16_kernel
        int t = threadIdx.x;
        asm volatile("" : "+v"(t));
        return t;
    };
    auto issue_x = [&](int h, int ln) {
        const bf16_t *xh = xbase + (size_t)h * P;
#pragma unroll
        for (int k = 0; k < XI; ++k) {
            const int i = k * NW + w;
            const int s = i * 64 + ln;
            const int r = s >> 3, q = (s & 7) ^ (r & 7);
            dma16(xh + (size_t)min(r, len - 1) * xrow + q * 8, xs + i * 512);
        }
    };
    auto issue_h = [&](int h, int ln) {
        const __bf16 *hc = hbase + (size_t)h * (P * N);
#pragma unroll
        for (int i = w; i < PPR; i += NW) {
            const int s = i * 64 + ln;
            const int p = s / PPR, q = (s % PPR) ^ h_swz<N>(p);
            dma16(hc + (size_t)p * N + q * 8, hbuf + i * 512);
        }
    };
    auto tab_load = [&](int h, int td, float &sv, float &se, float &d) {
        if (td < Q) {
            const float *s = sbase + (size_t)h * nC * Q;
            sv = s[td];
            se = s[td | 31];
            d = dbase[(size_t)h * nC * Q + td];
        }
    };
    // packed sequences: the rows' first tokens of their sequences, and whether
    // this thread's table token shares a sequence with its slice end
    const int *sg = seg + (size_t)(b * nC + c) * Q;
    const float cmask = VL && tid < Q ? (sg[tid | 31] <= tid ? 1.0f : 0.0f) : 1.0f;
    auto tab_store = [&](ScanTables<Q> &t, int td, float sv, float se, float d) {
        if (td < Q) {  // d = delta_j, zero past the end
            const float si_ = sv * kLog2e;
            t.sl[td] = si_;
            t.dtl[td] = si_ - __log2f(d);
            t.colf[td] = __builtin_amdgcn_exp2f(se * kLog2e - si_) * (VL ? d * cmask : d);
        }
    };

    // ---- prologue: the chunk's B rows (token rows past the end repeat the
    // last one; their products are multiplied by zero decay), the first
    // head's x and H_c, its tables, and the C rows of both tiles in registers
    for (int i = w; i < BI; i += NW) {
        const int s = i * 64 + l;
        const int j = s / PPR, q = (s % PPR) ^ h_swz<N>(j);
        dma16(Bc + (size_t)min(j, len - 1) * bcrow + q * 8, bsm + i * 512);
    }
    issue_x(hfirst, l);
    issue_h(hfirst, l);
    {
        float sv = 0.0f, se = 0.0f, d = 0.0f;
        tab_load(hfirst, tid, sv, se, d);
        tab_store(tab0, tid, sv, se, d);
    }
    Frag<bf16_t> cf[2][NK];
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
        const int il = ti ? il1 : il0;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            const int n0 = kk * 32 + 8 * g4;
            uint4 raw = *reinterpret_cast<const uint4 *>(Cc + (size_t)min(il, len - 1) * bcrow +
                                                         min(n0, N - 8));
            if (!(il < len && n0 < N)) raw = make_uint4(0, 0, 0, 0);
            cf[ti][kk].v = __builtin_bit_cast(bf16x8, raw);
        }
    }
    int xo[4];
    x_colfrag_offsets(xo, l);
    int so[NK];  // this lane's H_c / B fragment offsets
    swz_row_offsets<N>(so, l);
    int fs[2] = {-1, -1};  // first token (within the chunk) of rows il0's and il1's sequences
    if constexpr (VL) {
        fs[0] = sg[il0];
        fs[1] = sg[il1];
    }

    for (int k = 0; k < nh; ++k) {
        const int h = hfirst + k * nblk, hn = h + nblk;
        const bool more = k + 1 < nh;
        const ScanTables<Q> &tb = (k & 1) ? tab1 : tab0;
        wait_barrier<0>();  // x(h), H_c(h), tables(h) (and B) in LDS
        const int td = opaque_tid(), ln = td & 63;
        float nsv = 0.0f, nse = 0.0f, nd = 0.0f;
        if (more) tab_load(hn, td, nsv, nse, nd);

        // ---- state to output, scaled by exp(s_i) below
        floatx4 acc[2][4];
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) acc[ti][pt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                Frag<bf16_t> hf;
                hf.v = *reinterpret_cast<const bf16x8 *>(hbuf + so[kk] + pt * 16 * N);
                if (kk * 32 + 8 * g4 >= N) hf.zero();  // only N = 16
#pragma unroll
                for (int ti = 0; ti < 2; ++ti) mma(acc[ti][pt], hf, cf[ti][kk]);
            }
        }
        barrier_lds();  // every wavefront has read H_c(h)
        if (more) issue_h(hn, ln);

        float si[2];
        const float Dh = D ? D[h] : 0.0f;
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) {
            const int il = ti ? il1 : il0;
            si[ti] = tb.sl[il];
            float sc = __builtin_amdgcn_exp2f(si[ti]);
            if constexpr (VL) sc = fs[ti] < 0 ? sc : 0.0f;  // H_c belongs to row il's sequence
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                const bf16x4 xv = *reinterpret_cast<const bf16x4 *>(xs + x_at(il, pt * 16 + 4 * g4));
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[ti][pt][r] = acc[ti][pt][r] * sc + Dh * static_cast<float>(xv[r]);
            }
        }
        // ---- diagonal blocks
        pair_slices_of<N, Q, 0, VL>(M, acc, cf, bsm, so, xs, xo, tb, si, il0, il1, fs, g4, r16);

        // ---- next head's tables (see chunk_scan_bf16_kernel)
        asm volatile("" : "+v"(nsv), "+v"(nse), "+v"(nd));
        if (more) tab_store((k & 1) ? tab0 : tab1, td, nsv, nse, nd);

        // ---- outputs through the x buffer, stored as whole rows
        barrier_lds();
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) {
            const int il = ti ? il1 : il0;
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                const bf16x4 v{static_cast<__bf16>(acc[ti][pt][0]), static_cast<__bf16>(acc[ti][pt][1]),
                               static_cast<__bf16>(acc[ti][pt][2]), static_cast<__bf16>(acc[ti][pt][3])};
                *reinterpret_cast<bf16x4 *>(xs + x_at(il, pt * 16 + 4 * g4)) = v;
            }
        }
        barrier_lds();
        bf16_t *yh = ybase + (size_t)h * P;
#pragma unroll
        for (int kq = 0; kq < XI; ++kq) {
            const int i = kq * NW + w;
            const int s = i * 64 + ln;
            const int r = s >> 3, q = (s & 7) ^ (r & 7);
            const uint4 v = *reinterpret_cast<const uint4 *>(xs + s * 8);
            if (r < len) store_nt16(yh + (size_t)r * xrow + q * 8, v);
        }
        if (more) {
            barrier_lds();  // the outputs have left the x buffer
            issue_x(hn, ln);
        }
    }
}

template <int N, int Q, bool VL>
static void launch_scan_bf16(const void *x, const float *dl, const float *dA, const void *B,
                             const void *C, const float *D, const void *Hc, const int *seg,
                             int batch, int L, int H, int G, void *y, hipStream_t stream) {
    const int nC = (L + Q - 1) / Q;
    const int hpg = H / G;
    const int nU = batch * nC * G;
    constexpr bool kPair = PairLds<N, Q>::kFits;
    // resident workgroups per compute unit (LDS-bound), 256 compute units
    const size_t lds = kPair ? PairLds<N, Q>::kBytes : ScanBf16Lds<N, Q>::kBytes;
    const int per_cu = (int)((160 * 1024) / lds);
    const int target = 256 * (per_cu < 1 ? 1 : per_cu);
    int nblk = (target + nU - 1) / nU;
    nblk = nblk < 1 ? 1 : (nblk > hpg ? hpg : nblk);
    const dim3 grid((unsigned)(8 * nblk) * (unsigned)((nU + 7) / 8));
    if constexpr (kPair) {
        chunk_scan_bf16_pair_kernel<N, Q, VL><<<grid, Q * 2, 0, stream>>>(
            static_cast<const bf16_t *>(x), dl, dA,
            static_cast<const bf16_t *>(B), static_cast<const bf16_t *>(C), D,
            static_cast<const __bf16 *>(Hc), seg, L, H, G, nC, nU, nblk, static_cast<bf16_t *>(y));
    } else {
        chunk_scan_bf16_kernel<N, Q, VL><<<grid, Q * 4, 0, stream>>>(
            static_cast<const bf16_t *>(x), dl, dA,
            static_cast<const bf16_t *>(B), static_cast<const bf16_t *>(C), D,
            static_cast<const __bf16 *>(Hc), seg, L, H, G, nC, nU, nblk, static_cast<bf16_t *>(y));
    }
}

template <typename T, int N, int Q, bool VL>
static void launch_scan_vl(const void *x, const float *dl, const float *dA, const void *B,
                           const void *C, const void *cb, const float *D, const void *Hc,
                           const int *seg, int batch, int L, int H, int G, void *y,
                           hipStream_t stream) {
    if constexpr (sizeof(T) == 2) {
        launch_scan_bf16<N, Q, VL>(x, dl, dA, B, C, D, Hc, seg, batch, L, H, G, y, stream);
    } else {
        using E = typename LdsT<T>::type;
        const int nC = (L + Q - 1) / Q;
        const dim3 grid(nC, H, batch);
        chunk_scan_kernel<T, N, Q, VL><<<grid, Q * 2, 0, stream>>>(
            static_cast<const T *>(x), dl, dA, static_cast<const T *>(C),
            static_cast<const E *>(cb), D, static_cast<const E *>(Hc), seg, L, H, G, nC,
            static_cast<T *>(y));
    }
}

// seg (packed sequences, nullable): the kernels' masking variant
template <typename T, int N, int Q>
static void launch_scan(const void *x, const float *dl, const float *dA, const void *B,
                        const void *C, const void *cb, const float *D, const void *Hc,
                        const int *seg, int batch, int L, int H, int G, void *y,
                        hipStream_t stream) {
    if (seg)
        launch_scan_vl<T, N, Q, true>(x, dl, dA, B, C, cb, D, Hc, seg, batch, L, H, G, y, stream);
    else
        launch_scan_vl<T, N, Q, false>(x, dl, dA, B, C, cb, D, Hc, seg, batch, L, H, G, y, stream);
}

template <typename T, int N>
static bool scan_q(int Q, const void *x, const float *dl, const float *dA, const void *B,
                   const void *C, const void *cb, const float *D, const void *Hc, const int *seg,
                   int batch, int L, int H, int G, void *y, hipStream_t s) {
    switch (Q) {
        case 64: launch_scan<T, N, 64>(x, dl, dA, B, C, cb, D, Hc, seg, batch, L, H, G, y, s); return true;
        case 128: launch_scan<T, N, 128>(x, dl, dA, B, C, cb, D, Hc, seg, batch, L, H, G, y, s); return true;
        case 256: launch_scan<T, N, 256>(x, dl, dA, B, C, cb, D, Hc, seg, batch, L, H, G, y, s); return true;
        default: return false;
    }
}

template <typename T>
static hipError_t scan_dispatch(int N, int Q, const void *x, const float *dl, const float *dA,
                                const void *B, const void *C, const void *cb, const float *D,
                                const void *Hc, const int *seg, int batch, int L, int H, int G,
                                void *y, hipStream_t s) {
    bool ok = false;
    switch (N) {
        case 16: ok = scan_q<T, 16>(Q, x, dl, dA, B, C, cb, D, Hc, seg, batch, L, H, G, y, s); break;
        case 32: ok = scan_q<T, 32>(Q, x, dl, dA, B, C, cb, D, Hc, seg, batch, L, H, G, y, s); break;
        case 64: ok = scan_q<T, 64>(Q, x, dl, dA, B, C, cb, D, Hc, seg, batch, L, H, G, y, s); break;
        case 128: ok = scan_q<T, 128>(Q, x, dl, dA, B, C, cb, D, Hc, seg, batch, L, H, G, y, s); break;
        case 256: ok = scan_q<T, 256>(Q, x, dl, dA, B, C, cb, D, Hc, seg, batch, L, H, G, y, s); break;
        default: break;
    }
    if (!ok) return hipErrorInvalidValue;
    return hipGetLastError();
}

bool chunk_scan_reads_cb(bool bf16) { return !bf16; }

hipError_t launch_chunk_scan(const void *x, const float *delta, const float *dA_cumsum, const void *B,
                             const void *C, const void *cb, const float *D, const void *chunk_init,
                             const int *seg, int batch, int seqlen, int nheads, int ngroups,
                             int dstate, int chunk, bool bf16, void *y, hipStream_t stream) {
    if (bf16)
        return scan_dispatch<bf16_t>(dstate, chunk, x, delta, dA_cumsum, B, C, cb, D, chunk_init,
                                     seg, batch, seqlen, nheads, ngroups, y, stream);
    return scan_dispatch<float>(dstate, chunk, x, delta, dA_cumsum, B, C, cb, D, chunk_init, seg,
                                batch, seqlen, nheads, ngroups, y, stream);
}

}  // namespace ssd
