// The whole SSD forward in one pass over the sequence, for bf16 inputs: one
// workgroup per (batch, head) walks its sequence in blocks of T = 64 tokens
// and keeps the running state in registers, so every input row is read from
// HBM once and every output row written once, and no intermediate (prefix
// sums, input weights, per-chunk states) ever leaves the compute unit.
//
// It is the chunked SSD algorithm ("Mamba 模型", section 4.1; "Draft:Mamba2",
// SSD section; block decomposition of the "Mamba-2架构深度解析" page,
// section 2.2) with the chunk-to-chunk recurrence of stage 3 run inside the
// workgroup instead of by a separate pass. For block k with state H entering
// it (H = init state, or zero, at k = 0), with s_i the within-block prefix
// sums of step * A and w_j the input weights (step or its zero-order-hold
// weight):
//   y_i      = exp(s_i) C_i H^T + sum_{j<=i} (C_i . B_j) exp(s_i - s_j) w_j x_j + D x_i
//   H_next   = exp(s_end) H + sum_j exp(s_end - s_j) w_j x_j B_j^T
// Step sizes (bias, softplus, clamp) are formed from dt in the kernel, as in
// stage 1. The result equals the multi-stage path's for any chunk length up
// to rounding: the block length only decides which products run as the
// quadratic (attention-like) form and which through the state.
//
// Segments: with too few (batch, head) pairs to fill the GPU, each sequence
// is cut into segments of whole blocks, one workgroup per (batch, head,
// segment). A segment-state kernel first computes, for pieces of the earlier
// segments, the state each piece produces from zero and its total decay; a
// chain kernel folds them (H <- exp(d) H + H_piece: the same recurrence at a
// coarser grain) into the state entering each segment, from which that
// segment's workgroup starts.
// Packed sequences (VL) mask rows, pairs and the state update by each
// token's first token of its sequence, and take each sequence's final state
// at its last token.
//
// Layout: 4 wavefronts. Wavefront w owns the 16 output tokens 16w..16w+15
// (Y^T tiles for every head-dim column) and the head-dim columns
// 16w..16w+15 of the state H^T (float32 registers, MFMA accumulator layout).
// At N 256 (one workgroup per compute unit) 8 wavefronts: w and w + 4 share
// tile w: each holds half of the state's n (its half of the update), forms
// C H over the whole of N for two of the four head-dim tiles and C B^T over
// the whole of N for half of each slice's columns; the second hands its
// partial outputs to the first through LDS at the middle barrier, and the
// first stages and stores them. With one workgroup per compute unit nothing
// else hides LDS latency, so each product chain's operands are read before
// its products (the two C H chains interleaved, the C B^T slice's B and x
// operands ahead of a scheduling barrier).
// The block's x rows (three buffers where LDS allows, else two), B and C rows
// (single-buffered: they are shared by all heads of a group and come from
// L2), and the 8-head piece of dt holding this head's values arrive by direct
// global-to-LDS loads: x two blocks ahead (issued after the next block's B
// and C, so that the wait at a block's start leaves it in flight; one block
// ahead with two buffers), dt two blocks ahead, B and C one (issued mid-block,
// once the current ones are consumed). Memory instructions are spread over
// the block (the previous block's two output stores after the first
// products, B / C / dt / x after the middle barrier): issued in one burst
// they queue in the address unit and stall every wavefront behind them.
//
// Per block, per wavefront:
//   tables    s * log2(e), w and exp(s_end - s_j) w_j for the 64 tokens
//             (step sizes with bias, softplus, clamp; zero-order-hold weights;
//             one token per lane, wave-wide prefix sum): made once, by
//             wavefront 0, during the block before, into one of two LDS
//             tables that the barriers of that block publish;
//   C H       Y^T = H C_i^T for the wavefront's rows on MFMA (H from LDS in
//             bf16, where the previous block's update left it; C_i fragments
//             shared with the next step), scaled per token by exp(s_i);
//   C B^T     the row tile's causal tiles (slices j <= i), decayed by
//             exp(s_i - s_j) w_j (below the diagonal as exp(s_i - s_31) times
//             a per-token column factor), masked, kept in registers as the
//             B operand of Y^T += X^T M^T over every head-dim tile; D added
//             to M on the diagonal (j = i), so that the product carries D x;
//   state     H^T = exp(s_end) H^T + B^T (w' o x) on MFMA for the
//             wavefront's columns;
//   -- barrier: B, C, dt buffers free; next loads issued; H to LDS in bf16 --
//   outputs   this wavefront's 16 rows staged in the block's x buffer and
//             read back as whole 128-byte rows by the same wavefront (no
//             barrier), stored (non-temporal) during the next block.
#include <algorithm>

#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

constexpr int kOpT = 64;  // tokens per block

// Packed sequences (VL): one int4 per token, {first token of its sequence,
// sequence index, whether it is its sequence's last token, 0}.
template <bool VL>
struct VlTab {  // per block: each row's first token of its sequence (relative
                // to the block; negative: the sequence began earlier), the
                // state's decay across the block (0 where a sequence begins in
                // it) and the tokens that end a sequence
    int fs[kOpT];
    float dec;
    uint32_t ends[2];
    int pad;
};
template <>
struct VlTab<false> {};

// x buffers of the single-pass kernel: three (x two blocks ahead) where three
// workgroups per compute unit still fit, else two (x one block ahead).
template <int N, bool VL>
constexpr int onepass_xbufs() {
    return (N == 64 && VL) || N == 256 ? 2 : 3;  // packed sequences at N 64: their tables take the room
}

template <int N, bool VL>
struct OnepassLds {
    __bf16 xb[onepass_xbufs<N, VL>()][kOpT * 64];
    __bf16 bb[kOpT * N];
    __bf16 cs[kOpT * N];
    __bf16 hb[64 * N];     // the state entering the block, bf16, [p][n], pieces swizzled by p & 7
    __bf16 dts[2][kOpT * 8];  // dt pieces of blocks k, k+1: token j's 8 heads around this head
    // tables of blocks k, k+1: s * log2(e), w, exp(s_end - s_j) w_j, and for
    // the first 32 tokens exp(s_31 - s_j) w_j (column factor below the diagonal)
    struct {
        float sl[kOpT], wt[kOpT], wp[kOpT], cf[32];
    } tab[2];
    VlTab<VL> vt[2];
    int4 mts[VL ? 2 : 1][VL ? kOpT : 1];  // the tokens' int4 of blocks k, k+1
    // N 256: the second half-N wavefront of each tile pair hands its partial
    // outputs over here ([row tile][head-dim tile][lane])
    floatx4 xch[N == 256 ? 16 : 1][N == 256 ? 64 : 1];
    int touch[64];  // written by the L2 touches of B and C, never read
};

// One 16-byte-per-lane global-to-LDS load from the wave-uniform base `sbase`
// plus this lane's byte offset `voff` (lane l's 16 bytes land at lds_base +
// 16 l): the scalar-base form, so a block's loads cost no per-lane 64-bit
// address arithmetic.
__device__ __forceinline__ void dma16_sv(const void *sbase, uint32_t voff, const void *lds_base) {
    const uint32_t a = lds_addr32(lds_base);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(a)
                 : "memory", "m0");
}

// The same, marked non-temporal (streamed past the caches' retention).
__device__ __forceinline__ void dma16_sv_nt(const void *sbase, uint32_t voff,
                                            const void *lds_base) {
    const uint32_t a = lds_addr32(lds_base);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :
                 : "v"(voff), "s"(sbase), "s"(a)
                 : "memory", "m0");
}

// The same with 4 bytes per lane (lane l's word lands at lds_base + 4 l).
__device__ __forceinline__ void dma4_sv(const void *sbase, uint32_t voff, const void *lds_base) {
    const uint32_t a = lds_addr32(lds_base);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(a)
                 : "memory", "m0");
}

// Inclusive prefix sum over the 64 lanes: shifts within rows of 16 lanes,
// then row totals broadcast forward (DPP; no LDS round trips).
__device__ __forceinline__ float wave_prefix_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xa, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xc, 0xf, false));
    return v;
}

__device__ __forceinline__ float lane_value(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Eight floats -> one bf16 operand fragment (round to nearest even, in pairs).
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void pack8(Frag<bf16_t> &f, const float (&v)[8]) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        const bf16x2 p = __builtin_convertvector(floatx2{v[e], v[e + 1]}, bf16x2);
        f.v[e] = p[0];
        f.v[e + 1] = p[1];
    }
}

// Four floats -> one bf16 operand of the 16x16x16 product (the k = 16 half of
// a 32-wide slice; lane 16g + r holds k = 4g .. 4g + 3 of row r).
__device__ __forceinline__ bf16x4 pack4(const float (&v)[4]) {
    const bf16x2 a = __builtin_convertvector(floatx2{v[0], v[1]}, bf16x2);
    const bf16x2 b = __builtin_convertvector(floatx2{v[2], v[3]}, bf16x2);
    return bf16x4{a[0], a[1], b[0], b[1]};
}

__device__ __forceinline__ void mma16(floatx4 &acc, const bf16x4 &a, const bf16x4 &b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(shortx4, a),
                                                    __builtin_bit_cast(shortx4, b), acc, 0, 0, 0);
}

// Half of x_colfrag<JP>'s fragment: rows 32 jp + 16 hf + 4 g + 0..3 of
// head-dim column 16 pt + c for lane 16 g + c (one transposing read).
__device__ __forceinline__ bf16x4 x_colfrag_half(const __bf16 *xs, int off) {
    return __builtin_bit_cast(bf16x4,
                              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(xs + off)));
}

}  // namespace

// How a launch cuts each sequence. The single-pass kernel runs nseg segments
// of len tokens (the last may hold fewer), each starting from the state the
// kpc * seg pieces before it pass on; the segment-state kernel runs
// nseg = npc pieces of len tokens and stores for each the state it produces
// from a zero state and its total log2-decay.
struct OnepassSegs {
    int nseg, len, npc, kpc;
    float *state;  // float32 [Bt][H][npc][P][N]
    float *ld;     // float32 [Bt][H][npc]
    int chained;   // the chain kernel has left each segment's entering state in
                   // the slot of the last piece before it (else the single-pass
                   // kernel folds the pieces itself)
    int xnt;       // x loads non-temporal (see kStreamXBytes)
};

// x larger than this (the 256 MB last-level cache) is loaded with non-temporal
// loads: it cannot stay cached for a later reader anyway, and streaming it
// leaves the cache to B and C, which every head of a group reads. Smaller x is
// loaded normally, so that back-to-back calls find it still cached.
constexpr size_t kStreamXBytes = (size_t)256 << 20;

// The chain kernel runs when the last segment would have more than this many
// pieces to fold; below it the single-pass kernel folds them (one batch of loads).
constexpr int kChainPieces = 4;

// Packed sequences: the tokens' int4 (see VlTab) and each sequence's final
// state, float32 [nseq][H][P][N].
struct OnepassVl {
    const int4 *meta;
    float *seq_states;
};

// The masks of packed sequences (VL) from block k's token int4s, for rows and
// state weights: wavefront 0, lane j = token j of the block (len valid).
template <bool VL>
__device__ __forceinline__ void vl_tables(VlTab<VL> &vt, const int4 &m, int tblk, int len,
                                          float sle, float &wp) {
    if constexpr (VL) {
        const int l = lane_id();
        const bool valid = l < len;
        const int fs = m.x - tblk;  // first token of this token's sequence, block-relative
        const int fsl = __builtin_amdgcn_readlane(fs, len - 1);  // ... of the block's last token
        if (l < fsl) wp = 0.0f;  // a sequence the block's last token does not belong to
        const uint64_t ends = __ballot(valid && m.z != 0);
        vt.fs[l] = valid ? fs : kOpT;
        if (l == 0) {
            vt.dec = fsl < 0 ? __builtin_amdgcn_exp2f(sle) : 0.0f;
            vt.ends[0] = (uint32_t)ends;
            vt.ends[1] = (uint32_t)(ends >> 32);
        }
    }
}

template <int N, bool VL>
__global__ __launch_bounds__(N == 256 ? 512 : 256, N == 64 ? 3 : N == 128 ? 2 : 1) void ssd_forward_onepass_kernel(
    const bf16_t *__restrict__ x, const bf16_t *__restrict__ dt, const float *__restrict__ A,
    const bf16_t *__restrict__ B, const bf16_t *__restrict__ C, const float *__restrict__ D,
    const float *__restrict__ init, DtOpts o, int batch, int L, int H, int G, int per,
    OnepassSegs sg, OnepassVl vl, bf16_t *__restrict__ y, float *__restrict__ final_state) {
    constexpr int P = 64, T = kOpT;
    constexpr int PPR = N / 8, NT = N / 16, NK = N / 32;
    constexpr int HSW = PPR >= 16 ? 15 : PPR - 1;  // piece swizzle mask of the bf16 state rows
    constexpr int NXB = onepass_xbufs<N, VL>();
    // N 256: eight wavefronts, two per row / head-dim tile, each with half of N
    // (its half of the state, of the C H and C B^T sums and of the update)
    constexpr bool HALVES = N == 256;
    constexpr int NWV = HALVES ? 8 : 4;        // wavefronts
    constexpr int NTH = HALVES ? NT / 2 : NT;  // state tiles per wavefront
    constexpr int BL = T * PPR / 256;  // B (and C) loads per lane per block
    static_assert(N % 32 == 0 && BL >= 1, "state size");
    __shared__ __attribute__((aligned(16))) OnepassLds<N, VL> sm;

    // workgroup -> (batch, segment, head): consecutive workgroup ids go round
    // the 8 XCDs, so id -> (id % 8) * per + id / 8 gives each XCD a contiguous
    // range of units: the heads of one batch row and segment (and B/C group)
    // share an L2.
    const int nseg = sg.nseg;
    const int id = blockIdx.x;
    const int lin = (id & 7) * per + (id >> 3);
    if (lin >= batch * nseg * H) return;  // whole workgroup
    const int h = lin % H, bs = lin / H, seg = bs % nseg, b = bs / nseg, g = h / (H / G);
    // this workgroup's tokens: [tb, tb + Lw) of its batch row
    const int tb = seg * sg.len, Lw = min(sg.len, L - tb);
    const size_t bh = (size_t)b * H + h;
    // the wavefront index as a scalar (uniform branches and loop bounds)
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = HALVES ? (w & 3) : w;  // the row / head-dim tile
    const int nh = HALVES ? (w >> 2) : 0;  // the half of N
    const int l = lane_id(), g4 = l >> 4, cc = l & 15;
    const int nblk = (Lw + T - 1) / T;

    const size_t xrow = (size_t)H * P, brow = (size_t)G * N, row0 = (size_t)b * L + tb;
    const bf16_t *xh = x + row0 * xrow + (size_t)h * P;
    bf16_t *yh = y + row0 * xrow + (size_t)h * P;
    const bf16_t *bg = B + row0 * brow + (size_t)g * N;
    const bf16_t *cg = C + row0 * brow + (size_t)g * N;
    const bf16_t *dth = dt + row0 * H + (h & ~7);
    const float Ah = A[h];
    const float Dh = D ? D[h] : 0.0f;
    const float bias = o.bias ? o.bias[h] : 0.0f;

    // ---- direct loads: scalar base at the block's first token, per-lane byte
    // offsets of whole 16-byte pieces (rows past the end re-read the last row)
    const uint32_t xrb = (uint32_t)(xrow * 2), brb = (uint32_t)(brow * 2), drb = (uint32_t)H * 2;
    auto x_off = [&](int i, int len) {
        const int s = i * 64 + l, r = s >> 3, q = (s & 7) ^ (r & 7);
        return (uint32_t)min(r, len - 1) * xrb + q * 16;
    };
    auto bc_off = [&](int i, int len) {
        const int s = i * 64 + l, r = s / PPR, q = (s % PPR) ^ tr_swz<PPR>(r);
        return (uint32_t)min(r, len - 1) * brb + q * 16;
    };
    auto issue_x = [&](int k) {
        const int t0 = k * T, len = min(T, Lw - t0);
        const bf16_t *base = xh + (size_t)t0 * xrow;
        if (sg.xnt) {
#pragma unroll
            for (int i = w; i < 8; i += NWV)
                dma16_sv_nt(base, x_off(i, len), sm.xb[k % NXB] + i * 512);
        } else {
#pragma unroll
            for (int i = w; i < 8; i += NWV)
                dma16_sv(base, x_off(i, len), sm.xb[k % NXB] + i * 512);
        }
    };
    auto issue_dt = [&](int k) {  // wavefront 0 only
        const int t0 = k * T, len = min(T, Lw - t0);
        dma16_sv(dth + (size_t)t0 * H, (uint32_t)min(l, len - 1) * drb, sm.dts[k & 1]);
        if constexpr (VL)
            dma16_sv(vl.meta + row0 + t0, (uint32_t)min(l, len - 1) * 16, sm.mts[k & 1]);
    };
    // B and C of block k, after dt of block k+1 (so that waiting for block k's
    // B and C also brings the dt the next block's step sizes are made from)
    auto issue_bcd = [&](int k) {
        const int t0 = k * T, len = min(T, Lw - t0);
        if (w == 0 && k + 1 < nblk) issue_dt(k + 1);
        const bf16_t *bb_ = bg + (size_t)t0 * brow, *cb_ = cg + (size_t)t0 * brow;
#pragma unroll
        for (int i = w; i < T * PPR / 64; i += NWV) dma16_sv(bb_, bc_off(i, len), sm.bb + i * 512);
#pragma unroll
        for (int i = w; i < T * PPR / 64; i += NWV) dma16_sv(cb_, bc_off(i, len), sm.cs + i * 512);
    };
    // block k's tables from its dt piece (one wavefront; lane j is token t0 + j)
    auto make_tables = [&](int k) {
        const int len = min(T, Lw - k * T);
        const bool valid = l < len;
        const float raw = static_cast<float>(sm.dts[k & 1][l * 8 + (h & 7)]);
        const float st = valid ? step_size(o, raw, bias) : 0.0f;
        const float wgt = valid ? input_weight(o, st, Ah) : 0.0f;
        const float sl = wave_prefix_sum(st * Ah) * kLog2e;
        const float sle = lane_value(sl, 63), s31 = lane_value(sl, 31);
        auto &t = sm.tab[k & 1];
        float wp = __builtin_amdgcn_exp2f(sle - sl) * wgt;
        if constexpr (VL) vl_tables<VL>(sm.vt[k & 1], sm.mts[k & 1][l], tb + k * T, len, sle, wp);
        t.sl[l] = sl;
        t.wt[l] = wgt;
        t.wp[l] = wp;
        if (l < 32) t.cf[l] = __builtin_amdgcn_exp2f(s31 - sl) * wgt;

    };

    // the state H^T: lane (g4, cc) of wavefront w holds rows n = 16 nt + 4 g4 + r
    // of column p = 16 w + cc
    // (the initial state, brought through the pieces before this segment)
    floatx4 hreg[NTH];  // n tiles nh * NTH + 0 .. NTH-1
    // this lane's state offset (its column; its rows in the first n tile it holds)
    const size_t hoff = (size_t)(16 * wr + cc) * N + 4 * g4 + 16 * NTH * nh;
#pragma unroll
    for (int nt = 0; nt < NTH; ++nt) {
        hreg[nt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
        if (init && (seg == 0 || !sg.chained)) {
            const float4 v =
                *reinterpret_cast<const float4 *>(init + bh * P * N + hoff + 16 * nt);
            hreg[nt] = floatx4{v.x, v.y, v.z, v.w};
        }
    }
    // a later segment starts from the state the pieces before it pass on:
    // left by the chain kernel in the slot of the last of those pieces, or
    // (a few pieces) folded here, H <- exp(d_j) H + H_j, their loads issued
    // together
    if (seg > 0 && sg.chained) {  // uniform
        const float *sj = sg.state + (bh * sg.npc + seg * sg.kpc - 1) * P * N + hoff;
#pragma unroll
        for (int nt = 0; nt < NTH; ++nt) {
            const float4 v = *reinterpret_cast<const float4 *>(sj + 16 * nt);
            hreg[nt] = floatx4{v.x, v.y, v.z, v.w};
        }
    } else if (seg > 0) {
        const int nj = seg * sg.kpc;  // uniform, at most kChainPieces
        float4 v[kChainPieces][NTH];
        float f[kChainPieces];
#pragma unroll
        for (int j = 0; j < kChainPieces; ++j) {
            if (j < nj) {
                const float *sj = sg.state + (bh * sg.npc + j) * P * N + hoff;
                f[j] = sg.ld[bh * sg.npc + j];
#pragma unroll
                for (int nt = 0; nt < NTH; ++nt)
                    v[j][nt] = *reinterpret_cast<const float4 *>(sj + 16 * nt);
            }
        }
#pragma unroll
        for (int j = 0; j < kChainPieces; ++j) {
            if (j < nj) {
                const float a = __builtin_amdgcn_exp2f(f[j]);
#pragma unroll
                for (int nt = 0; nt < NTH; ++nt) {
                    hreg[nt][0] = hreg[nt][0] * a + v[j][nt].x;
                    hreg[nt][1] = hreg[nt][1] * a + v[j][nt].y;
                    hreg[nt][2] = hreg[nt][2] * a + v[j][nt].z;
                    hreg[nt][3] = hreg[nt][3] * a + v[j][nt].w;
                }
            }
        }
    }

    issue_x(0);
    if (w == 0) issue_dt(0);
    issue_bcd(0);
    if (NXB == 3 && nblk > 1) issue_x(1);

    int xo[4];
    x_colfrag_offsets(xo, l);
    // the output accumulators acc[q] hold p tile q ^ pflip: N 256, each half's
    // own two tiles first (the first half, which stages the rows, in order)
    const int pflip = HALVES ? 2 * nh : 0;
    int xol[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) xol[q] = pflip ? xo[q ^ 2] : xo[q];
    const int i = 16 * wr + cc;  // this lane's output token: row tile wr is rows 16wr..16wr+15

    // D on the diagonal slice (js = wr / 2) where j = i, added to M there so
    // that M x carries D x: lane (g4, cc) holds the slice's elements j = 32 js
    // + 4 g4 + e (e < 4) and 32 js + 12 + 4 g4 + e (e >= 4) of column i (N
    // 256: the wavefront's half nh of the slice, elements 4 nh + r)
    float dval[HALVES ? 4 : 8];
#pragma unroll
    for (int e = 0; e < (HALVES ? 4 : 8); ++e) {
        const int ee = HALVES ? 4 * nh + e : e;
        const int j = 32 * (wr >> 1) + 4 * g4 + (ee < 4 ? ee : 12 + ee);
        dval[e] = j == i ? Dh : 0.0f;
    }
    // this lane's two 16-byte pieces of its rows' outputs: byte offsets from
    // the block's first output row
    uint32_t yoff[2];
    int yrow[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const int s = 128 * wr + 64 * m + l, r = s >> 3, q = (s & 7) ^ (r & 7);
        yrow[m] = r;
        yoff[m] = (uint32_t)((r * xrow + q * 8) * 2);
    }

    // the state (bf16) into LDS for the next state-to-output product: this
    // wavefront's columns p = 16 w + cc, 4 consecutive n per accumulator tile
    auto put_h = [&]() {
        const int pp = 16 * wr + cc;
#pragma unroll
        for (int nq = 0; nq < NTH; ++nq) {
            const int nt = nh * NTH + nq;
            const int n0 = 16 * nt + 4 * g4, q = n0 >> 3;
            const bf16x2 lo = __builtin_convertvector(floatx2{hreg[nq][0], hreg[nq][1]}, bf16x2);
            const bf16x2 hi = __builtin_convertvector(floatx2{hreg[nq][2], hreg[nq][3]}, bf16x2);
            *reinterpret_cast<bf16x4 *>(sm.hb + pp * N + ((q ^ (pp & HSW)) << 3) + (n0 & 7)) =
                bf16x4{lo[0], lo[1], hi[0], hi[1]};
        }
    };
    put_h();  // published by the first block's barrier

    uint4 ystage[2];  // this lane's two 16-byte pieces of the previous block's outputs
    for (int k = 0; k < nblk; ++k) {
        const int t0 = k * T;
        // block k's x, B, C, this and the next block's dt have landed and the
        // stores issued before them have left; every wavefront has read the
        // previous block's staged outputs; the state entering the block is in
        // LDS. Three x buffers: block k+1's x (the last loads issued, two per
        // wavefront) may stay in flight. Two: it is issued now, into the
        // buffer of the previous block's staged outputs.
        if constexpr (NXB == 3) {
            if (k + 1 < nblk) wait_barrier<2>();
            else wait_barrier<0>();
        } else {
            wait_barrier<0>();
            if (k + 1 < nblk) issue_x(k + 1);
        }
        // B and C rows two blocks ahead are touched (one 4-byte direct load
        // per 128-byte line into a scratch LDS word, wavefronts 1 and 2 of
        // every eighth head of a group) so that their loads a block later
        // find them in L2
        if ((w == 1 || w == 2) && k + 2 < nblk && ((h % (H / G)) & 7) == 0) {  // uniform
            const int tp = t0 + 2 * T, lenp = min(T, Lw - tp);
            const bf16_t *src = (w == 1 ? bg : cg) + (size_t)tp * brow;
            const uint32_t off = (uint32_t)min(l, lenp - 1) * brb;
#pragma unroll
            for (int q = 0; q < N / 64; ++q) dma4_sv(src + 64 * q, off, sm.touch);
        }
        const __bf16 *xs = sm.xb[k % NXB];
        if (k == 0) {  // later blocks' tables are made during the block before
            if (w == 0) make_tables(0);
            barrier_lds();
        }
        const float *tsl = sm.tab[k & 1].sl, *twt = sm.tab[k & 1].wt, *twp = sm.tab[k & 1].wp,
                    *tcf = sm.tab[k & 1].cf;
        const float s31 = tsl[31], si = tsl[i];
        float dec;
        int fsi = 0;  // packed sequences: row i's first token of its sequence (block-relative)
        if constexpr (VL) {
            dec = sm.vt[k & 1].dec;
            fsi = sm.vt[k & 1].fs[i];
        } else {
            dec = __builtin_amdgcn_exp2f(tsl[T - 1]);
        }

        // C_i (n = 32 kk + 8 g4 .. +7) over the whole of N, the B operand of
        // both C H and C B^T
        Frag<bf16_t> cfr[NK];
#pragma unroll
        for (int kq = 0; kq < NK; ++kq)
            lds_frag8(cfr[kq], sm.cs + i * N + (((4 * kq + g4) ^ tr_swz<PPR>(i)) << 3));

        // ---- state to output: Y^T[p][i] = exp(s_i) sum_n H[p][n] C_i[n], every p
        // tile; acc[q] holds p tile q ^ pflip. N 256: the wavefront of half nh
        // takes its own p tiles 2 nh, 2 nh + 1 (acc[0], acc[1]), every H
        // fragment read before the two product chains, which run interleaved
        floatx4 acc[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (HALVES) {
            static_assert(HSW == 15, "rows pa and pa + 16 share their swizzle");
            const int pa = 32 * nh + cc;  // p tile 2 nh's row of this lane; 2 nh + 1: 16 rows on
            Frag<bf16_t> h0[NK], h1[NK];
#pragma unroll
            for (int kq = 0; kq < NK; ++kq) {
                const __bf16 *hp = sm.hb + pa * N + (((4 * kq + g4) ^ (pa & HSW)) << 3);
                lds_frag8(h0[kq], hp);
                lds_frag8(h1[kq], hp + 16 * N);
            }
#pragma unroll
            for (int kq = 0; kq < NK; ++kq) {
                mma(acc[0], h0[kq], cfr[kq]);
                mma(acc[1], h1[kq], cfr[kq]);
            }
        } else {
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                const int pp = 16 * pt + cc;
#pragma unroll
                for (int kq = 0; kq < NK; ++kq) {
                    Frag<bf16_t> hf;
                    lds_frag8(hf, sm.hb + pp * N + (((4 * kq + g4) ^ (pp & HSW)) << 3));
                    mma(acc[pt], hf, cfr[kq]);
                }
            }
        }
        {
            float e = __builtin_amdgcn_exp2f(si);
            if constexpr (VL) e = fsi < 0 ? e : 0.0f;  // H belongs to row i's sequence
#pragma unroll
            for (int q = 0; q < (HALVES ? 2 : 4); ++q)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[q][r] *= e;
        }

        // ---- the previous block's outputs leave here, between compute phases
        // (a full block: every row is in range)
        if (k > 0 && nh == 0) {
            char *yb = reinterpret_cast<char *>(yh + (size_t)(t0 - T) * xrow);
#pragma unroll
            for (int m = 0; m < 2; ++m) store_nt16(yb + yoff[m], ystage[m]);
        }

        // ---- the row tile's causal C B^T tiles (slices js <= w / 2), kept in
        // registers as the B operand of the diagonal products over every p tile:
        // M[i][j] = (C_i . B_j) exp(s_i - s_j) w_j, j <= i
        for (int js = 0; js <= (wr >> 1); ++js) {  // wave-uniform trip count
            const int j0 = 32 * js + 4 * g4;
            const bool diag = js == (wr >> 1);
            if constexpr (HALVES) {
                // N 256: the wavefront of half nh takes the 16 columns j =
                // 32 js + 16 nh + 0..15 of the slice, each C_i . B_j summed over
                // the whole of N in float32 (rounded to bf16 once, after the
                // decay), and their part of Y^T += X^T M^T as k = 16 products
                // (every B fragment read first; two chains, even and odd k)
                const int jn = 32 * js + 16 * nh + cc;
                Frag<bf16_t> bfr[NK];
#pragma unroll
                for (int kq = 0; kq < NK; ++kq)
                    lds_frag8(bfr[kq], sm.bb + jn * N + (((4 * kq + g4) ^ tr_swz<PPR>(jn)) << 3));
                // the x operands of this slice's part of Y^T += X^T M^T, read
                // with the B rows, ahead of the products
                const __bf16 *xsl = xs + js * 2048 + nh * 1024;
                bf16x4 xq[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) xq[q] = x_colfrag_half(xsl, xol[q]);
                __builtin_amdgcn_sched_barrier(0);  // the reads stay ahead of the products
                floatx4 m = floatx4{0.0f, 0.0f, 0.0f, 0.0f}, m1 = m;
#pragma unroll
                for (int kq = 0; kq < NK; kq += 2) {
                    mma(m, bfr[kq], cfr[kq]);
                    mma(m1, bfr[kq + 1], cfr[kq + 1]);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) m[r] += m1[r];
                // lane (g4, cc): rows j = jh + r of column i
                const int jh = j0 + 16 * nh;
                float v[4];
                if (diag) {
                    const floatx4 s0 = *reinterpret_cast<const floatx4 *>(tsl + jh);
                    const floatx4 w0 = *reinterpret_cast<const floatx4 *>(twt + jh);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float a0 = __builtin_fmaf(
                            m[r], __builtin_amdgcn_exp2f(si - s0[r]) * w0[r], dval[r]);
                        const bool on = jh + r <= i && (!VL || jh + r >= fsi);
                        v[r] = on ? a0 : 0.0f;
                    }
                } else {
                    const float rowf = __builtin_amdgcn_exp2f(si - s31);
                    const floatx4 c0 = *reinterpret_cast<const floatx4 *>(tcf + jh);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        v[r] = m[r] * (c0[r] * rowf);
                        if constexpr (VL) v[r] = jh + r >= fsi ? v[r] : 0.0f;
                    }
                }
                const bf16x4 mf = pack4(v);
#pragma unroll
                for (int q = 0; q < 4; ++q) mma16(acc[q], xq[q], mf);
                continue;
            }
            floatx4 m[2] = {floatx4{0.0f, 0.0f, 0.0f, 0.0f}, floatx4{0.0f, 0.0f, 0.0f, 0.0f}};
            // the diagonal slice of an even row tile: its second half lies above
            // the diagonal (j >= 32 js + 16 > i) and stays zero (packed sequences
            // take the general path)
            const bool zh1 = !VL && diag && !(wr & 1);  // uniform
            auto cb_half = [&](int half) {
#pragma unroll
                for (int kq = 0; kq < NK; ++kq) {
                    const int j = 32 * js + 16 * half + cc;
                    Frag<bf16_t> bf;
                    lds_frag8(bf, sm.bb + j * N + (((4 * kq + g4) ^ tr_swz<PPR>(j)) << 3));
                    mma(m[half], bf, cfr[kq]);
                }
            };
            if (zh1) {
                cb_half(0);
            } else if (N == 128) {
                // (two workgroups per compute unit: both halves' B fragments
                // read before the products, which then wait on no LDS read)
                Frag<bf16_t> bq[2][NK];
#pragma unroll
                for (int kq = 0; kq < NK; ++kq)
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        const int j = 32 * js + 16 * half + cc;
                        lds_frag8(bq[half][kq], sm.bb + j * N + (((4 * kq + g4) ^ tr_swz<PPR>(j)) << 3));
                    }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int kq = 0; kq < NK; ++kq)
#pragma unroll
                    for (int half = 0; half < 2; ++half) mma(m[half], bq[half][kq], cfr[kq]);
            } else {
#pragma unroll
                for (int kq = 0; kq < NK; ++kq) {
                    const int q = 4 * kq + g4;
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        const int j = 32 * js + 16 * half + cc;
                        Frag<bf16_t> bf;
                        lds_frag8(bf, sm.bb + j * N + ((q ^ tr_swz<PPR>(j)) << 3));
                        mma(m[half], bf, cfr[kq]);
                    }
                }
            }
            // lane (g4, cc): rows j = 32 js + 16 half + 4 g4 + r of column i
            float v[8];
            if (diag) {
                // holds the diagonal: exp per element, causal mask, D on j = i
                const floatx4 s0 = *reinterpret_cast<const floatx4 *>(tsl + j0);
                const floatx4 s1 = *reinterpret_cast<const floatx4 *>(tsl + j0 + 16);
                const floatx4 w0 = *reinterpret_cast<const floatx4 *>(twt + j0);
                const floatx4 w1 = *reinterpret_cast<const floatx4 *>(twt + j0 + 16);
                if (!VL && (wr & 1)) {
                    // odd row tile (i >= 32 js + 16): the first half lies wholly
                    // below the diagonal (no mask, no D; its decays exp(s_i - s_b)
                    // exp(s_b - s_j) w_j through the slice's 16th token b, both
                    // factors <= 1), the second holds the diagonal 16 x 16 block
                    // (j <= i: 4 g4 + r <= cc)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        v[r] = m[0][r] * (__builtin_amdgcn_exp2f(si - s0[r]) * w0[r]);
                        const float a1 = __builtin_fmaf(
                            m[1][r], __builtin_amdgcn_exp2f(si - s1[r]) * w1[r], dval[4 + r]);
                        v[4 + r] = 4 * g4 + r <= cc ? a1 : 0.0f;
                    }
                } else if (!VL) {
                    // even row tile: the first half holds the diagonal block, the
                    // second is zero
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float a0 = __builtin_fmaf(
                            m[0][r], __builtin_amdgcn_exp2f(si - s0[r]) * w0[r], dval[r]);
                        v[r] = 4 * g4 + r <= cc ? a0 : 0.0f;
                        v[4 + r] = 0.0f;
                    }
                } else {  // packed sequences: masks of causality and of each row's sequence
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float a0 = __builtin_fmaf(
                            m[0][r], __builtin_amdgcn_exp2f(si - s0[r]) * w0[r], dval[r]);
                        const float a1 = __builtin_fmaf(
                            m[1][r], __builtin_amdgcn_exp2f(si - s1[r]) * w1[r], dval[4 + r]);
                        const bool on0 = j0 + r <= i && j0 + r >= fsi;
                        const bool on1 = j0 + 16 + r <= i && j0 + 16 + r >= fsi;
                        v[r] = on0 ? a0 : 0.0f;
                        v[4 + r] = on1 ? a1 : 0.0f;
                    }
                }
            } else {
                // wholly below it (i >= 32 > j): exp(s_i - s_31) exp(s_31 - s_j) w_j,
                // both factors <= 1, no mask
                const float rowf = __builtin_amdgcn_exp2f(si - s31);
                const floatx4 c0 = *reinterpret_cast<const floatx4 *>(tcf + j0);
                const floatx4 c1 = *reinterpret_cast<const floatx4 *>(tcf + j0 + 16);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    v[r] = m[0][r] * (c0[r] * rowf);
                    v[4 + r] = m[1][r] * (c1[r] * rowf);
                    if constexpr (VL) {  // tokens of earlier sequences
                        v[r] = j0 + r >= fsi ? v[r] : 0.0f;
                        v[4 + r] = j0 + 16 + r >= fsi ? v[4 + r] : 0.0f;
                    }
                }
            }
            Frag<bf16_t> mf;
            pack8(mf, v);
            // Y^T[p][i] += sum_j x_j[p] M[i][j]
            const __bf16 *xsl = xs + js * 2048;
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                Frag<bf16_t> xf;
                x_colfrag<0>(xf, xsl, xo[pt]);
                mma(acc[pt], xf, mf);
            }
        }

        // ---- state (p tile w): H^T = exp(s_end) H^T + sum_j B_j (exp(s_end - s_j) w_j x_j)^T
        Frag<bf16_t> xr[2];
        x_colfrag<0>(xr[0], xs, xo[wr]);
        x_colfrag<1>(xr[1], xs, xo[wr]);
        const int lenk = min(T, Lw - t0);
        if constexpr (VL) {
            // sequences that end inside the block, before its last token je =
            // lenk - 1: the state after their last token e, [fs_e < 0] e^{s_e}
            // H + sum_{fs_e <= j <= e} e^{s_e - s_j} w_j x_j B_j^T, from the
            // state entering the block (this wavefront's columns)
            uint64_t ends = ((uint64_t)sm.vt[k & 1].ends[1] << 32) | sm.vt[k & 1].ends[0];
            ends &= ~(1ull << (lenk - 1));
            while (ends && vl.seq_states) {  // uniform
                const int e = __builtin_ctzll(ends);
                ends &= ends - 1;
                const int fe = sm.vt[k & 1].fs[e];
                const float se = tsl[e];
                const float f = fe < 0 ? __builtin_amdgcn_exp2f(se) : 0.0f;
                floatx4 he[NTH];
#pragma unroll
                for (int nt = 0; nt < NTH; ++nt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) he[nt][r] = hreg[nt][r] * f;
#pragma unroll
                for (int js = 0; js < 2; ++js) {
                    const int jb = 32 * js + 4 * g4;
                    float v[8];
#pragma unroll
                    for (int r = 0; r < 8; ++r) {
                        const int j = jb + (r < 4 ? r : 12 + r);
                        v[r] = j >= fe && j <= e ? xr[js].get(r) *
                                                       (__builtin_amdgcn_exp2f(se - tsl[j]) * twt[j])
                                                 : 0.0f;
                    }
                    Frag<bf16_t> xw;
                    pack8(xw, v);
#pragma unroll
                    for (int nt = 0; nt < NTH; ++nt) {
                        Frag<bf16_t> bf;
                        colfrag_swz<PPR>(bf, sm.bb, jb, jb + 16, (nh * NTH + nt) * 16);
                        mma(he[nt], bf, xw);
                    }
                }
                float *out = vl.seq_states + ((size_t)sm.mts[k & 1][e].y * H + h) * P * N + hoff;
#pragma unroll
                for (int nt = 0; nt < NTH; ++nt)
                    *reinterpret_cast<float4 *>(out + 16 * nt) =
                        make_float4(he[nt][0], he[nt][1], he[nt][2], he[nt][3]);
            }
        }
#pragma unroll
        for (int nt = 0; nt < NTH; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) hreg[nt][r] *= dec;
#pragma unroll
        for (int js = 0; js < 2; ++js) {
            const int jb = 32 * js + 4 * g4;
            const floatx4 p0 = *reinterpret_cast<const floatx4 *>(twp + jb);
            const floatx4 p1 = *reinterpret_cast<const floatx4 *>(twp + jb + 16);
            float v[8];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                v[r] = xr[js].get(r) * p0[r];
                v[4 + r] = xr[js].get(4 + r) * p1[r];
            }
            Frag<bf16_t> xw;
            pack8(xw, v);
            if constexpr (HALVES) {  // every B^T fragment read before the products
                Frag<bf16_t> bv[NTH];
#pragma unroll
                for (int nt = 0; nt < NTH; ++nt)
                    colfrag_swz<PPR>(bv[nt], sm.bb, jb, jb + 16, (nh * NTH + nt) * 16);
#pragma unroll
                for (int nt = 0; nt < NTH; ++nt) mma(hreg[nt], bv[nt], xw);
            } else {
#pragma unroll
                for (int nt = 0; nt < NTH; ++nt) {
                    Frag<bf16_t> bf;
                    colfrag_swz<PPR>(bf, sm.bb, jb, jb + 16, (nh * NTH + nt) * 16);
                    mma(hreg[nt], bf, xw);
                }
            }
        }
        if constexpr (VL) {
            // a sequence ending at the block's last token: the state is H itself
            const uint32_t eb = sm.vt[k & 1].ends[(lenk - 1) >> 5];
            if (((eb >> ((lenk - 1) & 31)) & 1u) && vl.seq_states) {  // uniform
                float *out =
                    vl.seq_states + ((size_t)sm.mts[k & 1][lenk - 1].y * H + h) * P * N + hoff;
#pragma unroll
                for (int nt = 0; nt < NTH; ++nt)
                    *reinterpret_cast<float4 *>(out + 16 * nt) =
                        make_float4(hreg[nt][0], hreg[nt][1], hreg[nt][2], hreg[nt][3]);
            }
        }

        // the next block's tables, by a wavefront with one C B^T tile
        if (w == 0 && k + 1 < nblk) make_tables(k + 1);

        if constexpr (HALVES) {  // the second half's partial outputs to the first
            if (nh == 1) {
#pragma unroll
                for (int q = 0; q < 4; ++q) sm.xch[4 * wr + (q ^ pflip)][l] = acc[q];
            }
        }

        // x, B, C, dt and the state of this block consumed by every wavefront
        barrier_lds();
        put_h();
        if (k + 1 < nblk) issue_bcd(k + 1);
        // (three buffers: x two blocks ahead, into the buffer of the previous
        // block, whose staged outputs every wavefront has read)
        if (NXB == 3 && k + 2 < nblk) issue_x(k + 2);

        if constexpr (HALVES) {
            if (nh == 1) continue;  // uniform: the first half stages and stores the rows
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                const floatx4 o = sm.xch[4 * wr + pt][l];
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[pt][r] += o[r];
            }
        }
        // ---- the outputs: this wavefront's rows, every column, into the x buffer
        __bf16 *xw_ = sm.xb[k % NXB];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
            const int off = x_at(i, 16 * pt + 4 * g4);
            const bf16x2 lo = __builtin_convertvector(floatx2{acc[pt][0], acc[pt][1]}, bf16x2);
            const bf16x2 hi = __builtin_convertvector(floatx2{acc[pt][2], acc[pt][3]}, bf16x2);
            *reinterpret_cast<bf16x4 *>(xw_ + off) = bf16x4{lo[0], lo[1], hi[0], hi[1]};
        }
        // this wavefront's 16 rows (staged by itself: no barrier) into
        // registers; stored during the next block
#pragma unroll
        for (int m = 0; m < 2; ++m)
            ystage[m] = *reinterpret_cast<const uint4 *>(xs + (128 * wr + 64 * m + l) * 8);
    }
    if (nh == 0) {  // the last block's outputs (possibly a partial block)
        const int t0 = (nblk - 1) * T, len = Lw - t0;
        char *yb = reinterpret_cast<char *>(yh + (size_t)t0 * xrow);
#pragma unroll
        for (int m = 0; m < 2; ++m)
            if (yrow[m] < len) store_nt16(yb + yoff[m], ystage[m]);
    }

    if (final_state && seg == nseg - 1) {
#pragma unroll
        for (int nt = 0; nt < NTH; ++nt)
            *reinterpret_cast<float4 *>(final_state + bh * P * N + hoff + 16 * nt) =
                make_float4(hreg[nt][0], hreg[nt][1], hreg[nt][2], hreg[nt][3]);
    }
}

// ---- segment states
//
// For each piece of the first S-1 segments of a (batch, head): the state the
// piece produces from a zero state, H = sum_t exp(s_end - s_t) w_t x_t B_t^T
// (the single-pass kernel's state update, block by block), and the piece's
// total log2-decay. Only x, B and dt are read. Small LDS footprints let
// several workgroups share a compute unit, enough for the loads of one to
// hide behind the others' work. Every block's inputs
// are loaded a whole block ahead into double buffers, issued as the block
// before starts, so one barrier per block suffices.
// At N 128, where a group has an even number of heads, a workgroup takes two
// heads of one group (HP = 2, four wavefronts each): they share the block's B
// rows (and dt piece), so B, two thirds of the bytes the kernel reads per
// head, crosses the texture path once per two heads. (At N 64, where B is a
// third of them, the pairs were slower.)
// Tokens per block of the segment-state kernel (the pieces still hold whole
// 64-token blocks of the single-pass kernel): 32 at N 128 (five workgroups per
// compute unit, three of head pairs); 64 at N 64 (four) and at N 256 (eight
// wavefronts, B rows of 512 bytes, one).
template <int N>
constexpr int seg_states_block() {
    return N == 128 ? 32 : 64;
}

template <int N, bool VL, int HP>
struct SegStateLds {
    static constexpr int TS = seg_states_block<N>();
    __bf16 xb[HP][2][TS * 64];
    __bf16 bb[2][TS * N];
    __bf16 dts[2][kOpT * 8];  // one 16-byte dt piece per lane (lanes past the block repeat its last)
    struct {
        float wp[TS];
        float dec, ld;  // the state's decay across the block and its log2 (-inf: a reset)
    } tab[HP][2];
    int4 mts[VL ? 2 : 1][VL ? kOpT : 1];  // packed sequences: the tokens' int4 of blocks k, k+1
};

// Workgroups per compute unit of the segment-state kernel (its launch bounds).
template <int N, int HP>
constexpr int seg_states_wgs_per_cu() {
    return HP == 2 ? 3 : N == 64 ? 4 : N == 128 ? 5 : 1;
}
// Heads per compute unit, as the plan counts them (with two heads per
// workgroup at N 128 the GPU holds six).
template <int N>
constexpr int seg_states_per_cu() {
    return N == 64 ? 4 : N == 128 ? 5 : 1;
}
// Two heads per workgroup of the segment-state kernel: N 128 and an even
// number of heads per group.
constexpr bool seg_states_pairs(int N, int H, int G) {
    return N == 128 && (H / G) % 2 == 0;
}

template <int N, bool VL, int HP>
__global__ __launch_bounds__(N == 256 ? 512 : 256 * HP, (seg_states_wgs_per_cu<N, HP>())) void ssd_segment_states_kernel(
    const bf16_t *__restrict__ x, const bf16_t *__restrict__ dt, const float *__restrict__ A,
    const bf16_t *__restrict__ B, DtOpts o, int batch, int L, int H, int G, int per,
    OnepassSegs sg, OnepassVl vl) {
    constexpr int P = 64, T = seg_states_block<N>();
    constexpr int PPR = N / 8, NT = N / 16;
    // N 256: eight wavefronts, w and w + 4 with halves of the state's n
    constexpr bool HALVES = N == 256;
    constexpr int NWV = HALVES ? 8 : 4, NTH = HALVES ? NT / 2 : NT;  // NWV: per head
    static_assert(N % 32 == 0 && T * PPR >= 64 && T * 8 % 64 == 0, "state size");
    static_assert(HP == 1 || (HP == 2 && N == 128), "head pairs at N 128 only");
    __shared__ __attribute__((aligned(16))) SegStateLds<N, VL, HP> sm;

    // workgroup -> (batch, piece, head pair or head), XCD-aware as in the
    // single-pass kernel; wavefronts NWV e .. NWV e + NWV - 1 take head HP hu + e
    const int id = blockIdx.x;
    const int lin = (id & 7) * per + (id >> 3);
    const int HU = H / HP;  // head units (the host launches HP = 2 only where HP divides H / G)
    if (lin >= batch * sg.nseg * HU) return;  // whole workgroup
    const int wa = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wavefront in the workgroup
    const int e = wa / NWV, w = wa % NWV;  // this wavefront's head of the unit, its index there
    const int hu = lin % HU, bs = lin / HU, pc = bs % sg.nseg, b = bs / sg.nseg;
    const int h = hu * HP + e, g = h / (H / G);
    const int tb = pc * sg.len, Lw = min(sg.len, L - tb);
    const size_t bh = (size_t)b * H + h;
    const int wr = HALVES ? (w & 3) : w, nh = HALVES ? (w >> 2) : 0;  // head-dim tile, n half
    const int l = lane_id(), g4 = l >> 4, cc = l & 15;
    const int nblk = (Lw + T - 1) / T;

    const size_t xrow = (size_t)H * P, brow = (size_t)G * N, row0 = (size_t)b * L + tb;
    const bf16_t *xh = x + row0 * xrow + (size_t)h * P;
    const bf16_t *bg = B + row0 * brow + (size_t)g * N;
    const bf16_t *dth = dt + row0 * H + (h & ~7);
    const float Ah = A[h];
    const float bias = o.bias ? o.bias[h] : 0.0f;
    const uint32_t xrb = (uint32_t)(xrow * 2), brb = (uint32_t)(brow * 2), drb = (uint32_t)H * 2;

    // (the unit's heads share the dt piece: HP hu and HP hu + 1 lie in one
    // aligned group of 8)
    auto issue_dt = [&](int k) {  // wavefront 0 of the workgroup only
        const int t0 = k * T, len = min(T, Lw - t0);
        dma16_sv(dth + (size_t)t0 * H, (uint32_t)min(l, len - 1) * drb, sm.dts[k & 1]);
        if constexpr (VL)
            dma16_sv(vl.meta + row0 + t0, (uint32_t)min(l, len - 1) * 16, sm.mts[k & 1]);
    };
    // block k's x (each head's own wavefronts) and B (every wavefront of the
    // workgroup), and (wavefront 0) the dt of block k + 1
    auto issue = [&](int k) {
        const int t0 = k * T, len = min(T, Lw - t0);
        if (wa == 0 && k + 1 < nblk) issue_dt(k + 1);
        const bf16_t *xk = xh + (size_t)t0 * xrow, *bk = bg + (size_t)t0 * brow;
#pragma unroll
        for (int i = w; i < T * 8 / 64; i += NWV) {
            const int s = i * 64 + l, r = s >> 3, q = (s & 7) ^ (r & 7);
            const uint32_t off = (uint32_t)min(r, len - 1) * xrb + q * 16;
            if (sg.xnt) dma16_sv_nt(xk, off, sm.xb[e][k & 1] + i * 512);
            else dma16_sv(xk, off, sm.xb[e][k & 1] + i * 512);
        }
#pragma unroll
        for (int i = wa; i < T * PPR / 64; i += HP * NWV) {
            const int s = i * 64 + l, r = s / PPR, q = (s % PPR) ^ tr_swz<PPR>(r);
            dma16_sv(bk, (uint32_t)min(r, len - 1) * brb + q * 16, sm.bb[k & 1] + i * 512);
        }
    };
    // block k's prefix sums and state weights (wavefront 0; lane j is token
    // t0 + j, lanes past the block add zero terms)
    auto make_tables = [&](int k) {
        const int len = min(T, Lw - k * T);
        const bool valid = l < len;
        const float raw = static_cast<float>(sm.dts[k & 1][l * 8 + (h & 7)]);
        const float st = valid ? step_size(o, raw, bias) : 0.0f;
        const float wgt = valid ? input_weight(o, st, Ah) : 0.0f;
        const float sl = wave_prefix_sum(st * Ah) * kLog2e;
        const float sle = lane_value(sl, 63);
        float wp = __builtin_amdgcn_exp2f(sle - sl) * wgt;
        bool reset = false;  // packed sequences: the block's last token's sequence begins in it
        if constexpr (VL) {
            const int fs = sm.mts[k & 1][l].x - (tb + k * T);
            const int fsl = __builtin_amdgcn_readlane(fs, len - 1);
            if (l < fsl) wp = 0.0f;
            reset = fsl >= 0;
        }
        if (l < T) sm.tab[e][k & 1].wp[l] = wp;
        if (l == 0) {
            sm.tab[e][k & 1].dec = reset ? 0.0f : __builtin_amdgcn_exp2f(sle);
            sm.tab[e][k & 1].ld = reset ? -__builtin_inff() : sle;
        }
    };

    floatx4 hreg[NTH];  // n tiles nh * NTH + 0 .. NTH-1
#pragma unroll
    for (int nt = 0; nt < NTH; ++nt) hreg[nt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    float ld = 0.0f;  // the piece's log2-decay so far
    int xo[4];
    x_colfrag_offsets(xo, l);
    const int jb = 4 * g4;

    if (wa == 0) issue_dt(0);
    issue(0);
    for (int k = 0; k < nblk; ++k) {
        // block k's inputs (and the dt of block k + 1) have landed; every
        // wavefront is done with block k - 1's buffers and tables
        wait_barrier<0>();
        if (k == 0) {  // later blocks' tables are made during the block before
            if (w == 0) make_tables(0);
            barrier_lds();
        }
        if (k + 1 < nblk) issue(k + 1);
        const __bf16 *xs = sm.xb[e][k & 1], *bs_ = sm.bb[k & 1];
        const float *twp = sm.tab[e][k & 1].wp;
        const float dec = sm.tab[e][k & 1].dec;
        ld += sm.tab[e][k & 1].ld;

        // H^T = exp(s_end) H^T + sum_j B_j (exp(s_end - s_j) w_j x_j)^T, p tile w
        Frag<bf16_t> xr[T / 32];
        x_colfrag<0>(xr[0], xs, xo[wr]);
        if constexpr (T == 64) x_colfrag<1>(xr[T / 32 - 1], xs, xo[wr]);
#pragma unroll
        for (int nt = 0; nt < NTH; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) hreg[nt][r] *= dec;
#pragma unroll
        for (int js = 0; js < T / 32; ++js) {
            const int jj = 32 * js + jb;
            const floatx4 p0 = *reinterpret_cast<const floatx4 *>(twp + jj);
            const floatx4 p1 = *reinterpret_cast<const floatx4 *>(twp + jj + 16);
            float v[8];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                v[r] = xr[js].get(r) * p0[r];
                v[4 + r] = xr[js].get(4 + r) * p1[r];
            }
            Frag<bf16_t> xw;
            pack8(xw, v);
#pragma unroll
            for (int nt = 0; nt < NTH; ++nt) {
                Frag<bf16_t> bf;
                colfrag_swz<PPR>(bf, bs_, jj, jj + 16, (nh * NTH + nt) * 16);
                mma(hreg[nt], bf, xw);
            }
        }
        // the next block's tables (its dt landed with this block's inputs)
        if (w == 0 && k + 1 < nblk) make_tables(k + 1);
    }

    float *sj = sg.state + (bh * sg.npc + pc) * P * N + (size_t)(16 * wr + cc) * N + 4 * g4 +
                16 * NTH * nh;
#pragma unroll
    for (int nt = 0; nt < NTH; ++nt)
        *reinterpret_cast<float4 *>(sj + 16 * nt) =
            make_float4(hreg[nt][0], hreg[nt][1], hreg[nt][2], hreg[nt][3]);
    if (w == 0 && l == 0) sg.ld[bh * sg.npc + pc] = ld;
}

// ---- the chain over the pieces
//
// For every (batch, head) and segment s = 1 .. S-1: the state entering the
// segment, E_s = fold over the pieces j < s k of E <- exp2(ld_j) E + H_j,
// from the initial state (or zero): the chunk-to-chunk recurrence at piece
// granularity, float32, each thread one float4 of one (batch, head)'s state.
// E_s overwrites the slot of piece s k - 1, which this thread has read by
// then; the single-pass kernel reads it from there.
__global__ __launch_bounds__(256) void ssd_segment_chain_kernel(const float *__restrict__ init,
                                                                OnepassSegs sg, int units, int PN) {
    const int q4 = PN / 4;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)units * q4) return;
    const size_t u = idx / q4, e = idx - u * q4;
    floatx4 acc = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    if (init) {
        const float4 v = reinterpret_cast<const float4 *>(init + u * PN)[e];
        acc = floatx4{v.x, v.y, v.z, v.w};
    }
    float4 *st = reinterpret_cast<float4 *>(sg.state + u * sg.npc * PN) + e;
    const float *ld = sg.ld + u * sg.npc;
    const int np = (sg.nseg - 1) * sg.kpc;
    // pieces in batches of eight: their loads issued together, then folded in order
    for (int j0 = 0; j0 < np; j0 += 8) {
        float4 v[8];
        float f[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            if (j0 + q < np) {
                v[q] = st[(size_t)(j0 + q) * q4];
                f[q] = ld[j0 + q];
            }
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int j = j0 + q;
            if (j < np) {
                const float a = __builtin_amdgcn_exp2f(f[q]);
                acc = floatx4{acc[0] * a + v[q].x, acc[1] * a + v[q].y, acc[2] * a + v[q].z,
                              acc[3] * a + v[q].w};
                if ((j + 1) % sg.kpc == 0)  // the last piece of a segment
                    st[(size_t)j * q4] = make_float4(acc[0], acc[1], acc[2], acc[3]);
            }
        }
    }
}

bool forward_onepass_ok(int batch, int nheads, int dstate, bool bf16, const void *dt) {
    // dt is read as 16-byte pieces of 8 heads; a block's byte offsets into x
    // and y (64 rows of nheads * 64 bf16) are 32-bit
    (void)batch;
    return bf16 && (dstate == 64 || dstate == 128 || dstate == 256) && nheads % 8 == 0 &&
           nheads < (1 << 19) && (reinterpret_cast<uintptr_t>(dt) & 15u) == 0;
}

namespace {

size_t piece_bytes(int dstate) { return (64 * (size_t)dstate + 1) * sizeof(float); }

}  // namespace

// Enough (batch, head) pairs fill the GPU with one workgroup each (three per
// compute unit at N = 64, two at N = 128, one at N = 256). With fewer, each
// sequence is cut into S segments of whole 64-token blocks, S the number of
// workgroups per pair that still fit in one round of workgroups, each segment
// at least 4 blocks long. The segment-state kernel, lighter (four workgroups
// per compute unit at N = 64, three at N = 128, one at N = 256), cuts each of
// the first S - 1 segments into k pieces of at least 2 blocks so that it, too,
// fills the GPU.
// The scratch holds one float32 state and one decay per piece of every
// (batch, head): batch * nheads * (S - 1) * k of them. A cap smaller than
// what that needs lowers k, then gives up the segments.
OnepassPlan forward_onepass_plan(int batch, int seqlen, int nheads, int dstate, size_t cap) {
    const int slots = (dstate == 64 ? 3 : dstate == 128 ? 2 : 1) * 256,
              so_slots = (dstate == 64    ? seg_states_per_cu<64>()
                          : dstate == 128 ? seg_states_per_cu<128>()
                                          : seg_states_per_cu<256>()) *
                         256;
    const size_t units = (size_t)batch * nheads;
    const int blocks = (seqlen + kOpT - 1) / kOpT;
    const OnepassPlan one{1, 0, blocks, blocks, 0};
    if (units >= (size_t)slots) return one;
    const int S0 = std::min((int)(slots / units), blocks / 4);
    if (S0 <= 1) return one;
    const int per = (blocks + S0 - 1) / S0;
    const size_t max_pieces = cap / piece_bytes(dstate);
    const int kmax = std::max(1, std::min((int)(so_slots / (units * (S0 - 1))), per / 2));
    // the k <= kmax that pads the segments least (k * ceil(per / k) blocks),
    // the largest of those: pieces of equal length, segments as even as the
    // sequence allows
    int k = 1;
    for (int kk = 1; kk <= kmax; ++kk)
        if (kk * ((per + kk - 1) / kk) <= k * ((per + k - 1) / k)) k = kk;
    for (;;) {
        const int psub = (per + k - 1) / k, per_seg = k * psub;
        const int S = (blocks + per_seg - 1) / per_seg;  // the last segment is not empty
        if (S <= 1) return one;
        const size_t pieces = units * (size_t)(S - 1) * k;
        if (pieces <= max_pieces) return OnepassPlan{S, k, per_seg, psub, pieces * piece_bytes(dstate)};
        if (k == 1) return one;
        k = std::max<int>(1, (int)std::min<size_t>(max_pieces / (units * (S - 1)), k - 1));
    }
}

template <int N, bool VL>
static hipError_t launch_onepass_n(const void *x, const void *dt, const float *A, const void *B,
                                   const void *C, const float *D, const float *init,
                                   const DtOpts &opts, int batch, int seqlen, int nheads,
                                   int ngroups, const OnepassPlan &pl, float *scratch,
                                   const OnepassVl &vl, void *y, float *final_state,
                                   hipEvent_t between, hipStream_t stream) {
    const auto xb = static_cast<const bf16_t *>(x);
    const auto dtb = static_cast<const bf16_t *>(dt);
    const auto Bb = static_cast<const bf16_t *>(B);
    const auto Cb = static_cast<const bf16_t *>(C);
    const int npc = pl.S > 1 ? (pl.S - 1) * pl.k : 0;
    float *ld = npc ? scratch + (size_t)batch * nheads * npc * 64 * N : nullptr;
    const int chained = npc > kChainPieces;  // the last segment folds npc pieces
    const int xnt = (size_t)batch * seqlen * nheads * 64 * sizeof(bf16_t) > kStreamXBytes;
    if (pl.S > 1) {
        const OnepassSegs pieces{npc, pl.psub * kOpT, npc, 0, scratch, ld, 0, xnt};
        bool pairs = false;
        if constexpr (N == 128) pairs = seg_states_pairs(N, nheads, ngroups);
        if (pairs) {
            if constexpr (N == 128) {
                const int per = (batch * nheads / 2 * npc + 7) / 8;
                ssd_segment_states_kernel<N, VL, 2><<<per * 8, 512, 0, stream>>>(
                    xb, dtb, A, Bb, opts, batch, seqlen, nheads, ngroups, per, pieces, vl);
            }
        } else {
            const int per = (batch * nheads * npc + 7) / 8;
            ssd_segment_states_kernel<N, VL, 1><<<per * 8, N == 256 ? 512 : 256, 0, stream>>>(
                xb, dtb, A, Bb, opts, batch, seqlen, nheads, ngroups, per, pieces, vl);
        }
        hipError_t e = hipGetLastError();
        if (e == hipSuccess && chained) {
            const OnepassSegs chain{pl.S, 0, npc, pl.k, scratch, ld, 1, 0};
            const size_t threads = (size_t)batch * nheads * 64 * N / 4;
            ssd_segment_chain_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, stream>>>(
                init, chain, batch * nheads, 64 * N);
            e = hipGetLastError();
        }
        if (e == hipSuccess && between) e = hipEventRecord(between, stream);
        if (e != hipSuccess) return e;
    }
    const OnepassSegs segs{pl.S, pl.per_seg * kOpT, npc, pl.k, scratch, ld, chained, xnt};
    const int units = batch * nheads * pl.S;
    const int per = (units + 7) / 8;
    ssd_forward_onepass_kernel<N, VL><<<per * 8, N == 256 ? 512 : 256, 0, stream>>>(
        xb, dtb, A, Bb, Cb, D, init, opts, batch, seqlen, nheads, ngroups, per, segs, vl,
        static_cast<bf16_t *>(y), final_state);
    return hipGetLastError();
}

hipError_t launch_forward_onepass(const void *x, const void *dt, const float *A, const void *B,
                                  const void *C, const float *D, const float *init,
                                  const DtOpts &opts, int batch, int seqlen, int nheads,
                                  int ngroups, int dstate, const OnepassPlan &pl, float *scratch,
                                  void *y, float *final_state, hipEvent_t between,
                                  hipStream_t stream, const void *varlen_meta,
                                  float *seq_states) {
    const OnepassVl vl{static_cast<const int4 *>(varlen_meta), seq_states};
    if (varlen_meta && (batch != 1 || init || final_state)) return hipErrorInvalidValue;
    if (pl.S > 1 && !scratch) return hipErrorInvalidValue;
#define SSD_ONEPASS(NN, VV)                                                                      \
    return launch_onepass_n<NN, VV>(x, dt, A, B, C, D, init, opts, batch, seqlen, nheads,       \
                                    ngroups, pl, scratch, vl, y, final_state, between, stream)
    if (dstate == 64) {
        if (varlen_meta) SSD_ONEPASS(64, true);
        SSD_ONEPASS(64, false);
    }
    if (dstate == 128) {
        if (varlen_meta) SSD_ONEPASS(128, true);
        SSD_ONEPASS(128, false);
    }
    if (dstate == 256) {
        if (varlen_meta) SSD_ONEPASS(256, true);
        SSD_ONEPASS(256, false);
    }
#undef SSD_ONEPASS
    return hipErrorInvalidValue;
}

// ---- packed sequences: the tokens' int4 and the states of empty sequences
//
// Workgroups 0 .. ceil(L / 256) - 1: meta[t] = {first token of t's sequence,
// its index, whether t is its last token, 0} for t < L (any cu_seqlens
// contents give in-range values: the index is the largest k < nseq with
// cu[k] <= t). The next nseq workgroups (when seq_states is given): zero
// states for the empty sequences, which no token ends.
__global__ __launch_bounds__(256) void onepass_varlen_prep_kernel(const int *__restrict__ cu,
                                                                  int nseq, int L, int H, int PN,
                                                                  int4 *__restrict__ meta,
                                                                  float *__restrict__ seq_states) {
    const int nb = (L + 255) / 256;
    if ((int)blockIdx.x >= nb) {
        const int k = blockIdx.x - nb;
        if (cu[k + 1] > cu[k]) return;  // whole workgroup
        float4 *out = reinterpret_cast<float4 *>(seq_states + (size_t)k * H * PN);
        for (int i = threadIdx.x; i < H * PN / 4; i += 256)
            out[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        return;
    }
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= L) return;
    int lo = 0, hi = nseq - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= t) lo = mid;
        else hi = mid - 1;
    }
    const int start = min(max(cu[lo], 0), t);
    const bool last = t == L - 1 || cu[lo + 1] == t + 1;
    meta[t] = make_int4(start, lo, last ? 1 : 0, 0);
}

hipError_t launch_onepass_varlen_prep(const int *cu_seqlens, int nseq, int seqlen, int nheads,
                                      int dstate, void *meta, float *seq_states,
                                      hipStream_t stream) {
    const int nb = (seqlen + 255) / 256;
    onepass_varlen_prep_kernel<<<nb + (seq_states ? nseq : 0), 256, 0, stream>>>(
        cu_seqlens, nseq, seqlen, nheads, 64 * dstate, static_cast<int4 *>(meta), seq_states);
    return hipGetLastError();
}

}  // namespace ssd
