// C B^T of every chunk, once per B/C group (part of stage 4).
//
// In the diagonal block of the semiseparable matrix, y_i = sum_{j<=i}
// (C_i . B_j) L_ij dt_j x_j ("Mamba 模型", section 4.1; "Draft:Mamba2", SSD
// section). C_i . B_j does not depend on the head: heads that share a B/C
// group (grouped-value heads, "Mamba 模型" section 4.3) share it. This kernel
// computes it once per (batch, chunk, group) for the causal 16x32 tiles and
// stores each tile in the exact register layout chunk_scan feeds to the MFMA
// (so chunk_scan loads one 16-byte fragment per lane and applies its head's
// decay).
//
// Tile (it, jp): output rows i = 16*it .. +15, tokens j = 32*jp .. +31, for
// jp <= it/2 (the 32-token slices that reach row 16*it+15). Tiles are stored
// row-tile-major; tile (it, jp) starts at entry (m(m+1) or (m+1)^2 for it =
// 2m or 2m+1) + jp. Within a tile, lane l = 16*g + r holds 8 values for row
// i = 16*it + r: element e < 4 is token 32*jp + 4*g + e and element e >= 4 is
// token 32*jp + 16 + 4*g + (e - 4). One wavefront computes one tile as two
// 16x16 MFMA products (B rows against C rows over the N state columns); the
// 16x16 result layout (lane 16*g + c holds rows 4g..4g+3 of column c) is
// exactly that fragment. Tokens past the sequence end read as zero.
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

template <typename T, int N, int Q>
__global__ __launch_bounds__(256) void chunk_cb_kernel(const T *__restrict__ B,
                                                       const T *__restrict__ C, int L, int G,
                                                       int nC, int nU,
                                                       typename LdsT<T>::type *__restrict__ cb) {
    using E = typename LdsT<T>::type;
    constexpr int NT = Q / 16;
    constexpr int ENTRIES = (NT / 2) * (NT / 2 + 1);
    constexpr int NK = (N + 31) / 32;
    // 1-D grid: unit u = c + nC * (g + G * b) has NTB workgroups of 4 tiles,
    // placed at ids q*8*NTB + tb*8 + u%8 (q = u/8) so that all of them run on
    // the same XCD (id % 8), which then reads that chunk's B and C once.
    constexpr int NTB = (ENTRIES + 3) / 4;
    const int id = blockIdx.x;
    const int q = id / (8 * NTB), rem = id % (8 * NTB);
    const int tb = rem / 8, u = q * 8 + rem % 8;
    if (u >= nU) return;  // whole workgroup exits together
    const int tile = tb * 4 + wave_id();
    if (tile >= ENTRIES) return;  // whole wavefront exits together
    const int c = u % nC, g = (u / nC) % G, b = u / (nC * G);
    // tile -> (it, jp)
    int it = 0;
    while (true) {
        const int m = (it + 1) / 2;
        const int next = ((it + 1) % 2 == 0) ? m * (m + 1) : (m + 1) * (m + 1);  // start of it+1
        if (tile < next) break;
        ++it;
    }
    const int m0 = it / 2;
    const int start = (it % 2 == 0) ? m0 * (m0 + 1) : (m0 + 1) * (m0 + 1);
    const int jp = tile - start;

    const int l = lane_id(), g4 = l >> 4, r16 = l & 15;
    const int t0 = c * Q, len = min(Q, L - t0);
    const size_t rs = (size_t)G * N;  // token stride of B and C
    const T *Bc = B + ((size_t)b * L + t0) * rs + (size_t)g * N;
    const T *Cc = C + ((size_t)b * L + t0) * rs + (size_t)g * N;

    // Loads are unconditional (row and column clamped into range); values
    // outside the chunk or past N are replaced by zero afterwards, so all
    // loads of the wavefront are in flight together.
    const int i = it * 16 + r16;
    Raw8<T> craw[NK], braw[2][NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
        const int n0 = min(kk * 32 + 8 * g4, N - 8);
        craw[kk].load(Cc + (size_t)min(i, len - 1) * rs + n0);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int j = jp * 32 + half * 16 + r16;
            braw[half][kk].load(Bc + (size_t)min(j, len - 1) * rs + n0);
        }
    }
    floatx4 m[2] = {floatx4{0.0f, 0.0f, 0.0f, 0.0f}, floatx4{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
        const bool kin = kk * 32 + 8 * g4 < N;
        Frag<T> cf;
#pragma unroll
        for (int e = 0; e < 8; ++e) cf.set(e, (kin && i < len) ? craw[kk].get(e) : 0.0f);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int j = jp * 32 + half * 16 + r16;
            Frag<T> bf;
#pragma unroll
            for (int e = 0; e < 8; ++e) bf.set(e, (kin && j < len) ? braw[half][kk].get(e) : 0.0f);
            mma(m[half], bf, cf);
        }
    }
    E *dst = cb + ((((size_t)b * nC + c) * G + g) * ENTRIES + tile) * (64 * 8) + l * 8;
    Frag<T> out;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        out.set(r, m[0][r]);
        out.set(4 + r, m[1][r]);
    }
    store_frag8(dst, out);
}

size_t chunk_cb_entries(int chunk) {
    const int nt = chunk / 16;
    return (size_t)(nt / 2) * (nt / 2 + 1);
}

size_t chunk_cb_bytes(int batch, int seqlen, int ngroups, int chunk, bool bf16) {
    const size_t nC = ((size_t)seqlen + chunk - 1) / chunk;
    return (size_t)batch * nC * ngroups * chunk_cb_entries(chunk) * 64 * 8 * (bf16 ? 2 : 4);
}

template <typename T, int N, int Q>
static void launch_cb(const void *B, const void *C, int batch, int L, int G, void *cb,
                      hipStream_t stream) {
    using E = typename LdsT<T>::type;
    const int nC = (L + Q - 1) / Q;
    constexpr int NT = Q / 16;
    constexpr int ENTRIES = (NT / 2) * (NT / 2 + 1);
    constexpr int NTB = (ENTRIES + 3) / 4;
    const int nU = batch * nC * G;
    const dim3 grid((unsigned)(8 * NTB) * (unsigned)((nU + 7) / 8));
    chunk_cb_kernel<T, N, Q><<<grid, 256, 0, stream>>>(static_cast<const T *>(B),
                                                        static_cast<const T *>(C), L, G, nC, nU,
                                                        static_cast<E *>(cb));
}

template <typename T, int N>
static bool cb_q(int Q, const void *B, const void *C, int batch, int L, int G, void *cb,
                 hipStream_t s) {
    switch (Q) {
        case 64: launch_cb<T, N, 64>(B, C, batch, L, G, cb, s); return true;
        case 128: launch_cb<T, N, 128>(B, C, batch, L, G, cb, s); return true;
        case 256: launch_cb<T, N, 256>(B, C, batch, L, G, cb, s); return true;
        default: return false;
    }
}

template <typename T>
static hipError_t cb_dispatch(int N, int Q, const void *B, const void *C, int batch, int L, int G,
                              void *cb, hipStream_t s) {
    bool ok = false;
    switch (N) {
        case 16: ok = cb_q<T, 16>(Q, B, C, batch, L, G, cb, s); break;
        case 32: ok = cb_q<T, 32>(Q, B, C, batch, L, G, cb, s); break;
        case 64: ok = cb_q<T, 64>(Q, B, C, batch, L, G, cb, s); break;
        case 128: ok = cb_q<T, 128>(Q, B, C, batch, L, G, cb, s); break;
        case 256: ok = cb_q<T, 256>(Q, B, C, batch, L, G, cb, s); break;
        default: break;
    }
    if (!ok) return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_chunk_cb(const void *B, const void *C, int batch, int seqlen, int ngroups,
                           int dstate, int chunk, bool bf16, void *cb, hipStream_t stream) {
    if (bf16) return cb_dispatch<bf16_t>(dstate, chunk, B, C, batch, seqlen, ngroups, cb, stream);
    return cb_dispatch<float>(dstate, chunk, B, C, batch, seqlen, ngroups, cb, stream);
}

}  // namespace ssd
