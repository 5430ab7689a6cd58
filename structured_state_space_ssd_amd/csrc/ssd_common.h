// Device-side helpers shared by the SSD kernels (gfx950 / CDNA4 only).
//
// Matrix products use the 16x16 MFMA family with a common fragment format:
// for a 16-row operand tile and a 32-wide slice of the contraction index k,
// lane l = 16*g + r (g = 0..3, r = 0..15) holds 8 elements of row r, at k
// positions kmap(g, e), e = 0..7, where kmap is any bijection onto the 32
// positions that both operands of one product share. One bf16 fragment pair
// is a single v_mfma_f32_16x16x32_bf16; one fp32 pair is eight
// v_mfma_f32_16x16x4_f32 (element e of every lane per instruction), so both
// dtypes sum exactly the same 32 products. The 16x16 float32 result lives in
// 4 registers per lane: lane 16*g + c holds rows 4*g + 0..3 of column c.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssd_launch.h"

namespace ssd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;  // bf16 storage in global memory

constexpr float kLog2e = 1.4426950408889634f;

// The step size for raw value v of a head whose bias is `bias` (0 if none).
__device__ __forceinline__ float step_size(const DtOpts &o, float v, float bias) {
    v += bias;
    if (o.softplus) v = fmaxf(v, 0.0f) + log1pf(expf(-fabsf(v)));  // log(1 + e^v)
    if (o.clamp) v = fminf(fmaxf(v, o.lo), o.hi);
    return v;
}

// Weight of the input term for step size d of a head with decay rate a.
__device__ __forceinline__ float input_weight(const DtOpts &o, float d, float a) {
    return (o.zoh && a != 0.0f) ? expm1f(d * a) / a : d;
}

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
    return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// Input element -> float.
template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }

// float -> output element (bf16: round to nearest even in hardware).
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) {
    __bf16 b = static_cast<__bf16>(v);
    return __builtin_bit_cast(bf16_t, b);
}

// ---- MFMA operand fragments ------------------------------------------------
//
// Frag<T>: the 8 elements one lane contributes to a 16x16x32 product, in the
// MFMA operand type for input dtype T (bf16 -> __bf16, float -> float).
template <typename T> struct Frag;

template <> struct Frag<bf16_t> {
    bf16x8 v;
    __device__ __forceinline__ void zero() {
        for (int e = 0; e < 8; ++e) v[e] = static_cast<__bf16>(0.0f);
    }
    __device__ __forceinline__ void set(int e, float f) { v[e] = static_cast<__bf16>(f); }
    __device__ __forceinline__ float get(int e) const { return static_cast<float>(v[e]); }
};

template <> struct Frag<float> {
    float v[8];
    __device__ __forceinline__ void zero() {
        for (int e = 0; e < 8; ++e) v[e] = 0.0f;
    }
    __device__ __forceinline__ void set(int e, float f) { v[e] = f; }
    __device__ __forceinline__ float get(int e) const { return v[e]; }
};

// acc += A * B over one 32-wide k slice (A rows and B columns each one lane's
// row index r; see the header comment).
__device__ __forceinline__ void mma(floatx4 &acc, const Frag<bf16_t> &a, const Frag<bf16_t> &b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(floatx4 &acc, const Frag<float> &a, const Frag<float> &b) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
}

// Load 8 consecutive elements (k = k0 .. k0+7) of one row from LDS, where the
// LDS copy is stored in the MFMA operand type. Requires 16-byte (bf16) or
// 32-byte (float) alignment of the address.
__device__ __forceinline__ void lds_frag8(Frag<bf16_t> &f, const __bf16 *p) {
    f.v = *reinterpret_cast<const bf16x8 *>(p);
}
__device__ __forceinline__ void lds_frag8(Frag<float> &f, const float *p) {
    const floatx4 a = *reinterpret_cast<const floatx4 *>(p);
    const floatx4 b = *reinterpret_cast<const floatx4 *>(p + 4);
    f.v[0] = a[0]; f.v[1] = a[1]; f.v[2] = a[2]; f.v[3] = a[3];
    f.v[4] = b[0]; f.v[5] = b[1]; f.v[6] = b[2]; f.v[7] = b[3];
}

// Load two runs of 4 consecutive elements (elements 0..3 from p0, 4..7 from p1).
__device__ __forceinline__ void lds_frag4x2(Frag<bf16_t> &f, const __bf16 *p0, const __bf16 *p1) {
    const bf16x4 a = *reinterpret_cast<const bf16x4 *>(p0);
    const bf16x4 b = *reinterpret_cast<const bf16x4 *>(p1);
    f.v[0] = a[0]; f.v[1] = a[1]; f.v[2] = a[2]; f.v[3] = a[3];
    f.v[4] = b[0]; f.v[5] = b[1]; f.v[6] = b[2]; f.v[7] = b[3];
}
__device__ __forceinline__ void lds_frag4x2(Frag<float> &f, const float *p0, const float *p1) {
    const floatx4 a = *reinterpret_cast<const floatx4 *>(p0);
    const floatx4 b = *reinterpret_cast<const floatx4 *>(p1);
    f.v[0] = a[0]; f.v[1] = a[1]; f.v[2] = a[2]; f.v[3] = a[3];
    f.v[4] = b[0]; f.v[5] = b[1]; f.v[6] = b[2]; f.v[7] = b[3];
}

// Store / load one lane's 8 fragment elements to / from memory (16 bytes for
// bf16, 32 bytes for float; the address must be aligned to that size).
__device__ __forceinline__ void store_frag8(__bf16 *p, const Frag<bf16_t> &f) {
    *reinterpret_cast<bf16x8 *>(p) = f.v;
}
__device__ __forceinline__ void store_frag8(float *p, const Frag<float> &f) {
    reinterpret_cast<floatx4 *>(p)[0] = floatx4{f.v[0], f.v[1], f.v[2], f.v[3]};
    reinterpret_cast<floatx4 *>(p)[1] = floatx4{f.v[4], f.v[5], f.v[6], f.v[7]};
}
__device__ __forceinline__ void load_frag8(Frag<bf16_t> &f, const __bf16 *p) {
    f.v = *reinterpret_cast<const bf16x8 *>(p);
}
__device__ __forceinline__ void load_frag8(Frag<float> &f, const float *p) {
    const floatx4 a = reinterpret_cast<const floatx4 *>(p)[0];
    const floatx4 b = reinterpret_cast<const floatx4 *>(p)[1];
    f.v[0] = a[0]; f.v[1] = a[1]; f.v[2] = a[2]; f.v[3] = a[3];
    f.v[4] = b[0]; f.v[5] = b[1]; f.v[6] = b[2]; f.v[7] = b[3];
}

// MFMA operand type held in LDS for input dtype T.
template <typename T> struct LdsT;
template <> struct LdsT<bf16_t> { using type = __bf16; };
template <> struct LdsT<float> { using type = float; };

__device__ __forceinline__ __bf16 to_lds(float v, __bf16 *) { return static_cast<__bf16>(v); }
__device__ __forceinline__ float to_lds(float v, float *) { return v; }

// 16-byte global load of 8 bf16 or 2x16 bytes of 8 floats, as floats.
__device__ __forceinline__ void load8(const bf16_t *p, float out[8]) {
    const uint4 u = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        out[2 * i] = __uint_as_float(w[i] << 16);
        out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void load8(const float *p, float out[8]) {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    const float4 b = *reinterpret_cast<const float4 *>(p + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

// Eight input elements as loaded from memory, still packed (bf16: one 16-byte
// load, 4 registers; float: two 16-byte loads, 8 registers).
template <typename T> struct Raw8;
template <> struct Raw8<bf16_t> {
    uint4 u;
    __device__ __forceinline__ void load(const bf16_t *p) { u = *reinterpret_cast<const uint4 *>(p); }
    __device__ __forceinline__ void zero() { u = make_uint4(0, 0, 0, 0); }
    __device__ __forceinline__ float get(int e) const {
        const uint32_t w = e < 2 ? u.x : e < 4 ? u.y : e < 6 ? u.z : u.w;
        return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    }
};
template <> struct Raw8<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float *p) {
        a = reinterpret_cast<const float4 *>(p)[0];
        b = reinterpret_cast<const float4 *>(p)[1];
    }
    __device__ __forceinline__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
    __device__ __forceinline__ float get(int e) const {
        const float4 &q = e < 4 ? a : b;
        const int k = e & 3;
        return k == 0 ? q.x : k == 1 ? q.y : k == 2 ? q.z : q.w;
    }
};

// 16-byte non-temporal store: for outputs nothing on the GPU reads again soon
// (the chunk scan's y), so that they do not displace inputs other workgroups
// are about to read from the caches.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_nt16(void *p, const uint4 &v) {
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4 *>(p));
}

// Copy 16 bytes.
__device__ __forceinline__ void copy16(void *dst, const void *src) {
    *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(src);
}

__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// ---- operand fragments whose contraction index is the ROW of an LDS matrix
//
// For a row-major LDS matrix M (row stride `stride` elements), lane 16*g + c
// receives column cb + c at rows r1 + 0..3 (elements 0..3) and r2 + 0..3
// (elements 4..7), where r1 and r2 are the values of the lane's own group g.
// bf16 uses the gfx950 transposing LDS read ds_read_b64_tr_b16: within each
// 16-lane group, lane j's element e comes from element j%4 of the 8 bytes
// read by lane 4e + j/4, so lane s of a group reads row r + s/4 at columns
// cb + 4*(s%4) .. +3. float reads the eight values one by one.
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

__device__ __forceinline__ void lds_colfrag(Frag<bf16_t> &f, const __bf16 *m, int stride, int r1,
                                            int r2, int cb) {
    const int s = lane_id() & 15;
    const int off = (s >> 2) * stride + cb + 4 * (s & 3);
    const shortx4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_shortx4 *)(m + r1 * stride + off));
    const shortx4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_shortx4 *)(m + r2 * stride + off));
    const bf16x4 ab = __builtin_bit_cast(bf16x4, a);
    const bf16x4 bb = __builtin_bit_cast(bf16x4, b);
    f.v = bf16x8{ab[0], ab[1], ab[2], ab[3], bb[0], bb[1], bb[2], bb[3]};
}
__device__ __forceinline__ void lds_colfrag(Frag<float> &f, const float *m, int stride, int r1,
                                            int r2, int cb) {
    const int c = lane_id() & 15;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f.v[e] = m[(r1 + e) * stride + cb + c];
        f.v[4 + e] = m[(r2 + e) * stride + cb + c];
    }
}

// LDS row stride (in elements of `bytes` each) for a matrix with `cols`
// columns read through lds_colfrag: the stride in 4-byte words is the
// smallest value >= the row length that is 8 mod 16, which spreads the 8
// rows one half-wavefront reads over distinct banks.
__host__ __device__ constexpr int colfrag_stride(int cols, int bytes) {
    int w = (cols * bytes + 3) / 4;
    while (w % 16 != 8) ++w;
    return w * 4 / bytes;
}

// ---- direct global-to-LDS loads and LDS-only barriers ------------------------
//
typedef __attribute__((address_space(3))) void lds_void;

// The LDS byte address of a generic pointer into LDS: the low 32 bits of its
// flat address (what the address-space cast yields for a non-null pointer,
// without the cast's null test, which the backend cannot always encode for a
// pointer at LDS offset 0), made wave-uniform.
__device__ __forceinline__ uint32_t lds_addr32(const void *p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}

// One 16-byte-per-lane global-to-LDS load: lane l's 16 bytes from `src` land
// at byte lds_base + 16*l (lds_base is the same for the whole wavefront). In
// inline assembly so that the compiler does not hold later reads of other LDS
// buffers behind it; completion is awaited explicitly (wait_barrier).
__device__ __forceinline__ void dma16(const void *src, const void *lds_base) {
    const uint32_t a = lds_addr32(lds_base);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(a)
                 : "memory", "m0");
}

// This wavefront's LDS operations complete and at most VM of its global
// memory operations (the most recently issued ones) remain outstanding; then
// the workgroup meets.
template <int VM>
__device__ __forceinline__ void wait_barrier() {
    static_assert(VM >= 0 && VM < 64, "vmcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4));  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
// LDS operations complete, global ones stay in flight; then the workgroup meets.
__device__ __forceinline__ void barrier_lds() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0) only
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// A 64-column bf16 matrix in LDS (a token tile of x: eight 16-byte pieces per
// 128-byte row); piece q of row r is stored at piece q ^ (r & 7). A half-wavefront's transposing read covers 8
// consecutive rows x 2 pieces, which this puts on 16 distinct bank groups.
__device__ __forceinline__ int x_at(int r, int col) {
    return r * 64 + ((((col >> 3) ^ r) & 7) << 3) + (col & 7);
}

// Piece swizzle of a bf16 LDS matrix with PPR 16-byte pieces per row that is
// read with the transposing read (lds_colfrag's pattern: a half-wavefront
// reads 8 consecutive rows x 2 adjacent pieces): the XOR mask for row r that
// puts those 16 pieces on distinct banks.
template <int PPR>
__device__ __forceinline__ int tr_swz(int r) {
    if constexpr (PPR <= 2) return 0;
    else if constexpr (PPR == 4) return ((r >> 2) & 1) << 1;
    else if constexpr (PPR == 8) return r & 7;
    else return (r & 7) << 1;
}

// Transposing read of a bf16 LDS matrix of PPR 16-byte pieces per row stored
// with the tr_swz<PPR> piece swizzle: lds_colfrag's result (column cb + c at
// rows r1 + 0..3 and r2 + 0..3 for lane 16*g + c).
template <int PPR>
__device__ __forceinline__ void colfrag_swz(Frag<bf16_t> &f, const __bf16 *m, int r1, int r2,
                                            int cb) {
    const int s = lane_id() & 15;
    const int col = cb + 4 * (s & 3);
    const int ra = r1 + (s >> 2), rb = r2 + (s >> 2);
    const int pa = ((col >> 3) ^ tr_swz<PPR>(ra)) << 3, pb = ((col >> 3) ^ tr_swz<PPR>(rb)) << 3;
    const shortx4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_shortx4 *)(m + ra * (PPR * 8) + pa + (col & 7)));
    const shortx4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_shortx4 *)(m + rb * (PPR * 8) + pb + (col & 7)));
    const bf16x4 ab = __builtin_bit_cast(bf16x4, a);
    const bf16x4 bb = __builtin_bit_cast(bf16x4, b);
    f.v = bf16x8{ab[0], ab[1], ab[2], ab[3], bb[0], bb[1], bb[2], bb[3]};
}

// Transposing reads of the swizzled x tile. Lane 16*g + s of a fragment for
// head-dim columns 16*pt + 0..15 reads row 32*jp + 4*g + s/4 (+16 for the
// second half) at column 16*pt + 4*(s%4); since 32*jp and 16 are multiples of
// 8, the swizzle term r & 7 = (4*g + s/4) & 7 is the same for every slice, and
// the element offset splits into a per-lane part, 16 * (pt ^ zt) with a
// per-lane zt, and compile-time multiples of 2048 (jp) and 1024 (second half).
__device__ __forceinline__ void x_colfrag_offsets(int (&xo)[4], int l) {
    const int s = l & 15, g = l >> 4;
    const int r = 4 * g + (s >> 2);
    const int z = r & 7;
    const int base = r * 64 + 8 * (((s >> 1) & 1) ^ (z & 1)) + 4 * (s & 1);
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) xo[pt] = base + 16 * (pt ^ (z >> 1));
}

// x^T operand fragment: lane 16*g + c receives x[32*jp + 4*g + 0..3][16*pt + c]
// (elements 0..3) and x[32*jp + 16 + 4*g + 0..3][16*pt + c] (elements 4..7).
template <int JP>
__device__ __forceinline__ void x_colfrag(Frag<bf16_t> &f, const __bf16 *xs, int xo) {
    const shortx4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(xs + xo + JP * 2048));
    const shortx4 b =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(xs + xo + JP * 2048 + 1024));
    const bf16x4 ab = __builtin_bit_cast(bf16x4, a);
    const bf16x4 bb = __builtin_bit_cast(bf16x4, b);
    f.v = bf16x8{ab[0], ab[1], ab[2], ab[3], bb[0], bb[1], bb[2], bb[3]};
}

}  // namespace ssd
