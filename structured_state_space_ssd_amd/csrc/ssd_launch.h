// Host-side launchers of the SSD kernels (one per kernel source file). They
// assume arguments were validated by the C-ABI layer (ssd_api.hip) and return
// the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace ssd {

// Step-size preprocessing and input discretisation, passed to the kernels by
// value. The selection mechanism makes the step size a projection of the
// input made positive by softplus ("从Transformer到Mamba" tutorial, section
// 3.2): `bias` is that projection's per-head constant term, added first; an
// optional clamp to [lo, hi] follows softplus (the tutorial's section 8.2
// adjusts the range step sizes are produced in). The input term is weighted by
// the step size (Euler) or, with `zoh`, by the zero-order hold's
// (exp(dt A) - 1) / A (tutorial section 2.2; "Mamba 模型" section 2.3.1).
struct DtOpts {
    const float *bias;  // [H], or nullptr
    float lo, hi;       // clamp bounds, read when clamp != 0
    int softplus, clamp, zoh;
};

// delta (nullable): each token's input weight (the preprocessed step size, or
// its zero-order-hold weight) as float32 in dA_cumsum's chunk-padded layout,
// zero past the end. The later stages read it in place of dt.
hipError_t launch_chunk_cumsum(const void *dt, const float *A, int batch, int seqlen, int nheads,
                               int chunk, bool bf16, const DtOpts &opts, float *dA_cumsum,
                               float *delta, hipStream_t stream);

// seg (nullable): packed sequences, one int per token in dA_cumsum's chunk-padded
// layout: the first token of the token's sequence relative to its chunk's first
// token, or -1 if that sequence began in an earlier chunk (launch_varlen_seg).
// dout (backward): the same contraction with token weights exp(s_j) instead of
// exp(s_end - s_j) delta_j, i.e. sum_j exp(s_j) x_j B_j^T with x := dy and
// B := C: how a chunk's outputs depend on the state entering it (delta unused).
hipError_t launch_chunk_state(const void *x, const void *B, const float *delta,
                              const float *dA_cumsum, const int *seg,
                              int batch, int seqlen, int nheads, int ngroups, int dstate, int chunk,
                              bool bf16, float *states, hipStream_t stream, bool dout = false);

// The single-pass bf16 forward (fwd_onepass.hip): whether it applies; how
// it cuts each sequence; and the launch (two kernels when there are several
// segments: the segment states, then the forward proper; `between`
// (nullable) is recorded between them).
bool forward_onepass_ok(int batch, int nheads, int dstate, bool bf16, const void *dt);
// S segments of per_seg 64-token blocks each (the last may hold fewer); when
// S > 1 the first S - 1 segments are cut into k pieces of psub blocks, whose
// states (float32 [Bt][H][(S-1)k][P][N]) and log2-decays (float32
// [Bt][H][(S-1)k]) take scratch_bytes of scratch. S == 1: k == 0, no scratch.
struct OnepassPlan {
    int S, k, per_seg, psub;
    size_t scratch_bytes;
};
// cap: the most scratch the plan may take (SIZE_MAX: no limit); a smaller cap
// lowers k, then gives up the segments.
OnepassPlan forward_onepass_plan(int batch, int seqlen, int nheads, int dstate, size_t cap);
// Packed sequences (batch 1, no init_state / final_state): `varlen_meta`
// holds one int4 per token made by launch_onepass_varlen_prep from cu_seqlens
// (16 * seqlen bytes, 16-byte aligned); each sequence's final state goes to
// seq_states (nullable) [nseq][H][P][N]; the prep also zeroes the empty ones.
// `scratch` must hold pl.scratch_bytes (it may be NULL when that is 0).
hipError_t launch_forward_onepass(const void *x, const void *dt, const float *A, const void *B,
                                  const void *C, const float *D, const float *init,
                                  const DtOpts &opts, int batch, int seqlen, int nheads,
                                  int ngroups, int dstate, const OnepassPlan &pl, float *scratch,
                                  void *y, float *final_state, hipEvent_t between,
                                  hipStream_t stream, const void *varlen_meta = nullptr,
                                  float *seq_states = nullptr);
hipError_t launch_onepass_varlen_prep(const int *cu_seqlens, int nseq, int seqlen, int nheads,
                                      int dstate, void *meta, float *seq_states,
                                      hipStream_t stream);

// Stages 2 and 3 in one kernel (bf16 only; used when state_passing_fused()):
// writes chunk_init (bf16) and final_state (nullable) directly, without the
// per-chunk float32 states. Reads dA_cumsum and delta (stage 1's outputs).
bool state_passing_fused(int batch, int nheads, bool bf16);
// reverse (backward): the adjoint pass (x = dy, B = C, init = dfinal; chunk_init
// receives the gradient of the state leaving each chunk, final_state G_0).
hipError_t launch_chunk_state_passing(const void *x, const void *B, const float *dA_cumsum,
                                      const float *delta, const float *init, int batch,
                                      int seqlen, int nheads, int ngroups, int dstate, int chunk,
                                      void *chunk_init, float *final_state, hipStream_t stream,
                                      bool reverse = false);

// chunk_init is written in the MFMA operand type of the forward's dtype
// (bf16 when bf16 is true, else float32). reverse (backward): the adjoint pass,
// from init = dfinal over the chunks in reverse (see state_passing.hip).
hipError_t launch_state_passing(const float *states, const float *dA_cumsum, const float *init,
                                const int *seg, int batch, int seqlen, int nheads, int dstate, int chunk,
                                bool bf16, void *chunk_init, float *final_state,
                                hipStream_t stream, bool reverse = false);

size_t chunk_cb_bytes(int batch, int seqlen, int ngroups, int chunk, bool bf16);

hipError_t launch_chunk_cb(const void *B, const void *C, int batch, int seqlen, int ngroups,
                           int dstate, int chunk, bool bf16, void *cb, hipStream_t stream);

// The bf16 path forms C B^T itself (reads B, ignores cb); the float path reads
// the C B^T tiles of launch_chunk_cb (reads cb, ignores B).
bool chunk_scan_reads_cb(bool bf16);

hipError_t launch_chunk_scan(const void *x, const float *delta, const float *dA_cumsum, const void *B,
                             const void *C, const void *cb, const float *D, const void *chunk_init,
                             const int *seg, int batch, int seqlen, int nheads, int ngroups, int dstate, int chunk,
                             bool bf16, void *y, hipStream_t stream);

// Packed sequences (batch 1): seg of every token position (nC*Q ints) from
// cu_seqlens [nseq + 1]; and each sequence's state after its last token,
// seq_states [nseq][H][P][N] float32, from the stage outputs (chunk_init in the
// operand type of the forward's dtype).
hipError_t launch_varlen_seg(const int *cu_seqlens, int nseq, int seqlen, int chunk, int *seg,
                             hipStream_t stream);
hipError_t launch_varlen_final_states(const void *x, const void *B, const float *delta,
                                      const float *dA_cumsum, const int *cu_seqlens,
                                      const int *seg, const void *chunk_init, int nseq,
                                      int seqlen, int nheads, int ngroups, int dstate, int chunk,
                                      bool bf16, float *seq_states, hipStream_t stream);

// ---- backward (chunk_bwd.hip)
// Chunk length the backward runs with (0: unsupported) and its head blocks.
int bwd_chunk(int dstate, bool bf16);
int bwd_head_blocks(int batch, int seqlen, int nheads, int ngroups, int chunk);

struct BwdArgs {
    const void *x, *dy, *B, *C;
    const float *dA_cumsum, *delta, *D;
    const void *chunk_init, *grad_next;  // operand type: H_c and the adjoint G_{c+1}
    int batch, seqlen, nheads, ngroups, dstate, chunk, nblk;
    bool bf16;
    void *dx;
    float *ds, *dw;                 // [Bt][H][nC*Q]
    float *dB_part, *dC_part;       // [nblk][Bt][L][G][N]
    float *dD_part;                 // [Bt][nC][H]
};
hipError_t launch_chunk_bwd(const BwdArgs &a, hipStream_t stream);
// out0, out1 (input dtype, count elements each, count a multiple of 4) = the
// sums over nblk of part0[k][count], part1[k][count], in one launch
hipError_t launch_bwd_reduce(const float *part0, const float *part1, int nblk, size_t count,
                             bool bf16, void *out0, void *out1, hipStream_t stream);
hipError_t launch_bwd_dt(const void *dt, const float *A, const float *ds, const float *dw,
                         int batch, int seqlen, int nheads, int chunk, bool bf16,
                         const DtOpts &opts, void *ddt, float *dA_part, float *dbias_part,
                         hipStream_t stream);
// out[j][h] = sum_i part[j][i][h], i < nbc, for the j < n (at most 3) whose out[j] is
// not NULL, in one launch
hipError_t launch_bwd_head_sum(const float *const *part, float *const *out, int n, int nbc,
                               int nheads, hipStream_t stream);

// State-size padding (pad.hip): the N the kernels run with for dstate (the
// smallest of 16, 32, 64, 128, 256 not below it; 0 above 256), and a copy of
// `rows` rows of src_cols elements into rows of dst_cols elements, zero-filled
// past src_cols or cut to dst_cols (both column counts times elem_bytes must
// be multiples of 16; src and dst 16-byte aligned).
int kernel_dstate(int dstate);
hipError_t launch_pad_rows(const void *src, void *dst, size_t rows, int src_cols, int dst_cols,
                           int elem_bytes, hipStream_t stream);

// dstate: any multiple of 16 up to 256 (the kernel for 16, 32, 64, 128, 256
// keeps the state's rows in lanes that share them by powers of two; the other
// sizes reduce each row's products through LDS).
hipError_t launch_decode_step(float *state, const void *x, const void *dt, const float *A,
                              const void *B, const void *C, const float *D, int batch, int nheads,
                              int ngroups, int dstate, bool bf16, const DtOpts &opts, void *y,
                              hipStream_t stream);

}  // namespace ssd
