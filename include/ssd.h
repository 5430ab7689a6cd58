/*
 * ssd.h - C ABI of the MI355X (gfx950) SSD layer library (libssd.so).
 *
 * The layer is the per-head selective state-space model of Mamba-2:
 *
 *   h_t = exp(dt_t * A_h) * h_{t-1} + w_t * x_t B_t^T       state, P x N per head
 *   y_t = h_t C_t + D_h * x_t                               output after the update
 *
 * ("从Transformer到Mamba" tutorial, sections 2.1-2.2: discrete recurrence and
 * feed-through D; "深挖-Mamba", core concept 3: dt, B, C depend on the token.)
 * The input weight w_t is dt_t (Euler, the default) or, with the zero-order
 * hold option, (exp(dt_t A_h) - 1) / A_h. dt_t is the caller's dt, optionally
 * preprocessed first (bias, softplus, clamp; see ssd_options).
 * The forward pass computes it with the block decomposition of the
 * semiseparable matrix ("Mamba 模型", section 4.1 and "Draft:Mamba2", SSD
 * section): diagonal blocks (chunks of Q tokens) as masked matrix products,
 * off-diagonal blocks through the hidden state carried from chunk to chunk.
 * The decode step is the recurrence for a single token (linear mode of the
 * "Mamba-2架构深度解析" page, section 2.2 table).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor argument is a DEVICE pointer to dense row-major memory, last
 *   dimension contiguous, owned by the caller. The library never allocates;
 *   scratch memory for the forward pass is the caller's workspace.
 * - Layouts (Bt batch, L seqlen, H heads, P headdim, G groups, N dstate,
 *   Q chunk, nC = ceil(L / Q)):
 *     x, y          [Bt][L][H][P]        dtype
 *     dt            [Bt][L][H]           dtype (positive, unless ssd_options applies softplus)
 *     B, C          [Bt][L][G][N]        dtype; head h reads group h / (H / G)
 *     A, D          [H]                  float32 (A < 0 for a decaying state)
 *     states        [Bt][H][P][N]        float32 (init / final / decode state)
 *   Decode (ssd_step) drops the L dimension: x, y [Bt][H][P], dt [Bt][H],
 *   B, C [Bt][G][N].
 * - dtype is SSD_F32 (all of x, dt, B, C, y float32) or SSD_BF16 (all bf16);
 *   A, D and every state are float32. Products run on MFMA in the input
 *   dtype with float32 accumulation.
 * - Supported set: headdim == 64; dstate any multiple of 16 from 16 to 256
 *   (ssd_forward*, ssd_backward*, ssd_step*; the kernels are built for 16, 32,
 *   64, 128 and 256, and the forward and backward run other sizes
 *   zero-padded to the next of these, which changes nothing but the work: the
 *   padded columns of B, C and the states are zeros and add exact zeros to
 *   every sum over the state dimension; the workspace then also holds the
 *   padded copies); the separate stage entry points and ssd_forward_varlen
 *   take dstate in {16, 32, 64, 128, 256} only; chunk in {64, 128, 256}; any
 *   seqlen >= 1 (the last chunk may be short); nheads % ngroups == 0.
 *   Anything else returns SSD_ERR_UNSUPPORTED.
 * - stream is a hipStream_t (NULL: the null stream). Calls only enqueue work
 *   and return before it finishes; no host synchronisation happens inside.
 * - Arguments are checked before anything is enqueued; a failed check returns
 *   a negative status and enqueues nothing. A launch failure returns
 *   SSD_ERR_HIP. NaN / Inf inputs are not checked and propagate.
 * - There is no global mutable state: concurrent calls on different streams
 *   are safe as long as they use different workspaces and outputs.
 */
#ifndef SSD_H
#define SSD_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;

typedef enum {
    SSD_OK = 0,
    SSD_ERR_NULL = -1,        /* a required pointer is NULL                        */
    SSD_ERR_SHAPE = -2,       /* a size is non-positive or nheads % ngroups != 0   */
    SSD_ERR_UNSUPPORTED = -3, /* outside the supported set above                   */
    SSD_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required        */
    SSD_ERR_HIP = -5,         /* the HIP runtime reported an error at launch       */
    SSD_ERR_OPTION = -6,      /* an ssd_options field holds an invalid value       */
    SSD_ERR_TOO_LARGE = -7    /* ssd_forward_static: needs more than its fixed scratch */
} ssd_status;

/* Discretisation of the input term. */
typedef enum {
    SSD_DISC_EULER = 0, /* w_t = dt_t: the Mamba-2 layer's form                       */
    SSD_DISC_ZOH = 1    /* w_t = (exp(dt_t A) - 1) / A (dt_t at A = 0): zero-order hold,
                           "从Transformer到Mamba" tutorial section 2.2 and
                           "Mamba 模型" section 2.3.1, for a scalar A                   */
} ssd_discretization;

/*
 * Step-size preprocessing and discretisation (a host struct, passed by
 * pointer; a NULL pointer means every field off / SSD_DISC_EULER). The
 * selection mechanism of the "从Transformer到Mamba" tutorial (section 3.2)
 * produces the step size by a linear projection of the input and softplus;
 * the library takes the projection's output as dt and applies, per token, in
 * this order:
 *   dt <- dt + dt_bias[h]                    if dt_bias != NULL (the projection's
 *                                            per-head constant term)
 *   dt <- log(1 + exp(dt))                   if dt_softplus
 *   dt <- min(max(dt, dt_min), dt_max)       if dt_clamp (the step-size range the
 *                                            tutorial's section 8.2 adjusts)
 * in float32. The decay uses the result; the input term uses it (Euler) or its
 * zero-order-hold weight (SSD_DISC_ZOH).
 *   dt_bias         DEVICE pointer, float32 [H], 4-byte aligned, or NULL.
 *   dt_min, dt_max  read only when dt_clamp; need dt_min <= dt_max (infinite
 *                   bounds allowed), else SSD_ERR_OPTION.
 *   discretization  an ssd_discretization, else SSD_ERR_OPTION.
 */
typedef struct {
    const float *dt_bias;
    int dt_softplus;
    int dt_clamp;
    float dt_min, dt_max;
    int discretization;
} ssd_options;

/* Human-readable text for a status code (static storage; never NULL). */
const char *ssd_strerror(int status);

/*
 * How ssd_forward runs for given sizes and dt pointer (ssd_forward_plan_info).
 *   path            SSD_PATH_SINGLE_PASS: the single-pass kernel (SSD_BF16, dstate
 *                   64, 128 or 256, nheads a multiple of 8, 16-byte aligned dt);
 *                   SSD_PATH_STAGES: the stage kernels listed under ssd_forward.
 *   segments        S >= 1 segments per sequence on the single-pass kernel; 0 on
 *                   the stage kernels.
 *   pieces          K: pieces per segment of the first S-1 segments (0 when S == 1).
 *   block_tokens    tokens per block: 64 on the single-pass kernel (whatever
 *                   `chunk` says), the chunk length on the stage kernels.
 *   segment_blocks  blocks per segment (the last segment may hold fewer).
 *   piece_blocks    blocks per piece (0 when S == 1).
 *   workspace_bytes workspace ssd_forward needs for exactly these arguments.
 */
typedef enum { SSD_PATH_STAGES = 0, SSD_PATH_SINGLE_PASS = 1 } ssd_path;
typedef struct {
    int path, segments, pieces, block_tokens, segment_blocks, piece_blocks;
    int kernel_dstate; /* the state size the kernels run with (dstate, or the next of
                          16, 32, 64, 128, 256 when dstate is zero-padded)          */
    size_t workspace_bytes;
} ssd_plan;

/*
 * Fills *out with the plan of ssd_forward (and ssd_forward_ex / _timed) for
 * these sizes and this dt pointer (only its alignment is looked at; it is not
 * read). Returns SSD_OK, SSD_ERR_NULL for a NULL `out`, or the status
 * ssd_forward would return for these sizes (then *out is zeroed).
 *
 * Workspace layout. On the single-pass path it is the segment scratch only,
 * and only when S > 1: float32 [Bt][H][(S-1)K][P][N], the state each piece of
 * the first S-1 segments produces from a zero state, then float32
 * [Bt][H][(S-1)K], each piece's total log2-decay (sum of dt*A over the piece,
 * times log2(e)); when (S-1)K > 4 a chain pass then overwrites the slot of
 * the last piece of each segment s-1 with the state entering segment s (the
 * initial state carried through every earlier piece). With S == 1 no
 * workspace is needed
 * (NULL is accepted). On
 * the stage path it holds, at 256-byte aligned offsets in this order (with
 * N = kernel_dstate):
 *   dA_cumsum   float32 [Bt][H][nC*Q]      within-chunk prefix sums of dt*A
 *   delta       float32 [Bt][H][nC*Q]      each token's input weight w_t, same layout
 *                                          (zero past seqlen)
 *   states      float32 [Bt][nC][H][P][N]  each chunk's own state contribution
 *   chunk_init  [Bt][nC][H][P][N]          state entering each chunk, in the MFMA
 *                                          operand type (bf16 for SSD_BF16, else float32)
 *   cb          SSD_F32 only: ssd_chunk_cb_size(...) bytes, C B^T tiles of every
 *               chunk (the SSD_BF16 chunk scan forms them itself; no space)
 * After a stage-path forward these hold the intermediate results of the
 * stages (a caller may read them, e.g. to test a stage), except that for
 * SSD_BF16 with batch * nheads >= 512 stages 2 and 3 run as one kernel that
 * keeps the per-chunk states on chip (`states` is then not written).
 * When kernel_dstate != dstate, the kernels' part above is followed (at a
 * 256-byte aligned offset) by the zero-padded copies of B and C
 * ([Bt][L][G][kernel_dstate] in dtype) and of the initial and final states
 * ([Bt][H][P][kernel_dstate] float32), each 256-byte aligned.
 */
int ssd_forward_plan_info(int batch, int seqlen, int nheads, int headdim, int ngroups,
                          int dstate, int chunk, int dtype, const void *dt, ssd_plan *out);

/*
 * Bytes of workspace ssd_forward needs for these sizes with a 16-byte aligned
 * dt (0 for invalid sizes, and 0 where the forward needs none). An unaligned
 * dt makes the forward take the stage kernels, whose larger need
 * ssd_forward_plan_info reports for that pointer.
 */
size_t ssd_forward_workspace_size(int batch, int seqlen, int nheads, int headdim,
                                  int ngroups, int dstate, int chunk, int dtype);

/*
 * Full SSD layer forward: enqueues ssd_chunk_cumsum, ssd_chunk_state,
 * ssd_state_passing, ssd_chunk_cb (SSD_F32 only) and ssd_chunk_scan on
 * `stream`. For SSD_BF16 with dstate 64, 128 or 256, nheads a multiple of 8 and
 * a 16-byte aligned dt, it enqueues instead one single-pass kernel that
 * computes the same result (up to rounding): one workgroup per (batch, head)
 * walks the sequence in blocks of 64 tokens, carrying the state from block to
 * block in registers (the chunk-to-chunk recurrence of the "Mamba 模型" page,
 * section 4.1, run within the workgroup), so x is read from memory once.
 * With too few (batch, head) pairs to fill the GPU, each sequence is cut into
 * S segments of whole blocks (ssd_forward_plan gives S): a first kernel
 * computes the state that each piece of the first S-1 segments produces from
 * a zero state, and the single-pass kernel then runs one workgroup per
 * (batch, head, segment), each starting from the state the pieces before it
 * pass on (the same recurrence at piece granularity). `chunk` must still be valid but does
 * not set that kernel's block length. ssd_forward_plan_info reports the path,
 * the cut and the workspace.
 *   D           nullable: no feed-through term.
 *   init_state  nullable: the state before token 0 is zero.
 *   y           output, [Bt][L][H][P] in dtype.
 *   final_state nullable: if given, receives the state after token L-1.
 *   workspace   at least ssd_plan.workspace_bytes for these arguments (for an
 *               aligned dt: ssd_forward_workspace_size(...)), 256-byte aligned;
 *               NULL when that is 0. Too small: SSD_ERR_WORKSPACE.
 */
int ssd_forward(const void *x, const void *dt, const float *A, const void *B,
                const void *C, const float *D, int batch, int seqlen, int nheads,
                int headdim, int ngroups, int dstate, int chunk, int dtype,
                const float *init_state, void *y, float *final_state,
                void *workspace, size_t workspace_bytes, void *stream);

/*
 * ssd_forward_ex for callers that cannot allocate memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): no
 * workspace argument and no events. Its scratch is one device array of
 * SSD_STATIC_SCRATCH_BYTES (32 MiB) that the library holds on every GPU it
 * runs on until the process ends; this call allocates nothing. It uses the
 * array of the current device (hipGetDevice); `stream` must belong to it.
 * The plan is ssd_forward_ex's with the segment scratch capped at the
 * array's size; arguments whose forward needs more (ssd_plan.workspace_bytes,
 * e.g. a large shape on the stage kernels) return SSD_ERR_TOO_LARGE and
 * enqueue nothing. Every call on one GPU shares that GPU's array, which keeps
 * the last call's contents (nothing in it must start at zero: each kernel
 * writes what a later one reads): calls that overlap on one GPU (on
 * different streams or from different host threads) race and give wrong
 * results.
 */
#define SSD_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
int ssd_forward_static(const void *x, const void *dt, const float *A, const void *B,
                       const void *C, const float *D, int batch, int seqlen, int nheads,
                       int headdim, int ngroups, int dstate, int chunk, int dtype,
                       const float *init_state, void *y, float *final_state,
                       const ssd_options *opts, void *stream);

/*
 * Which path ssd_forward takes for these sizes and this dt pointer (only its
 * alignment is looked at; it is not read): the number S >= 1 of segments per
 * sequence when it runs the single-pass kernel, 0 when it runs the stage
 * kernels, or a negative ssd_status for sizes ssd_forward rejects. The same
 * for ssd_forward_ex and ssd_forward_timed.
 */
int ssd_forward_plan(int batch, int seqlen, int nheads, int headdim, int ngroups,
                     int dstate, int chunk, int dtype, const void *dt);

/*
 * ssd_forward with options: `opts` (nullable, see ssd_options) preprocesses dt
 * and chooses the discretisation; `events` are the timing hooks of
 * ssd_forward_timed (nullable). ssd_forward is this call with opts = NULL and
 * events = NULL.
 */
int ssd_forward_ex(const void *x, const void *dt, const float *A, const void *B,
                   const void *C, const float *D, int batch, int seqlen, int nheads,
                   int headdim, int ngroups, int dstate, int chunk, int dtype,
                   const float *init_state, void *y, float *final_state,
                   void *workspace, size_t workspace_bytes, const ssd_options *opts,
                   void *stream, void *const *events);

/*
 * ssd_forward with per-stage timing hooks for profilers and benchmarks.
 * `events` is NULL (then this is exactly ssd_forward) or an array of 6
 * hipEvent_t owned by the caller, any of which may be NULL (not recorded):
 * events[k] is recorded on `stream` right before stage k+1 is enqueued and
 * events[5] after the last stage, so the
 * elapsed time between consecutive events is each stage's GPU time (stages in
 * the order listed for ssd_forward; for SSD_BF16 the ssd_chunk_cb interval is
 * empty, that work being part of ssd_chunk_scan). When the forward runs as the
 * single-pass kernel (see ssd_forward), events[0] is recorded before it and
 * events[1..5] after it: its time is the first interval; with S > 1 segments,
 * events[0] before the segment-state kernel, events[1] between the two
 * kernels and events[2..5] after the single-pass kernel.
 */
int ssd_forward_timed(const void *x, const void *dt, const float *A, const void *B,
                      const void *C, const float *D, int batch, int seqlen, int nheads,
                      int headdim, int ngroups, int dstate, int chunk, int dtype,
                      const float *init_state, void *y, float *final_state,
                      void *workspace, size_t workspace_bytes, void *stream,
                      void *const *events);

/*
 * Backward pass: the gradients of
 *   loss = sum(dy * y) + sum(dfinal_state * final_state)
 * for ssd_forward_ex with the same inputs and options. The adjoint of the
 * state runs backward in time, g_t = dy_t C_t^T + a_{t+1} g_{t+1}, chunked like
 * the forward: the forward's per-chunk states are recomputed (not stored), a
 * reverse pass over the chunks carries the adjoint, and one kernel per
 * (batch, chunk, group, block of heads) forms every gradient of the chunk on
 * MFMA. The pages motivate the layer by its training speed ("Mamba-2架构深度解析"
 * section 1) and recompute states in the backward pass instead of storing
 * them (the "从Transformer到Mamba" tutorial section 4.2; "Mamba 模型" section 3.4).
 *   dy           [Bt][L][H][P] in dtype (x's layout).
 *   dfinal_state nullable, float32 [Bt][H][P][N]: the final state's gradient.
 *   init_state   nullable, as for ssd_forward.
 * Outputs (overwritten):
 *   dx [Bt][L][H][P], ddt [Bt][L][H] (with respect to the raw dt, through the
 *   options), dB, dC [Bt][L][G][N] (summed over the heads of each group): dtype.
 *   dA [H] float32. dD [H] float32 (nullable; sum of dy.x whether or not D is
 *   given). dinit_state [Bt][H][P][N] float32 (nullable). ddt_bias [H] float32
 *   (nullable; the gradient of opts->dt_bias, which is the sum of ddt per head).
 * The backward picks its own chunk length for the state size (its LDS holds
 * a chunk's x, dy, B, C and two states): 256 tokens for N <= 32, 128 for N 64
 * and 128, 64 for N 256 (bf16); float32 supports N <= 64 only (else
 * SSD_ERR_UNSUPPORTED). The result does not depend on it beyond rounding.
 * Clamp bounds pass the gradient (d clamp / d dt = 1 for dt_min <= dt <= dt_max).
 * workspace: at least ssd_backward_workspace_size(...) bytes, 256-byte aligned.
 * x, dy, B, C, dx, dB, dC and the state arguments need 16-byte alignment.
 */
size_t ssd_backward_workspace_size(int batch, int seqlen, int nheads, int headdim, int ngroups,
                                   int dstate, int dtype);
/*
 * ssd_backward with timing hooks: `events` is NULL (then this is exactly
 * ssd_backward) or an array of 5 hipEvent_t owned by the caller, any of which
 * may be NULL (not recorded), recorded on `stream`: [0] before the forward
 * recompute (prefix sums, weights, the state entering each chunk), [1] before
 * the adjoint pass over the chunks, [2] before the chunk-gradient kernel,
 * [3] after it, [4] after the last kernel (the dB / dC sums and the dt, A,
 * bias stage).
 */
int ssd_backward_timed(const void *x, const void *dt, const float *A, const void *B,
                       const void *C, const float *D, const float *init_state, const void *dy,
                       const float *dfinal_state, int batch, int seqlen, int nheads, int headdim,
                       int ngroups, int dstate, int dtype, void *dx, void *ddt, float *dA,
                       void *dB, void *dC, float *dD, float *dinit_state, float *ddt_bias,
                       void *workspace, size_t workspace_bytes, const ssd_options *opts,
                       void *stream, void *const *events);
int ssd_backward(const void *x, const void *dt, const float *A, const void *B, const void *C,
                 const float *D, const float *init_state, const void *dy,
                 const float *dfinal_state, int batch, int seqlen, int nheads, int headdim,
                 int ngroups, int dstate, int dtype, void *dx, void *ddt, float *dA, void *dB,
                 void *dC, float *dD, float *dinit_state, float *ddt_bias, void *workspace,
                 size_t workspace_bytes, const ssd_options *opts, void *stream);

/*
 * Packed variable-length sequences (the dynamic packing of variable-length
 * sequences named on the "Mamba-2架构深度解析" page, section 5). The token
 * axis of a batch-1 input holds nseq sequences one after another: sequence k
 * is tokens cu_seqlens[k] .. cu_seqlens[k+1]-1. Each has its own recurrence
 * from the zero state; nothing flows from one sequence into the next.
 *   x, y        [L][H][P] (= [1][L][H][P]) in dtype; dt [L][H]; B, C [L][G][N].
 *   cu_seqlens  DEVICE int32 [nseq + 1], 4-byte aligned: cu_seqlens[0] = 0,
 *               non-decreasing, cu_seqlens[nseq] = seqlen (empty sequences
 *               allowed). The library does not read device memory on the host,
 *               so it cannot check these values: other contents give
 *               unspecified results, but every access stays in bounds.
 *   seq_states  nullable, float32 [nseq][H][P][N], 16-byte aligned: each
 *               sequence's state after its last token (zero if empty).
 *   opts        nullable, as for ssd_forward_ex.
 *   workspace   at least ssd_forward_varlen_workspace_size(...) bytes,
 *               256-byte aligned: ssd_forward's layout at batch 1, then one
 *               int32 per token position of the chunk-padded layout.
 * Where ssd_forward would run its single-pass kernel at batch 1
 * (ssd_forward_plan(1, ...) > 0: SSD_BF16, dstate 64, 128 or 256, nheads a
 * multiple of 8, 16-byte aligned dt) it runs that kernel with sequence masks
 * (over segments of the token axis, with the segment-state kernel first):
 * rows ignore the state of earlier sequences, the state restarts from zero
 * where a sequence begins, and each sequence's final state is taken at its
 * last token. The workspace then holds one int4 per token (first token of
 * its sequence, sequence index, last-token flag) where dA_cumsum would be,
 * and the segment scratch as for ssd_forward. Otherwise it enqueues the
 * separate stages (never the fused stage 2 + 3 kernel), each masking pairs of
 * tokens from different sequences, then one kernel for the per-sequence
 * states. nseq < 1 returns SSD_ERR_SHAPE.
 */
size_t ssd_forward_varlen_workspace_size(int seqlen, int nheads, int headdim, int ngroups,
                                         int dstate, int chunk, int dtype);
int ssd_forward_varlen(const void *x, const void *dt, const float *A, const void *B,
                       const void *C, const float *D, const int *cu_seqlens, int nseq,
                       int seqlen, int nheads, int headdim, int ngroups, int dstate, int chunk,
                       int dtype, void *y, float *seq_states, void *workspace,
                       size_t workspace_bytes, const ssd_options *opts, void *stream);

/*
 * One recurrent (decode) step for every (batch, head): updates `state`
 * [Bt][H][P][N] float32 in place,
 *   state <- exp(dt*A_h) * state + dt * x B^T,   y = state C + D_h x,
 * and writes y [Bt][H][P] in dtype. D is nullable. `state` and `y` must not
 * overlap the inputs.
 */
int ssd_step(float *state, const void *x, const void *dt, const float *A,
             const void *B, const void *C, const float *D, int batch, int nheads,
             int headdim, int ngroups, int dstate, int dtype, void *y, void *stream);

/*
 * ssd_step with options (nullable, see ssd_options): dt is preprocessed as in
 * ssd_forward_ex and the input term weighted by w = dt or, for SSD_DISC_ZOH,
 * (exp(dt A_h) - 1) / A_h:
 *   state <- exp(dt*A_h) * state + w * x B^T,   y = state C + D_h x.
 */
int ssd_step_ex(float *state, const void *x, const void *dt, const float *A,
                const void *B, const void *C, const float *D, int batch, int nheads,
                int headdim, int ngroups, int dstate, int dtype, void *y,
                const ssd_options *opts, void *stream);

/* ---- The forward pass stage by stage (what ssd_forward enqueues) ---------- */

/*
 * Stage 1: dA_cumsum[b][h][c*Q + k] = sum_{t=cQ..cQ+k} dt_t * A[h], with dt_t
 * the step size of token t after `opts`' preprocessing (opts nullable; see
 * ssd_options), in natural-log units; entries past seqlen continue the sum
 * with zero terms. Output float32 [Bt][H][nC*Q]. `delta` (nullable, 16-byte
 * aligned) receives each token's input weight w_t (dt_t, or its zero-order-hold
 * weight for SSD_DISC_ZOH) in the same layout, as float32, zero past seqlen:
 * the later stages read it in place of dt.
 */
int ssd_chunk_cumsum(const void *dt, const float *A, int batch, int seqlen, int nheads,
                     int chunk, int dtype, float *dA_cumsum, float *delta,
                     const ssd_options *opts, void *stream);

/*
 * Stage 2: each chunk's state contribution from a zero state,
 *   states[b][c][h][p][n] = sum_{t in c} exp(s_end(c) - s_t) * w_t * x_t[p] * B_t[n],
 * with s from dA_cumsum, s_end(c) its value at the chunk's last token, and
 * w from `delta` (stage 1's float32 [Bt][H][nC*Q], 16-byte aligned).
 * Output float32 [Bt][nC][H][P][N].
 */
int ssd_chunk_state(const void *x, const void *B, const float *delta, const float *dA_cumsum,
                    int batch, int seqlen, int nheads, int headdim, int ngroups, int dstate,
                    int chunk, int dtype, float *states, void *stream);

/*
 * Stage 3: the sequential pass over chunks, in float32,
 *   H_0 = init_state (NULL: zero),  H_{c+1} = exp(s_end(c)) * H_c + states_c,
 * writing chunk_init[b][c] = H_c ([Bt][nC][H][P][N] in the operand type of
 * dtype: bf16 for SSD_BF16, the precision ssd_chunk_scan multiplies it in;
 * float32 for SSD_F32) and, if final_state is not NULL, final_state = H_nC
 * (float32 [Bt][H][P][N]).
 */
int ssd_state_passing(const float *states, const float *dA_cumsum, const float *init_state,
                      int batch, int seqlen, int nheads, int headdim, int dstate, int chunk,
                      int dtype, void *chunk_init, float *final_state, void *stream);

/*
 * Stage 4a: C_i . B_j for every pair of tokens j <= i (in 32-token slices) of
 * every chunk, once per B/C group; this does not depend on the head. `cb` is
 * scratch of ssd_chunk_cb_size(...) bytes (32-byte aligned) in the layout
 * ssd_chunk_scan reads (MFMA operand fragments, in dtype's operand type: bf16
 * or float32). The content is only meant for ssd_chunk_scan.
 */
size_t ssd_chunk_cb_size(int batch, int seqlen, int ngroups, int chunk, int dtype);
int ssd_chunk_cb(const void *B, const void *C, int batch, int seqlen, int ngroups, int dstate,
                 int chunk, int dtype, void *cb, void *stream);

/*
 * Stage 4b: outputs of every chunk,
 *   y_i = sum_{j in c, j <= i} (C_i . B_j) exp(s_i - s_j) w_j x_j    (diagonal block)
 *       + exp(s_i) H_c C_i                                           (off-diagonal blocks)
 *       + D_h x_i,
 * writing y [Bt][L][H][P] in dtype, with w from `delta` (stage 1's float32
 * [Bt][H][nC*Q], 16-byte aligned). D is nullable. C_i . B_j comes from
 *   SSD_BF16: B itself ([Bt][L][G][N], 16-byte aligned): the kernel forms the
 *             C B^T tiles of each chunk on chip; `cb` is not read (may be NULL);
 *   SSD_F32:  `cb`, the output of ssd_chunk_cb (stage 4a); `B` is not read
 *             (may be NULL).
 */
int ssd_chunk_scan(const void *x, const float *delta, const float *dA_cumsum, const void *B,
                   const void *C, const void *cb, const float *D, const void *chunk_init,
                   int batch, int seqlen, int nheads, int headdim, int ngroups, int dstate,
                   int chunk, int dtype, void *y, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H */
