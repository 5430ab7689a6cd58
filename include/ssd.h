/*
 * ssd.h - C ABI of the MI355X (gfx950) SSD layer library (libssd.so).
 *
 * The layer is the per-head selective state-space model of Mamba-2:
 *
 *   h_t = exp(dt_t * A_h) * h_{t-1} + dt_t * x_t B_t^T      state, P x N per head
 *   y_t = h_t C_t + D_h * x_t                               output after the update
 *
 * ("从Transformer到Mamba" tutorial, sections 2.1-2.2: discrete recurrence and
 * feed-through D; "深挖-Mamba", core concept 3: dt, B, C depend on the token.)
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
 *     dt            [Bt][L][H]           dtype (already positive; no softplus)
 *     B, C          [Bt][L][G][N]        dtype; head h reads group h / (H / G)
 *     A, D          [H]                  float32 (A < 0 for a decaying state)
 *     states        [Bt][H][P][N]        float32 (init / final / decode state)
 *   Decode (ssd_step) drops the L dimension: x, y [Bt][H][P], dt [Bt][H],
 *   B, C [Bt][G][N].
 * - dtype is SSD_F32 (all of x, dt, B, C, y float32) or SSD_BF16 (all bf16);
 *   A, D and every state are float32. Products run on MFMA in the input
 *   dtype with float32 accumulation.
 * - Supported set: headdim == 64; dstate in {16, 32, 64, 128, 256};
 *   chunk in {64, 128, 256}; any seqlen >= 1 (the last chunk may be short);
 *   nheads % ngroups == 0. Anything else returns SSD_ERR_UNSUPPORTED.
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
    SSD_ERR_HIP = -5          /* the HIP runtime reported an error at launch       */
} ssd_status;

/* Human-readable text for a status code (static storage; never NULL). */
const char *ssd_strerror(int status);

/*
 * Bytes of workspace ssd_forward needs (0 for invalid sizes). The workspace
 * holds, at 256-byte aligned offsets in this order:
 *   dA_cumsum   float32 [Bt][H][nC*Q]      within-chunk prefix sums of dt*A
 *   delta       float32 [Bt][H][nC*Q]      dt in the same layout (zero past seqlen)
 *   states      float32 [Bt][nC][H][P][N]  each chunk's own state contribution
 *   chunk_init  [Bt][nC][H][P][N]          state entering each chunk, in the MFMA
 *                                          operand type (bf16 for SSD_BF16, else float32)
 *   cb          SSD_F32 only: ssd_chunk_cb_size(...) bytes, C B^T tiles of every
 *               chunk (the SSD_BF16 chunk scan forms them itself; no space)
 * After the forward pass has run, these hold the intermediate results of the
 * stages below (a caller may read them, e.g. to test a stage), except that
 * for SSD_BF16 with batch * nheads >= 512 stages 2 and 3 run as one kernel
 * that keeps the per-chunk states on chip: `states` is then not written.
 */
size_t ssd_forward_workspace_size(int batch, int seqlen, int nheads, int headdim,
                                  int ngroups, int dstate, int chunk, int dtype);

/*
 * Full SSD layer forward: enqueues ssd_chunk_cumsum, ssd_chunk_state,
 * ssd_state_passing, ssd_chunk_cb (SSD_F32 only) and ssd_chunk_scan on
 * `stream`.
 *   D           nullable: no feed-through term.
 *   init_state  nullable: the state before token 0 is zero.
 *   y           output, [Bt][L][H][P] in dtype.
 *   final_state nullable: if given, receives the state after token L-1.
 *   workspace   at least ssd_forward_workspace_size(...) bytes, 256-byte aligned.
 */
int ssd_forward(const void *x, const void *dt, const float *A, const void *B,
                const void *C, const float *D, int batch, int seqlen, int nheads,
                int headdim, int ngroups, int dstate, int chunk, int dtype,
                const float *init_state, void *y, float *final_state,
                void *workspace, size_t workspace_bytes, void *stream);

/*
 * ssd_forward with per-stage timing hooks for profilers and benchmarks.
 * `events` is NULL (then this is exactly ssd_forward) or an array of 6
 * hipEvent_t owned by the caller, any of which may be NULL (not recorded):
 * events[k] is recorded on `stream` right before stage k+1 is enqueued and
 * events[5] after the last stage, so the
 * elapsed time between consecutive events is each stage's GPU time (stages in
 * the order listed for ssd_forward; for SSD_BF16 the ssd_chunk_cb interval is
 * empty, that work being part of ssd_chunk_scan).
 */
int ssd_forward_timed(const void *x, const void *dt, const float *A, const void *B,
                      const void *C, const float *D, int batch, int seqlen, int nheads,
                      int headdim, int ngroups, int dstate, int chunk, int dtype,
                      const float *init_state, void *y, float *final_state,
                      void *workspace, size_t workspace_bytes, void *stream,
                      void *const *events);

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

/* ---- The forward pass stage by stage (what ssd_forward enqueues) ---------- */

/*
 * Stage 1: dA_cumsum[b][h][c*Q + k] = sum_{t=cQ..cQ+k} dt[b][t][h] * A[h]
 * (natural-log units; entries past seqlen continue the sum with zero terms).
 * Output float32 [Bt][H][nC*Q]. `delta` (nullable) receives dt itself in the
 * same layout, as float32, zero past seqlen: a copy of dt that the later
 * stages read contiguously per head.
 */
int ssd_chunk_cumsum(const void *dt, const float *A, int batch, int seqlen, int nheads,
                     int chunk, int dtype, float *dA_cumsum, float *delta, void *stream);

/*
 * Stage 2: each chunk's state contribution from a zero state,
 *   states[b][c][h][p][n] = sum_{t in c} exp(s_end(c) - s_t) * dt_t * x_t[p] * B_t[n],
 * with s from dA_cumsum and s_end(c) its value at the chunk's last token.
 * Output float32 [Bt][nC][H][P][N].
 */
int ssd_chunk_state(const void *x, const void *B, const void *dt, const float *dA_cumsum,
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
 *   y_i = sum_{j in c, j <= i} (C_i . B_j) exp(s_i - s_j) dt_j x_j   (diagonal block)
 *       + exp(s_i) H_c C_i                                           (off-diagonal blocks)
 *       + D_h x_i,
 * writing y [Bt][L][H][P] in dtype. D is nullable. C_i . B_j comes from
 *   SSD_BF16: B itself ([Bt][L][G][N], 16-byte aligned): the kernel forms the
 *             C B^T tiles of each chunk on chip; `cb` is not read (may be NULL);
 *   SSD_F32:  `cb`, the output of ssd_chunk_cb (stage 4a); `B` is not read
 *             (may be NULL).
 */
int ssd_chunk_scan(const void *x, const void *dt, const float *dA_cumsum, const void *B,
                   const void *C, const void *cb, const float *D, const void *chunk_init,
                   int batch, int seqlen, int nheads, int headdim, int ngroups, int dstate,
                   int chunk, int dtype, void *y, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H */
