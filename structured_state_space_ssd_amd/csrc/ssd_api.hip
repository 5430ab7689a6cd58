// C ABI of libssd.so: argument checks, workspace layout and launch order.
// Every declaration and its contract is in include/ssd.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "ssd.h"
#include "ssd_launch.h"

namespace {

constexpr size_t kAlign = 256;
constexpr int kHeaddim = 64;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// N the kernels are built for; every other multiple of 16 up to 256 runs the
// forward, the backward and the decode step zero-padded to the next of these
// (pad.hip)
bool kernel_dstate_ok(int n) { return n == 16 || n == 32 || n == 64 || n == 128 || n == 256; }
bool supported_dstate(int n) { return n >= 16 && n <= 256 && n % 16 == 0; }
bool supported_chunk(int q) { return q == 64 || q == 128 || q == 256; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool valid_dtype(int d) { return d == SSD_F32 || d == SSD_BF16; }

struct Workspace {
    size_t cumsum_off, delta_off, states_off, init_off, cb_off, total;
};

Workspace layout(int batch, int seqlen, int nheads, int headdim, int ngroups, int dstate, int chunk,
                 bool bf16) {
    const size_t nC = (static_cast<size_t>(seqlen) + chunk - 1) / chunk;
    const size_t cumsum = static_cast<size_t>(batch) * nheads * nC * chunk * sizeof(float);
    const size_t elems = static_cast<size_t>(batch) * nC * nheads * headdim * dstate;
    const size_t st = elems * sizeof(float);
    const size_t ci = elems * (bf16 ? 2 : 4);
    Workspace w;
    w.cumsum_off = 0;
    w.delta_off = align_up(cumsum);
    w.states_off = w.delta_off + align_up(cumsum);
    w.init_off = w.states_off + align_up(st);
    w.cb_off = w.init_off + align_up(ci);
    w.total = w.cb_off;
    if (ssd::chunk_scan_reads_cb(bf16))
        w.total += align_up(ssd::chunk_cb_bytes(batch, seqlen, ngroups, chunk, bf16));
    return w;
}

// Packed sequences: the forward's workspace at batch 1, then seg (one int per
// token position of the chunk-padded layout).
Workspace varlen_layout(int seqlen, int nheads, int headdim, int ngroups, int dstate, int chunk,
                        bool bf16, size_t *seg_off) {
    Workspace w = layout(1, seqlen, nheads, headdim, ngroups, dstate, chunk, bf16);
    const size_t nC = (static_cast<size_t>(seqlen) + chunk - 1) / chunk;
    *seg_off = w.total;
    w.total += align_up(nC * chunk * sizeof(int));
    return w;
}

// The backward's workspace (its own chunk length, see ssd::bwd_chunk).
struct BwdWorkspace {
    size_t s_off, delta_off, states_off, init_off, gnext_off, ds_off, dw_off, dB_off, dC_off,
        dA_off, dbias_off, dD_off, total;
    int chunk, nblk;
};

BwdWorkspace bwd_layout(int batch, int seqlen, int nheads, int headdim, int ngroups, int dstate,
                        bool bf16) {
    BwdWorkspace w{};
    w.chunk = ssd::bwd_chunk(dstate, bf16);
    if (!w.chunk) return w;
    w.nblk = ssd::bwd_head_blocks(batch, seqlen, nheads, ngroups, w.chunk);
    const size_t nC = (static_cast<size_t>(seqlen) + w.chunk - 1) / w.chunk;
    const size_t tok = static_cast<size_t>(batch) * nheads * nC * w.chunk * sizeof(float);
    const size_t elems = static_cast<size_t>(batch) * nC * nheads * headdim * dstate;
    const size_t part = static_cast<size_t>(w.nblk) * batch * seqlen * ngroups * dstate * sizeof(float);
    const size_t per_chunk = static_cast<size_t>(batch) * nC * nheads * sizeof(float);
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o += align_up(bytes);
        return at;
    };
    w.s_off = take(tok);
    w.delta_off = take(tok);
    w.states_off = take(elems * sizeof(float));
    w.init_off = take(elems * (bf16 ? 2 : 4));
    w.gnext_off = take(elems * (bf16 ? 2 : 4));
    w.ds_off = take(tok);
    w.dw_off = take(tok);
    w.dB_off = take(part);
    w.dC_off = take(part);
    w.dA_off = take(per_chunk);
    w.dbias_off = take(per_chunk);
    w.dD_off = take(per_chunk);
    w.total = o;
    return w;
}

// The path ssd_forward takes and the workspace it needs. The single-pass
// kernel needs scratch only for the pieces' states when the sequences are cut
// into segments (at most `cap` bytes of it); the stage kernels need the whole
// layout above.
// With a state size outside the kernels' set, the kernels run at nk (the
// next size of the set) on zero-padded copies of B, C and the initial state
// held after the kernels' own part of the workspace, from pad_off on: B', C'
// [Bt][L][G][nk] in the input dtype, then the initial and final states
// [Bt][H][P][nk] float32.
struct FwdPlan {
    bool onepass;
    ssd::OnepassPlan op;
    Workspace ws;
    int nk;
    size_t pad_off, need;
};

struct PadLayout {
    size_t bc, st;  // bytes of one padded B / C, and of one padded state (aligned)
};
PadLayout pad_layout(int batch, int seqlen, int nheads, int headdim, int ngroups, int nk,
                     bool bf16) {
    return PadLayout{align_up((size_t)batch * seqlen * ngroups * nk * (bf16 ? 2 : 4)),
                     align_up((size_t)batch * nheads * headdim * nk * sizeof(float))};
}

FwdPlan plan_forward(int batch, int seqlen, int nheads, int headdim, int ngroups, int dstate,
                     int chunk, bool bf16, const void *dt, size_t cap) {
    FwdPlan f{};
    f.nk = ssd::kernel_dstate(dstate);
    size_t pad_total = 0;
    if (f.nk != dstate) {
        const PadLayout pl = pad_layout(batch, seqlen, nheads, headdim, ngroups, f.nk, bf16);
        pad_total = 2 * pl.bc + 2 * pl.st + kAlign;
    }
    f.onepass = ssd::forward_onepass_ok(batch, nheads, f.nk, bf16, dt);
    if (f.onepass) {
        f.op = ssd::forward_onepass_plan(batch, seqlen, nheads, f.nk,
                                         cap > pad_total ? cap - pad_total : 0);
        f.need = f.op.scratch_bytes;
    } else {
        f.ws = layout(batch, seqlen, nheads, headdim, ngroups, f.nk, chunk, bf16);
        f.need = f.ws.total;
    }
    if (f.nk != dstate) {
        const PadLayout pl = pad_layout(batch, seqlen, nheads, headdim, ngroups, f.nk, bf16);
        f.pad_off = align_up(f.need);
        f.need = f.pad_off + 2 * pl.bc + 2 * pl.st;
    }
    return f;
}

// Any 16-byte aligned address: what the sizing calls assume for dt.
const void *const kAlignedDt = reinterpret_cast<const void *>(uintptr_t{256});

int check_dims(int batch, int seqlen, int nheads, int headdim, int ngroups, int dstate) {
    if (batch < 1 || seqlen < 1 || nheads < 1 || headdim < 1 || ngroups < 1 || dstate < 1)
        return SSD_ERR_SHAPE;
    if (nheads % ngroups != 0) return SSD_ERR_SHAPE;
    if (headdim != kHeaddim || !supported_dstate(dstate)) return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? SSD_OK : SSD_ERR_HIP; }

// The backward's workspace: its kernels' layout at nk, then (nk != dstate)
// the padded copies B', C', dB', dC' and three padded states.
size_t bwd_need(const BwdWorkspace &ws, int batch, int seqlen, int nheads, int headdim,
                int ngroups, int dstate, int nk, bool bf16) {
    if (nk == dstate) return ws.total;
    const PadLayout pl = pad_layout(batch, seqlen, nheads, headdim, ngroups, nk, bf16);
    return align_up(ws.total) + 4 * pl.bc + 3 * pl.st;
}

// Checks an ssd_options (NULL: every option off) and converts it for the kernels.
int dt_opts(const ssd_options *o, ssd::DtOpts &d) {
    d = ssd::DtOpts{nullptr, 0.0f, 0.0f, 0, 0, 0};
    if (!o) return SSD_OK;
    if (o->discretization != SSD_DISC_EULER && o->discretization != SSD_DISC_ZOH)
        return SSD_ERR_OPTION;
    if (o->dt_clamp && !(o->dt_min <= o->dt_max)) return SSD_ERR_OPTION;  // NaN bounds fail too
    if ((reinterpret_cast<uintptr_t>(o->dt_bias) & 3u) != 0) return SSD_ERR_UNSUPPORTED;
    d.bias = o->dt_bias;
    d.lo = o->dt_min;
    d.hi = o->dt_max;
    d.softplus = o->dt_softplus != 0;
    d.clamp = o->dt_clamp != 0;
    d.zoh = o->discretization == SSD_DISC_ZOH;
    return SSD_OK;
}

}  // namespace

extern "C" {

const char *ssd_strerror(int status) {
    switch (status) {
        case SSD_OK: return "ok";
        case SSD_ERR_NULL: return "a required pointer is NULL";
        case SSD_ERR_SHAPE: return "invalid sizes (non-positive, or nheads not a multiple of ngroups)";
        case SSD_ERR_UNSUPPORTED:
            return "unsupported configuration (need headdim 64, dstate a multiple of 16 up to "
                   "256 (16, 32, 64, 128 or 256 for the stage entry points and packed "
                   "sequences), chunk in {64,128,256}, dtype SSD_F32/SSD_BF16, 16-byte aligned "
                   "buffers)";
        case SSD_ERR_WORKSPACE: return "workspace missing or too small";
        case SSD_ERR_HIP: return "HIP runtime error at kernel launch";
        case SSD_ERR_OPTION:
            return "invalid ssd_options (discretization not SSD_DISC_EULER/SSD_DISC_ZOH, or "
                   "dt_clamp with dt_min > dt_max or a NaN bound)";
        case SSD_ERR_TOO_LARGE:
            return "the forward needs more scratch than ssd_forward_static's fixed device array "
                   "holds (SSD_STATIC_SCRATCH_BYTES); use ssd_forward with a workspace";
        default: return "unknown status";
    }
}

size_t ssd_forward_workspace_size(int batch, int seqlen, int nheads, int headdim, int ngroups,
                                  int dstate, int chunk, int dtype) {
    ssd_plan p;
    if (ssd_forward_plan_info(batch, seqlen, nheads, headdim, ngroups, dstate, chunk, dtype,
                              kAlignedDt, &p) != SSD_OK)
        return 0;
    return p.workspace_bytes;
}

int ssd_forward_plan_info(int batch, int seqlen, int nheads, int headdim, int ngroups, int dstate,
                          int chunk, int dtype, const void *dt, ssd_plan *out) {
    if (!out) return SSD_ERR_NULL;
    *out = ssd_plan{};
    const int rc = check_dims(batch, seqlen, nheads, headdim, ngroups, dstate);
    if (rc != SSD_OK) return rc;
    if (!supported_chunk(chunk) || !valid_dtype(dtype)) return SSD_ERR_UNSUPPORTED;
    const FwdPlan f = plan_forward(batch, seqlen, nheads, headdim, ngroups, dstate, chunk,
                                   dtype == SSD_BF16, dt, SIZE_MAX);
    out->path = f.onepass ? SSD_PATH_SINGLE_PASS : SSD_PATH_STAGES;
    out->segments = f.onepass ? f.op.S : 0;
    out->pieces = f.onepass ? f.op.k : 0;
    out->block_tokens = f.onepass ? 64 : chunk;
    out->segment_blocks = f.onepass ? f.op.per_seg : 0;
    out->piece_blocks = f.onepass && f.op.S > 1 ? f.op.psub : 0;
    out->kernel_dstate = f.nk;
    out->workspace_bytes = f.need;
    return SSD_OK;
}

int ssd_forward_plan(int batch, int seqlen, int nheads, int headdim, int ngroups, int dstate,
                     int chunk, int dtype, const void *dt) {
    ssd_plan p;
    const int rc = ssd_forward_plan_info(batch, seqlen, nheads, headdim, ngroups, dstate, chunk,
                                         dtype, dt, &p);
    return rc != SSD_OK ? rc : p.segments;
}

size_t ssd_forward_varlen_workspace_size(int seqlen, int nheads, int headdim, int ngroups,
                                         int dstate, int chunk, int dtype) {
    if (check_dims(1, seqlen, nheads, headdim, ngroups, dstate) != SSD_OK ||
        !kernel_dstate_ok(dstate) || !supported_chunk(chunk) || !valid_dtype(dtype))
        return 0;
    size_t seg_off;
    return varlen_layout(seqlen, nheads, headdim, ngroups, dstate, chunk, dtype == SSD_BF16,
                         &seg_off).total;
}

size_t ssd_backward_workspace_size(int batch, int seqlen, int nheads, int headdim, int ngroups,
                                   int dstate, int dtype) {
    if (check_dims(batch, seqlen, nheads, headdim, ngroups, dstate) != SSD_OK || !valid_dtype(dtype))
        return 0;
    const int nk = ssd::kernel_dstate(dstate);
    const bool bf16 = dtype == SSD_BF16;
    const BwdWorkspace ws = bwd_layout(batch, seqlen, nheads, headdim, ngroups, nk, bf16);
    if (!ws.chunk) return 0;
    return bwd_need(ws, batch, seqlen, nheads, headdim, ngroups, dstate, nk, bf16);
}

size_t ssd_chunk_cb_size(int batch, int seqlen, int ngroups, int chunk, int dtype) {
    if (batch < 1 || seqlen < 1 || ngroups < 1 || !supported_chunk(chunk) || !valid_dtype(dtype))
        return 0;
    return ssd::chunk_cb_bytes(batch, seqlen, ngroups, chunk, dtype == SSD_BF16);
}

int ssd_chunk_cb(const void *B, const void *C, int batch, int seqlen, int ngroups, int dstate,
                 int chunk, int dtype, void *cb, void *stream) {
    if (!B || !C || !cb) return SSD_ERR_NULL;
    if (batch < 1 || seqlen < 1 || ngroups < 1 || dstate < 1) return SSD_ERR_SHAPE;
    if (!kernel_dstate_ok(dstate) || !supported_chunk(chunk) || !valid_dtype(dtype))
        return SSD_ERR_UNSUPPORTED;
    if (!aligned16(B) || !aligned16(C) || (reinterpret_cast<uintptr_t>(cb) % 32) != 0)
        return SSD_ERR_UNSUPPORTED;
    return status_of(ssd::launch_chunk_cb(B, C, batch, seqlen, ngroups, dstate, chunk,
                                          dtype == SSD_BF16, cb, static_cast<hipStream_t>(stream)));
}

int ssd_chunk_cumsum(const void *dt, const float *A, int batch, int seqlen, int nheads, int chunk,
                     int dtype, float *dA_cumsum, float *delta, const ssd_options *opts,
                     void *stream) {
    if (!dt || !A || !dA_cumsum) return SSD_ERR_NULL;
    if (batch < 1 || seqlen < 1 || nheads < 1) return SSD_ERR_SHAPE;
    if (!supported_chunk(chunk) || !valid_dtype(dtype)) return SSD_ERR_UNSUPPORTED;
    if (delta && !aligned16(delta)) return SSD_ERR_UNSUPPORTED;
    ssd::DtOpts o;
    const int rc = dt_opts(opts, o);
    if (rc != SSD_OK) return rc;
    return status_of(ssd::launch_chunk_cumsum(dt, A, batch, seqlen, nheads, chunk,
                                              dtype == SSD_BF16, o, dA_cumsum, delta,
                                              static_cast<hipStream_t>(stream)));
}

int ssd_chunk_state(const void *x, const void *B, const float *delta, const float *dA_cumsum,
                    int batch, int seqlen, int nheads, int headdim, int ngroups, int dstate,
                    int chunk, int dtype, float *states, void *stream) {
    if (!x || !B || !delta || !dA_cumsum || !states) return SSD_ERR_NULL;
    int rc = check_dims(batch, seqlen, nheads, headdim, ngroups, dstate);
    if (rc != SSD_OK) return rc;
    if (!kernel_dstate_ok(dstate)) return SSD_ERR_UNSUPPORTED;
    if (!supported_chunk(chunk) || !valid_dtype(dtype)) return SSD_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(B) || !aligned16(states) || !aligned16(delta))
        return SSD_ERR_UNSUPPORTED;
    return status_of(ssd::launch_chunk_state(x, B, delta, dA_cumsum, nullptr, batch, seqlen, nheads, ngroups,
                                             dstate, chunk, dtype == SSD_BF16, states,
                                             static_cast<hipStream_t>(stream)));
}

int ssd_state_passing(const float *states, const float *dA_cumsum, const float *init_state,
                      int batch, int seqlen, int nheads, int headdim, int dstate, int chunk,
                      int dtype, void *chunk_init, float *final_state, void *stream) {
    if (!states || !dA_cumsum || !chunk_init) return SSD_ERR_NULL;
    int rc = check_dims(batch, seqlen, nheads, headdim, 1, dstate);
    if (rc != SSD_OK) return rc;
    if (!kernel_dstate_ok(dstate)) return SSD_ERR_UNSUPPORTED;
    if (!supported_chunk(chunk) || !valid_dtype(dtype)) return SSD_ERR_UNSUPPORTED;
    if (!aligned16(states) || !aligned16(chunk_init) || (init_state && !aligned16(init_state)) ||
        (final_state && !aligned16(final_state)))
        return SSD_ERR_UNSUPPORTED;
    return status_of(ssd::launch_state_passing(states, dA_cumsum, init_state, nullptr, batch, seqlen, nheads,
                                               dstate, chunk, dtype == SSD_BF16, chunk_init,
                                               final_state, static_cast<hipStream_t>(stream)));
}

int ssd_chunk_scan(const void *x, const float *delta, const float *dA_cumsum, const void *B,
                   const void *C, const void *cb, const float *D, const void *chunk_init,
                   int batch, int seqlen, int nheads, int headdim, int ngroups, int dstate,
                   int chunk, int dtype, void *y, void *stream) {
    if (!x || !delta || !dA_cumsum || !C || !chunk_init || !y) return SSD_ERR_NULL;
    int rc = check_dims(batch, seqlen, nheads, headdim, ngroups, dstate);
    if (rc != SSD_OK) return rc;
    if (!kernel_dstate_ok(dstate)) return SSD_ERR_UNSUPPORTED;
    if (!supported_chunk(chunk) || !valid_dtype(dtype)) return SSD_ERR_UNSUPPORTED;
    const bool bf16 = dtype == SSD_BF16;
    const bool reads_cb = ssd::chunk_scan_reads_cb(bf16);
    if (reads_cb ? !cb : !B) return SSD_ERR_NULL;
    if (!aligned16(x) || !aligned16(C) || !aligned16(chunk_init) || !aligned16(y) ||
        !aligned16(dA_cumsum) || !aligned16(delta) ||
        (reads_cb ? (reinterpret_cast<uintptr_t>(cb) % 32) != 0 : !aligned16(B)))
        return SSD_ERR_UNSUPPORTED;
    return status_of(ssd::launch_chunk_scan(x, delta, dA_cumsum, B, C, cb, D, chunk_init, nullptr, batch,
                                            seqlen, nheads, ngroups, dstate, chunk, bf16, y,
                                            static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

hipError_t static_scratch(void **out);

// The forward's launches for a plan at the kernels' own state size f.nk,
// with B, C and the states already of that size; `base` holds the plan's
// workspace (f.need bytes before any padding region).
hipError_t forward_run(const FwdPlan &f, const void *x, const void *dt, const float *A,
                       const void *B, const void *C, const float *D, int batch, int seqlen,
                       int nheads, int ngroups, int chunk, bool bf16, const float *init_state,
                       void *y, float *final_state, char *base, const ssd::DtOpts &o,
                       hipStream_t s, void *const *events) {
    const int dstate = f.nk;
    auto mark = [&](int k) -> hipError_t {
        return events && events[k] ? hipEventRecord(static_cast<hipEvent_t>(events[k]), s)
                                   : hipSuccess;
    };
    hipError_t e = mark(0);
    if (f.onepass) {
        // every stage in one kernel (after the segment-state kernel when the
        // sequences are cut into segments): intervals 0 (and 1), the others empty
        const int segments = f.op.S;
        if (e == hipSuccess)
            e = ssd::launch_forward_onepass(
                x, dt, A, B, C, D, init_state, o, batch, seqlen, nheads, ngroups, dstate, f.op,
                reinterpret_cast<float *>(base), y, final_state,
                segments > 1 && events ? static_cast<hipEvent_t>(events[1]) : nullptr, s);
        for (int k = segments > 1 ? 2 : 1; k <= 5 && e == hipSuccess; ++k) e = mark(k);
        return e;
    }
    const Workspace &ws = f.ws;
    float *cumsum = reinterpret_cast<float *>(base + ws.cumsum_off);
    float *delta = reinterpret_cast<float *>(base + ws.delta_off);
    float *states = reinterpret_cast<float *>(base + ws.states_off);
    void *cinit = base + ws.init_off;
    void *cb = base + ws.cb_off;
    if (e == hipSuccess)
        e = ssd::launch_chunk_cumsum(dt, A, batch, seqlen, nheads, chunk, bf16, o, cumsum, delta,
                                     s);
    if (e == hipSuccess) e = mark(1);
    if (ssd::state_passing_fused(batch, nheads, bf16)) {
        // stages 2 and 3 in one kernel; the state_passing interval stays empty
        if (e == hipSuccess)
            e = ssd::launch_chunk_state_passing(x, B, cumsum, delta, init_state, batch, seqlen,
                                                nheads, ngroups, dstate, chunk, cinit,
                                                final_state, s);
        if (e == hipSuccess) e = mark(2);
    } else {
        if (e == hipSuccess)
            e = ssd::launch_chunk_state(x, B, delta, cumsum, nullptr, batch, seqlen, nheads,
                                        ngroups, dstate, chunk, bf16, states, s);
        if (e == hipSuccess) e = mark(2);
        if (e == hipSuccess)
            e = ssd::launch_state_passing(states, cumsum, init_state, nullptr, batch, seqlen,
                                          nheads, dstate, chunk, bf16, cinit, final_state, s);
    }
    if (e == hipSuccess) e = mark(3);
    if (e == hipSuccess && ssd::chunk_scan_reads_cb(bf16))
        e = ssd::launch_chunk_cb(B, C, batch, seqlen, ngroups, dstate, chunk, bf16, cb, s);
    if (e == hipSuccess) e = mark(4);
    if (e == hipSuccess)
        e = ssd::launch_chunk_scan(x, delta, cumsum, B, C, cb, D, cinit, nullptr, batch, seqlen,
                                   nheads, ngroups, dstate, chunk, bf16, y, s);
    if (e == hipSuccess) e = mark(5);
    return e;
}

// ssd_forward_ex with the plan's scratch capped at `cap` bytes; with
// `fixed_scratch` the workspace is the current device's fixed scratch array
// (ssd_forward_static), and `workspace` / `workspace_bytes` are not read.
int forward_impl(const void *x, const void *dt, const float *A, const void *B, const void *C,
                 const float *D, int batch, int seqlen, int nheads, int headdim, int ngroups,
                 int dstate, int chunk, int dtype, const float *init_state, void *y,
                 float *final_state, void *workspace, size_t workspace_bytes,
                 const ssd_options *opts, void *stream, void *const *events, size_t cap,
                 bool fixed_scratch = false) {
    if (!x || !dt || !A || !B || !C || !y) return SSD_ERR_NULL;
    int rc = check_dims(batch, seqlen, nheads, headdim, ngroups, dstate);
    if (rc != SSD_OK) return rc;
    if (!supported_chunk(chunk) || !valid_dtype(dtype)) return SSD_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(B) || !aligned16(C) || !aligned16(y) ||
        (init_state && !aligned16(init_state)) || (final_state && !aligned16(final_state)))
        return SSD_ERR_UNSUPPORTED;
    ssd::DtOpts o;
    rc = dt_opts(opts, o);
    if (rc != SSD_OK) return rc;
    const bool bf16 = dtype == SSD_BF16;
    const FwdPlan f =
        plan_forward(batch, seqlen, nheads, headdim, ngroups, dstate, chunk, bf16, dt, cap);
    if (fixed_scratch) {
        if (f.need > cap) return SSD_ERR_TOO_LARGE;
        workspace = nullptr;
        if (f.need > 0) {
            const hipError_t e = static_scratch(&workspace);
            if (e != hipSuccess) return SSD_ERR_HIP;
        }
        workspace_bytes = cap;
    }
    if (f.need > cap) return SSD_ERR_WORKSPACE;
    if (f.need > 0 && (!workspace || workspace_bytes < f.need)) return SSD_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0) return SSD_ERR_WORKSPACE;

    char *base = static_cast<char *>(workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (f.nk == dstate)
        return status_of(forward_run(f, x, dt, A, B, C, D, batch, seqlen, nheads, ngroups, chunk,
                                     bf16, init_state, y, final_state, base, o, s, events));
    // zero-padded to the kernels' state size (pad.hip): B, C, the initial state
    // in; the final state cut back to dstate
    const PadLayout pl = pad_layout(batch, seqlen, nheads, headdim, ngroups, f.nk, bf16);
    char *pb = base + f.pad_off;
    void *Bp = pb, *Cp = pb + pl.bc;
    float *ip = reinterpret_cast<float *>(pb + 2 * pl.bc);
    float *fp = reinterpret_cast<float *>(pb + 2 * pl.bc + pl.st);
    const size_t bc_rows = (size_t)batch * seqlen * ngroups, st_rows = (size_t)batch * nheads * headdim;
    const int es = bf16 ? 2 : 4;
    hipError_t e = ssd::launch_pad_rows(B, Bp, bc_rows, dstate, f.nk, es, s);
    if (e == hipSuccess) e = ssd::launch_pad_rows(C, Cp, bc_rows, dstate, f.nk, es, s);
    if (e == hipSuccess && init_state)
        e = ssd::launch_pad_rows(init_state, ip, st_rows, dstate, f.nk, 4, s);
    if (e == hipSuccess)
        e = forward_run(f, x, dt, A, Bp, Cp, D, batch, seqlen, nheads, ngroups, chunk, bf16,
                        init_state ? ip : nullptr, y, final_state ? fp : nullptr, base, o, s,
                        events);
    if (e == hipSuccess && final_state)
        e = ssd::launch_pad_rows(fp, final_state, st_rows, f.nk, dstate, 4, s);
    return status_of(e);
}

// ---- the fixed scratch of ssd_forward_static
//
// One array per GPU the library runs on, held until the process ends. Host
// code never uses the array's name as an address (on the host it names a
// stand-in, not device memory): the device address comes from
// hipGetSymbolAddress, once per device with that device current, and only
// that address reaches the kernels.
static __device__ __align__(256) unsigned char scratch[SSD_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];  // device address of `scratch`, per device

hipError_t static_scratch(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

int ssd_forward_static(const void *x, const void *dt, const float *A, const void *B,
                       const void *C, const float *D, int batch, int seqlen, int nheads,
                       int headdim, int ngroups, int dstate, int chunk, int dtype,
                       const float *init_state, void *y, float *final_state,
                       const ssd_options *opts, void *stream) {
    return forward_impl(x, dt, A, B, C, D, batch, seqlen, nheads, headdim, ngroups, dstate, chunk,
                        dtype, init_state, y, final_state, nullptr, 0, opts, stream, nullptr,
                        SSD_STATIC_SCRATCH_BYTES, /*fixed_scratch=*/true);
}

int ssd_forward_ex(const void *x, const void *dt, const float *A, const void *B, const void *C,
                   const float *D, int batch, int seqlen, int nheads, int headdim, int ngroups,
                   int dstate, int chunk, int dtype, const float *init_state, void *y,
                   float *final_state, void *workspace, size_t workspace_bytes,
                   const ssd_options *opts, void *stream, void *const *events) {
    return forward_impl(x, dt, A, B, C, D, batch, seqlen, nheads, headdim, ngroups, dstate, chunk,
                        dtype, init_state, y, final_state, workspace, workspace_bytes, opts,
                        stream, events, SIZE_MAX);
}

int ssd_forward_varlen(const void *x, const void *dt, const float *A, const void *B,
                       const void *C, const float *D, const int *cu_seqlens, int nseq,
                       int seqlen, int nheads, int headdim, int ngroups, int dstate, int chunk,
                       int dtype, void *y, float *seq_states, void *workspace,
                       size_t workspace_bytes, const ssd_options *opts, void *stream) {
    if (!x || !dt || !A || !B || !C || !y || !cu_seqlens) return SSD_ERR_NULL;
    if (nseq < 1) return SSD_ERR_SHAPE;
    int rc = check_dims(1, seqlen, nheads, headdim, ngroups, dstate);
    if (rc != SSD_OK) return rc;
    if (!kernel_dstate_ok(dstate)) return SSD_ERR_UNSUPPORTED;
    if (!supported_chunk(chunk) || !valid_dtype(dtype)) return SSD_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(B) || !aligned16(C) || !aligned16(y) ||
        (seq_states && !aligned16(seq_states)) ||
        (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0)
        return SSD_ERR_UNSUPPORTED;
    ssd::DtOpts o;
    rc = dt_opts(opts, o);
    if (rc != SSD_OK) return rc;
    const bool bf16 = dtype == SSD_BF16;
    size_t seg_off;
    const Workspace ws =
        varlen_layout(seqlen, nheads, headdim, ngroups, dstate, chunk, bf16, &seg_off);
    if (!workspace || workspace_bytes < ws.total) return SSD_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0) return SSD_ERR_WORKSPACE;

    char *base = static_cast<char *>(workspace);
    float *cumsum = reinterpret_cast<float *>(base + ws.cumsum_off);
    float *delta = reinterpret_cast<float *>(base + ws.delta_off);
    float *states = reinterpret_cast<float *>(base + ws.states_off);
    void *cinit = base + ws.init_off;
    void *cb = base + ws.cb_off;
    int *seg = reinterpret_cast<int *>(base + seg_off);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (ssd::forward_onepass_ok(1, nheads, dstate, bf16, dt)) {
        // the single-pass kernel with sequence masks; the tokens' int4s (16
        // bytes per token) go where dA_cumsum would (H >= 8 floats per token),
        // the pieces' states into the `states` region (the plan fits them there)
        void *meta = base + ws.cumsum_off;
        const ssd::OnepassPlan pl =
            ssd::forward_onepass_plan(1, seqlen, nheads, dstate, ws.init_off - ws.states_off);
        hipError_t e = ssd::launch_onepass_varlen_prep(cu_seqlens, nseq, seqlen, nheads, dstate,
                                                       meta, seq_states, s);
        if (e == hipSuccess)
            e = ssd::launch_forward_onepass(x, dt, A, B, C, D, nullptr, o, 1, seqlen, nheads,
                                            ngroups, dstate, pl, states, y, nullptr, nullptr, s,
                                            meta, seq_states);
        return status_of(e);
    }
    // the separate stages, each masking by seg (no fused stage 2 + 3 here)
    hipError_t e = ssd::launch_varlen_seg(cu_seqlens, nseq, seqlen, chunk, seg, s);
    if (e == hipSuccess)
        e = ssd::launch_chunk_cumsum(dt, A, 1, seqlen, nheads, chunk, bf16, o, cumsum, delta, s);
    if (e == hipSuccess)
        e = ssd::launch_chunk_state(x, B, delta, cumsum, seg, 1, seqlen, nheads, ngroups, dstate,
                                    chunk, bf16, states, s);
    if (e == hipSuccess)
        e = ssd::launch_state_passing(states, cumsum, nullptr, seg, 1, seqlen, nheads, dstate,
                                      chunk, bf16, cinit, nullptr, s);
    if (e == hipSuccess && ssd::chunk_scan_reads_cb(bf16))
        e = ssd::launch_chunk_cb(B, C, 1, seqlen, ngroups, dstate, chunk, bf16, cb, s);
    if (e == hipSuccess)
        e = ssd::launch_chunk_scan(x, delta, cumsum, B, C, cb, D, cinit, seg, 1, seqlen, nheads,
                                   ngroups, dstate, chunk, bf16, y, s);
    if (e == hipSuccess && seq_states)
        e = ssd::launch_varlen_final_states(x, B, delta, cumsum, cu_seqlens, seg, cinit, nseq,
                                            seqlen, nheads, ngroups, dstate, chunk, bf16,
                                            seq_states, s);
    return status_of(e);
}

int ssd_backward(const void *x, const void *dt, const float *A, const void *B, const void *C,
                 const float *D, const float *init_state, const void *dy,
                 const float *dfinal_state, int batch, int seqlen, int nheads, int headdim,
                 int ngroups, int dstate, int dtype, void *dx, void *ddt, float *dA, void *dB,
                 void *dC, float *dD, float *dinit_state, float *ddt_bias, void *workspace,
                 size_t workspace_bytes, const ssd_options *opts, void *stream) {
    return ssd_backward_timed(x, dt, A, B, C, D, init_state, dy, dfinal_state, batch, seqlen,
                              nheads, headdim, ngroups, dstate, dtype, dx, ddt, dA, dB, dC, dD,
                              dinit_state, ddt_bias, workspace, workspace_bytes, opts, stream,
                              nullptr);
}

}  // extern "C"

namespace {

// The backward's launches at the kernels' own state size (dstate here is
// one of 16, 32, 64, 128, 256), with `base` holding the layout `ws`.
hipError_t backward_run(const BwdWorkspace &ws, const void *x, const void *dt, const float *A,
                        const void *B, const void *C, const float *D, const float *init_state,
                        const void *dy, const float *dfinal_state, int batch, int seqlen,
                        int nheads, int ngroups, int dstate, bool bf16, void *dx, void *ddt,
                        float *dA, void *dB, void *dC, float *dD, float *dinit_state,
                        float *ddt_bias, char *base, const ssd::DtOpts &o, hipStream_t st,
                        void *const *events) {
    auto f32 = [&](size_t off) { return reinterpret_cast<float *>(base + off); };
    float *s_ = f32(ws.s_off), *delta = f32(ws.delta_off), *states = f32(ws.states_off);
    void *cinit = base + ws.init_off, *gnext = base + ws.gnext_off;
    const int Q = ws.chunk, nC = (seqlen + Q - 1) / Q;
    auto mark = [&](int k) -> hipError_t {
        return events && events[k] ? hipEventRecord(static_cast<hipEvent_t>(events[k]), st)
                                   : hipSuccess;
    };

    // forward recompute: prefix sums, input weights, the state entering each chunk
    hipError_t e = mark(0);
    if (e == hipSuccess)
        e = ssd::launch_chunk_cumsum(dt, A, batch, seqlen, nheads, Q, bf16, o, s_, delta, st);
    if (e == hipSuccess) {
        if (ssd::state_passing_fused(batch, nheads, bf16)) {
            e = ssd::launch_chunk_state_passing(x, B, s_, delta, init_state, batch, seqlen, nheads,
                                                ngroups, dstate, Q, cinit, nullptr, st);
        } else {
            e = ssd::launch_chunk_state(x, B, delta, s_, nullptr, batch, seqlen, nheads, ngroups,
                                        dstate, Q, bf16, states, st);
            if (e == hipSuccess)
                e = ssd::launch_state_passing(states, s_, init_state, nullptr, batch, seqlen,
                                              nheads, dstate, Q, bf16, cinit, nullptr, st);
        }
    }
    // the adjoint of the state leaving each chunk: dS_c, then the reverse pass
    // (one kernel per (b, h) walking the chunks backward when that fills the GPU)
    if (e == hipSuccess) e = mark(1);
    if (ssd::state_passing_fused(batch, nheads, bf16)) {
        if (e == hipSuccess)
            e = ssd::launch_chunk_state_passing(dy, C, s_, nullptr, dfinal_state, batch, seqlen,
                                                nheads, ngroups, dstate, Q, gnext, dinit_state,
                                                st, /*reverse=*/true);
    } else {
        if (e == hipSuccess)
            e = ssd::launch_chunk_state(dy, C, nullptr, s_, nullptr, batch, seqlen, nheads,
                                        ngroups, dstate, Q, bf16, states, st, /*dout=*/true);
        if (e == hipSuccess)
            e = ssd::launch_state_passing(states, s_, dfinal_state, nullptr, batch, seqlen,
                                          nheads, dstate, Q, bf16, gnext, dinit_state, st,
                                          /*reverse=*/true);
    }
    // the chunks' gradients
    ssd::BwdArgs a{};
    a.x = x; a.dy = dy; a.B = B; a.C = C; a.dA_cumsum = s_; a.delta = delta; a.D = D;
    a.chunk_init = cinit; a.grad_next = gnext;
    a.batch = batch; a.seqlen = seqlen; a.nheads = nheads; a.ngroups = ngroups;
    a.dstate = dstate; a.chunk = Q; a.nblk = ws.nblk; a.bf16 = bf16;
    a.dx = dx; a.ds = f32(ws.ds_off); a.dw = f32(ws.dw_off);
    a.dB_part = f32(ws.dB_off); a.dC_part = f32(ws.dC_off); a.dD_part = f32(ws.dD_off);
    if (e == hipSuccess) e = mark(2);
    if (e == hipSuccess) e = ssd::launch_chunk_bwd(a, st);
    if (e == hipSuccess) e = mark(3);
    const size_t bc = static_cast<size_t>(batch) * seqlen * ngroups * dstate;
    if (e == hipSuccess)
        e = ssd::launch_bwd_reduce(a.dB_part, a.dC_part, ws.nblk, bc, bf16, dB, dC, st);
    // stage 1: dt, A, dt bias
    if (e == hipSuccess)
        e = ssd::launch_bwd_dt(dt, A, a.ds, a.dw, batch, seqlen, nheads, Q, bf16, o, ddt,
                               f32(ws.dA_off), f32(ws.dbias_off), st);
    const int nbc = batch * nC;
    if (e == hipSuccess) {
        const float *parts[3] = {f32(ws.dA_off), f32(ws.dbias_off), a.dD_part};
        float *outs[3] = {dA, ddt_bias, dD};
        e = ssd::launch_bwd_head_sum(parts, outs, 3, nbc, nheads, st);
    }
    if (e == hipSuccess) e = mark(4);
    return e;
}

}  // namespace

extern "C" {


int ssd_backward_timed(const void *x, const void *dt, const float *A, const void *B,
                       const void *C, const float *D, const float *init_state, const void *dy,
                       const float *dfinal_state, int batch, int seqlen, int nheads, int headdim,
                       int ngroups, int dstate, int dtype, void *dx, void *ddt, float *dA,
                       void *dB, void *dC, float *dD, float *dinit_state, float *ddt_bias,
                       void *workspace, size_t workspace_bytes, const ssd_options *opts,
                       void *stream, void *const *events) {
    if (!x || !dt || !A || !B || !C || !dy || !dx || !ddt || !dA || !dB || !dC) return SSD_ERR_NULL;
    int rc = check_dims(batch, seqlen, nheads, headdim, ngroups, dstate);
    if (rc != SSD_OK) return rc;
    if (!valid_dtype(dtype)) return SSD_ERR_UNSUPPORTED;
    const bool bf16 = dtype == SSD_BF16;
    const int nk = ssd::kernel_dstate(dstate);
    if (!ssd::bwd_chunk(nk, bf16)) return SSD_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(B) || !aligned16(C) || !aligned16(dy) || !aligned16(dx) ||
        !aligned16(dB) || !aligned16(dC) || (init_state && !aligned16(init_state)) ||
        (dfinal_state && !aligned16(dfinal_state)) || (dinit_state && !aligned16(dinit_state)))
        return SSD_ERR_UNSUPPORTED;
    ssd::DtOpts o;
    rc = dt_opts(opts, o);
    if (rc != SSD_OK) return rc;
    const BwdWorkspace ws = bwd_layout(batch, seqlen, nheads, headdim, ngroups, nk, bf16);
    const size_t need = bwd_need(ws, batch, seqlen, nheads, headdim, ngroups, dstate, nk, bf16);
    if (!workspace || workspace_bytes < need) return SSD_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0) return SSD_ERR_WORKSPACE;
    char *base = static_cast<char *>(workspace);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (nk == dstate)
        return status_of(backward_run(ws, x, dt, A, B, C, D, init_state, dy, dfinal_state, batch,
                                      seqlen, nheads, ngroups, nk, bf16, dx, ddt, dA, dB, dC, dD,
                                      dinit_state, ddt_bias, base, o, st, events));
    // zero-padded to the kernels' state size (pad.hip): B, C and the states
    // in, their gradients cut back to dstate. After the kernels' workspace:
    // B', C', dB', dC' [Bt][L][G][nk] (input dtype), then the initial state,
    // the final state's gradient and the initial state's gradient [Bt][H][P][nk]
    const PadLayout pl = pad_layout(batch, seqlen, nheads, headdim, ngroups, nk, bf16);
    char *pb = base + align_up(ws.total);
    void *Bp = pb, *Cp = pb + pl.bc, *dBp = pb + 2 * pl.bc, *dCp = pb + 3 * pl.bc;
    float *ip = reinterpret_cast<float *>(pb + 4 * pl.bc);
    float *dfp = reinterpret_cast<float *>(pb + 4 * pl.bc + pl.st);
    float *dip = reinterpret_cast<float *>(pb + 4 * pl.bc + 2 * pl.st);
    const size_t bc_rows = (size_t)batch * seqlen * ngroups, st_rows = (size_t)batch * nheads * headdim;
    const int es = bf16 ? 2 : 4;
    hipError_t e = ssd::launch_pad_rows(B, Bp, bc_rows, dstate, nk, es, st);
    if (e == hipSuccess) e = ssd::launch_pad_rows(C, Cp, bc_rows, dstate, nk, es, st);
    if (e == hipSuccess && init_state)
        e = ssd::launch_pad_rows(init_state, ip, st_rows, dstate, nk, 4, st);
    if (e == hipSuccess && dfinal_state)
        e = ssd::launch_pad_rows(dfinal_state, dfp, st_rows, dstate, nk, 4, st);
    if (e == hipSuccess)
        e = backward_run(ws, x, dt, A, Bp, Cp, D, init_state ? ip : nullptr, dy,
                         dfinal_state ? dfp : nullptr, batch, seqlen, nheads, ngroups, nk, bf16,
                         dx, ddt, dA, dBp, dCp, dD, dinit_state ? dip : nullptr, ddt_bias, base, o,
                         st, events);
    if (e == hipSuccess) e = ssd::launch_pad_rows(dBp, dB, bc_rows, nk, dstate, es, st);
    if (e == hipSuccess) e = ssd::launch_pad_rows(dCp, dC, bc_rows, nk, dstate, es, st);
    if (e == hipSuccess && dinit_state)
        e = ssd::launch_pad_rows(dip, dinit_state, st_rows, nk, dstate, 4, st);
    return status_of(e);
}

int ssd_forward_timed(const void *x, const void *dt, const float *A, const void *B,
                      const void *C, const float *D, int batch, int seqlen, int nheads,
                      int headdim, int ngroups, int dstate, int chunk, int dtype,
                      const float *init_state, void *y, float *final_state, void *workspace,
                      size_t workspace_bytes, void *stream, void *const *events) {
    return ssd_forward_ex(x, dt, A, B, C, D, batch, seqlen, nheads, headdim, ngroups, dstate,
                          chunk, dtype, init_state, y, final_state, workspace, workspace_bytes,
                          nullptr, stream, events);
}

int ssd_forward(const void *x, const void *dt, const float *A, const void *B, const void *C,
                const float *D, int batch, int seqlen, int nheads, int headdim, int ngroups,
                int dstate, int chunk, int dtype, const float *init_state, void *y,
                float *final_state, void *workspace, size_t workspace_bytes, void *stream) {
    return ssd_forward_ex(x, dt, A, B, C, D, batch, seqlen, nheads, headdim, ngroups, dstate,
                          chunk, dtype, init_state, y, final_state, workspace, workspace_bytes,
                          nullptr, stream, nullptr);
}

int ssd_step_ex(float *state, const void *x, const void *dt, const float *A, const void *B,
                const void *C, const float *D, int batch, int nheads, int headdim, int ngroups,
                int dstate, int dtype, void *y, const ssd_options *opts, void *stream) {
    if (!state || !x || !dt || !A || !B || !C || !y) return SSD_ERR_NULL;
    int rc = check_dims(batch, 1, nheads, headdim, ngroups, dstate);
    if (rc != SSD_OK) return rc;
    if (!valid_dtype(dtype)) return SSD_ERR_UNSUPPORTED;
    if (!aligned16(state)) return SSD_ERR_UNSUPPORTED;
    ssd::DtOpts o;
    rc = dt_opts(opts, o);
    if (rc != SSD_OK) return rc;
    return status_of(ssd::launch_decode_step(state, x, dt, A, B, C, D, batch, nheads, ngroups,
                                             dstate, dtype == SSD_BF16, o, y,
                                             static_cast<hipStream_t>(stream)));
}

int ssd_step(float *state, const void *x, const void *dt, const float *A, const void *B,
             const void *C, const float *D, int batch, int nheads, int headdim, int ngroups,
             int dstate, int dtype, void *y, void *stream) {
    return ssd_step_ex(state, x, dt, A, B, C, D, batch, nheads, headdim, ngroups, dstate, dtype, y,
                       nullptr, stream);
}

}  // extern "C"
