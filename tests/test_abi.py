"""The C-ABI library on the CPU: it loads, exports every declared symbol, sizes
its workspace as documented, and rejects bad arguments before touching the GPU
(every call here fails validation, so no HIP call is made)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")
LIB = os.path.join(ROOT, "structured_state_space_ssd_amd", "libssd.so")

SSD_OK, SSD_ERR_NULL, SSD_ERR_SHAPE, SSD_ERR_UNSUPPORTED, SSD_ERR_WORKSPACE, SSD_ERR_HIP = 0, -1, -2, -3, -4, -5
SSD_ERR_OPTION = -6


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|size_t|int)\s*(ssd_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libssd.so is not built (run __graft_entry__.build())")
    import torch  # noqa: F401  (binds the HIP runtime the way the package does)
    from structured_state_space_ssd_amd import _native
    return _native.lib


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("ssd_forward", "ssd_step", "ssd_forward_workspace_size", "ssd_strerror",
                     "ssd_chunk_cumsum", "ssd_chunk_state", "ssd_state_passing", "ssd_chunk_cb",
                     "ssd_chunk_scan", "ssd_forward_timed", "ssd_chunk_cb_size", "ssd_forward_ex",
                     "ssd_step_ex", "ssd_forward_varlen", "ssd_forward_varlen_workspace_size",
                     "ssd_backward", "ssd_backward_workspace_size", "ssd_forward_plan",
                     "ssd_forward_plan_info"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(LIB)
    for name in declared_functions():
        assert hasattr(raw, name), f"{name} declared in ssd.h but not exported"


def test_strerror(lib):
    for code in (SSD_OK, SSD_ERR_NULL, SSD_ERR_SHAPE, SSD_ERR_UNSUPPORTED, SSD_ERR_WORKSPACE, SSD_ERR_HIP,
                 SSD_ERR_OPTION, 42):
        s = lib.ssd_strerror(code)
        assert isinstance(s, bytes) and len(s) > 0
    assert lib.ssd_strerror(42) == b"unknown status"


def _cb_expected(Bt, L, G, Q, dtype):
    nC = -(-L // Q)
    nt = Q // 16
    return Bt * nC * G * (nt // 2) * (nt // 2 + 1) * 64 * 8 * (2 if dtype == 1 else 4)


def _ws_expected(Bt, L, H, P, G, N, Q, dtype):
    al = lambda v: (v + 255) // 256 * 256
    nC = -(-L // Q)
    cs = Bt * H * nC * Q * 4  # dA_cumsum, and the same again for delta
    st = Bt * nC * H * P * N * 4
    ci = Bt * nC * H * P * N * (2 if dtype == 1 else 4)
    # the C B^T scratch is needed by the float path only (bf16 forms the tiles on chip)
    cb = al(_cb_expected(Bt, L, G, Q, dtype)) if dtype == 0 else 0
    return al(cs) + al(cs) + al(st) + al(ci) + cb


class Plan(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int), ("segments", ctypes.c_int), ("pieces", ctypes.c_int),
                ("block_tokens", ctypes.c_int), ("segment_blocks", ctypes.c_int),
                ("piece_blocks", ctypes.c_int), ("kernel_dstate", ctypes.c_int),
                ("workspace_bytes", ctypes.c_size_t)]


def plan_info(lib, Bt, L, H, P, G, N, Q, dtype, dt=256):
    p = Plan()
    rc = ctypes.CDLL(LIB).ssd_forward_plan_info(Bt, L, H, P, G, N, Q, dtype, ctypes.c_void_p(dt),
                                                ctypes.byref(p))
    return rc, p


def _scratch_expected(Bt, H, N, S, K):
    """The single-pass path's scratch: one float32 P x N state and one float32
    log2-decay per piece of the first S-1 segments of every (batch, head)."""
    pieces = Bt * H * (S - 1) * K
    return pieces * 64 * N * 4 + pieces * 4


@pytest.mark.parametrize("dims", [(3, 77, 5, 64, 5, 32, 128, 0), (1, 1, 1, 64, 1, 16, 64, 0),
                                  (8, 2048, 68, 64, 4, 64, 256, 1), (2, 300, 4, 64, 2, 128, 64, 1)])
def test_workspace_size_stage_path(lib, dims):
    # float32, N 16 / 32, heads not a multiple of 8: the stage kernels and their layout
    assert lib.ssd_forward_workspace_size(*dims) == _ws_expected(*dims)
    rc, p = plan_info(lib, *dims)
    assert rc == SSD_OK and p.path == 0 and p.segments == 0 and p.block_tokens == dims[6]
    assert p.workspace_bytes == _ws_expected(*dims)
    Bt, L, H, P, G, N, Q, dt = dims
    assert lib.ssd_chunk_cb_size(Bt, L, G, Q, dt) == _cb_expected(Bt, L, G, Q, dt)


SINGLE_PASS = [(8, 2048, 80, 64, 1, 64, 256, 1), (1, 65536, 80, 64, 8, 128, 256, 1),
               (4, 4096, 32, 64, 1, 256, 128, 1), (1, 2000, 16, 64, 1, 64, 256, 1),
               (1, 1000, 16, 64, 2, 64, 256, 1), (1, 37 * 64 + 13, 16, 64, 2, 128, 256, 1),
               (1, 16384, 16, 64, 2, 256, 128, 1), (1, 100, 8, 64, 1, 64, 64, 1)]


@pytest.mark.parametrize("dims", SINGLE_PASS)
def test_workspace_size_single_pass(lib, dims):
    """The single-pass path needs exactly the scratch its plan writes: nothing
    with one segment, one state and decay per piece otherwise (the segment
    kernels write units * (S-1) * K pieces, so this is the bound every write
    stays inside)."""
    Bt, L, H, P, G, N, Q, dt = dims
    rc, p = plan_info(lib, *dims)
    assert rc == SSD_OK and p.path == 1 and p.block_tokens == 64
    blocks = -(-L // 64)
    assert p.segments >= 1 and p.segment_blocks * (p.segments - 1) < blocks <= p.segment_blocks * p.segments
    if p.segments == 1:
        assert p.pieces == 0 and p.workspace_bytes == 0
    else:
        assert p.pieces >= 1 and p.piece_blocks * p.pieces == p.segment_blocks
        assert p.workspace_bytes == _scratch_expected(Bt, H, N, p.segments, p.pieces)
    assert lib.ssd_forward_workspace_size(*dims) == p.workspace_bytes
    # an unaligned dt takes the stage kernels, with their layout
    rc, q = plan_info(lib, *dims, dt=258)
    assert rc == SSD_OK and q.path == 0 and q.workspace_bytes == _ws_expected(*dims)


def test_plan_info_sweep(lib):
    """Over a sweep of shapes: segments only when the (batch, head) pairs alone
    leave the GPU part idle, at least 4 blocks per segment, pieces of at least
    2 blocks, and never more pieces than the segment-state kernel fills the GPU
    with (so the scratch stays a few tens of MB)."""
    slots = {64: 3 * 256, 128: 2 * 256, 256: 256}
    for N in (64, 128, 256):
        for Bt, H in ((1, 8), (1, 16), (2, 16), (1, 80), (4, 32), (8, 80), (3, 64)):
            for L in (1, 64, 255, 256, 1000, 4096, 20000, 65536):
                rc, p = plan_info(lib, Bt, L, H, 64, 1, N, 256, 1)
                assert rc == SSD_OK and p.path == 1
                blocks = -(-L // 64)
                if Bt * H >= slots[N] or blocks < 8:
                    assert p.segments == 1, (N, Bt, H, L)
                if p.segments > 1:
                    assert p.segment_blocks >= 4 and p.piece_blocks >= 2 or p.pieces == 1
                    assert Bt * H * p.segments <= slots[N] + Bt * H
                    assert p.workspace_bytes <= 64 << 20, (N, Bt, H, L, p.workspace_bytes)
                    assert p.workspace_bytes == _scratch_expected(Bt, H, N, p.segments, p.pieces)


def test_plan_info_rejects(lib):
    rc, p = plan_info(lib, 0, 10, 8, 64, 1, 64, 64, 1)
    assert rc == SSD_ERR_SHAPE and p.workspace_bytes == 0
    rc, _ = plan_info(lib, 1, 10, 8, 64, 1, 40, 64, 1)
    assert rc == SSD_ERR_UNSUPPORTED
    assert ctypes.CDLL(LIB).ssd_forward_plan_info(1, 10, 8, 64, 1, 64, 64, 1, None, None) == SSD_ERR_NULL


@pytest.mark.parametrize("dims", [(16384, 80, 64, 1, 64, 256, 1), (700, 4, 64, 2, 64, 64, 0),
                                  (1, 1, 64, 1, 16, 64, 1)])
def test_varlen_workspace_size(lib, dims):
    L, H, P, G, N, Q, dt = dims
    al = lambda v: (v + 255) // 256 * 256
    seg = al(-(-L // Q) * Q * 4)  # one int32 per token position
    assert lib.ssd_forward_varlen_workspace_size(*dims) == _ws_expected(1, L, H, P, G, N, Q, dt) + seg


def test_workspace_size_invalid(lib):
    assert lib.ssd_forward_workspace_size(0, 10, 1, 64, 1, 16, 64, 1) == 0
    assert lib.ssd_forward_workspace_size(1, 10, 1, 64, 1, 40, 64, 1) == 0
    assert lib.ssd_forward_workspace_size(1, 10, 1, 64, 1, 272, 64, 1) == 0
    assert lib.ssd_forward_workspace_size(1, 10, 1, 64, 1, 16, 0, 1) == 0
    assert lib.ssd_forward_workspace_size(1, 10, 1, 64, 1, 16, 64, 5) == 0
    assert lib.ssd_chunk_cb_size(1, 10, 1, 96, 1) == 0


FAKE = ctypes.c_void_p(0x100000)  # aligned, never dereferenced: every call below fails its checks first


def _fwd(lib, **kw):
    a = dict(x=FAKE, dt=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, batch=1, seqlen=128, nheads=4,
             headdim=64, ngroups=1, dstate=64, chunk=64, dtype=1, init=None, y=FAKE, fs=None,
             ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return lib.ssd_forward(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["batch"], a["seqlen"],
                           a["nheads"], a["headdim"], a["ngroups"], a["dstate"], a["chunk"], a["dtype"],
                           a["init"], a["y"], a["fs"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), SSD_ERR_NULL),
    (dict(y=None), SSD_ERR_NULL),
    (dict(A=None), SSD_ERR_NULL),
    (dict(batch=0), SSD_ERR_SHAPE),
    (dict(seqlen=0), SSD_ERR_SHAPE),
    (dict(nheads=6, ngroups=4), SSD_ERR_SHAPE),
    (dict(headdim=32), SSD_ERR_UNSUPPORTED),
    (dict(dstate=40), SSD_ERR_UNSUPPORTED),
    (dict(dstate=272), SSD_ERR_UNSUPPORTED),
    (dict(chunk=96), SSD_ERR_UNSUPPORTED),
    (dict(dtype=7), SSD_ERR_UNSUPPORTED),
    (dict(x=ctypes.c_void_p(0x100002)), SSD_ERR_UNSUPPORTED),
    (dict(ws=None), SSD_ERR_WORKSPACE),
    (dict(wsb=1024), SSD_ERR_WORKSPACE),
    (dict(ws=ctypes.c_void_p(0x100010)), SSD_ERR_WORKSPACE),
])
def test_forward_rejects(lib, kw, code):
    assert _fwd(lib, **kw) == code


def test_step_rejects(lib):
    args = [FAKE] * 7 + [4, 8, 64, 2, 128, 1, FAKE, None]
    ok = list(args)
    bad = list(ok); bad[0] = None
    assert lib.ssd_step(*bad) == SSD_ERR_NULL
    bad = list(ok); bad[8] = 6; bad[10] = 4  # nheads 6, ngroups 4
    assert lib.ssd_step(*bad) == SSD_ERR_SHAPE
    bad = list(ok); bad[11] = 100
    assert lib.ssd_step(*bad) == SSD_ERR_UNSUPPORTED
    bad = list(ok); bad[9] = 128
    assert lib.ssd_step(*bad) == SSD_ERR_UNSUPPORTED


def test_stage_entry_points_reject(lib):
    assert lib.ssd_chunk_cumsum(None, FAKE, 1, 10, 2, 64, 1, FAKE, None, None, None) == SSD_ERR_NULL
    assert lib.ssd_chunk_cumsum(FAKE, FAKE, 1, 10, 2, 100, 1, FAKE, None, None, None) == SSD_ERR_UNSUPPORTED
    assert lib.ssd_chunk_cumsum(FAKE, FAKE, 1, 10, 2, 64, 1, FAKE, ctypes.c_void_p(0x100004),
                                None, None) == SSD_ERR_UNSUPPORTED  # misaligned delta
    assert lib.ssd_chunk_state(FAKE, FAKE, FAKE, FAKE, 1, 10, 3, 64, 2, 64, 64, 1, FAKE, None) == SSD_ERR_SHAPE
    assert lib.ssd_chunk_state(FAKE, FAKE, None, FAKE, 1, 10, 2, 64, 2, 64, 64, 1, FAKE, None) == SSD_ERR_NULL
    assert lib.ssd_chunk_state(FAKE, FAKE, ctypes.c_void_p(0x100004), FAKE, 1, 10, 2, 64, 2, 64, 64, 1,
                               FAKE, None) == SSD_ERR_UNSUPPORTED  # misaligned delta
    assert lib.ssd_state_passing(FAKE, FAKE, None, 1, 10, 2, 64, 64, 64, 1, None, None, None) == SSD_ERR_NULL
    assert lib.ssd_state_passing(FAKE, FAKE, None, 1, 10, 2, 64, 64, 64, 4, FAKE, None, None) == SSD_ERR_UNSUPPORTED
    # ssd_chunk_scan(x, delta, dA, B, C, cb, D, chunk_init, Bt, L, H, P, G, N, Q, dtype, y, stream)
    assert lib.ssd_chunk_scan(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 10, 2, 64, 1, 64, 256, 9,
                              FAKE, None) == SSD_ERR_UNSUPPORTED
    assert lib.ssd_chunk_scan(FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, 1, 10, 2, 64, 1, 64, 256, 1,
                              FAKE, None) == SSD_ERR_NULL
    # bf16 reads B (not cb), float reads cb (not B)
    assert lib.ssd_chunk_scan(FAKE, FAKE, FAKE, None, FAKE, FAKE, None, FAKE, 1, 10, 2, 64, 1, 64, 256, 1,
                              FAKE, None) == SSD_ERR_NULL
    assert lib.ssd_chunk_scan(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 1, 10, 2, 64, 1, 64, 256, 0,
                              FAKE, None) == SSD_ERR_NULL
    assert lib.ssd_chunk_scan(FAKE, FAKE, FAKE, ctypes.c_void_p(0x100008), FAKE, None, None, FAKE, 1, 10,
                              2, 64, 1, 64, 256, 1, FAKE, None) == SSD_ERR_UNSUPPORTED
    assert lib.ssd_chunk_scan(FAKE, None, FAKE, FAKE, FAKE, None, None, FAKE, 1, 10, 2, 64, 1, 64, 256, 1,
                              FAKE, None) == SSD_ERR_NULL
    assert lib.ssd_chunk_scan(FAKE, ctypes.c_void_p(0x100004), FAKE, FAKE, FAKE, None, None, FAKE, 1, 10,
                              2, 64, 1, 64, 256, 1, FAKE, None) == SSD_ERR_UNSUPPORTED  # misaligned delta
    assert lib.ssd_chunk_cb(FAKE, None, 1, 10, 1, 64, 64, 1, FAKE, None) == SSD_ERR_NULL
    assert lib.ssd_chunk_cb(FAKE, FAKE, 1, 10, 1, 48, 64, 1, FAKE, None) == SSD_ERR_UNSUPPORTED


def _opts(**kw):
    from structured_state_space_ssd_amd import _native
    o = _native.SsdOptions(None, 0, 0, 0.0, 0.0, 0)
    for k, v in kw.items():
        setattr(o, k, v)
    return ctypes.byref(o)


BAD_OPTIONS = [
    (dict(discretization=2), SSD_ERR_OPTION),
    (dict(discretization=-1), SSD_ERR_OPTION),
    (dict(dt_clamp=1, dt_min=0.5, dt_max=0.1), SSD_ERR_OPTION),
    (dict(dt_clamp=1, dt_min=float("nan"), dt_max=0.1), SSD_ERR_OPTION),
    (dict(dt_clamp=1, dt_min=0.0, dt_max=float("nan")), SSD_ERR_OPTION),
    (dict(dt_bias=0x100002), SSD_ERR_UNSUPPORTED),  # misaligned float pointer
]


@pytest.mark.parametrize("kw,code", BAD_OPTIONS)
def test_options_rejected(lib, kw, code):
    """Invalid ssd_options are refused by every entry point that takes them
    (all other arguments valid, so the options check is what fails)."""
    o = _opts(**kw)
    ws = lib.ssd_forward_workspace_size(1, 128, 4, 64, 1, 64, 64, 1)
    rc = lib.ssd_forward_ex(FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 128, 4, 64, 1, 64, 64, 1, None, FAKE,
                            None, FAKE, ws, o, None, None)
    assert rc == code
    rc = lib.ssd_step_ex(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 4, 8, 64, 2, 128, 1, FAKE, o, None)
    assert rc == code
    rc = lib.ssd_chunk_cumsum(FAKE, FAKE, 1, 10, 2, 64, 1, FAKE, FAKE, o, None)
    assert rc == code


def test_options_checked_after_shapes(lib):
    """A bad size is reported as such even when the options are bad too."""
    o = _opts(discretization=7)
    rc = lib.ssd_forward_ex(FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 128, 4, 64, 1, 64, 64, 1, None, FAKE,
                            None, FAKE, 1 << 40, o, None, None)
    assert rc == SSD_ERR_SHAPE
    rc = lib.ssd_step_ex(None, FAKE, FAKE, FAKE, FAKE, FAKE, None, 4, 8, 64, 2, 128, 1, FAKE, o, None)
    assert rc == SSD_ERR_NULL


def _varlen(lib, **kw):
    a = dict(x=FAKE, dt=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, cu=FAKE, nseq=3, L=128, H=4, P=64,
             G=1, N=64, Q=64, dtype=1, y=FAKE, ss=None, ws=FAKE, wsb=1 << 40, opts=None)
    a.update(kw)
    return lib.ssd_forward_varlen(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["cu"], a["nseq"],
                                  a["L"], a["H"], a["P"], a["G"], a["N"], a["Q"], a["dtype"], a["y"],
                                  a["ss"], a["ws"], a["wsb"], a["opts"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(cu=None), SSD_ERR_NULL),
    (dict(x=None), SSD_ERR_NULL),
    (dict(nseq=0), SSD_ERR_SHAPE),
    (dict(L=0), SSD_ERR_SHAPE),
    (dict(H=6, G=4), SSD_ERR_SHAPE),
    (dict(N=48), SSD_ERR_UNSUPPORTED),
    (dict(Q=32), SSD_ERR_UNSUPPORTED),
    (dict(cu=ctypes.c_void_p(0x100002)), SSD_ERR_UNSUPPORTED),
    (dict(ss=ctypes.c_void_p(0x100008)), SSD_ERR_UNSUPPORTED),
    (dict(ws=None), SSD_ERR_WORKSPACE),
    (dict(wsb=4096), SSD_ERR_WORKSPACE),
])
def test_varlen_rejects(lib, kw, code):
    assert _varlen(lib, **kw) == code


def test_varlen_rejects_bad_options(lib):
    assert _varlen(lib, opts=_opts(discretization=3)) == SSD_ERR_OPTION


def _bwd(lib, **kw):
    a = dict(x=FAKE, dt=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, init=None, dy=FAKE, dfinal=None,
             Bt=1, L=128, H=4, P=64, G=1, N=64, dtype=1, dx=FAKE, ddt=FAKE, dA=FAKE, dB=FAKE,
             dC=FAKE, dD=None, dinit=None, dbias=None, ws=FAKE, wsb=1 << 40, opts=None)
    a.update(kw)
    return lib.ssd_backward(*(a[k] for k in ("x", "dt", "A", "B", "C", "D", "init", "dy", "dfinal",
                                             "Bt", "L", "H", "P", "G", "N", "dtype", "dx", "ddt",
                                             "dA", "dB", "dC", "dD", "dinit", "dbias", "ws", "wsb",
                                             "opts")), None)


@pytest.mark.parametrize("kw,code", [
    (dict(dy=None), SSD_ERR_NULL),
    (dict(dx=None), SSD_ERR_NULL),
    (dict(dA=None), SSD_ERR_NULL),
    (dict(Bt=0), SSD_ERR_SHAPE),
    (dict(H=6, G=4), SSD_ERR_SHAPE),
    (dict(N=40), SSD_ERR_UNSUPPORTED),
    (dict(dtype=0, N=128), SSD_ERR_UNSUPPORTED),   # float32 backward: N <= 64
    (dict(dtype=0, N=96), SSD_ERR_UNSUPPORTED),    # ... padded to 128
    (dict(dx=ctypes.c_void_p(0x100008)), SSD_ERR_UNSUPPORTED),
    (dict(ws=None), SSD_ERR_WORKSPACE),
    (dict(wsb=4096), SSD_ERR_WORKSPACE),
    (dict(opts=_opts(discretization=9)), SSD_ERR_OPTION),
])
def test_backward_rejects(lib, kw, code):
    assert _bwd(lib, **kw) == code


def test_backward_workspace_size(lib):
    assert lib.ssd_backward_workspace_size(8, 2048, 80, 64, 1, 64, 1) > 0
    assert lib.ssd_backward_workspace_size(1, 256, 2, 64, 1, 128, 0) == 0  # unsupported
    assert lib.ssd_backward_workspace_size(1, 256, 2, 64, 1, 64, 0) > 0


def test_forward_plan(lib):
    # which path ssd_forward takes (host arithmetic only): segments of the
    # single-pass kernel, 0 for the stage kernels, a status for bad sizes
    al, off = 256, 258  # an aligned and a misaligned dt address (never read)
    plan = lambda Bt, L, H, G, N, Q, dtype=1, dt=al: lib.ssd_forward_plan(Bt, L, H, 64, G, N, Q,
                                                                           dtype, dt)
    assert plan(8, 2048, 80, 1, 64, 256) == 1       # enough (batch, head) pairs
    assert plan(1, 65536, 80, 8, 128, 256) > 1     # few pairs, long sequence: segments
    assert plan(1, 100, 8, 1, 64, 64) == 1         # too short to cut
    assert plan(4, 4096, 32, 1, 256, 128) == 2     # N 256: one workgroup per CU, 2 segments
    assert plan(8, 2048, 80, 1, 32, 256) == 0      # N 32: stage kernels
    assert plan(8, 2048, 80, 1, 64, 256, dtype=0) == 0   # float32: stage kernels
    assert plan(8, 2048, 68, 4, 64, 256) == 0      # heads not a multiple of 8
    assert plan(8, 2048, 80, 1, 64, 256, dt=off) == 0    # dt not 16-byte aligned
    assert plan(0, 2048, 80, 1, 64, 256) == SSD_ERR_SHAPE
    assert plan(8, 2048, 80, 1, 64, 100) == SSD_ERR_UNSUPPORTED
    # segments never outnumber the 4-block minimum, and grow as pairs shrink
    for L in (256, 1000, 4096, 65536):
        s = [plan(1, L, H, 1, 64, 256) for H in (512, 64, 16, 8)]
        assert s == sorted(s) and s[-1] <= max(1, -(-L // 64) // 4), (L, s)


SSD_ERR_TOO_LARGE = -7


def _static(lib, **kw):
    a = dict(x=FAKE, dt=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, batch=1, seqlen=128, nheads=4,
             headdim=64, ngroups=1, dstate=64, chunk=64, dtype=1, init=None, y=FAKE, fs=None,
             opts=None, stream=None)
    a.update(kw)
    return lib.ssd_forward_static(*(a[k] for k in ("x", "dt", "A", "B", "C", "D", "batch", "seqlen",
                                                   "nheads", "headdim", "ngroups", "dstate", "chunk",
                                                   "dtype", "init", "y", "fs", "opts", "stream")))


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), SSD_ERR_NULL),
    (dict(batch=0), SSD_ERR_SHAPE),
    (dict(dstate=40), SSD_ERR_UNSUPPORTED),
    (dict(opts=_opts(discretization=4)), SSD_ERR_OPTION),
    # the stage kernels' workspace for 8 x 2048 tokens x 80 heads in float32 is far
    # beyond the fixed 32 MiB array: refused before anything touches the GPU
    (dict(batch=8, seqlen=2048, nheads=80, dtype=0), SSD_ERR_TOO_LARGE),
    (dict(batch=1, seqlen=65536, nheads=80, ngroups=8, dstate=128, dt=ctypes.c_void_p(0x100002)),
     SSD_ERR_TOO_LARGE),
])
def test_forward_static_rejects(lib, kw, code):
    assert _static(lib, **kw) == code
    assert lib.ssd_strerror(SSD_ERR_TOO_LARGE) != b"unknown status"


@pytest.mark.parametrize("N", [48, 80, 96, 112, 144, 160, 176, 192, 208, 224, 240])
def test_plan_info_padded_dstate(lib, N):
    """A state size outside 16, 32, 64, 128, 256 runs the kernels of the next
    of these on zero-padded copies of B, C and the states: the plan names the
    kernels' size, and the workspace is the kernels' own need plus the copies
    (B' and C' in the input dtype, two float32 states)."""
    al = lambda v: (v + 255) // 256 * 256
    nk = next(k for k in (64, 128, 256) if N <= k)
    for dims, dtype in (((8, 2048, 80, 64, 1), 1), ((1, 4096, 16, 64, 2), 1), ((2, 300, 4, 64, 2), 0)):
        Bt, L, H, P, G = dims
        rc, p = plan_info(lib, Bt, L, H, P, G, N, 128, dtype)
        assert rc == SSD_OK and p.kernel_dstate == nk
        rc, q = plan_info(lib, Bt, L, H, P, G, nk, 128, dtype)
        assert (p.path, p.segments, p.pieces) == (q.path, q.segments, q.pieces)
        e = 2 if dtype == 1 else 4
        pad = 2 * al(Bt * L * G * nk * e) + 2 * al(Bt * H * P * nk * 4)
        assert p.workspace_bytes == al(q.workspace_bytes) + pad
        assert lib.ssd_forward_workspace_size(Bt, L, H, P, G, N, 128, dtype) == p.workspace_bytes
    # the backward: its kernels' layout at nk plus B', C', dB', dC' and three states
    Bt, L, H, P, G = 2, 300, 4, 64, 2
    if nk <= 256:
        w0 = lib.ssd_backward_workspace_size(Bt, L, H, P, G, nk, 1)
        w1 = lib.ssd_backward_workspace_size(Bt, L, H, P, G, N, 1)
        assert w1 == al(w0) + 4 * al(Bt * L * G * nk * 2) + 3 * al(Bt * H * P * nk * 4)


def test_padded_dstate_kernel_sizes_only_on_stages_and_varlen(lib):
    # the stage entry points and the packed forward take the kernels' sizes only
    assert lib.ssd_chunk_cb(FAKE, FAKE, 1, 10, 1, 48, 64, 1, FAKE, None) == SSD_ERR_UNSUPPORTED
    assert lib.ssd_chunk_state(FAKE, FAKE, FAKE, FAKE, 1, 10, 2, 64, 2, 96, 64, 1, FAKE, None) == SSD_ERR_UNSUPPORTED
    assert _varlen(lib, N=48) == SSD_ERR_UNSUPPORTED
    assert lib.ssd_forward_varlen_workspace_size(100, 4, 64, 1, 48, 64, 1) == 0
