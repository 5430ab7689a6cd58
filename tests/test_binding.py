"""The Python binding's argument checks, on the CPU: the C ABI takes sizes,
not shapes, so every tensor whose shape the binding does not check against
the others could be read or written out of bounds by the kernels. Each
mis-shaped argument must raise ValueError naming it, before any device check
(so CPU tensors reach these checks); well-shaped CPU tensors then fail the
device check instead."""
import pytest

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ssd():
    import structured_state_space_ssd_amd as m
    return m


Bt, L, H, P, G, N = 2, 10, 8, 64, 2, 64
f32, bf = torch.float32, torch.bfloat16


def fwd_args(**over):
    a = dict(x=torch.zeros(Bt, L, H, P, dtype=bf), dt=torch.zeros(Bt, L, H, dtype=bf),
             A=torch.zeros(H), B=torch.zeros(Bt, L, G, N, dtype=bf),
             C=torch.zeros(Bt, L, G, N, dtype=bf), D=torch.zeros(H))
    a.update(over)
    return a


FORWARD_BAD = [
    ("A", dict(A=torch.zeros(H + 1))),
    ("D", dict(D=torch.zeros(H - 1))),
    ("init_state", dict(init_state=torch.zeros(Bt, H, P, N + 16))),
    ("init_state", dict(init_state=torch.zeros(Bt + 1, H, P, N))),
    ("dt_bias", dict(dt_bias=torch.zeros(2 * H))),
    ("shape mismatch", dict(dt=torch.zeros(Bt, L, H + 1, dtype=bf))),
    ("shape mismatch", dict(C=torch.zeros(Bt, L, G, 2 * N, dtype=bf))),
    ("shape mismatch", dict(B=torch.zeros(Bt + 1, L, G, N, dtype=bf))),
    ("y", dict(y=torch.zeros(Bt, L, H, P + 1, dtype=bf))),
]


@pytest.mark.parametrize("name,over", FORWARD_BAD, ids=[f"{n}-{i}" for i, (n, _) in enumerate(FORWARD_BAD)])
def test_forward_rejects_shapes(ssd, name, over):
    with pytest.raises(ValueError, match=name):
        ssd.forward(**fwd_args(**over))


def test_forward_well_shaped_cpu_tensors_fail_device_check(ssd):
    with pytest.raises(ValueError, match="GPU"):
        ssd.forward(**fwd_args(init_state=torch.zeros(Bt, H, P, N)))


BACKWARD_BAD = [
    ("A", dict(A=torch.zeros(1))),
    ("D", dict(D=torch.zeros(2 * H))),
    ("init_state", dict(init_state=torch.zeros(Bt, H, N, P + 1))),
    ("dfinal_state", dict(dfinal_state=torch.zeros(Bt, H + 1, P, N))),
    ("shape mismatch", dict(dy=torch.zeros(Bt, L - 1, H, P, dtype=bf))),
]


@pytest.mark.parametrize("name,over", BACKWARD_BAD, ids=[n for n, _ in BACKWARD_BAD])
def test_backward_rejects_shapes(ssd, name, over):
    a = fwd_args(dy=torch.zeros(Bt, L, H, P, dtype=bf))
    a.update(over)
    with pytest.raises(ValueError, match=name):
        ssd.backward(**a)


def test_varlen_rejects_shapes(ssd):
    a = dict(x=torch.zeros(L, H, P, dtype=bf), dt=torch.zeros(L, H, dtype=bf), A=torch.zeros(H),
             B=torch.zeros(L, G, N, dtype=bf), C=torch.zeros(L, G, N, dtype=bf), D=torch.zeros(H),
             cu_seqlens=torch.tensor([0, 4, L], dtype=torch.int32))
    for name, over in (("A", dict(A=torch.zeros(H + 2))), ("D", dict(D=torch.zeros(3))),
                       ("batch 1", dict(x=torch.zeros(2, L, H, P, dtype=bf))),
                       ("shape mismatch", dict(dt=torch.zeros(L, H - 1, dtype=bf)))):
        b = dict(a)
        b.update(over)
        with pytest.raises(ValueError, match=name):
            ssd.forward_varlen(**b)


def step_args(**over):
    a = dict(state=torch.zeros(Bt, H, P, N), x=torch.zeros(Bt, H, P, dtype=bf),
             dt=torch.zeros(Bt, H, dtype=bf), A=torch.zeros(H),
             B=torch.zeros(Bt, G, N, dtype=bf), C=torch.zeros(Bt, G, N, dtype=bf),
             D=torch.zeros(H))
    a.update(over)
    return a


STEP_BAD = [
    ("shape mismatch", dict(B=torch.zeros(1, G, N, dtype=bf), C=torch.zeros(1, G, N, dtype=bf))),
    ("shape mismatch", dict(state=torch.zeros(Bt, H, P, N + 16))),
    ("A", dict(A=torch.zeros(H // 2))),
    ("D", dict(D=torch.zeros(H + 8))),
    ("y", dict(y=torch.zeros(Bt, H + 1, P, dtype=bf))),
]


@pytest.mark.parametrize("name,over", STEP_BAD, ids=[f"{n}-{i}" for i, (n, _) in enumerate(STEP_BAD)])
def test_step_rejects_shapes(ssd, name, over):
    with pytest.raises(ValueError, match=name):
        ssd.step(**step_args(**over))


def test_step_well_shaped_cpu_tensors_fail_device_check(ssd):
    with pytest.raises(ValueError, match="GPU"):
        ssd.step(**step_args())
