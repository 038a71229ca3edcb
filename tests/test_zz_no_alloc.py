"""scan_fwd_noalloc, the forward that allocates nothing (its scratch is a
static device array), against scan_fwd_ex, the forward it is a variant of:
the same kernels on the same inputs, so the results must agree bit for bit.

Two calls in a row on one stream, the second on a smaller input (the static
array keeps the first call's contents, which the second call must not
depend on), for the automatic choice, the three-launch form and the state
options; and the argument errors of the entry point."""
import ctypes

import pytest

import workloads as W
from _gpu import dev, dev_f32, log

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import linear_recurrence_sequence_diag_amd as lr  # noqa: E402

NOALLOC_BYTES = 16 << 20


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lr.library()


def forward(fn, a, b, opts):
    B, T, D = a.shape
    out = torch.empty_like(a)
    last = torch.empty((B, D), device=a.device, dtype=torch.float32)
    fn(a.data_ptr(), b.data_ptr(), out.data_ptr(), last.data_ptr(), B, T, D,
       lr.dtype_code(a.dtype), torch.cuda.current_stream().cuda_stream, opts)
    return out, last


def inputs(B, T, D, dt, seed):
    r = W.random_inputs(B, T, D, dt, seed=seed, a_lo=0.5, a_hi=0.999)
    return dev(r.a, dt), dev(r.b, dt)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("algo", ["auto", "chunked"])
def test_noalloc_equals_the_allocating_forward(dt, algo):
    big = inputs(4, 8192, 1024, dt, seed=81)
    small = inputs(2, 3001, 200, dt, seed=82)   # ragged T and D
    o = lr.make_opts(algo=algo, chunk=64 if algo == "chunked" else 0)
    for x in (big, small):
        B, T, D = x[0].shape
        need = lr.scan_workspace_bytes(B, T, D, lr.dtype_code(x[0].dtype), o)
        assert 0 < need <= NOALLOC_BYTES, need
    # two calls in a row on one stream, no synchronisation between them
    got = [forward(lr.scan_fwd_noalloc, *big, o), forward(lr.scan_fwd_noalloc, *small, o)]
    ref = [forward(lr.scan_fwd_ex, *big, o), forward(lr.scan_fwd_ex, *small, o)]
    torch.cuda.synchronize()
    for k, (g, r) in enumerate(zip(got, ref)):
        assert torch.equal(g[0], r[0]), f"call {k}: out differs"
        assert torch.equal(g[1], r[1]), f"call {k}: last differs"
    log(f"noalloc {dt} {algo}: two calls bitwise equal to scan_fwd_ex")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_noalloc_with_state_and_resets(dt):
    B, T, D = 3, 5000, 520
    a, b = inputs(B, T, D, dt, seed=83)
    h0 = dev_f32(W.random_inputs(B, 1, D, "f32", seed=84).b[:, 0])
    g = torch.Generator().manual_seed(85)
    reset = (torch.rand((B, T), generator=g) < 0.01).to(torch.uint8).cuda()
    o = lr.make_opts(h0=h0, reset=reset)
    first = forward(lr.scan_fwd_noalloc, a, b, o)
    second = forward(lr.scan_fwd_noalloc, a[:, :1700].contiguous(), b[:, :1700].contiguous(),
                     lr.make_opts(h0=h0))
    ref1 = forward(lr.scan_fwd_ex, a, b, o)
    ref2 = forward(lr.scan_fwd_ex, a[:, :1700].contiguous(), b[:, :1700].contiguous(),
                   lr.make_opts(h0=h0))
    torch.cuda.synchronize()
    for g_, r_ in ((first, ref1), (second, ref2)):
        assert torch.equal(g_[0], r_[0]) and torch.equal(g_[1], r_[1])
    log(f"noalloc {dt}: h0 and resets bitwise equal to scan_fwd_ex")


def test_noalloc_argument_errors():
    lib = lr.library()
    # a shape whose forward scratch exceeds the static array: refused before any work
    B, T, D = 64, 4096, 2560
    o = lr.make_opts()
    assert lr.scan_workspace_bytes(B, T, D, lr.BF16, o) > NOALLOC_BYTES
    a = torch.empty((B, T, D), device="cuda", dtype=torch.bfloat16)
    b = torch.empty_like(a)
    out = torch.empty_like(a)
    last = torch.empty((B, D), device="cuda", dtype=torch.float32)
    st = torch.cuda.current_stream().cuda_stream
    rc = lib.scan_fwd_noalloc(a.data_ptr(), b.data_ptr(), out.data_ptr(), last.data_ptr(), B, T, D,
                              lr.BF16, st, ctypes.byref(o))
    assert rc == -9, rc
    assert "static buffer" in lr.status_string(rc)
    # a caller workspace contradicts the entry point's purpose
    ws = torch.empty(1 << 20, device="cuda", dtype=torch.uint8)
    o2 = lr.make_opts(workspace=ws)
    rc = lib.scan_fwd_noalloc(a.data_ptr(), b.data_ptr(), out.data_ptr(), last.data_ptr(), 2, 64,
                              64, lr.BF16, st, ctypes.byref(o2))
    assert rc == -5, rc
    assert lib.scan_fwd_noalloc(None, b.data_ptr(), out.data_ptr(), None, 2, 8, 4, lr.F32, st,
                                None) == -1
    torch.cuda.synchronize()
