"""Extreme shapes against the fp64 oracle: one very long chain (a single lane
block walking about a million steps, so every tile's look-back waits on the
one before it), a single time step across four million lanes, and the
complex and fused-transition forms on long single-lane chains.  Transitions
are drawn in U(0.5, 0.99) so that no lane's memory spans the whole chain."""
import numpy as np
import pytest

import oracle
import workloads as W
from _gpu import log

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import linear_recurrence_sequence_diag_amd as lr  # noqa: E402
from test_gpu_parity import check_against_oracle, run_pair  # noqa: E402


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lr.library()


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,D", [(1, (1 << 20) + 3, 1), (1, (1 << 18) + 7, 8), (2, 100003, 3)],
                         ids=["T1M_D1", "T256k_D8", "B2_T100k_D3"])
@pytest.mark.parametrize("algo,chunk", [("auto", 0), ("fused", 0), ("chunked", 1024), ("seq", 0)],
                         ids=["auto", "fused", "chunked1024", "seq"])
def test_long_single_chain(B, T, D, dt, algo, chunk):
    # AUTO takes the three-launch form on the million-step one-block chain;
    # the fused form is run explicitly for its chained look-backs
    inp = W.random_inputs(B, T, D, dt, seed=51, a_lo=0.5, a_hi=0.99)
    res = run_pair(inp, algo, chunk, chunk)
    check_against_oracle(inp, res)
    log(f"{algo} {dt} B{B} T{T} D{D}: within tolerance")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("algo", ["auto", "seq", "fused"])
def test_many_lanes_unaligned_rows(dt, algo):
    """Rows that are not 16-byte aligned over 300K lanes and a few steps: the
    walk writes blocks shared between neighbouring lanes (and wavefronts and
    batch rows end mid-block), the tiles write blocks shared across their
    row groups; every element against the oracle, with h0 and grad_last."""
    B, T, D = 300, 5, 1001
    inp = W.random_inputs(B, T, D, dt, seed=59, a_lo=0.5, a_hi=0.99)
    rng = np.random.default_rng(60)
    h0 = rng.standard_normal((B, D)).astype(np.float32)
    gl = rng.standard_normal((B, D)).astype(np.float32)
    check_against_oracle(inp, run_pair(inp, algo, 0, 0, h0=h0, gl=gl), h0=h0, gl=gl)
    log(f"{algo} {dt} B{B} T{T} D{D}: within tolerance")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("algo,chunk", [("auto", 0), ("chunked", 16), ("seq", 0)],
                         ids=["auto", "chunked16", "seq"])
def test_single_step_many_lanes(dt, algo, chunk):
    inp = W.random_inputs(1, 1, (1 << 22) + 5, dt, seed=52, a_lo=0.5, a_hi=0.99)
    res = run_pair(inp, algo, chunk, chunk)
    check_against_oracle(inp, res)
    rng = np.random.default_rng(55)
    h0 = rng.standard_normal((1, (1 << 22) + 5)).astype(np.float32)
    gl = rng.standard_normal((1, (1 << 22) + 5)).astype(np.float32)
    check_against_oracle(inp, run_pair(inp, algo, chunk, chunk, h0=h0, gl=gl), h0=h0, gl=gl)
    res = run_pair(inp, algo, chunk, chunk)
    # one step from a zero state: out = b exactly, grad_b = grad_out exactly
    assert torch.equal(res[0], torch.from_numpy(np.ascontiguousarray(inp.b).view(
        np.int16 if dt == "bf16" else np.float32)).cuda().view(res[0].dtype))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_complex_long_single_lane(dt):
    from test_gpu_complex import check_c, check_c_grad_a, chost, cprev, run
    inp = W.complex_inputs(1, (1 << 18) + 5, 1, dt, seed=53, r_lo=0.5, r_hi=0.99, theta=np.pi)
    a, b, g = inp.c128("a"), inp.c128("b"), inp.c128("g")
    h, hl = oracle.complex_fwd(a, b)
    oga, ogb, _ = oracle.complex_bwd(a, h, g)
    for algo in ("fused", "seq"):
        res = run(inp, algo, need_grad_h0=False)
        check_c(f"{algo} out", chost(res[0], res[1]), h, dt)
        check_c(f"{algo} grad_b", chost(res[6], res[7]), ogb, dt)
        check_c_grad_a(chost(res[4], res[5]), oga, ogb, cprev(h, None), dt)
    log(f"complex {dt} T{(1 << 18) + 5} M1: within tolerance")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_fused_transition_long_single_lane(dt):
    from test_gpu_samu import Bounds, check_all, run
    inp = W.samu_inputs(1, (1 << 17) + 5, 1, dt, seed=54)
    eta, delta, nu_log, theta_log = inp.controls()
    bd = Bounds(eta, delta, nu_log, theta_log, inp.c128("b"), inp.c128("g"), dt)
    check_all(f"samu {dt} long", run(inp, need_grad_h0=False), bd)
    log(f"fused-transition {dt} T{(1 << 17) + 5} M1: within the derived bounds")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,D", [(100000, 3, 1), (4099, 5, 9), (1, 2, (1 << 21) + 1)],
                         ids=["B100k_T3_D1", "B4099_T5_D9", "T2_D2M"])
def test_many_short_series(B, T, D, dt):
    """Very many series of a few steps (one tile per series, tens of thousands
    of ticket holders per counter), and a two-step scan over two million lanes."""
    inp = W.random_inputs(B, T, D, dt, seed=56, a_lo=0.5, a_hi=0.99)
    for algo, chunk in (("auto", 0), ("chunked", 16)):
        check_against_oracle(inp, run_pair(inp, algo, chunk, chunk))
    log(f"{dt} B{B} T{T} D{D}: within tolerance")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_complex_many_short_series(dt):
    from test_gpu_complex import check_c, chost, run
    inp = W.complex_inputs(30000, 3, 3, dt, seed=57, r_lo=0.5, r_hi=0.99, theta=np.pi)
    a, b, g = inp.c128("a"), inp.c128("b"), inp.c128("g")
    h, _ = oracle.complex_fwd(a, b)
    _, ogb, _ = oracle.complex_bwd(a, h, g)
    for algo in ("fused", "seq"):
        res = run(inp, algo, need_grad_h0=False)
        check_c(f"{algo} out", chost(res[0], res[1]), h, dt)
        check_c(f"{algo} grad_b", chost(res[6], res[7]), ogb, dt)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,M", [(2, 1, (1 << 20) + 3), (20000, 2, 3)], ids=["T1_M1M", "B20k_T2_M3"])
def test_fused_transition_wide_and_many(B, T, M, dt):
    """Many modes in one step (per-mode partials over a single tile row) and
    many short series (per-token partials over a single lane block)."""
    from test_gpu_samu import Bounds, check_all, run
    inp = W.samu_inputs(B, T, M, dt, seed=58)
    eta, delta, nu_log, theta_log = inp.controls()
    bd = Bounds(eta, delta, nu_log, theta_log, inp.c128("b"), inp.c128("g"), dt)
    check_all(f"samu {dt} B{B} T{T} M{M}", run(inp, need_grad_h0=False), bd)


def offset_copy(t, elems=1):
    """The same values in a buffer whose data pointer is `elems` elements past
    a 16-byte boundary (a contiguous view with a storage offset)."""
    buf = torch.empty(t.numel() + elems, dtype=t.dtype, device=t.device)
    v = buf[elems:].view(t.shape)
    v.copy_(t)
    return v


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("algo,chunk,width", [("auto", 0, 0), ("fused", 256, 8), ("chunked", 64, 0),
                                              ("seq", 0, 0)],
                         ids=["auto", "fused256w8", "chunked64", "seq"])
def test_misaligned_pointers_with_aligned_rows(dt, algo, chunk, width):
    """D a multiple of the vector width but every array starting one element
    past a 16-byte boundary: the element-wise paths, through the raw C ABI
    (inputs and outputs misaligned)."""
    from _gpu import dev, host
    B, T, D = 2, 777, 128
    inp = W.random_inputs(B, T, D, dt, seed=59, a_lo=0.5, a_hi=0.99)
    a, b, g = (offset_copy(dev(x, dt)) for x in (inp.a, inp.b, inp.g))
    out, ga, gb = (offset_copy(torch.zeros_like(a)) for _ in range(3))
    last = torch.empty((B, D), device="cuda", dtype=torch.float32)
    assert a.data_ptr() % 16 != 0 and out.data_ptr() % 16 != 0
    code = lr.F32 if dt == "f32" else lr.BF16
    st = torch.cuda.current_stream().cuda_stream
    o = lr.make_opts(algo=algo, chunk=chunk, width=width)
    lr.scan_fwd_ex(a.data_ptr(), b.data_ptr(), out.data_ptr(), last.data_ptr(), B, T, D, code, st, o)
    lr.scan_bwd_ex(a.data_ptr(), out.data_ptr(), g.data_ptr(), None, ga.data_ptr(), gb.data_ptr(),
                   B, T, D, code, st, o)
    torch.cuda.synchronize()
    from _gpu import check_close, check_grad_a, prev_state
    h, hl = oracle.scan_fwd(inp.f64("a"), inp.f64("b"))
    oga, ogb, _ = oracle.scan_bwd(inp.f64("a"), h, inp.f64("g"))
    check_close("out", host(out), h, dt)
    check_close("last", host(last), hl, "f32")
    check_close("grad_b", host(gb), ogb, dt)
    check_grad_a(host(ga), oga, ogb, prev_state(h), dt)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_misaligned_pointers_complex_and_fused_transition(dt):
    """The complex and fused-transition forms on inputs that start one element
    past a 16-byte boundary (their outputs are allocated aligned)."""
    from _gpu import dev, dev_f32, host
    from test_gpu_complex import check_c, chost
    B, T, M = 2, 600, 64
    c = W.complex_inputs(B, T, M, dt, seed=60, r_lo=0.5, r_hi=0.99, theta=np.pi)
    t = {n: offset_copy(dev(getattr(c, n), dt)) for n in ("ar", "ai", "br", "bi", "gr", "gi")}
    o = lr.complex_scan(t["ar"], t["ai"], t["br"], t["bi"])
    g = lr.complex_scan_backward(t["ar"], t["ai"], offset_copy(o[0]), offset_copy(o[1]),
                                 t["gr"], t["gi"])
    torch.cuda.synchronize()
    a, b, gg = c.c128("a"), c.c128("b"), c.c128("g")
    h, _ = oracle.complex_fwd(a, b)
    _, ogb, _ = oracle.complex_bwd(a, h, gg)
    check_c("complex out", chost(o[0], o[1]), h, dt)
    check_c("complex grad_b", chost(g[2], g[3]), ogb, dt)

    from test_gpu_samu import Bounds, check
    from _gpu import TOL
    s = W.samu_inputs(B, T, M, dt, seed=61)
    ts = {n: offset_copy(dev(getattr(s, n), dt)) for n in ("eta", "delta", "br", "bi", "gr", "gi")}
    nl, tl = offset_copy(dev_f32(s.nu_log)), offset_copy(dev_f32(s.theta_log))
    ctl = (ts["eta"], ts["delta"], nl, tl)
    so = lr.samu_scan(*ctl, ts["br"], ts["bi"])
    sg = lr.samu_scan_backward(*ctl, offset_copy(so[0]), offset_copy(so[1]), ts["gr"], ts["gi"])
    torch.cuda.synchronize()
    eta, delta, nu_log, theta_log = s.controls()
    bd = Bounds(eta, delta, nu_log, theta_log, s.c128("b"), s.c128("g"), dt)
    rtol, atol = TOL[dt]
    check("samu out", host(so[0]) + 1j * host(so[1]), bd.h, atol + rtol * np.abs(bd.h) + bd.E_h)
    check("samu grad_eta", host(sg[0]), bd.ge, bd.tol_ge)
    check("samu grad_nu_log", host(sg[2]), bd.gn, bd.tol_gn)
