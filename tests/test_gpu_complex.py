"""Complex diagonal scan (planar real / imaginary arrays) through the C ABI
against the fp64 complex oracle: every form, ragged and unaligned shapes,
h0 / grad_last / grad_h0 and the reset mask; bitwise determinism and
bitwise-identical look-back derivation; the real special case bit for bit;
the autograd wrapper; the full-size complex workload on sampled lanes.

Tolerances are those of the real scan applied to complex moduli: a part's
error is bounded by atol + rtol*|ref| with |ref| the complex modulus (a
part-wise relative bound would fail wherever one part cancels while the
other is large); grad_a by atol*(1 + |lambda| + |h_{t-1}|) + 2*rtol*|grad_a|."""
import numpy as np
import pytest

import oracle
import workloads as W
from _gpu import TOL, dev, dev_f32, host, log

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import linear_recurrence_sequence_diag_amd as lr  # noqa: E402


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lr.library()


def cdev(inp, name):
    dt = inp.workload.dtype
    return dev(getattr(inp, name + "r"), dt), dev(getattr(inp, name + "i"), dt)


def chost(re, im):
    return host(re) + 1j * host(im)


def check_c(name, got, ref, dtype):
    rtol, atol = TOL[dtype]
    err = np.maximum(np.abs(got.real - ref.real), np.abs(got.imag - ref.imag))
    tol = atol + rtol * np.abs(ref)
    bad = ~(err <= tol)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err / tol, 0)), err.shape)
        raise AssertionError(f"{name}: {int(bad.sum())} of {bad.size} outside tolerance; worst at "
                             f"{i}: got {got[i]!r} ref {ref[i]!r}")


def check_c_grad_a(got, ref, lam, hprev, dtype):
    rtol, atol = TOL[dtype]
    err = np.maximum(np.abs(got.real - ref.real), np.abs(got.imag - ref.imag))
    tol = atol * (1 + np.abs(lam) + np.abs(hprev)) + 2 * rtol * np.abs(ref)
    bad = ~(err <= tol)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err / tol, 0)), err.shape)
        raise AssertionError(f"grad_a: {int(bad.sum())} outside the propagated bound; worst at {i}:"
                             f" got {got[i]!r} ref {ref[i]!r}")


def cprev(h, h0):
    B, T, M = h.shape
    first = np.zeros((B, 1, M), complex) if h0 is None else h0[:, None, :]
    return np.concatenate([first, h[:, :-1]], axis=1)


def run(inp, algo, h0=None, gl=None, mask=None, polls=0, need_grad_h0=True):
    ar, ai = cdev(inp, "a")
    br, bi = cdev(inp, "b")
    gr, gi = cdev(inp, "g")
    th0 = None if h0 is None else (dev_f32(h0.real), dev_f32(h0.imag))
    tgl = None if gl is None else (dev_f32(gl.real), dev_f32(gl.imag))
    tm = None if mask is None else torch.from_numpy(mask.astype(np.uint8)).cuda()
    out_r, out_i, last_r, last_i = lr.complex_scan(ar, ai, br, bi, h0=th0, algo=algo, polls=polls,
                                                   reset=tm)
    gar, gai, gbr, gbi, gh0 = lr.complex_scan_backward(ar, ai, out_r, out_i, gr, gi, grad_last=tgl,
                                                       h0=th0, algo=algo, polls=polls, reset=tm,
                                                       need_grad_h0=need_grad_h0)
    torch.cuda.synchronize()
    return out_r, out_i, last_r, last_i, gar, gai, gbr, gbi, gh0


def state_pair(B, M, seed):
    r = np.random.default_rng(seed)
    z = r.standard_normal((B, M)) + 1j * r.standard_normal((B, M))
    return (z.real.astype(np.float32) + 1j * z.imag.astype(np.float32))


SHAPES = [(2, 300, 72), (3, 1000, 130), (1, 4096, 256), (2, 333, 13), (1, 1, 1), (2, 129, 1),
          (300, 12, 1024), (140, 40, 2048)]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,M", SHAPES, ids=[f"B{b}T{t}M{m}" for b, t, m in SHAPES])
def test_complex_against_oracle(B, T, M, dt):
    inp = W.complex_inputs(B, T, M, dt, seed=5, r_lo=0.5, theta=np.pi)
    h0, gl = state_pair(B, M, 6), state_pair(B, M, 7)
    mask = np.random.default_rng(8).random((B, T)) < 0.03
    mask[0, 0] = True
    a, b, g = inp.c128("a"), inp.c128("b"), inp.c128("g")
    for m in (None, mask):
        h, hl = oracle.complex_fwd(a, b, h0=h0, reset=m)
        oga, ogb, ogh0 = oracle.complex_bwd(a, h, g, h0=h0, grad_last=gl, reset=m)
        for algo in ("seq", "fused", "auto"):
            res = run(inp, algo, h0=h0, gl=gl, mask=m)
            out, last = chost(res[0], res[1]), chost(res[2], res[3])
            ga, gb = chost(res[4], res[5]), chost(res[6], res[7])
            gh0 = host(res[8][0]) + 1j * host(res[8][1])
            tag = f"{algo}{'+reset' if m is not None else ''}"
            check_c(f"{tag} out", out, h, dt)
            check_c(f"{tag} last", last, hl, "f32" if dt == "bf16" else dt)
            check_c(f"{tag} grad_b", gb, ogb, dt)
            check_c_grad_a(ga, oga, ogb, cprev(h, h0), dt)
            rtol, atol = TOL[dt]
            assert np.all(np.abs(gh0 - ogh0) <= atol * (1 + np.abs(ogb[:, 0])) + 2 * rtol * np.abs(ogh0)), tag
            if m is not None:
                assert np.all(ga[m] == 0), f"{tag}: grad_a at a reset step"
    log(f"complex {dt} B{B} T{T} M{M}: seq and fused within tolerance, with and without resets")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_complex_fused_deterministic_and_derivation_bitwise(dt):
    inp = W.complex_inputs(2, 4096, 256, dt, seed=9, r_lo=0.9)
    h0, gl = state_pair(2, 256, 10), state_pair(2, 256, 11)
    mask = np.random.default_rng(12).random((2, 4096)) < 0.01
    r1 = run(inp, "fused", h0=h0, gl=gl, mask=mask)
    r2 = run(inp, "fused", h0=h0, gl=gl, mask=mask)
    r3 = run(inp, "fused", h0=h0, gl=gl, mask=mask, polls=1)
    names = ("out_r", "out_i", "last_r", "last_i", "grad_ar", "grad_ai", "grad_br", "grad_bi")
    for n, x, y, z in zip(names, r1[:8], r2[:8], r3[:8]):
        assert torch.equal(x, y), f"{n} not bitwise repeatable"
        assert torch.equal(x, z), f"{n} differs with polls=1"
    for x, y in zip(r1[8], r3[8]):
        assert torch.equal(x, y), "grad_h0 differs with polls=1"


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_complex_with_zero_imaginary_parts_is_the_real_walk(dt):
    """Zero imaginary parts: the complex per-lane walk reproduces the real
    per-lane walk bit for bit (its products with zero parts are exact)."""
    B, T, M = 2, 500, 72
    rin = W.random_inputs(B, T, M, dt, seed=13, a_lo=0.5)
    zeros = np.zeros_like(rin.a)
    cin = W.ComplexInputs(rin.workload, rin.a, zeros, rin.b, zeros, rin.g, zeros)
    res = run(cin, "seq", need_grad_h0=False)
    a, b = dev(rin.a, dt), dev(rin.b, dt)
    out, last = lr.scan(a, b, algo="seq")
    torch.cuda.synchronize()
    assert torch.equal(res[0], out) and torch.equal(res[2], last)
    assert not torch.any(res[1].float()) and not torch.any(res[3])


def test_complex_autograd_wrapper():
    inp = W.complex_inputs(2, 200, 64, "f32", seed=14, r_lo=0.5, theta=np.pi)
    ar, ai = (t.clone().requires_grad_(True) for t in cdev(inp, "a"))
    br, bi = (t.clone().requires_grad_(True) for t in cdev(inp, "b"))
    gr, gi = cdev(inp, "g")
    out_r, out_i = lr.complex_diagonal_scan(ar, ai, br, bi)
    loss = (out_r * gr).sum() + (out_i * gi).sum()
    loss.backward()
    a, b, g = inp.c128("a"), inp.c128("b"), inp.c128("g")
    h, _ = oracle.complex_fwd(a, b)
    oga, ogb, _ = oracle.complex_bwd(a, h, g)
    check_c("grad_b", host(br.grad) + 1j * host(bi.grad), ogb, "f32")
    check_c_grad_a(host(ar.grad) + 1j * host(ai.grad), oga, ogb, cprev(h, None), "f32")


def test_complex_full_size_workload_sampled():
    """cwide (B8 T2048 M2560 bf16) through AUTO: sampled lanes against the
    oracle, and the state-only forward's last bitwise equal to the full one."""
    wl = W.COMPLEX_WORKLOADS["cwide"]
    inp = W.generate_complex(wl, seed=0)
    res = run(inp, "auto", need_grad_h0=False)
    ar, ai = cdev(inp, "a")
    br, bi = cdev(inp, "b")
    _, _, lr_only, li_only = lr.complex_scan(ar, ai, br, bi, with_out=False)
    torch.cuda.synchronize()
    assert torch.equal(lr_only, res[2]) and torch.equal(li_only, res[3])
    lanes = W.sample_lanes(wl, 24, seed=3)
    bs = [l[0] for l in lanes]
    ms = [l[1] for l in lanes]
    a, b, g = inp.c128("a", lanes), inp.c128("b", lanes), inp.c128("g", lanes)
    h, hl = oracle.complex_fwd(a, b)
    oga, ogb, _ = oracle.complex_bwd(a, h, g)
    pick = lambda t: host(t[bs, :, ms]).T[None]  # [1, T, L]
    check_c("out", pick(res[0]) + 1j * pick(res[1]), h, "bf16")
    check_c("grad_b", pick(res[6]) + 1j * pick(res[7]), ogb, "bf16")
    check_c_grad_a(pick(res[4]) + 1j * pick(res[5]), oga, ogb, cprev(h, None), "bf16")
    lastc = host(res[2])[bs, ms] + 1j * host(res[3])[bs, ms]
    check_c("last", lastc[None], hl, "f32")
    log(f"cwide: {len(lanes)} lanes within tolerance")
