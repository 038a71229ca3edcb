"""Segment resets (a [B, T] mask that starts a new segment where it is set)
on every algorithm, through the C ABI, against the fp64 oracle; a reset
step's a gets exactly zero gradient; the masked workload at full size with
its own reset positions as the mask; and the fused look-back's derivation
path stays bitwise identical under resets."""
import numpy as np
import pytest

import oracle
import workloads as W
from _gpu import TOL, check_close, check_grad_a, dev, dev_f32, host, log, prev_state
from test_gpu_parity import ALGOS, ALGO_IDS, FUSED, aligned_only

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import linear_recurrence_sequence_diag_amd as lr  # noqa: E402


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lr.library()


def reset_mask(B, T, seed, p=0.05):
    m = np.random.default_rng(seed).random((B, T)) < p
    m[0, 0] = True           # drops h0 of row 0 (grad_h0 = 0 there)
    m[-1, T - 1] = True      # a reset on the very last step
    if B > 1:
        m[1, 0] = False      # row 1 keeps h0
    return m


def oracle_ref(inp, h0, gl, mask):
    a, b, g = inp.f64("a"), inp.f64("b"), inp.f64("g")
    h, hl = oracle.scan_fwd(a, b, h0=h0, reset=mask)
    oga, ogb, ogh0 = oracle.scan_bwd(a, h, g, h0=h0, grad_last=gl, reset=mask)
    return h, hl, oga, ogb, ogh0


# (2, 10317, 64): two chains of 41 tiles, so the backward's window of 16
# predecessors is crossed twice under resets
SHAPES = [(2, 1000, 72), (3, 777, 130), (1, 4096, 256), (4, 300, 4096), (2, 10317, 64)]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,D", SHAPES, ids=[f"B{b}T{t}D{d}" for b, t, d in SHAPES])
def test_reset_mask_every_algorithm(B, T, D, dt):
    inp, h0, gl = W.random_inputs(B, T, D, dt, seed=7, a_lo=0.5, with_state=True)
    mask = reset_mask(B, T, 8)
    h, hl, oga, ogb, ogh0 = oracle_ref(inp, h0, gl, mask)
    a, b, g = dev(inp.a, dt), dev(inp.b, dt), dev(inp.g, dt)
    th0, tgl = dev_f32(h0), dev_f32(gl)
    tm = torch.from_numpy(mask.astype(np.uint8)).cuda()
    tmb = torch.from_numpy(mask).cuda()  # the binding takes bool as well
    rtol, atol = TOL[dt]
    for algo, cf, cb, wf, wb in ALGOS:
        if aligned_only(algo, cf, cb, wf, wb, D, dt):
            continue
        m = tmb if algo == "auto" else tm
        out, last = lr.scan(a, b, h0=th0, algo=algo, chunk=cf, width=wf, reset=m)
        ga, gb, gh0 = lr.scan_backward(a, out, g, grad_last=tgl, h0=th0, algo=algo, chunk=cb,
                                       need_grad_h0=True, width=wb, reset=m)
        torch.cuda.synchronize()
        what = f"{algo}{cf}w{wf}"
        check_close(f"{what} out", host(out), h, dt)
        check_close(f"{what} last", host(last), hl, "f32" if dt == "bf16" else dt)
        check_close(f"{what} grad_b", host(gb), ogb, dt)
        check_grad_a(host(ga), oga, ogb, prev_state(h, h0), dt)
        # a reset step does not use a_t: its gradient is exactly zero
        gah = host(ga)
        assert np.all(gah[mask] == 0.0), f"{what}: nonzero grad_a at a reset step"
        assert np.all(host(gh0)[0] == 0.0), f"{what}: grad_h0 of a row reset at t = 0"
        assert np.all(np.abs(host(gh0) - ogh0)
                      <= atol * (1 + np.abs(ogb[:, 0])) + 2 * rtol * np.abs(ogh0)), what
        # the step after a reset starts from b_t exactly (forward)
        hb = host(out)
        bb = inp.f64("b")
        assert np.array_equal(hb[mask], W.storage_to_f64(W.to_storage(bb[mask], dt), dt)), what
    log(f"{dt} B{B} T{T} D{D}: {int(mask.sum())} resets, every algorithm within tolerance")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,D", [(2, 4096, 256), (1, 10317, 64)], ids=["B2T4096D256", "B1T10317D64"])
def test_reset_derivation_is_bitwise_identical(B, T, D, dt):
    inp, h0, gl = W.random_inputs(B, T, D, dt, seed=12, a_lo=0.9, with_state=True)
    mask = reset_mask(B, T, 13, p=0.01)
    a, b, g = dev(inp.a, dt), dev(inp.b, dt), dev(inp.g, dt)
    th0, tgl = dev_f32(h0), dev_f32(gl)
    tm = torch.from_numpy(mask.astype(np.uint8)).cuda()
    for algo, cf, cb, wf, wb in FUSED:
        res = []
        for polls in (0, 1):
            out, last = lr.scan(a, b, h0=th0, algo=algo, chunk=cf, width=wf, polls=polls, reset=tm)
            ga, gb, gh0 = lr.scan_backward(a, out, g, grad_last=tgl, h0=th0, algo=algo, chunk=cb,
                                           need_grad_h0=True, width=wb, polls=polls, reset=tm)
            torch.cuda.synchronize()
            res.append((out, last, ga, gb, gh0))
        for name, x, y in zip(("out", "last", "grad_a", "grad_b", "grad_h0"), *res):
            assert torch.equal(x, y), f"fused f{cf}w{wf}: {name} differs with polls=1 under resets"


def test_masked_workload_with_its_reset_mask():
    """The masked workload (B16 T4096 D2560 bf16) with its own reset tokens
    passed as the mask, through AUTO: sampled lanes against the oracle, and
    zero grad_a on every reset token."""
    wl = W.WORKLOADS["masked"]
    inp = W.generate(wl, seed=0)
    mask = inp.reset
    a, b, g = dev(inp.a, "bf16"), dev(inp.b, "bf16"), dev(inp.g, "bf16")
    tm = torch.from_numpy(mask.astype(np.uint8)).cuda()
    out, last = lr.scan(a, b, reset=tm)
    ga, gb, _ = lr.scan_backward(a, out, g, reset=tm)
    torch.cuda.synchronize()
    lanes = W.sample_lanes(wl, 24, seed=3)
    for bi, d in lanes:
        la, lb, lg = (inp.f64(n, [(bi, d)]) for n in ("a", "b", "g"))
        m = mask[bi:bi + 1]
        h, hl = oracle.scan_fwd(la, lb, reset=m)
        oga, ogb, _ = oracle.scan_bwd(la, h, lg, reset=m)
        check_close("out", host(out[bi, :, d])[None, :, None], h, "bf16")
        check_close("grad_b", host(gb[bi, :, d])[None, :, None], ogb, "bf16")
        check_grad_a(host(ga[bi, :, d])[None, :, None], oga, ogb, prev_state(h), "bf16")
    gz = ga.view(torch.int16)[tm.bool()]
    assert int(torch.count_nonzero(gz & 0x7FFF)) == 0
    log(f"masked workload: {int(mask.sum())} reset tokens, {len(lanes)} lanes checked")
