"""Inference paths through the C ABI: the one-step decode update (scan_step)
and the state-only forward (out = NULL).  Chained steps reproduce the
per-lane walk bit for bit; a single step and the state-only `last` agree
with the fp64 oracle; the state-only `last` is bitwise the full forward's."""
import numpy as np
import pytest

import oracle
import workloads as W
from _gpu import TOL, check_close, dev, dev_f32, host, log
from test_gpu_parity import ALGOS, ALGO_IDS, aligned_only

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import linear_recurrence_sequence_diag_amd as lr  # noqa: E402


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lr.library()


STEP_SHAPES = [(3, 40, 72), (2, 16, 4096), (5, 30, 13)]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,D", STEP_SHAPES, ids=[f"B{b}T{t}D{d}" for b, t, d in STEP_SHAPES])
def test_chained_steps_equal_the_per_lane_walk_bitwise(B, T, D, dt):
    inp = W.random_inputs(B, T, D, dt, seed=3, a_lo=0.5)
    mask = np.random.default_rng(4).random((B, T)) < 0.1
    a, b = dev(inp.a, dt), dev(inp.b, dt)
    tm = torch.from_numpy(mask.astype(np.uint8)).cuda()
    ref_out, ref_last = lr.scan(a, b, algo="seq", reset=tm)
    state = torch.zeros((B, D), device="cuda", dtype=torch.float32)
    outs = []
    for t in range(T):
        o, state = lr.step(a[:, t].contiguous(), b[:, t].contiguous(), state=state,
                           reset=tm[:, t].contiguous(), out_state=state)
        outs.append(o)
    torch.cuda.synchronize()
    got = torch.stack(outs, dim=1)
    assert torch.equal(got, ref_out), "chained steps differ from the per-lane walk"
    assert torch.equal(state, ref_last), "final state differs from last"
    log(f"{dt} B{B} T{T} D{D}: {T} chained steps bitwise equal to the walk")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_single_step_against_oracle(dt):
    B, D = 6, 2560
    inp = W.random_inputs(B, 1, D, dt, seed=9, a_lo=0.0, a_hi=1.0)
    s0 = np.random.default_rng(10).standard_normal((B, D)).astype(np.float32)
    rs = np.array([0, 1, 0, 0, 1, 0], dtype=np.uint8)
    a, b = dev(inp.a[:, 0], dt), dev(inp.b[:, 0], dt)
    out, new = lr.step(a, b, state=dev_f32(s0), reset=torch.from_numpy(rs).cuda())
    only_state = lr.step(a, b, state=dev_f32(s0), reset=torch.from_numpy(rs).cuda(),
                         with_out=False)[1]
    zero = lr.step(a, b)[1]
    torch.cuda.synchronize()
    h, hl = oracle.scan_fwd(inp.f64("a"), inp.f64("b"), h0=s0, reset=rs[:, None])
    check_close("out", host(out), h[:, 0], dt)
    check_close("state", host(new), hl, "f32")
    assert torch.equal(new, only_state)
    h0z, _ = oracle.scan_fwd(inp.f64("a"), inp.f64("b"))
    check_close("state from zero", host(zero), h0z[:, 0], "f32")
    rtol, atol = TOL["f32"]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,D", [(2, 1000, 72), (3, 777, 130), (1, 4096, 256)],
                         ids=["B2T1000D72", "B3T777D130", "B1T4096D256"])
def test_state_only_forward(B, T, D, dt):
    inp, h0, _ = W.random_inputs(B, T, D, dt, seed=15, a_lo=0.5, with_state=True)
    mask = np.random.default_rng(16).random((B, T)) < 0.03
    a, b = dev(inp.a, dt), dev(inp.b, dt)
    th0 = dev_f32(h0)
    tm = torch.from_numpy(mask.astype(np.uint8)).cuda()
    _, hl = oracle.scan_fwd(inp.f64("a"), inp.f64("b"), h0=h0, reset=mask)
    for algo, cf, cb, wf, wb in ALGOS:
        if aligned_only(algo, cf, cb, wf, wb, D, dt):
            continue
        for m in (None, tm):
            _, full = lr.scan(a, b, h0=th0, algo=algo, chunk=cf, width=wf, reset=m)
            out, only = lr.scan(a, b, h0=th0, algo=algo, chunk=cf, width=wf, reset=m,
                                with_out=False)
            torch.cuda.synchronize()
            assert out is None
            assert torch.equal(only, full), f"{algo}{cf}w{wf}: state-only last differs"
        check_close(f"{algo}{cf}w{wf} last", host(only), hl, "f32" if dt == "bf16" else dt)
