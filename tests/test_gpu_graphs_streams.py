"""The single-launch forms under HIP graph capture and on concurrent streams.

Graphs: fused forward + backward captured on a stream whose library
workspace is already set up, replayed several times with eager calls on the
same stream (and so the same workspace) in between; every replay must equal
the eager result bit for bit (the workspace cleans itself on the device, so
replays need no initialisation step and capture no memset).

Capture without a set-up workspace: a capturing stream gets no library
allocation, so a first call under capture is refused (LRSCAN_ERR_CAPTURE)
with nothing enqueued.  A larger eager call after a capture gets a new
workspace while the captured graph keeps replaying on the old one, which the
library never frees.

Streams: two streams run different scans at the same time, each on its own
library workspace; the results equal those of the same calls made alone."""
import ctypes

import numpy as np
import pytest

import workloads as W
from _gpu import dev, dev_f32, log

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import linear_recurrence_sequence_diag_amd as lr  # noqa: E402


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lr.library()


def real_step(a, b, g):
    out, last = lr.scan(a, b)
    ga, gb, _ = lr.scan_backward(a, out, g)
    return [out, last, ga, gb]


def samu_step(t):
    ctl = (t["eta"], t["delta"], t["nu_log"], t["theta_log"])
    o = lr.samu_scan(*ctl, t["br"], t["bi"])
    gr = lr.samu_scan_backward(*ctl, o[0], o[1], t["gr"], t["gi"])
    return list(o) + list(gr[:6])


def samu_tensors(s):
    dt = s.workload.dtype
    t = {n: dev(getattr(s, n), dt) for n in ("eta", "delta", "br", "bi", "gr", "gi")}
    t["nu_log"], t["theta_log"] = dev_f32(s.nu_log), dev_f32(s.theta_log)
    return t


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_graph_replays_equal_eager(dt):
    r = W.random_inputs(2, 3000, 256, dt, seed=71, a_lo=0.5, a_hi=0.99)
    a, b, g = dev(r.a, dt), dev(r.b, dt), dev(r.g, dt)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        ref = [x.clone() for x in real_step(a, b, g)]   # also sets up this stream's workspace
        sm = samu_tensors(W.samu_inputs(2, 700, 64, dt, seed=72))
        sref = [x.clone() for x in samu_step(sm)]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=st):
        res = real_step(a, b, g)
        sres = samu_step(sm)
    for rep in range(4):
        graph.replay()
        torch.cuda.synchronize()
        for k, (x, y) in enumerate(zip(res, ref)):
            assert torch.equal(x, y), f"replay {rep}: real output {k} differs from eager"
        for k, (x, y) in enumerate(zip(sres, sref)):
            assert torch.equal(x, y), f"replay {rep}: fused-transition output {k} differs from eager"
        with torch.cuda.stream(st):   # eager work on the same workspace between replays
            again = real_step(a, b, g)
        torch.cuda.synchronize()
        assert all(torch.equal(x, y) for x, y in zip(again, ref)), f"eager call after replay {rep}"
    log(f"graph {dt}: 4 replays bitwise equal to eager")


def fresh_stream():
    """A new HIP stream (never handed out before, so the library has no
    workspace for it), wrapped for torch.  Not destroyed: the library keeps
    its workspaces keyed by the handle."""
    hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch already loaded
    h = ctypes.c_void_p()
    assert hip.hipStreamCreate(ctypes.byref(h)) == 0
    return torch.cuda.ExternalStream(h.value)


def test_capture_first_call_is_refused():
    r = W.random_inputs(2, 700, 256, "f32", seed=76, a_lo=0.5, a_hi=0.99)
    a, b = dev(r.a, "f32"), dev(r.b, "f32")
    st = fresh_stream()
    x = torch.arange(4096, device="cuda", dtype=torch.float32)
    y = torch.zeros_like(x)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=st):
        y.copy_(x)
        with pytest.raises(lr.LRScanError) as err:
            lr.scan(a, b)
    assert err.value.status == -8, err.value
    for _ in range(2):
        y.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, x)
    # an eager call sets the stream up; then the same call captures and replays
    with torch.cuda.stream(st):
        ref = [t.clone() for t in lr.scan(a, b)]
    torch.cuda.synchronize()
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2, stream=st):
        res = lr.scan(a, b)
    for rep in range(3):
        g2.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(u, v) for u, v in zip(res, ref)), f"replay {rep}"
    log("capture: a first call is refused; after an eager call it captures and replays")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_capture_survives_a_larger_eager_call(dt):
    """Capture at one size, then make a much larger eager call on the same
    stream (the stream's workspace is replaced): the graph's replays still
    equal eager results bit for bit."""
    small = W.random_inputs(2, 3000, 256, dt, seed=77, a_lo=0.5, a_hi=0.99)
    big = W.random_inputs(4, 4096, 2560, dt, seed=78, a_lo=0.5, a_hi=0.99)
    a, b, g = dev(small.a, dt), dev(small.b, dt), dev(small.g, dt)
    A, Bv, G = dev(big.a, dt), dev(big.b, dt), dev(big.g, dt)
    st = fresh_stream()
    with torch.cuda.stream(st):
        ref = [x.clone() for x in real_step(a, b, g)]
        big_ref = [x.clone() for x in real_step(A, Bv, G)]
        small_again = [x.clone() for x in real_step(a, b, g)]
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(ref, small_again))
    st2 = fresh_stream()
    with torch.cuda.stream(st2):
        real_step(a, b, g)   # sets st2's workspace up at the small size only
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=st2):
        res = real_step(a, b, g)
    for rep in range(3):
        with torch.cuda.stream(st2):   # needs a bigger workspace than the captured one
            out_big = real_step(A, Bv, G)
        graph.replay()
        torch.cuda.synchronize()
        for k, (x, y) in enumerate(zip(res, ref)):
            assert torch.equal(x, y), f"replay {rep}: output {k} differs from eager"
        assert all(torch.equal(x, y) for x, y in zip(out_big, big_ref)), f"large call {rep}"
        with torch.cuda.stream(st2):
            again = real_step(a, b, g)
        torch.cuda.synchronize()
        assert all(torch.equal(x, y) for x, y in zip(again, ref)), f"eager after replay {rep}"
    log(f"capture {dt}: replays unaffected by a larger eager call on the capture stream")


def test_concurrent_streams_equal_solo():
    r1 = W.random_inputs(4, 2048, 1024, "bf16", seed=73, a_lo=0.5, a_hi=0.99)
    r2 = W.random_inputs(1, 20000, 512, "f32", seed=74, a_lo=0.5, a_hi=0.99)
    x1 = [dev(v, "bf16") for v in (r1.a, r1.b, r1.g)]
    x2 = [dev(v, "f32") for v in (r2.a, r2.b, r2.g)]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(s1):
        solo1 = [t.clone() for t in real_step(*x1)]
    torch.cuda.synchronize()
    with torch.cuda.stream(s2):
        solo2 = [t.clone() for t in real_step(*x2)]
    torch.cuda.synchronize()
    for rep in range(3):
        outs1, outs2 = [], []
        for _ in range(3):   # interleave launches on the two streams
            with torch.cuda.stream(s1):
                outs1.append(real_step(*x1))
            with torch.cuda.stream(s2):
                outs2.append(real_step(*x2))
        torch.cuda.synchronize()
        for o in outs1:
            assert all(torch.equal(x, y) for x, y in zip(o, solo1)), "stream 1 differs"
        for o in outs2:
            assert all(torch.equal(x, y) for x, y in zip(o, solo2)), "stream 2 differs"
    log("two concurrent streams: bitwise equal to solo runs")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_captured_decode_loop(dt):
    """Sixteen decode steps captured in one graph (state updated in place,
    one token's a and b per step) replay to the eager chain bit for bit, and
    the last state equals the state-only forward over the same tokens."""
    B, T, D = 4, 16, 1000
    r = W.random_inputs(B, T, D, dt, seed=75, a_lo=0.5, a_hi=0.99)
    a, b = dev(r.a, dt), dev(r.b, dt)
    at = [a[:, t].contiguous() for t in range(T)]
    bt = [b[:, t].contiguous() for t in range(T)]
    st = torch.cuda.Stream()
    state = torch.zeros((B, D), device="cuda", dtype=torch.float32)
    with torch.cuda.stream(st):
        eager = []
        for t in range(T):
            o, _ = lr.step(at[t], bt[t], state=state, out_state=state)
            eager.append(o.clone())
        eager_state = state.clone()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    gstate = torch.zeros((B, D), device="cuda", dtype=torch.float32)
    with torch.cuda.graph(graph, stream=st):
        outs = [lr.step(at[t], bt[t], state=gstate, out_state=gstate)[0] for t in range(T)]
    for rep in range(3):
        gstate.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(x, y) for x, y in zip(outs, eager)), f"replay {rep} outputs"
        assert torch.equal(gstate, eager_state), f"replay {rep} state"
    _, last = lr.scan(a, b, algo="seq")
    torch.cuda.synchronize()
    assert torch.equal(last, eager_state)


def test_one_workspace_across_shapes():
    """One stream's library workspace serves calls whose tiles come from
    different numbers of ticket counters (1, 2, 4 and 64 lane-block chains
    per counter set) and different directions, one after another, twice
    round: every result equals the same call made on a stream of its own,
    bit for bit (each launch must find its region clean and leave the
    counters and the other region's count right for the next one)."""
    shapes = [(1, 3000, 64, "bf16"), (4, 1500, 1024, "bf16"), (3, 777, 200, "f32"),
              (2, 5000, 130, "bf16"), (2, 2100, 96, "f32")]
    data = []
    for n, (B, T, D, dt) in enumerate(shapes):
        r = W.random_inputs(B, T, D, dt, seed=200 + n, a_lo=0.5, a_hi=0.99)
        data.append((dev(r.a, dt), dev(r.b, dt), dev(r.g, dt)))
    refs = []
    for x in data:
        st = fresh_stream()
        with torch.cuda.stream(st):
            refs.append([t.clone() for t in real_step(*x)])
        torch.cuda.synchronize()
    shared = fresh_stream()
    for rnd in range(2):
        for n, x in enumerate(data):
            with torch.cuda.stream(shared):
                res = real_step(*x)
            torch.cuda.synchronize()
            for k, (u, v) in enumerate(zip(res, refs[n])):
                assert torch.equal(u, v), f"round {rnd}, shape {shapes[n]}: output {k} differs"
    log(f"one workspace, {len(shapes)} shapes x 2 rounds: bitwise equal to separate streams")
