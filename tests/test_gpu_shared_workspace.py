"""The library's self-cleaning workspace shared by every single-launch form on
one stream: real, complex and fused-transition calls of different shapes,
interleaved on the same library workspace, give bit for bit the results of
the same calls made on their own (each launch clears what the previous launch
on the workspace wrote, whatever kind of scan that was), also with
polls = 1 (every look-back derives its predecessors' maps itself)."""
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


def real_call(a, b, g, polls):
    out, last = lr.scan(a, b, algo="fused", polls=polls)
    ga, gb, _ = lr.scan_backward(a, out, g, algo="fused", polls=polls)
    return [out, last, ga, gb]


def complex_call(t, polls):
    o = lr.complex_scan(t["ar"], t["ai"], t["br"], t["bi"], polls=polls)
    g = lr.complex_scan_backward(t["ar"], t["ai"], o[0], o[1], t["gr"], t["gi"], polls=polls)
    return list(o) + list(g[:4])


def samu_call(t, polls):
    ctl = (t["eta"], t["delta"], t["nu_log"], t["theta_log"])
    o = lr.samu_scan(*ctl, t["br"], t["bi"], polls=polls)
    g = lr.samu_scan_backward(*ctl, o[0], o[1], t["gr"], t["gi"], polls=polls)
    return list(o) + list(g[:6])


@pytest.mark.parametrize("polls", [0, 1])
def test_interleaved_families_on_one_workspace(polls):
    r = W.random_inputs(3, 1500, 200, "bf16", seed=41)
    a, b, g = dev(r.a, "bf16"), dev(r.b, "bf16"), dev(r.g, "bf16")
    r2 = W.random_inputs(1, 5000, 96, "f32", seed=42)
    a2, b2, g2 = dev(r2.a, "f32"), dev(r2.b, "f32"), dev(r2.g, "f32")
    c = W.complex_inputs(2, 900, 130, "bf16", seed=43)
    tc = {n: dev(getattr(c, n), "bf16") for n in ("ar", "ai", "br", "bi", "gr", "gi")}
    sm = W.samu_inputs(2, 1100, 72, "f32", seed=44)
    ts = {n: dev(getattr(sm, n), "f32") for n in ("eta", "delta", "br", "bi", "gr", "gi")}
    ts["nu_log"], ts["theta_log"] = dev_f32(sm.nu_log), dev_f32(sm.theta_log)
    calls = [lambda: real_call(a, b, g, polls), lambda: complex_call(tc, polls),
             lambda: samu_call(ts, polls), lambda: real_call(a2, b2, g2, polls)]
    # each call alone, twice (the second run reuses a workspace the first dirtied)
    alone = []
    for f in calls:
        f()
        res = f()
        torch.cuda.synchronize()
        alone.append([x.clone() for x in res])
    # interleaved, several rounds, in two orders
    for order in ([0, 1, 2, 3], [3, 2, 1, 0, 2, 0, 1]):
        for i in order:
            res = calls[i]()
            torch.cuda.synchronize()
            for k, (x, y) in enumerate(zip(res, alone[i])):
                assert torch.equal(x, y), f"call {i} output {k} differs after the other families ran"
    log(f"interleaved real/complex/fused-transition calls bitwise equal (polls={polls})")
