"""Parity at the full sizes of the five specified workloads, in the launch
configuration the benchmark times (the library's automatic choice).

Lanes are independent, so the oracle recomputes a sample of whole lanes
(every step of T) exactly; properties that hold at any size are checked on
every element: the final state against the last stored row, the adjoint
identity <grad_out, out> = <grad_b, b>, and for the masked workload the reset
and padding invariants.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from _gpu import TOL, check_close, check_grad_a, dev, host, log, prev_state

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import linear_recurrence_sequence_diag_amd as lr  # noqa: E402


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lr.library()


def lane_view(t, lanes):
    bs = torch.tensor([l[0] for l in lanes], device=t.device)
    ds = torch.tensor([l[1] for l in lanes], device=t.device)
    return host(t[bs, :, ds].transpose(0, 1).unsqueeze(0).contiguous())  # [1, T, L]


@pytest.mark.parametrize("name", ["small", "wide", "long32", "longseq", "masked"])
def test_full_size_workload(name):
    wl = W.WORKLOADS[name]
    dt = wl.dtype
    log(f"{name}: generating B={wl.B} T={wl.T} D={wl.D} {dt}")
    inp = W.generate(wl, seed=0)
    a, b, g = dev(inp.a, dt), dev(inp.b, dt), dev(inp.g, dt)
    log(f"{name}: running")
    out, last = lr.scan(a, b)
    ga, gb, _ = lr.scan_backward(a, out, g)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(gb.float()).all()

    # sampled whole lanes against the oracle
    lanes = W.sample_lanes(wl, 48 if wl.T > 10000 else 96)
    la, lb, lg = inp.f64("a", lanes), inp.f64("b", lanes), inp.f64("g", lanes)
    h, hl = oracle.scan_fwd(la, lb)
    r_out = check_close("out", lane_view(out, lanes), h, dt)
    hl_gpu = host(last)[[l[0] for l in lanes], [l[1] for l in lanes]]
    check_close("last", hl_gpu, hl[0], "f32")
    oga, ogb, _ = oracle.scan_bwd(la, h, lg)
    r_gb = check_close("grad_b", lane_view(gb, lanes), ogb, dt)
    r_ga = check_grad_a(lane_view(ga, lanes), oga, ogb, prev_state(h), dt)
    log(f"{name}: worst err/tol out {r_out:.3f} grad_b {r_gb:.3f} grad_a {r_ga:.3f}")

    # every element: final state vs the last stored row
    lo = out[:, -1].float()
    if dt == "f32":
        assert torch.equal(last, lo)
    else:
        assert torch.equal(last.to(torch.bfloat16), out[:, -1])

    # adjoint identity over the whole tensor, in fp64 on the device
    lhs = (g.double() * out.double()).sum()
    rhs = (gb.double() * b.double()).sum()
    scale = (g.double() * out.double()).abs().sum() + (gb.double() * b.double()).abs().sum()
    rel = float((lhs - rhs).abs() / scale)
    log(f"{name}: adjoint identity |lhs - rhs| / sum|terms| = {rel:.3g}")
    assert rel < 2 * TOL[dt][0]

    if name == "masked":
        pad = torch.from_numpy(inp.pad).cuda()
        reset = torch.from_numpy(inp.reset).cuda()
        assert torch.equal(out[reset], b[reset])  # a reset restarts from b exactly
        prev = torch.roll(out, 1, dims=1)
        pad_inner = pad.clone()
        pad_inner[:, 0] = False
        check_close("padding carries the state", host(out[pad_inner]), host(prev[pad_inner]), dt)
        # gradients do not cross a reset: lambda at a reset is g plus the carry from the right,
        # and nothing flows further left (checked through the oracle lanes above)
