"""Parity of the HIP path (through the C ABI) with the fp64 oracle: small and
ragged shapes, every algorithm, every chunk step on its own, edge cases and
determinism.  Full-size workloads are in test_gpu_workloads.py."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads as W
from _gpu import TOL, check_close, check_grad_a, dev, dev_f32, host, log, prev_state

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import linear_recurrence_sequence_diag_amd as lr  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))

# (name, forward chunk/tile, backward chunk/tile, forward width, backward width)
ALGOS = [("seq", 0, 0, 0, 0), ("chunked", 16, 16, 0, 0), ("chunked", 64, 64, 0, 0),
         ("chunked", 256, 256, 0, 0), ("chunked", 1024, 1024, 0, 0),
         ("fused", 256, 256, 8, 8), ("fused", 512, 128, 8, 8), ("fused", 128, 128, 16, 16),
         ("fused", 256, 128, 16, 16), ("fused", 64, 64, 32, 32), ("fused", 128, 32, 32, 32),
         ("fused", 32, 32, 32, 32),
         ("auto", 0, 0, 0, 0)]
ALGO_IDS = [f"{a}{c}w{w}" if c else a for a, c, _, w, _ in ALGOS]


# fused tile shapes (width, rows) that rows not 16-byte aligned take
UNALIGNED_FWD = {(8, 256), (16, 128), (32, 64)}
UNALIGNED_BWD = {(8, 256), (16, 128), (32, 64), (8, 128)}


def aligned_only(algo, cf, cb, wf, wb, D, dt):
    """Fused tile shapes that need 16-byte aligned rows."""
    rows_aligned = (D * (4 if dt == "f32" else 2)) % 16 == 0
    return (algo == "fused" and not rows_aligned
            and ((wf, cf) not in UNALIGNED_FWD or (wb, cb) not in UNALIGNED_BWD))


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lr.library()


def run_pair(inp, algo, cf, cb, wf=0, wb=0, h0=None, gl=None):
    """GPU forward then backward (the backward reads the GPU's own out)."""
    dt = inp.workload.dtype
    a, b, g = dev(inp.a, dt), dev(inp.b, dt), dev(inp.g, dt)
    th0 = None if h0 is None else dev_f32(h0)
    tgl = None if gl is None else dev_f32(gl)
    out, last = lr.scan(a, b, h0=th0, algo=algo, chunk=cf, width=wf)
    ga, gb, gh0 = lr.scan_backward(a, out, g, grad_last=tgl, h0=th0, algo=algo, chunk=cb,
                                   need_grad_h0=True, width=wb)
    torch.cuda.synchronize()
    return out, last, ga, gb, gh0


def check_against_oracle(inp, res, h0=None, gl=None):
    dt = inp.workload.dtype
    out, last, ga, gb, gh0 = res
    a, b, g = inp.f64("a"), inp.f64("b"), inp.f64("g")
    h, hl = oracle.scan_fwd(a, b, h0=h0)
    check_close("out", host(out), h, dt)
    check_close("last", host(last), hl, dt if dt == "f32" else "f32")
    oga, ogb, ogh0 = oracle.scan_bwd(a, h, g, h0=h0, grad_last=gl)
    check_close("grad_b", host(gb), ogb, dt)
    check_grad_a(host(ga), oga, ogb, prev_state(h, h0), dt)
    rtol, atol = TOL[dt]
    # grad_h0 = a_0 * lambda_0 (fp32 output): checked like a product of a stored a and lambda
    assert np.all(np.abs(host(gh0) - ogh0) <= atol * (1 + np.abs(ogb[:, 0])) + 2 * rtol * np.abs(ogh0))
    # the final state agrees with the last stored row
    lo = host(out)[:, -1]
    if dt == "f32":
        assert np.array_equal(host(last), lo)
    else:
        assert np.array_equal(W.f32_to_bf16_bits(host(last).astype(np.float32)),
                              W.f32_to_bf16_bits(lo.astype(np.float32)))


# ----------------------------------------------------------------------------
def test_golden_hand_example_exact():
    with open(os.path.join(HERE, "golden", "hand_example.json")) as f:
        ex = json.load(f)
    arr = lambda k: np.array(ex[k], dtype=np.float64)[None]
    for dt in ("f32", "bf16"):
        inp = W.Inputs(W.Workload("hand", 1, 4, 2, dt, "hand"), W.to_storage(arr("a"), dt),
                       W.to_storage(arr("b"), dt), W.to_storage(arr("g"), dt))
        gl = np.array(ex["grad_last"], np.float32)[None]
        for algo, cf, cb, wf, wb in ALGOS:
            if aligned_only(algo, cf, cb, wf, wb, 2, dt):
                continue
            log(f"golden {dt} {algo}{cf} w{wf}")
            out, last, ga, gb, gh0 = run_pair(inp, algo, cf, cb, wf, wb)
            assert np.array_equal(host(out), arr("out")), (dt, algo)
            assert np.array_equal(host(last)[0], np.array(ex["last"])), (dt, algo)
            assert np.array_equal(host(ga), arr("grad_a")), (dt, algo)
            assert np.array_equal(host(gb), arr("grad_b")), (dt, algo)
            assert np.array_equal(host(gh0)[0], np.array(ex["grad_h0"])), (dt, algo)
            out, last, ga, gb, gh0 = run_pair(inp, algo, cf, cb, wf, wb, gl=gl)
            w = ex["with_grad_last"]
            assert np.array_equal(host(ga)[0], np.array(w["grad_a"])), (dt, algo)
            assert np.array_equal(host(gb)[0], np.array(w["grad_b"])), (dt, algo)
            assert np.array_equal(host(gh0)[0], np.array(w["grad_h0"])), (dt, algo)


@pytest.mark.parametrize("algo,cf,cb,wf,wb", ALGOS, ids=ALGO_IDS)
def test_small_workload(algo, cf, cb, wf, wb):
    """The B=2, T=256, D=64 fp32 workload, whole tensors, every algorithm."""
    inp = W.generate(W.WORKLOADS["small"], seed=0)
    log(f"small {algo}{cf} w{wf}")
    check_against_oracle(inp, run_pair(inp, algo, cf, cb, wf, wb))


# AUTO's tile shapes: (2, 20, 304) and (3, 33, 520) its short-sequence tiles
# with 512-byte rows (rows past T and lanes past D in every tile), (3, 257, 64)
# a forward chain of one 512-row tile, the last two its 512-row forward tiles
# for long sequences with few lane blocks
SHAPES = [(1, 1, 1), (1, 2, 3), (2, 63, 7), (2, 64, 8), (1, 65, 9), (2, 20, 304), (3, 33, 520),
          (3, 257, 64), (2, 300, 65), (1, 1000, 100), (2, 513, 129), (1, 1100, 16),
          (2, 2049, 40), (3, 4099, 136), (1, 4097, 40)]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,D", SHAPES, ids=[f"B{b}T{t}D{d}" for b, t, d in SHAPES])
def test_ragged_shapes_all_algos(B, T, D, dt):
    """Tails in T (partial chunks and tiles) and in D (partial vectors and
    lane blocks, unaligned rows), with an initial state and grad_last."""
    inp, h0, gl = W.random_inputs(B, T, D, dt, seed=B * 1000 + T * 10 + D, with_state=True)
    for algo, cf, cb, wf, wb in ALGOS:
        if aligned_only(algo, cf, cb, wf, wb, D, dt):
            continue
        log(f"ragged B{B} T{T} D{D} {dt} {algo}{cf} w{wf}")
        check_against_oracle(inp, run_pair(inp, algo, cf, cb, wf, wb, h0=h0, gl=gl), h0=h0, gl=gl)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("C", [16, 64, 256])
@pytest.mark.parametrize("T", [256, 1000])
def test_chunk_steps_each_against_oracle(dt, C, T):
    """Every step of the three-launch form through its own entry point."""
    B, D = 2, 72
    inp, h0, gl = W.random_inputs(B, T, D, dt, seed=C + T, a_lo=0.8, with_state=True)
    log(f"steps {dt} C{C} T{T}")
    a, b, g = inp.f64("a"), inp.f64("b"), inp.f64("g")
    ta, tb, tg = dev(inp.a, dt), dev(inp.b, dt), dev(inp.g, dt)
    # forward summary: P is a product of stored values, Q a short scan
    P, Q = lr.chunk_summary(ta, tb, C)
    oP, oQ = oracle.chunk_summary(a, b, C)
    check_close("P", host(P), oP, "f32")
    check_close("Q", host(Q), oQ, "f32")
    # prefix on the oracle's own maps (so this step is checked on its own)
    cin, fin = lr.chunk_prefix(dev_f32(oP), dev_f32(oQ), init=dev_f32(h0))
    ocin, ofin = oracle.chunk_prefix(oP.astype(np.float32), oQ.astype(np.float32), h0=h0)
    check_close("chunk_in", host(cin), ocin, "f32")
    check_close("prefix last", host(fin), ofin, "f32")
    # replay from the oracle's entering states
    out, last = lr.chunk_replay(ta, tb, dev_f32(ocin), C)
    oout, olast = oracle.chunk_replay(a, b, ocin.astype(np.float32), C)
    check_close("replay out", host(out), oout, dt)
    check_close("replay last", host(last), olast, "f32")
    # reverse trio
    h, _ = oracle.scan_fwd(a, b, h0=h0)
    rP, rQ = lr.chunk_summary(ta, tg, C, reverse=True)
    orP, orQ = oracle.reverse_chunk_summary(a, g, C)
    check_close("reverse P", host(rP), orP, "f32")
    check_close("reverse Q", host(rQ), orQ, "f32")
    fut, gh0 = lr.chunk_prefix(dev_f32(orP), dev_f32(orQ), init=dev_f32(gl), reverse=True)
    ofut, ogh0 = oracle.reverse_chunk_prefix(orP.astype(np.float32), orQ.astype(np.float32),
                                             grad_last=gl)
    check_close("future", host(fut), ofut, "f32")
    check_close("grad_h0", host(gh0), ogh0, "f32")
    hs = W.to_storage(h, dt)
    ga, gb = lr.reverse_chunk_replay(ta, dev(hs, dt), tg, dev_f32(ofut), C, h0=dev_f32(h0))
    hq = W.storage_to_f64(hs, dt)
    oga, ogb = oracle.reverse_chunk_replay(a, hq, g, ofut.astype(np.float32), C, h0=h0)
    check_close("reverse grad_b", host(gb), ogb, dt)
    check_grad_a(host(ga), oga, ogb, prev_state(hq, h0), dt)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_deterministic_and_paths_agree(dt):
    B, T, D = 2, 4096, 256
    inp = W.random_inputs(B, T, D, dt, seed=5, a_lo=0.9)
    runs = {}
    for algo, cf, cb, wf, wb in ALGOS:
        r1 = run_pair(inp, algo, cf, cb, wf, wb)
        r2 = run_pair(inp, algo, cf, cb, wf, wb)
        for x, y in zip(r1, r2):
            assert torch.equal(x, y), f"{algo}{cf} w{wf} not bitwise repeatable"
        runs[(algo, cf, wf)] = [host(x) for x in r1]
    ref = runs[("seq", 0, 0)]
    worst = 0.0
    for key, r in runs.items():
        for x, y in zip(r, ref):
            worst = max(worst, float(np.max(np.abs(x - y) / (1 + np.abs(y)))))
    log(f"{dt}: max |path - seq| / (1 + |seq|) = {worst:.3g}")
    assert worst < (1e-4 if dt == "f32" else 2e-2)


FUSED = [c for c in ALGOS if c[0] == "fused"]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,D", [(2, 4096, 256), (3, 1000, 201), (1, 20000, 64)],
                         ids=["B2T4096D256", "B3T1000D201", "B1T20000D64"])
def test_lookback_derivation_is_bitwise_identical(B, T, D, dt):
    """With a single poll, a fused tile whose predecessors have not published
    yet derives their maps from the inputs (the path taken when a
    predecessor's workgroup stays descheduled).  Every output must be bitwise
    the one the default, waiting, path gives, with h0 and grad_last set."""
    inp, h0n, gln = W.random_inputs(B, T, D, dt, seed=11, a_lo=0.9, with_state=True)
    a, b, g = dev(inp.a, dt), dev(inp.b, dt), dev(inp.g, dt)
    h0, gl = dev_f32(h0n), dev_f32(gln)
    for algo, cf, cb, wf, wb in FUSED:
        if aligned_only(algo, cf, cb, wf, wb, D, dt):
            continue
        res = []
        for polls in (0, 1):
            out, last = lr.scan(a, b, h0=h0, algo=algo, chunk=cf, width=wf, polls=polls)
            ga, gb, gh0 = lr.scan_backward(a, out, g, grad_last=gl, h0=h0, algo=algo, chunk=cb,
                                           need_grad_h0=True, width=wb, polls=polls)
            torch.cuda.synchronize()
            res.append((out, last, ga, gb, gh0))
        for name, x, y in zip(("out", "last", "grad_a", "grad_b", "grad_h0"), *res):
            assert torch.equal(x, y), f"fused f{cf}w{wf} b{cb}w{wb}: {name} differs with polls=1"
    log(f"{dt} B{B} T{T} D{D}: derived look-back maps bitwise equal on {len(FUSED)} configs")


def test_identity_and_reset_steps():
    """a = 0 steps restart the scan bit for bit on every path; a = 1 steps
    carry the state unchanged bit for bit on the sequential path (chunked
    paths may enter a segment at such a step with a state re-associated from
    the chunk maps, so there they agree to the tolerance)."""
    B, T, D = 2, 3000, 64
    for dt in ("f32", "bf16"):
        inp = W.random_inputs(B, T, D, dt, seed=11, a_lo=0.5)
        a = inp.f64("a")
        pads = np.arange(7, T, 13)
        resets = np.setdiff1d(np.arange(5, T, 97), np.concatenate([pads, pads + 1]))
        a[:, pads] = 1.0
        a[:, resets] = 0.0
        b = inp.f64("b")
        b[:, pads] = 0.0
        inp = W.Inputs(inp.workload, W.to_storage(a, dt), W.to_storage(b, dt), inp.g)
        for algo, cf, cb, wf, wb in ALGOS:
            out, last, ga, gb, _ = run_pair(inp, algo, cf, cb, wf, wb)
            o = host(out)
            assert np.array_equal(o[:, resets], W.storage_to_f64(inp.b, dt)[:, resets]), (dt, algo)
            if algo == "seq":
                assert np.array_equal(o[:, pads], o[:, pads - 1]), (dt, algo)
            else:
                check_close(f"pad carry {algo}{cf}", o[:, pads], o[:, pads - 1], dt)


def test_autograd_wrapper_matches_oracle():
    inp = W.random_inputs(2, 300, 48, "f32", seed=3, a_lo=0.7)
    a = dev(inp.a, "f32").requires_grad_()
    b = dev(inp.b, "f32").requires_grad_()
    g = dev(inp.g, "f32")
    out = lr.diagonal_scan(a, b)
    out.backward(g)
    h, _ = oracle.scan_fwd(inp.f64("a"), inp.f64("b"))
    oga, ogb, _ = oracle.scan_bwd(inp.f64("a"), h, inp.f64("g"))
    check_close("out", host(out), h, "f32")
    check_close("grad_b", host(b.grad), ogb, "f32")
    check_grad_a(host(a.grad), oga, ogb, prev_state(h), "f32")


def test_caller_workspace_and_errors():
    B, T, D = 2, 700, 40
    inp = W.random_inputs(B, T, D, "bf16", seed=9)
    a, b = dev(inp.a, "bf16"), dev(inp.b, "bf16")
    for algo, chunk, width in (("chunked", 64, 0), ("fused", 256, 8), ("fused", 64, 32)):
        o = lr.make_opts(algo=algo, chunk=chunk, width=width)
        n = lr.scan_workspace_bytes(B, T, D, lr.BF16, o)
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        out = torch.empty_like(a)
        last = torch.empty((B, D), device="cuda")
        opts = lr.make_opts(algo=algo, chunk=chunk, workspace=ws, width=width)
        lr.scan_fwd_ex(a.data_ptr(), b.data_ptr(), out.data_ptr(), last.data_ptr(), B, T, D,
                       lr.BF16, torch.cuda.current_stream().cuda_stream, opts)
        torch.cuda.synchronize()
        h, hl = oracle.scan_fwd(inp.f64("a"), inp.f64("b"))
        check_close("out", host(out), h, "bf16")
        small = lr.make_opts(algo=algo, chunk=chunk, workspace=ws[: n // 2], width=width)
        with pytest.raises(lr.LRScanError):
            lr.scan_fwd_ex(a.data_ptr(), b.data_ptr(), out.data_ptr(), None, B, T, D, lr.BF16,
                           torch.cuda.current_stream().cuda_stream, small)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_plain_entry_points_on_data(dt):
    """The two entry points the boundary is named by, scan_fwd and scan_bwd
    (no options: the automatic choice), on a ragged shape with grad_last,
    against the oracle element by element; and bitwise equal to scan_fwd_ex /
    scan_bwd_ex with the same automatic choice."""
    inp, h0, gl = W.random_inputs(3, 5000, 300, dt, seed=91, a_lo=0.5, a_hi=0.999,
                                  with_state=True)
    a, b, g = dev(inp.a, dt), dev(inp.b, dt), dev(inp.g, dt)
    tgl = dev_f32(gl)
    B, T, D = a.shape
    code = lr.dtype_code(a.dtype)
    sh = torch.cuda.current_stream().cuda_stream
    out, ga, gb = torch.empty_like(a), torch.empty_like(a), torch.empty_like(a)
    last = torch.empty((B, D), device="cuda", dtype=torch.float32)
    assert lr.scan_fwd(a.data_ptr(), b.data_ptr(), out.data_ptr(), last.data_ptr(), B, T, D, code,
                       sh) == 0
    assert lr.scan_bwd(a.data_ptr(), out.data_ptr(), g.data_ptr(), tgl.data_ptr(), ga.data_ptr(),
                       gb.data_ptr(), B, T, D, code, sh) == 0
    torch.cuda.synchronize()
    a64, b64, g64 = inp.f64("a"), inp.f64("b"), inp.f64("g")
    h, hl = oracle.scan_fwd(a64, b64)
    oga, ogb, _ = oracle.scan_bwd(a64, h, g64, grad_last=gl)
    r = [check_close("out", host(out), h, dt), check_close("last", host(last), hl, "f32"),
         check_close("grad_b", host(gb), ogb, dt),
         check_grad_a(host(ga), oga, ogb, prev_state(h), dt)]
    ex_out, ex_last = lr.scan(a, b)
    ex_ga, ex_gb, _ = lr.scan_backward(a, ex_out, g, grad_last=tgl)
    torch.cuda.synchronize()
    assert torch.equal(out, ex_out) and torch.equal(last, ex_last)
    assert torch.equal(ga, ex_ga) and torch.equal(gb, ex_gb)
    log(f"plain scan_fwd/scan_bwd {dt}: worst err/tol {max(r):.3f}")
