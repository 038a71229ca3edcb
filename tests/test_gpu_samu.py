"""Fused-transition (SAMU-form) complex scan through the C ABI against the fp64
oracle (page "triton_training_scan.py", _samu_forward / _samu_backward):
ragged and unaligned shapes, h0 / grad_last / grad_h0, the reset mask, the
four parameter gradients; bitwise determinism and bitwise-identical look-back
derivation; caller workspace; the autograd wrapper; the full-size workload on
whole batch rows.

Tolerances.  The kernel rebuilds every transition a in fp32 from the
controls, so besides the rounding the plain complex scan already has (the
atol + rtol|ref| bounds of the complex tests) each a carries a relative error
eps_a.  With x = e^{nu_log} e^{eta}, theta = e^{theta_log} and u = 2^-24:
the modulus exp(-x) inherits the relative error of x (about 3u: two
exponentials and a product) times |x|, plus its own rounding; the rotation
by theta + delta inherits the absolute error of the angle (about
u (|theta| + |delta|) from forming theta and rounding the angle-addition
products) plus a few roundings.  So eps_a = 2^-22 (4 + 3x + theta + |delta|),
four times u times these counts.  That error propagates through the
recurrence to first order:
  E_h[t] = |a_t| E_h[t-1] + eps_a[t] |a_t| |h_{t-1}|         (forward)
  E_l[t] = |a_{t+1}| E_l[t+1] + eps_a[t+1] |a_{t+1}| |lambda_{t+1}|  (reverse)
and is added to the out / grad_b bounds.  A parameter-gradient term is
c |a| |lambda| |h_{t-1}| times a unit-modulus factor (c = nu e^eta for eta and
nu_log, 1 for delta, theta for theta_log); its error is bounded by
c |a| (err_lambda |h_{t-1}| + |lambda| err_h + |lambda| |h_{t-1}| (eps_a + 2^-21)).
A sum of n such terms, added in fp32 in any order, errs by at most
(n - 1) u times the sum of |terms| more (the bound of recursive summation,
which covers every association): n = M for grad_eta and grad_delta (one
token's modes), n = B*T for grad_nu_log and grad_theta_log (one mode's
tokens).  The bound depends on the method and the shapes only, not on how
the kernels tile the sums.
"""
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


def sdev(inp):
    dt = inp.workload.dtype
    return dict(eta=dev(inp.eta, dt), delta=dev(inp.delta, dt), nu_log=dev_f32(inp.nu_log),
                theta_log=dev_f32(inp.theta_log), br=dev(inp.br, dt), bi=dev(inp.bi, dt),
                gr=dev(inp.gr, dt), gi=dev(inp.gi, dt))


def run(inp, h0=None, gl=None, mask=None, polls=0, need_grad_h0=True, workspace=None,
        algo="auto"):
    t = sdev(inp)
    th0 = None if h0 is None else (dev_f32(h0.real), dev_f32(h0.imag))
    tgl = None if gl is None else (dev_f32(gl.real), dev_f32(gl.imag))
    tm = None if mask is None else torch.from_numpy(mask.astype(np.uint8)).cuda()
    ctl = (t["eta"], t["delta"], t["nu_log"], t["theta_log"])
    out_r, out_i, last_r, last_i = lr.samu_scan(*ctl, t["br"], t["bi"], h0=th0, polls=polls,
                                                reset=tm, workspace=workspace, algo=algo)
    ge, gd, gn, gt, gbr, gbi, gh0 = lr.samu_scan_backward(
        *ctl, out_r, out_i, t["gr"], t["gi"], grad_last=tgl, h0=th0, polls=polls, reset=tm,
        need_grad_h0=need_grad_h0, workspace=workspace, algo=algo)
    torch.cuda.synchronize()
    return dict(out_r=out_r, out_i=out_i, last_r=last_r, last_i=last_i, ge=ge, gd=gd, gn=gn,
                gt=gt, gbr=gbr, gbi=gbi, gh0=gh0)


def state_pair(B, M, seed):
    r = np.random.default_rng(seed)
    z = r.standard_normal((B, M)) + 1j * r.standard_normal((B, M))
    return z.real.astype(np.float32) + 1j * z.imag.astype(np.float32)


def propagate(coef, src, reverse=False):
    """E[t] = coef[t] E[t-1] + src[t] over axis 1 (or the mirror in reverse)."""
    E = np.empty_like(src)
    acc = np.zeros_like(src[:, 0])
    steps = range(src.shape[1] - 1, -1, -1) if reverse else range(src.shape[1])
    for t in steps:
        acc = coef[:, t] * acc + src[:, t]
        E[:, t] = acc
    return E


class Bounds:
    """Oracle results for one input set plus the tolerance bounds derived above."""

    def __init__(self, eta, delta, nu_log, theta_log, b, g, dt, h0=None, gl=None, mask=None,
                 mode_terms=None):
        """mode_terms: the number of (b, t) terms in each mode's sum (default B*T;
        larger when these rows are part of a bigger batch)."""
        self.h, self.last = oracle.samu_fwd(eta, delta, nu_log, theta_log, b, h0=h0, reset=mask)
        (self.ge, self.gd, self.gn, self.gt, self.lam,
         self.gh0) = oracle.samu_bwd(eta, delta, nu_log, theta_log, self.h, g, h0=h0,
                                     grad_last=gl, reset=mask)
        B, T, M = b.shape
        rtol, atol = TOL[dt]
        x = np.exp(nu_log)[None, None, :] * np.exp(eta)[..., None]
        theta = np.exp(theta_log)[None, None, :]
        absa = np.exp(-x)
        eps = 2.0 ** -22 * (4 + 3 * x + theta + np.abs(delta)[..., None])
        if mask is not None:
            absa = np.where(mask[..., None], 0.0, absa)
        hp = np.concatenate([np.zeros((B, 1, M), complex) if h0 is None else h0[:, None, :],
                             self.h[:, :-1]], axis=1)
        if mask is not None:
            hp = np.where(mask[..., None], 0.0, hp)
        self.absa = absa
        self.E_h = propagate(absa, eps * absa * np.abs(hp))
        a_next = np.concatenate([absa[:, 1:], np.zeros((B, 1, M))], axis=1)
        src = np.concatenate([(eps * absa * np.abs(self.lam))[:, 1:], np.zeros((B, 1, M))], axis=1)
        self.E_l = propagate(a_next, src, reverse=True)
        err_l = atol + rtol * np.abs(self.lam) + self.E_l
        err_h = atol + rtol * np.abs(hp) + np.concatenate(
            [np.zeros((B, 1, M)), self.E_h[:, :-1]], axis=1)
        mag = absa * np.abs(self.lam) * np.abs(hp)
        unit = absa * (err_l * np.abs(hp) + np.abs(self.lam) * err_h) + mag * (eps + 2.0 ** -21)
        c_rad = np.exp(nu_log)[None, None, :] * np.exp(eta)[..., None]
        u = 2.0 ** -24
        n_tok = M - 1  # additions in one token's sum over modes
        n_mode = (B * T if mode_terms is None else mode_terms) - 1  # in one mode's sum over tokens
        self.tol_ge = atol + (c_rad * unit).sum(2) + n_tok * u * (c_rad * mag).sum(2)
        self.tol_gd = atol + unit.sum(2) + n_tok * u * mag.sum(2)
        self.tol_gn = atol + (c_rad * unit).sum((0, 1)) + n_mode * u * (c_rad * mag).sum((0, 1))
        self.tol_gt = atol + (theta * unit).sum((0, 1)) + n_mode * u * (theta * mag).sum((0, 1))
        self.eps0 = eps[:, 0]
        self.dt = dt


def check(name, got, ref, tol):
    err = np.abs(got - ref) if np.isrealobj(got) else np.maximum(
        np.abs(got.real - ref.real), np.abs(got.imag - ref.imag))
    bad = ~(err <= tol)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err / tol, 0)), err.shape)
        raise AssertionError(f"{name}: {int(bad.sum())} of {bad.size} outside the bound; worst at "
                             f"{i}: got {got[i]!r} ref {ref[i]!r} tol {tol[i]!r}")


def check_all(tag, res, bd, rows=slice(None), check_params=True):
    rtol, atol = TOL[bd.dt]
    rtol32, atol32 = TOL["f32"]
    out = host(res["out_r"][rows]) + 1j * host(res["out_i"][rows])
    check(f"{tag} out", out, bd.h, atol + rtol * np.abs(bd.h) + bd.E_h)
    last = host(res["last_r"][rows]) + 1j * host(res["last_i"][rows])
    check(f"{tag} last", last, bd.last, atol32 + rtol32 * np.abs(bd.last) + bd.E_h[:, -1])
    gb = host(res["gbr"][rows]) + 1j * host(res["gbi"][rows])
    check(f"{tag} grad_b", gb, bd.lam, atol + rtol * np.abs(bd.lam) + bd.E_l)
    if res["gh0"] is not None:
        gh0 = host(res["gh0"][0][rows]) + 1j * host(res["gh0"][1][rows])
        l0 = np.abs(bd.lam[:, 0])
        tol = (atol * (1 + l0) + 2 * rtol * np.abs(bd.gh0)
               + bd.absa[:, 0] * (bd.E_l[:, 0] + bd.eps0 * l0))
        check(f"{tag} grad_h0", gh0, bd.gh0, tol)
    check(f"{tag} grad_eta", host(res["ge"][rows]), bd.ge, bd.tol_ge)
    check(f"{tag} grad_delta", host(res["gd"][rows]), bd.gd, bd.tol_gd)
    if check_params:
        check(f"{tag} grad_nu_log", host(res["gn"]), bd.gn, bd.tol_gn)
        check(f"{tag} grad_theta_log", host(res["gt"]), bd.gt, bd.tol_gt)


# (64, 7, 512) ... (5, 100, 200) run the short-sequence tiles: 8, 16, 32 and
# 64 rows of 512-byte rows (rows of 300 bf16 values are not 16-byte aligned)
# and 128 rows of 256-byte rows; (520, 6, 520) is walked by AUTO (270K lanes),
# a row's second wavefront mostly padding
SHAPES = [(2, 300, 72), (3, 1000, 130), (1, 4096, 256), (2, 333, 13), (1, 1, 1), (2, 129, 1),
          (64, 7, 512), (30, 13, 300), (40, 20, 300), (9, 50, 520), (5, 100, 200),
          (520, 6, 520)]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,M", SHAPES, ids=[f"B{b}T{t}M{m}" for b, t, m in SHAPES])
def test_samu_against_oracle(B, T, M, dt):
    inp = W.samu_inputs(B, T, M, dt, seed=21)
    h0, gl = state_pair(B, M, 22), state_pair(B, M, 23)
    mask = np.random.default_rng(24).random((B, T)) < 0.03
    mask[0, 0] = True
    eta, delta, nu_log, theta_log = inp.controls()
    b, g = inp.c128("b"), inp.c128("g")
    for m in (None, mask):
        bd = Bounds(eta, delta, nu_log, theta_log, b, g, dt, h0=h0, gl=gl, mask=m)
        for algo in ("fused", "seq", "auto"):
            res = run(inp, h0=h0, gl=gl, mask=m, algo=algo)
            tag = f"{dt} B{B}T{T}M{M}{'+reset' if m is not None else ''} {algo}"
            check_all(tag, res, bd)
            if m is not None:
                assert np.all(host(res["ge"])[m] == 0) and np.all(host(res["gd"])[m] == 0), tag
    log(f"samu {dt} B{B} T{T} M{M}: tiles, walk and AUTO within the derived bounds, with and "
        f"without resets")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_samu_deterministic_and_derivation_bitwise(dt):
    """Two runs, and a run that derives every predecessor map itself
    (polls=1), agree bit for bit, parameter gradients included."""
    inp = W.samu_inputs(2, 4096, 256, dt, seed=25)
    h0, gl = state_pair(2, 256, 26), state_pair(2, 256, 27)
    mask = np.random.default_rng(28).random((2, 4096)) < 0.01
    r1 = run(inp, h0=h0, gl=gl, mask=mask)
    r2 = run(inp, h0=h0, gl=gl, mask=mask)
    r3 = run(inp, h0=h0, gl=gl, mask=mask, polls=1)
    for k in r1:
        if k == "gh0":
            for x, y, z in zip(r1[k], r2[k], r3[k]):
                assert torch.equal(x, y) and torch.equal(x, z), k
        else:
            assert torch.equal(r1[k], r2[k]), f"{k} not bitwise repeatable"
            assert torch.equal(r1[k], r3[k]), f"{k} differs with polls=1"


def test_samu_caller_workspace_and_state_only_forward():
    """A caller workspace of scan_samu_workspace_bytes() gives the same bits as
    the library's; the state-only forward's last equals the full forward's."""
    B, T, M = 2, 700, 96
    inp = W.samu_inputs(B, T, M, "bf16", seed=29)
    need = lr.scan_samu_workspace_bytes(B, T, M, lr.BF16)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    r1 = run(inp)
    r2 = run(inp, workspace=ws)
    for k in r1:
        if k != "gh0":
            assert torch.equal(r1[k], r2[k]), k
    t = sdev(inp)
    _, _, lr_only, li_only = lr.samu_scan(t["eta"], t["delta"], t["nu_log"], t["theta_log"],
                                          t["br"], t["bi"], with_out=False)
    torch.cuda.synchronize()
    assert torch.equal(lr_only, r1["last_r"]) and torch.equal(li_only, r1["last_i"])
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(lr.LRScanError):
        run(inp, workspace=small)


def test_samu_autograd_wrapper():
    B, T, M = 2, 200, 64
    inp = W.samu_inputs(B, T, M, "f32", seed=30)
    t = sdev(inp)
    leaves = [t[k].clone().requires_grad_(True)
              for k in ("eta", "delta", "nu_log", "theta_log", "br", "bi")]
    out_r, out_i = lr.samu_diagonal_scan(*leaves)
    loss = (out_r * t["gr"]).sum() + (out_i * t["gi"]).sum()
    loss.backward()
    eta, delta, nu_log, theta_log = inp.controls()
    bd = Bounds(eta, delta, nu_log, theta_log, inp.c128("b"), inp.c128("g"), "f32")
    rtol, atol = TOL["f32"]
    check("grad_eta", host(leaves[0].grad), bd.ge, bd.tol_ge)
    check("grad_delta", host(leaves[1].grad), bd.gd, bd.tol_gd)
    check("grad_nu_log", host(leaves[2].grad), bd.gn, bd.tol_gn)
    check("grad_theta_log", host(leaves[3].grad), bd.gt, bd.tol_gt)
    gb = host(leaves[4].grad) + 1j * host(leaves[5].grad)
    check("grad_b", gb, bd.lam, atol + rtol * np.abs(bd.lam) + bd.E_l)


def test_samu_full_size_workload_by_rows():
    """swide (B8 T2048 M2560 bf16) in the launch configuration the benchmark
    times: every batch row against the oracle (out, last, grad_b, grad_eta,
    grad_delta, every element), and grad_nu_log / grad_theta_log against the
    sum of the oracle's per-row contributions (the loss is a sum over rows)."""
    wl = W.SAMU_WORKLOADS["swide"]
    inp = W.generate_samu(wl, seed=0)
    res = run(inp, need_grad_h0=False)
    gn_ref = np.zeros(wl.D)
    gt_ref = np.zeros(wl.D)
    tol_gn = np.zeros(wl.D)
    tol_gt = np.zeros(wl.D)
    for row in range(wl.B):
        rows = [row]
        eta, delta, nu_log, theta_log = inp.controls(rows)
        bd = Bounds(eta, delta, nu_log, theta_log, inp.c128("b", rows), inp.c128("g", rows),
                    "bf16", mode_terms=wl.B * wl.T)
        gn_ref += bd.gn
        gt_ref += bd.gt
        tol_gn += bd.tol_gn
        tol_gt += bd.tol_gt
        check_all(f"swide row {row}", res, bd, rows=slice(row, row + 1), check_params=False)
    log(f"swide: every batch row within the derived bounds")
    check("swide grad_nu_log", host(res["gn"]), gn_ref, tol_gn)
    check("swide grad_theta_log", host(res["gt"]), gt_ref, tol_gt)
    log("swide parameter gradients within the derived bounds")
