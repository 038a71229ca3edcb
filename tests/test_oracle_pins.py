"""Pins of the fp64 oracle against what the mathematics fixes (CPU only).

Each test checks the oracle against something other than itself: a value
derived by hand, a closed form, a library routine (numpy cumsum, torch
autograd), exact rational arithmetic, finite differences, or an identity that
a dropped term, a wrong sign or a shifted index would break.  The recurrence
and its adjoint are the ones the page "triton_training_scan.py"
(botwwt.github.io/SAMU_GPU/benchmark) defines in _real_forward and
_real_backward; the chunk forms are its _real_chunk_* and
_real_reverse_chunk_* kernels.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def rand(shape, seed, lo=-1.0, hi=1.0):
    return np.random.default_rng(seed).uniform(lo, hi, size=shape)


def dyadic(shape, seed, scale=8):
    """Random dyadic rationals k/scale, exact in binary floating point."""
    r = np.random.default_rng(seed)
    return r.integers(-scale, scale + 1, size=shape) / float(scale)


# ----------------------------------------------------------------------------
# hand-worked example (tests/golden/hand_example.json, derivation inside)
# ----------------------------------------------------------------------------
def load_golden():
    with open(os.path.join(HERE, "golden", "hand_example.json")) as f:
        ex = json.load(f)
    arr = lambda k: np.array(ex[k], dtype=np.float64)[None]  # [1, T, D]
    return ex, arr


def test_golden_forward_backward():
    ex, arr = load_golden()
    a, b, g = arr("a"), arr("b"), arr("g")
    out, last = oracle.scan_fwd(a, b)
    assert np.array_equal(out, arr("out"))
    assert np.array_equal(last[0], np.array(ex["last"]))
    ga, gb, gh0 = oracle.scan_bwd(a, out, g)
    assert np.array_equal(gb, arr("grad_b"))
    assert np.array_equal(ga, arr("grad_a"))
    assert np.array_equal(gh0[0], np.array(ex["grad_h0"]))
    gl = np.array(ex["grad_last"])[None]
    ga, gb, gh0 = oracle.scan_bwd(a, out, g, grad_last=gl)
    w = ex["with_grad_last"]
    assert np.array_equal(gb[0], np.array(w["grad_b"]))
    assert np.array_equal(ga[0], np.array(w["grad_a"]))
    assert np.array_equal(gh0[0], np.array(w["grad_h0"]))


def test_golden_chunks():
    ex, arr = load_golden()
    a, b, g = arr("a"), arr("b"), arr("g")
    C = ex["chunk"]
    P, Q = oracle.chunk_summary(a, b, C)
    assert np.array_equal(P, arr("P")) and np.array_equal(Q, arr("Q"))
    cin, last = oracle.chunk_prefix(P, Q)
    assert np.array_equal(cin, arr("chunk_in"))
    assert np.array_equal(last[0], np.array(ex["last"]))
    out, last2 = oracle.chunk_replay(a, b, cin, C)
    assert np.array_equal(out, arr("out")) and np.array_equal(last2, last)
    rP, rQ = oracle.reverse_chunk_summary(a, g, C)
    assert np.array_equal(rP, arr("reverse_P")) and np.array_equal(rQ, arr("reverse_Q"))
    fut, gh0 = oracle.reverse_chunk_prefix(rP, rQ)
    assert np.array_equal(fut, arr("future"))
    assert np.array_equal(gh0[0], np.array(ex["grad_h0"]))
    ga, gb = oracle.reverse_chunk_replay(a, out, g, fut, C)
    assert np.array_equal(ga, arr("grad_a")) and np.array_equal(gb, arr("grad_b"))


# ----------------------------------------------------------------------------
# special cases that reduce to textbook results
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [0, 1])
def test_a_one_is_cumulative_sum(seed):
    B, T, D = 2, 37, 5
    a = np.ones((B, T, D))
    b = rand((B, T, D), seed)
    g = rand((B, T, D), seed + 10)
    gl = rand((B, D), seed + 20)
    out, last = oracle.scan_fwd(a, b)
    np.testing.assert_allclose(out, np.cumsum(b, axis=1), rtol=0, atol=1e-12)
    np.testing.assert_allclose(last, b.sum(axis=1), rtol=0, atol=1e-12)
    ga, gb, gh0 = oracle.scan_bwd(a, out, g, grad_last=gl)
    rev = np.flip(np.cumsum(np.flip(g, axis=1), axis=1), axis=1) + gl[:, None, :]
    np.testing.assert_allclose(gb, rev, rtol=0, atol=1e-12)
    prev = np.concatenate([np.zeros((B, 1, D)), out[:, :-1]], axis=1)
    np.testing.assert_allclose(ga, rev * prev, rtol=0, atol=1e-12)
    np.testing.assert_allclose(gh0, rev[:, 0], rtol=0, atol=1e-12)


def test_a_zero_returns_b():
    B, T, D = 3, 20, 4
    a = np.zeros((B, T, D))
    b = rand((B, T, D), 3)
    g = rand((B, T, D), 4)
    out, last = oracle.scan_fwd(a, b, h0=rand((B, D), 5))
    assert np.array_equal(out, b) and np.array_equal(last, b[:, -1])
    ga, gb, gh0 = oracle.scan_bwd(a, out, g)
    assert np.array_equal(gb, g)
    assert np.array_equal(ga[:, 1:], g[:, 1:] * b[:, :-1])
    assert np.array_equal(ga[:, 0], np.zeros((B, D)))
    assert np.array_equal(gh0, np.zeros((B, D)))


@pytest.mark.parametrize("alpha,beta,gamma", [(0.9, 1.0, 1.0), (0.5, -2.0, 0.25), (1.5, 0.5, -1.0),
                                              (-0.7, 1.0, 2.0)])
def test_constant_coefficients_geometric_sum(alpha, beta, gamma):
    B, T, D = 1, 40, 3
    a = np.full((B, T, D), alpha)
    b = np.full((B, T, D), beta)
    g = np.full((B, T, D), gamma)
    t = np.arange(T)[None, :, None]
    out, last = oracle.scan_fwd(a, b)
    h = beta * (1 - alpha ** (t + 1)) / (1 - alpha)
    np.testing.assert_allclose(out, np.broadcast_to(h, out.shape), rtol=1e-12, atol=1e-12)
    ga, gb, _ = oracle.scan_bwd(a, out, g)
    lam = gamma * (1 - alpha ** (T - t)) / (1 - alpha)
    np.testing.assert_allclose(gb, np.broadcast_to(lam, gb.shape), rtol=1e-12, atol=1e-12)
    hprev = np.where(t > 0, beta * (1 - alpha ** t) / (1 - alpha), 0.0)
    np.testing.assert_allclose(ga, np.broadcast_to(lam * hprev, ga.shape), rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# brute force on tiny inputs
# ----------------------------------------------------------------------------
def test_forward_matches_explicit_sum_exactly():
    """h_t = sum_{k<=t} (prod_{j=k+1..t} a_j) b_k + (prod_{j=0..t} a_j) h0,
    evaluated in exact rational arithmetic on dyadic inputs."""
    B, T, D = 2, 9, 3
    a = dyadic((B, T, D), 7, scale=4)
    b = dyadic((B, T, D), 8, scale=4)
    h0 = dyadic((B, D), 9, scale=4)
    out, last = oracle.scan_fwd(a, b, h0=h0)
    for bi in range(B):
        for d in range(D):
            A = [Fraction(x) for x in a[bi, :, d]]
            Bv = [Fraction(x) for x in b[bi, :, d]]
            for t in range(T):
                s = Fraction(h0[bi, d])
                for j in range(0, t + 1):
                    s *= A[j]
                for k in range(t + 1):
                    p = Bv[k]
                    for j in range(k + 1, t + 1):
                        p *= A[j]
                    s += p
                assert out[bi, t, d] == float(s)  # dyadic, few bits: exact in fp64
            assert last[bi, d] == out[bi, T - 1, d]


def test_forward_jacobian_in_b():
    """d out_s / d b_t = prod_{j=t+1..s} a_j for t <= s, zero for t > s."""
    T = 8
    a = rand((1, T, 1), 11, 0.3, 1.2)
    for t in range(T):
        e = np.zeros((1, T, 1))
        e[0, t, 0] = 1.0
        col, _ = oracle.scan_fwd(a, e)
        for s in range(T):
            want = np.prod(a[0, t + 1:s + 1, 0]) if s >= t else 0.0
            assert col[0, s, 0] == pytest.approx(want, rel=1e-14, abs=0)


def _loss(a, b, g, gl, h0):
    out, last = oracle.scan_fwd(a, b, h0=h0)
    return float(np.sum(g * out) + np.sum(gl * last))


def test_backward_matches_central_finite_differences():
    B, T, D = 2, 6, 2
    a = rand((B, T, D), 21, 0.2, 1.1)
    b = rand((B, T, D), 22)
    g = rand((B, T, D), 23)
    gl = rand((B, D), 24)
    h0 = rand((B, D), 25)
    out, _ = oracle.scan_fwd(a, b, h0=h0)
    ga, gb, gh0 = oracle.scan_bwd(a, out, g, h0=h0, grad_last=gl)
    eps = 1e-6
    for name, x, grad in (("a", a, ga), ("b", b, gb), ("h0", h0, gh0)):
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            ix = it.multi_index
            args = {"a": a.copy(), "b": b.copy(), "h0": h0.copy()}
            args[name][ix] += eps
            up = _loss(args["a"], args["b"], g, gl, args["h0"])
            args[name][ix] -= 2 * eps
            dn = _loss(args["a"], args["b"], g, gl, args["h0"])
            fd = (up - dn) / (2 * eps)
            assert grad[ix] == pytest.approx(fd, rel=1e-7, abs=1e-8), (name, ix)


def test_backward_matches_torch_autograd():
    torch = pytest.importorskip("torch")
    B, T, D = 2, 11, 3
    a = rand((B, T, D), 31, -1.1, 1.1)
    b = rand((B, T, D), 32)
    g = rand((B, T, D), 33)
    gl = rand((B, D), 34)
    h0 = rand((B, D), 35)
    ta = torch.tensor(a, requires_grad=True)
    tb = torch.tensor(b, requires_grad=True)
    th0 = torch.tensor(h0, requires_grad=True)
    h = th0
    outs = []
    for t in range(T):
        h = ta[:, t] * h + tb[:, t]
        outs.append(h)
    tout = torch.stack(outs, dim=1)
    loss = (tout * torch.tensor(g)).sum() + (h * torch.tensor(gl)).sum()
    loss.backward()
    out, last = oracle.scan_fwd(a, b, h0=h0)
    np.testing.assert_allclose(out, tout.detach().numpy(), rtol=1e-13, atol=1e-13)
    ga, gb, gh0 = oracle.scan_bwd(a, out, g, h0=h0, grad_last=gl)
    np.testing.assert_allclose(ga, ta.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(gb, tb.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(gh0, th0.grad.numpy(), rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# identities at moderate size
# ----------------------------------------------------------------------------
def test_adjoint_identity():
    """out is linear in (b, h0): <g,out> + <gl,last> = <grad_b,b> + <grad_h0,h0>."""
    B, T, D = 3, 500, 7
    a = rand((B, T, D), 41, 0.8, 1.0)
    b = rand((B, T, D), 42)
    g = rand((B, T, D), 43)
    gl = rand((B, D), 44)
    h0 = rand((B, D), 45)
    out, last = oracle.scan_fwd(a, b, h0=h0)
    ga, gb, gh0 = oracle.scan_bwd(a, out, g, h0=h0, grad_last=gl)
    lhs = np.sum(g * out) + np.sum(gl * last)
    rhs = np.sum(gb * b) + np.sum(gh0 * h0)
    assert lhs == pytest.approx(rhs, rel=1e-11)


def test_time_reversal_duality():
    """grad_b is the forward scan run backwards in time: with
    at_tau = a_{T-tau} (tau >= 1), at_0 = 1, bt_tau = g_{T-1-tau} and initial
    state grad_last, flip(scan(at, bt)) = grad_b."""
    B, T, D = 2, 64, 5
    a = rand((B, T, D), 51, 0.5, 1.0)
    b = rand((B, T, D), 52)
    g = rand((B, T, D), 53)
    gl = rand((B, D), 54)
    out, _ = oracle.scan_fwd(a, b)
    _, gb, gh0 = oracle.scan_bwd(a, out, g, grad_last=gl)
    at = np.concatenate([np.ones((B, 1, D)), np.flip(a[:, 1:], axis=1)], axis=1)
    bt = np.flip(g, axis=1)
    dual, dual_last = oracle.scan_fwd(at, bt, h0=gl)
    np.testing.assert_allclose(np.flip(dual, axis=1), gb, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(a[:, 0] * dual_last, gh0, rtol=1e-12, atol=1e-12)


def test_linearity_in_b():
    B, T, D = 2, 100, 3
    a = rand((B, T, D), 61, 0.5, 1.0)
    b1 = rand((B, T, D), 62)
    b2 = rand((B, T, D), 63)
    o1, _ = oracle.scan_fwd(a, b1)
    o2, _ = oracle.scan_fwd(a, b2)
    o3, _ = oracle.scan_fwd(a, 2.0 * b1 - 3.0 * b2)
    np.testing.assert_allclose(o3, 2.0 * o1 - 3.0 * o2, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# chunk forms: associativity against the sequential definition
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("T,C", [(64, 16), (100, 16), (65, 64), (1, 16), (256, 256), (300, 128)])
def test_chunk_forms_equal_sequential(T, C):
    B, D = 2, 3
    a = rand((B, T, D), 71, 0.6, 1.05)
    b = rand((B, T, D), 72)
    g = rand((B, T, D), 73)
    gl = rand((B, D), 74)
    h0 = rand((B, D), 75)
    out, last = oracle.scan_fwd(a, b, h0=h0)
    P, Q = oracle.chunk_summary(a, b, C)
    NC = oracle.n_chunks(T, C)
    assert P.shape == (B, NC, D)
    # P is a plain product over the chunk (numpy prod), Q the chunk scanned from zero
    for k in range(NC):
        sl = slice(k * C, min(k * C + C, T))
        np.testing.assert_allclose(P[:, k], np.prod(a[:, sl], axis=1), rtol=1e-13)
        q, _ = oracle.scan_fwd(a[:, sl], b[:, sl])
        np.testing.assert_allclose(Q[:, k], q[:, -1], rtol=1e-13)
    cin, plast = oracle.chunk_prefix(P, Q, h0=h0)
    np.testing.assert_allclose(cin[:, 0], h0, rtol=0, atol=0)
    np.testing.assert_allclose(plast, last, rtol=1e-12, atol=1e-12)
    ro, rl = oracle.chunk_replay(a, b, cin, C)
    np.testing.assert_allclose(ro, out, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(rl, last, rtol=1e-12, atol=1e-12)
    for k in range(1, NC):
        np.testing.assert_allclose(cin[:, k], out[:, k * C - 1], rtol=1e-12, atol=1e-12)

    ga, gb, gh0 = oracle.scan_bwd(a, out, g, h0=h0, grad_last=gl)
    rP, rQ = oracle.reverse_chunk_summary(a, g, C)
    for k in range(NC):
        sl = slice(k * C, min(k * C + C, T))
        np.testing.assert_allclose(rP[:, k], np.prod(a[:, sl], axis=1), rtol=1e-13)
    fut, rg0 = oracle.reverse_chunk_prefix(rP, rQ, grad_last=gl)
    np.testing.assert_allclose(fut[:, NC - 1], gl, rtol=0, atol=0)
    np.testing.assert_allclose(rg0, gh0, rtol=1e-12, atol=1e-12)
    # the carry entering chunk k from the right is a_{t} lambda_{t} at its first row after it
    for k in range(NC - 1):
        t = (k + 1) * C
        np.testing.assert_allclose(fut[:, k], a[:, t] * gb[:, t], rtol=1e-12, atol=1e-12)
    rga, rgb = oracle.reverse_chunk_replay(a, out, g, fut, C, h0=h0)
    np.testing.assert_allclose(rga, ga, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(rgb, gb, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# masked workload invariants: resets and padding
# ----------------------------------------------------------------------------
def test_reset_and_padding_invariants():
    rng = np.random.default_rng(81)
    B, T, D = 2, 60, 4
    a = rng.uniform(0.5, 1.0, (B, T, D))
    b = rng.standard_normal((B, T, D))
    g = rng.standard_normal((B, T, D))
    r = 23  # reset step in every batch row
    pads = [5, 6, 40, 41, 42]
    a[:, r] = 0.0
    a[:, pads] = 1.0
    b[:, pads] = 0.0
    g[:, pads] = 0.0
    out, _ = oracle.scan_fwd(a, b)
    ga, gb, _ = oracle.scan_bwd(a, out, g)
    # a reset restarts the scan: out_r = b_r, and the suffix equals a fresh scan
    assert np.array_equal(out[:, r], b[:, r])
    fresh, _ = oracle.scan_fwd(a[:, r:], b[:, r:])
    np.testing.assert_allclose(out[:, r:], fresh, rtol=1e-13, atol=1e-13)
    # gradients before the reset do not see grad_out after it
    g2 = g.copy()
    g2[:, r + 1:] = rng.standard_normal((B, T - r - 1, D))
    ga2, gb2, _ = oracle.scan_bwd(a, out, g2)
    assert np.array_equal(gb2[:, :r], gb[:, :r])
    assert np.array_equal(ga2[:, :r], ga[:, :r])
    # padding steps pass the state through
    for p in pads:
        np.testing.assert_allclose(out[:, p], out[:, p - 1], rtol=0, atol=0)
    # compaction: dropping padding steps leaves every kept output unchanged
    keep = [t for t in range(T) if t not in pads]
    oc, _ = oracle.scan_fwd(a[:, keep], b[:, keep])
    np.testing.assert_allclose(oc, out[:, keep], rtol=1e-13, atol=1e-13)
    gac, gbc, _ = oracle.scan_bwd(a[:, keep], oc, g[:, keep])
    np.testing.assert_allclose(gbc, gb[:, keep], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(gac, ga[:, keep], rtol=1e-12, atol=1e-12)


def test_last_equals_final_state_and_threads_agree():
    B, T, D = 3, 200, 33
    a = rand((B, T, D), 91, 0.8, 1.0)
    b = rand((B, T, D), 92)
    g = rand((B, T, D), 93)
    out, last = oracle.scan_fwd(a, b)
    assert np.array_equal(last, out[:, -1])
    out4, last4 = oracle.scan_fwd(a, b, threads=4)
    assert np.array_equal(out4, out) and np.array_equal(last4, last)
    r1 = oracle.scan_bwd(a, out, g)
    r4 = oracle.scan_bwd(a, out, g, threads=5)
    for x, y in zip(r1, r4):
        assert np.array_equal(x, y)


# ----------------------------------------------------------------------------
# segment resets: a [B, T] mask whose nonzero entries start a new segment
# (the state entering that step is dropped, as a forced a = 0)
# ----------------------------------------------------------------------------
def _segments(mask_row):
    """[start, end) of every segment of one batch row."""
    T = mask_row.shape[0]
    starts = [0] + [t for t in range(1, T) if mask_row[t]]
    return list(zip(starts, starts[1:] + [T]))


def _reset_case(B=3, T=40, D=5, seed=21):
    a, b, g = rand((B, T, D), seed, 0.3, 1.2), rand((B, T, D), seed + 1), rand((B, T, D), seed + 2)
    h0, gl = rand((B, D), seed + 3), rand((B, D), seed + 4)
    mask = np.random.default_rng(seed + 5).random((B, T)) < 0.15
    mask[0, 0] = True       # a reset on the very first step drops h0
    mask[1, 0] = False
    mask[1, T - 1] = True   # and one on the very last step
    return a, b, g, h0, gl, mask


def test_reset_mask_splits_into_independent_segments():
    """Forward and backward with a reset mask equal the plain scan run on
    each segment on its own: zero entering state (h0 only for a first segment
    that is not reset), grad_last only for the final segment, no gradient
    reaching a reset step's a, and none crossing a reset."""
    a, b, g, h0, gl, mask = _reset_case()
    B, T, D = a.shape
    out, last = oracle.scan_fwd(a, b, h0=h0, reset=mask)
    ga, gb, gh0 = oracle.scan_bwd(a, out, g, h0=h0, grad_last=gl, reset=mask)
    for bi in range(B):
        for s, e in _segments(mask[bi]):
            first = s == 0 and not mask[bi, 0]
            sh0 = h0[bi:bi + 1] if first else None
            so, sl = oracle.scan_fwd(a[bi:bi + 1, s:e], b[bi:bi + 1, s:e], h0=sh0)
            assert np.array_equal(out[bi, s:e], so[0]), (bi, s, e)
            sgl = gl[bi:bi + 1] if e == T else None
            sga, sgb, sgh0 = oracle.scan_bwd(a[bi:bi + 1, s:e], so, g[bi:bi + 1, s:e], h0=sh0,
                                             grad_last=sgl)
            assert np.array_equal(gb[bi, s:e], sgb[0]), (bi, s, e)
            assert np.array_equal(ga[bi, s:e], sga[0]), (bi, s, e)
            if s == 0:
                expect = sgh0[0] if first else np.zeros(D)
                assert np.array_equal(gh0[bi], expect), bi
            else:
                assert np.all(ga[bi, s] == 0.0)
        assert np.array_equal(last[bi], out[bi, T - 1])


def test_reset_gradients_match_finite_differences():
    """dL/da, dL/db and dL/dh0 of L = <g, out> + <grad_last, last> under a
    reset mask, by central differences in fp64 (a is not used at a reset
    step, so its derivative there is exactly 0)."""
    a, b, g, h0, gl, mask = _reset_case(B=2, T=9, D=2, seed=33)
    mask[0, 4] = True

    def loss(a_, b_, h0_):
        o, l = oracle.scan_fwd(a_, b_, h0=h0_, reset=mask)
        return float(np.sum(g * o) + np.sum(gl * l))

    out, _ = oracle.scan_fwd(a, b, h0=h0, reset=mask)
    ga, gb, gh0 = oracle.scan_bwd(a, out, g, h0=h0, grad_last=gl, reset=mask)
    eps = 1e-6
    for arr, grad, which in ((a, ga, 0), (b, gb, 1), (h0, gh0, 2)):
        for idx in np.ndindex(arr.shape):
            up, dn = arr.copy(), arr.copy()
            up[idx] += eps
            dn[idx] -= eps
            args_up = [a, b, h0]
            args_dn = [a, b, h0]
            args_up[which], args_dn[which] = up, dn
            fd = (loss(*args_up) - loss(*args_dn)) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-7 * (1 + abs(fd)), (which, idx, fd, grad[idx])
    assert np.all(ga[mask[:, :, None].repeat(a.shape[2], 2)] == 0.0)


def test_reset_all_clear_mask_is_the_plain_scan():
    a, b, g, h0, gl, _ = _reset_case(seed=41)
    mask = np.zeros(a.shape[:2], dtype=bool)
    o1, l1 = oracle.scan_fwd(a, b, h0=h0, reset=mask)
    o2, l2 = oracle.scan_fwd(a, b, h0=h0)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    r1 = oracle.scan_bwd(a, o1, g, h0=h0, grad_last=gl, reset=mask)
    r2 = oracle.scan_bwd(a, o2, g, h0=h0, grad_last=gl)
    for x, y in zip(r1, r2):
        assert np.array_equal(x, y)


# ----------------------------------------------------------------------------
# complex diagonal scan (page "triton_training_scan.py", _complex_forward /
# _complex_backward): h_t = a_t h_{t-1} + b_t over complex values, adjoint
# through conj(a)
# ----------------------------------------------------------------------------
def crand(shape, seed, scale=1.0):
    r = np.random.default_rng(seed)
    return scale * (r.uniform(-1, 1, shape) + 1j * r.uniform(-1, 1, shape))


def test_complex_with_real_values_is_the_real_scan():
    """Real a, b, g, h0, grad_last: every complex result has a zero imaginary
    part and a real part bitwise equal to the real oracle's."""
    B, T, D = 2, 37, 5
    a, b, g = rand((B, T, D), 50, 0.2, 1.1), rand((B, T, D), 51), rand((B, T, D), 52)
    h0, gl = rand((B, D), 53), rand((B, D), 54)
    mask = np.random.default_rng(55).random((B, T)) < 0.1
    o, l = oracle.complex_fwd(a + 0j, b + 0j, h0=h0 + 0j, reset=mask)
    ro, rl = oracle.scan_fwd(a, b, h0=h0, reset=mask)
    assert np.array_equal(o.real, ro) and not np.any(o.imag)
    assert np.array_equal(l.real, rl) and not np.any(l.imag)
    ga, gb, gh0 = oracle.complex_bwd(a + 0j, o, g + 0j, h0=h0 + 0j, grad_last=gl + 0j, reset=mask)
    rga, rgb, rgh0 = oracle.scan_bwd(a, ro, g, h0=h0, grad_last=gl, reset=mask)
    for z, r in ((ga, rga), (gb, rgb), (gh0, rgh0)):
        assert np.array_equal(z.real, r) and not np.any(z.imag)


def test_complex_real_transition_splits_into_two_real_scans():
    """With real a, the real and imaginary parts of b scan independently."""
    B, T, D = 3, 29, 4
    a = rand((B, T, D), 60, 0.1, 1.0)
    b, g = crand((B, T, D), 61), crand((B, T, D), 62)
    o, _ = oracle.complex_fwd(a + 0j, b)
    assert np.array_equal(o.real, oracle.scan_fwd(a, b.real)[0])
    assert np.array_equal(o.imag, oracle.scan_fwd(a, b.imag)[0])
    ga, gb, _ = oracle.complex_bwd(a + 0j, o, g)
    assert np.array_equal(gb.real, oracle.scan_bwd(a, o.real, g.real)[1])
    assert np.array_equal(gb.imag, oracle.scan_bwd(a, o.imag, g.imag)[1])


def test_complex_rotation_closed_form():
    """a_t = r e^{i theta} for every t and b = (b0, 0, 0, ...): h_t = a^t b0."""
    T = 400
    r_, th = 0.999, 0.3
    a = np.full((1, T, 1), r_ * np.exp(1j * th))
    b = np.zeros((1, T, 1), complex)
    b[0, 0, 0] = 0.7 - 0.2j
    o, _ = oracle.complex_fwd(a, b)
    t = np.arange(T)
    expect = (r_ ** t) * np.exp(1j * th * t) * b[0, 0, 0]
    assert np.allclose(o[0, :, 0], expect, rtol=1e-12 * T, atol=1e-15)
    # |a| = 1: the modulus is preserved
    o1, _ = oracle.complex_fwd(np.full((1, T, 1), np.exp(1j * th)), b)
    assert np.allclose(np.abs(o1[0, :, 0]), abs(b[0, 0, 0]), rtol=1e-12 * T)


def test_complex_gradients_match_finite_differences():
    """dL/dRe + i dL/dIm of L = sum Re(conj(g) h) + Re(conj(grad_last) h_{T-1})
    for a, b and h0, by central differences in fp64, with a reset mask."""
    B, T, M = 2, 7, 2
    a, b, g = crand((B, T, M), 70, 0.8), crand((B, T, M), 71), crand((B, T, M), 72)
    h0, gl = crand((B, M), 73), crand((B, M), 74)
    mask = np.zeros((B, T), bool)
    mask[1, 3] = True

    def loss(a_, b_, h0_):
        o, l = oracle.complex_fwd(a_, b_, h0=h0_, reset=mask)
        return float(np.sum((np.conj(g) * o).real) + np.sum((np.conj(gl) * l).real))

    o, _ = oracle.complex_fwd(a, b, h0=h0, reset=mask)
    ga, gb, gh0 = oracle.complex_bwd(a, o, g, h0=h0, grad_last=gl, reset=mask)
    eps = 1e-6
    for which, (arr, grad) in enumerate(((a, ga), (b, gb), (h0, gh0))):
        for idx in np.ndindex(arr.shape):
            for unit, part in ((1.0, "re"), (1j, "im")):
                up, dn = arr.copy(), arr.copy()
                up[idx] += eps * unit
                dn[idx] -= eps * unit
                args_up, args_dn = [a, b, h0], [a, b, h0]
                args_up[which], args_dn[which] = up, dn
                fd = (loss(*args_up) - loss(*args_dn)) / (2 * eps)
                got = grad[idx].real if part == "re" else grad[idx].imag
                assert abs(fd - got) <= 1e-7 * (1 + abs(fd)), (which, idx, part, fd, got)
    assert ga[1, 3, 0] == 0 and ga[1, 3, 1] == 0


# ----------------------------------------------------------------------------
# fused-transition (SAMU-form) scan (page "triton_training_scan.py",
# _samu_forward / _samu_backward): a = exp(-nu e^eta) e^{i(theta + delta)},
# nu = e^{nu_log}, theta = e^{theta_log}
# ----------------------------------------------------------------------------
def test_samu_hand_values_closed_form():
    """nu_log = 0, eta = ln ln 2 gives rho = 1/2; theta = delta = pi/2 gives a
    phase of pi: a = -1/2 on every step.  With b = 1 the scan is the geometric
    sum h_t = (1 - (-1/2)^(t+1)) / (3/2); with b = i it is i times that."""
    T = 60
    eta = np.full((1, T), np.log(np.log(2.0)))
    delta = np.full((1, T), np.pi / 2)
    nu_log, theta_log = np.zeros(2), np.full(2, np.log(np.pi / 2))
    b = np.zeros((1, T, 2), complex)
    b[..., 0] = 1.0
    b[..., 1] = 1j
    out, last = oracle.samu_fwd(eta, delta, nu_log, theta_log, b)
    t = np.arange(T)
    geo = (1 - (-0.5) ** (t + 1)) / 1.5
    assert np.allclose(out[0, :, 0], geo, rtol=0, atol=1e-14)
    assert np.allclose(out[0, :, 1], 1j * geo, rtol=0, atol=1e-14)
    assert np.allclose(last[0], [geo[-1], 1j * geo[-1]], atol=1e-14)


def test_samu_gradients_match_finite_differences():
    """grad_eta, grad_delta (per token), grad_nu_log, grad_theta_log (per
    mode), grad_b and grad_h0 of L = sum Re(conj(g) h) + Re(conj(g_last) h_{T-1})
    by central differences in fp64, with a reset mask."""
    B, T, M = 2, 6, 3
    r = np.random.default_rng(80)
    eta, delta = r.uniform(-2.0, 0.5, (B, T)), r.uniform(-1.0, 1.0, (B, T))
    nu_log, theta_log = r.uniform(-1.0, 0.5, M), r.uniform(-1.0, 1.0, M)
    b, g = crand((B, T, M), 81), crand((B, T, M), 82)
    h0, gl = crand((B, M), 83), crand((B, M), 84)
    mask = np.zeros((B, T), bool)
    mask[0, 2] = True

    def loss(e, d, nl, tl, bb, hh0):
        o, l = oracle.samu_fwd(e, d, nl, tl, bb, h0=hh0, reset=mask)
        return float(np.sum((np.conj(g) * o).real) + np.sum((np.conj(gl) * l).real))

    out, _ = oracle.samu_fwd(eta, delta, nu_log, theta_log, b, h0=h0, reset=mask)
    ge, gd, gn, gt, gb, gh0 = oracle.samu_bwd(eta, delta, nu_log, theta_log, out, g, h0=h0,
                                             grad_last=gl, reset=mask)
    args = [eta, delta, nu_log, theta_log, b, h0]
    eps = 1e-6
    for which, grad in ((0, ge), (1, gd), (2, gn), (3, gt)):
        for idx in np.ndindex(args[which].shape):
            up = [x.copy() for x in args]
            dn = [x.copy() for x in args]
            up[which][idx] += eps
            dn[which][idx] -= eps
            fd = (loss(*up) - loss(*dn)) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-7 * (1 + abs(fd)), (which, idx, fd, grad[idx])
    for which, grad in ((4, gb), (5, gh0)):
        for idx in np.ndindex(args[which].shape):
            for unit in (1.0, 1j):
                up = [x.copy() for x in args]
                dn = [x.copy() for x in args]
                up[which][idx] += eps * unit
                dn[which][idx] -= eps * unit
                fd = (loss(*up) - loss(*dn)) / (2 * eps)
                got = grad[idx].real if unit == 1.0 else grad[idx].imag
                assert abs(fd - got) <= 1e-7 * (1 + abs(fd)), (which, idx, unit, fd, got)
    # a reset step's transition does not depend on its controls
    assert ge[0, 2] == 0.0 and gd[0, 2] == 0.0
