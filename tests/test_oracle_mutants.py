"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of oracle.c (a dropped term, a swapped
operand, a shifted index, a wrong seed, an inclusive-for-exclusive scan),
compiles it with gcc into a temporary directory, and runs the pin suite
against it in a subprocess.  The suite must fail for every mutant; the clean
source must pass.
"""
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "oracle.c")
SRC_COMPLEX = os.path.join(ROOT, "oracle", "oracle_complex.c")

# (name, text in oracle.c, replacement, occurrence index or None for all)
MUTANTS = [
    ("fwd_drop_b", "h = at * h + b[i];\n            if (out)", "h = at * h;\n            if (out)"),
    ("fwd_swap_ab", "h = at * h + b[i];\n            if (out)", "h = b[i] * h + at;\n            if (out)"),
    ("fwd_ignore_h0", "double h = h0 ? h0[lane] : 0.0;", "double h = 0.0;"),
    ("bwd_drop_carry", "double lam = g[i] + carry;\n            double h_prev = (t > 0) ? h[idx3(bi, t - 1, d, T, D)] : (h0 ? h0[lane] : 0.0);",
     "double lam = g[i];\n            double h_prev = (t > 0) ? h[idx3(bi, t - 1, d, T, D)] : (h0 ? h0[lane] : 0.0);"),
    ("bwd_hprev_same_step", "double h_prev = (t > 0) ? h[idx3(bi, t - 1, d, T, D)] : (h0 ? h0[lane] : 0.0);",
     "double h_prev = h[idx3(bi, t, d, T, D)];"),
    ("bwd_carry_uses_g", "carry = (r ? 0.0 : a[i]) * lam;", "carry = (r ? 0.0 : a[i]) * g[i];"),
    ("bwd_ignore_grad_last", "double carry = grad_last ? grad_last[lane] : 0.0;", "double carry = 0.0;"),
    ("bwd_grad_h0_lambda", "if (grad_h0) grad_h0[lane] = carry;", "if (grad_h0) grad_h0[lane] = carry / 2;"),
    ("summary_drop_decay", "q = a[i] * q + b[i];", "q = q + b[i];"),
    ("prefix_inclusive", "chunk_in[i] = s;\n                s = P[i] * s + Q[i];", "s = P[i] * s + Q[i];\n                chunk_in[i] = s;"),
    ("replay_zero_start", "double h = chunk_in[idx3(bi, k, d, NC, D)];", "double h = 0.0;"),
    ("rsummary_drop_a_on_g", "q = a[i] * q + a[i] * g[i];", "q = a[i] * q + g[i];"),
    ("rprefix_inclusive", "future[i] = s;\n                s = P[i] * s + Q[i];", "s = P[i] * s + Q[i];\n                future[i] = s;"),
    ("rreplay_no_decay", "carry = a[i] * lam;\n                }", "carry = lam;\n                }"),
    ("reset_ignored_fwd", "double at = is_reset(reset, bi, t, T) ? 0.0 : a[i];", "double at = a[i];"),
    ("reset_zeroes_b", "double at = is_reset(reset, bi, t, T) ? 0.0 : a[i];\n            h = at * h + b[i];",
     "double at = a[i];\n            h = at * h + (is_reset(reset, bi, t, T) ? 0.0 : b[i]);"),
    ("reset_shifted", "double at = is_reset(reset, bi, t, T) ? 0.0 : a[i];",
     "double at = is_reset(reset, bi, t > 0 ? t - 1 : 0, T) ? 0.0 : a[i];"),
    ("reset_keeps_grad_a", "grad_a[i] = r ? 0.0 : lam * h_prev;", "grad_a[i] = lam * h_prev;"),
    ("reset_keeps_carry", "carry = (r ? 0.0 : a[i]) * lam;", "carry = a[i] * lam;"),
    # complex oracle (the mutation applies to oracle_complex.c)
    ("c:fwd_conj_a", "h = at * h + CMPLX(br[i], bi[i]);", "h = conj(at) * h + CMPLX(br[i], bi[i]);"),
    ("c:fwd_swap_re_im_b", "h = at * h + CMPLX(br[i], bi[i]);", "h = at * h + CMPLX(bi[i], br[i]);"),
    ("c:bwd_carry_no_conj", "carry = conj(at) * lam;", "carry = at * lam;"),
    ("c:bwd_grad_a_no_conj", "lam * conj(prev);", "lam * prev;"),
    ("c:bwd_grad_a_conj_lam", "lam * conj(prev);", "conj(lam) * prev;"),
    ("c:reset_ignored", "double complex at = c_reset(reset, b, t, T) ? CMPLX(0.0, 0.0) : CMPLX(ar[i], ai[i]);",
     "double complex at = CMPLX(ar[i], ai[i]);"),
    ("c:h0_imag_dropped", "double complex h = h0r ? CMPLX(h0r[lane], h0i[lane]) : CMPLX(0.0, 0.0);",
     "double complex h = h0r ? CMPLX(h0r[lane], 0.0) : CMPLX(0.0, 0.0);"),
    # the same slips in the fused-transition oracle, which spells these lines
    # identically ("c2:" mutates the second occurrence)
    ("c2:fwd_conj_a", "h = at * h + CMPLX(br[i], bi[i]);", "h = conj(at) * h + CMPLX(br[i], bi[i]);"),
    ("c2:fwd_swap_re_im_b", "h = at * h + CMPLX(br[i], bi[i]);", "h = at * h + CMPLX(bi[i], br[i]);"),
    ("c2:bwd_carry_no_conj", "carry = conj(at) * lam;", "carry = at * lam;"),
    ("c2:bwd_grad_a_no_conj", "lam * conj(prev);", "lam * prev;"),
    ("c2:bwd_grad_a_conj_lam", "lam * conj(prev);", "conj(lam) * prev;"),
    ("c2:h0_imag_dropped", "double complex h = h0r ? CMPLX(h0r[lane], h0i[lane]) : CMPLX(0.0, 0.0);",
     "double complex h = h0r ? CMPLX(h0r[lane], 0.0) : CMPLX(0.0, 0.0);"),
    ("c:samu_nu_not_exp", "double nu = exp(nu_log), theta = exp(theta_log);",
     "double nu = nu_log, theta = exp(theta_log);"),
    ("c:samu_phase_sign", "return rho * cexp(CMPLX(0.0, theta + delta));",
     "return rho * cexp(CMPLX(0.0, theta - delta));"),
    ("c:samu_radial_no_nu", "double radial = -nu * exp(eta[tok]) * creal(w);",
     "double radial = -exp(eta[tok]) * creal(w);"),
    ("c:samu_theta_grad_no_theta", "grad_theta_log[m] += theta * phase;",
     "grad_theta_log[m] += phase;"),
    ("c:samu_phase_real_part", "double phase = cimag(w);", "double phase = creal(w);"),
    ("reset_mask_transposed", "return reset != NULL && reset[(size_t)bi * (size_t)T + (size_t)t] != 0;",
     "return reset != NULL && reset[(size_t)bi * (size_t)T + (size_t)(T - 1 - t)] != 0;"),
]


def _run_pins(lib_path):
    env = dict(os.environ)
    env["ORACLE_LIBRARY_OVERRIDE"] = lib_path
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           os.path.join(HERE, "test_oracle_pins.py")],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


def _compile(src_text, tmp_path, name, complex_text=None):
    c = tmp_path / f"{name}.c"
    cc = tmp_path / f"{name}_complex.c"
    so = tmp_path / f"{name}.so"
    c.write_text(src_text)
    cc.write_text(complex_text if complex_text is not None else open(SRC_COMPLEX).read())
    subprocess.check_call(["gcc", *oracle.GCC_FLAGS, str(c), str(cc), "-o", str(so), "-lm"])
    return str(so)


def test_clean_oracle_passes_pins(tmp_path):
    src = open(SRC).read()
    r = _run_pins(_compile(src, tmp_path, "clean"))
    assert r.returncode == 0, r.stdout[-2000:]


def _mutate(src, old, new, nth):
    """Replace the nth occurrence of old (1-based)."""
    at = -1
    for _ in range(nth):
        at = src.index(old, at + 1)
    return src[:at] + new + src[at + len(old):]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, tmp_path):
    path = SRC_COMPLEX if name.startswith(("c:", "c2:")) else SRC
    src = open(path).read()
    # a site is either unique or spelled once in each complex oracle (two)
    nth = 2 if name.startswith("c2:") else 1
    assert src.count(old) in ((1, 2) if path == SRC_COMPLEX else (1,)), \
        f"mutation site for {name} appears {src.count(old)} times"
    assert src.count(old) >= nth, f"{name}: no occurrence {nth}"
    mutated = _mutate(src, old, new, nth)
    tag = name.replace(":", "_")
    if path == SRC_COMPLEX:
        so = _compile(open(SRC).read(), tmp_path, tag, complex_text=mutated)
    else:
        so = _compile(mutated, tmp_path, tag)
    r = _run_pins(so)
    assert r.returncode != 0, f"mutant {name} survived the pins"
