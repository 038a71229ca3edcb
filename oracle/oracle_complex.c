/*
 * oracle_complex.c -- plain, slow, fp64 CPU oracle for the complex diagonal
 *                     recurrence  h_t = a_t * h_{t-1} + b_t  (complex a, b, h).
 *
 * TEST INFRASTRUCTURE ONLY, like oracle.c: nothing in the product path may
 * include, link, load or call it, and it shares no code with the HIP library.
 *
 * Source: the page "triton_training_scan.py" (botwwt.github.io/SAMU_GPU/
 * benchmark), kernels _complex_forward and _complex_backward and the class
 * _ComplexScan.  Storage is planar there: real and imaginary parts of a, b,
 * out (and of every gradient) are separate [B, T, M] arrays, element
 * (b, t, m) at (b*T + t)*M + m; the final state is two fp32 [B, M] arrays.
 *
 * Definitions, written here with C99 complex arithmetic:
 *   forward   h_{-1} = h0 (zero when absent),  h_t = a_t h_{t-1} + b_t.
 *   backward  for the real loss L = sum Re(conj(g_t) h_t) + Re(conj(g_last) h_{T-1})
 *             (g = grad_out_r + i grad_out_i, likewise g_last), the gradient
 *             with respect to z = x + i y is dL/dx + i dL/dy, and
 *               lambda_{T-1} = g_{T-1} + g_last,
 *               lambda_t     = g_t + conj(a_{t+1}) lambda_{t+1},
 *               grad_b_t = lambda_t,  grad_a_t = lambda_t conj(h_{t-1}),
 *               grad_h0  = conj(a_0) lambda_0.
 *   (_complex_backward: adds the direct gradient, emits grad_a from the
 *    previous state and grad_b from the adjoint, then carries the adjoint
 *    back through the conjugate of a_t.)
 * A segment-reset mask (as in oracle.c: [B, T] bytes, nonzero = a new
 * segment starts at step t) takes the transition of that step as 0; its
 * grad_a is then 0 and no adjoint is carried past it.
 */
#include <complex.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

static size_t cidx(int64_t b, int64_t t, int64_t m, int64_t T, int64_t M) {
    return ((size_t)b * (size_t)T + (size_t)t) * (size_t)M + (size_t)m;
}

static int c_reset(const uint8_t* reset, int64_t b, int64_t t, int64_t T) {
    return reset != NULL && reset[(size_t)b * (size_t)T + (size_t)t] != 0;
}

void oracle_complex_fwd(int64_t B, int64_t T, int64_t M, const double* ar, const double* ai,
                        const double* br, const double* bi, const double* h0r,
                        const double* h0i, const uint8_t* reset, double* out_r, double* out_i,
                        double* last_r, double* last_i) {
    for (int64_t b = 0; b < B; ++b)
        for (int64_t m = 0; m < M; ++m) {
            size_t lane = (size_t)b * (size_t)M + (size_t)m;
            double complex h = h0r ? CMPLX(h0r[lane], h0i[lane]) : CMPLX(0.0, 0.0);
            for (int64_t t = 0; t < T; ++t) {
                size_t i = cidx(b, t, m, T, M);
                double complex at = c_reset(reset, b, t, T) ? CMPLX(0.0, 0.0) : CMPLX(ar[i], ai[i]);
                h = at * h + CMPLX(br[i], bi[i]);
                out_r[i] = creal(h);
                out_i[i] = cimag(h);
            }
            last_r[lane] = creal(h);
            last_i[lane] = cimag(h);
        }
}

void oracle_complex_bwd(int64_t B, int64_t T, int64_t M, const double* ar, const double* ai,
                        const double* hr, const double* hi, const double* gr, const double* gi,
                        const double* h0r, const double* h0i, const double* glr,
                        const double* gli, const uint8_t* reset, double* gar, double* gai,
                        double* gbr, double* gbi, double* gh0r, double* gh0i) {
    for (int64_t b = 0; b < B; ++b)
        for (int64_t m = 0; m < M; ++m) {
            size_t lane = (size_t)b * (size_t)M + (size_t)m;
            /* carry = conj(a_{t+1}) lambda_{t+1} */
            double complex carry = glr ? CMPLX(glr[lane], gli[lane]) : CMPLX(0.0, 0.0);
            for (int64_t t = T - 1; t >= 0; --t) {
                size_t i = cidx(b, t, m, T, M);
                int r = c_reset(reset, b, t, T);
                double complex lam = CMPLX(gr[i], gi[i]) + carry;
                double complex prev;
                if (t > 0) {
                    size_t ip = cidx(b, t - 1, m, T, M);
                    prev = CMPLX(hr[ip], hi[ip]);
                } else {
                    prev = h0r ? CMPLX(h0r[lane], h0i[lane]) : CMPLX(0.0, 0.0);
                }
                double complex ga = r ? CMPLX(0.0, 0.0) : lam * conj(prev);
                gbr[i] = creal(lam);
                gbi[i] = cimag(lam);
                gar[i] = creal(ga);
                gai[i] = cimag(ga);
                double complex at = r ? CMPLX(0.0, 0.0) : CMPLX(ar[i], ai[i]);
                carry = conj(at) * lam;
            }
            if (gh0r) {
                gh0r[lane] = creal(carry);
                gh0i[lane] = cimag(carry);
            }
        }
}

/*
 * Fused-transition (SAMU-form) complex scan.  Source: the same page,
 * kernels _samu_forward and _samu_backward.  The transition is rebuilt from
 * per-token controls eta[b,t], delta[b,t] and per-mode parameters
 * nu_log[m], theta_log[m]:
 *   nu = exp(nu_log),  theta = exp(theta_log),
 *   rho = exp(-nu * exp(eta)),  a = rho * exp(i (theta + delta)),
 *   h_t = a_t h_{t-1} + b_t   (complex, as above; a reset step takes a = 0).
 * Backward, for the same real loss as the plain complex scan, with
 * grad_a = lambda conj(h_{t-1}) as above:
 *   radial = -nu exp(eta) Re(conj(a) grad_a),   phase = Im(conj(a) grad_a),
 *   grad_eta[b,t]   = sum over m of radial,     grad_delta[b,t] = sum over m of phase,
 *   grad_nu_log[m]  = sum over (b,t) of radial, grad_theta_log[m] = sum over (b,t) of theta phase,
 *   grad_b = lambda.
 * (radial is dL/d eta through rho; dL/d nu_log = nu dL/d nu has the same
 * expression; phase is dL/d delta, and dL/d theta_log = theta dL/d theta.)
 */
static double complex samu_a(double eta, double delta, double nu_log, double theta_log) {
    double nu = exp(nu_log), theta = exp(theta_log);
    double rho = exp(-nu * exp(eta));
    return rho * cexp(CMPLX(0.0, theta + delta));
}

void oracle_samu_fwd(int64_t B, int64_t T, int64_t M, const double* eta, const double* delta,
                     const double* nu_log, const double* theta_log, const double* br,
                     const double* bi, const double* h0r, const double* h0i,
                     const uint8_t* reset, double* out_r, double* out_i, double* last_r,
                     double* last_i) {
    for (int64_t b = 0; b < B; ++b)
        for (int64_t m = 0; m < M; ++m) {
            size_t lane = (size_t)b * (size_t)M + (size_t)m;
            double complex h = h0r ? CMPLX(h0r[lane], h0i[lane]) : CMPLX(0.0, 0.0);
            for (int64_t t = 0; t < T; ++t) {
                size_t i = cidx(b, t, m, T, M);
                size_t tok = (size_t)b * (size_t)T + (size_t)t;
                double complex at = c_reset(reset, b, t, T)
                                        ? CMPLX(0.0, 0.0)
                                        : samu_a(eta[tok], delta[tok], nu_log[m], theta_log[m]);
                h = at * h + CMPLX(br[i], bi[i]);
                out_r[i] = creal(h);
                out_i[i] = cimag(h);
            }
            last_r[lane] = creal(h);
            last_i[lane] = cimag(h);
        }
}

void oracle_samu_bwd(int64_t B, int64_t T, int64_t M, const double* eta, const double* delta,
                     const double* nu_log, const double* theta_log, const double* hr,
                     const double* hi, const double* gr, const double* gi, const double* h0r,
                     const double* h0i, const double* glr, const double* gli,
                     const uint8_t* reset, double* grad_eta, double* grad_delta,
                     double* grad_nu_log, double* grad_theta_log, double* gbr, double* gbi,
                     double* gh0r, double* gh0i) {
    for (int64_t i = 0; i < B * T; ++i) grad_eta[i] = grad_delta[i] = 0.0;
    for (int64_t m = 0; m < M; ++m) grad_nu_log[m] = grad_theta_log[m] = 0.0;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t m = 0; m < M; ++m) {
            size_t lane = (size_t)b * (size_t)M + (size_t)m;
            double nu = exp(nu_log[m]), theta = exp(theta_log[m]);
            double complex carry = glr ? CMPLX(glr[lane], gli[lane]) : CMPLX(0.0, 0.0);
            for (int64_t t = T - 1; t >= 0; --t) {
                size_t i = cidx(b, t, m, T, M);
                size_t tok = (size_t)b * (size_t)T + (size_t)t;
                int r = c_reset(reset, b, t, T);
                double complex lam = CMPLX(gr[i], gi[i]) + carry;
                double complex prev;
                if (t > 0) {
                    size_t ip = cidx(b, t - 1, m, T, M);
                    prev = CMPLX(hr[ip], hi[ip]);
                } else {
                    prev = h0r ? CMPLX(h0r[lane], h0i[lane]) : CMPLX(0.0, 0.0);
                }
                double complex at = r ? CMPLX(0.0, 0.0)
                                      : samu_a(eta[tok], delta[tok], nu_log[m], theta_log[m]);
                double complex ga = r ? CMPLX(0.0, 0.0) : lam * conj(prev);
                double complex w = conj(at) * ga;
                double radial = -nu * exp(eta[tok]) * creal(w);
                double phase = cimag(w);
                grad_eta[tok] += radial;
                grad_delta[tok] += phase;
                grad_nu_log[m] += radial;
                grad_theta_log[m] += theta * phase;
                gbr[i] = creal(lam);
                gbi[i] = cimag(lam);
                carry = conj(at) * lam;
            }
            if (gh0r) {
                gh0r[lane] = creal(carry);
                gh0i[lane] = cimag(carry);
            }
        }
}
