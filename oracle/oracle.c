/*
 * oracle.c -- plain, slow, fp64 CPU oracle for the diagonal affine recurrence
 *             scan  h_t = a_t * h_{t-1} + b_t  over [B, T, D] tensors.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no code, header, table or
 * helper with the HIP library.
 *
 * Source of the definitions: the page "triton_training_scan.py"
 * (botwwt.github.io/SAMU_GPU/benchmark), which states the recurrence in its
 * module docstring and in the kernels _real_forward, _real_backward,
 * _real_chunk_summary, _real_chunk_prefix, _real_chunk_replay and their
 * _real_reverse_* counterparts.  The initial-state / final-gradient seeding
 * follows the same page's _samu_tiled_serial_forward/_backward (an optional
 * initial state, and an adjoint seeded from the gradient of the last state).
 *
 * Everything is written out exactly as defined, one lane at a time, in
 * double precision.  There is no blocking, fusion or reordering beyond what
 * the definitions state.  Layout of every [B, T, D] array is row-major with D
 * fastest: element (b, t, d) lives at (b*T + t)*D + d.  [B, D] arrays (h0,
 * last, grad_last, grad_h0) live at b*D + d.  Chunk arrays are [B, NC, D]
 * with NC = ceil(T / C); element (b, k, d) lives at (b*NC + k)*D + d.
 *
 * A lane-range worker is run over a partition of the (b, d) lanes by
 * oracle_parallel_*; the partition only splits independent lanes and does not
 * change any arithmetic.
 */
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

static size_t idx3(int64_t b, int64_t t, int64_t d, int64_t T, int64_t D) {
    return ((size_t)b * (size_t)T + (size_t)t) * (size_t)D + (size_t)d;
}

/* ------------------------------------------------------------------------ */
/* Segment resets (optional).  reset is a [B, T] byte mask, element (b, t) at */
/* b*T + t; a nonzero byte marks step t of batch row b as the first step of a */
/* new segment.  The state entering that step is dropped: the step's          */
/* transition is taken as 0 in place of a_t, so h_t = b_t.  (Page            */
/* "triton_training_scan.py", _samu_tiled_serial_forward: a step whose        */
/* segment position is 0 forces the decay to 0; the same page's token mask   */
/* is per (b, t) across all D.)  In the backward, a_t does not enter a reset  */
/* step, so grad_a_t = 0 there, and the adjoint carried to earlier steps is   */
/* 0 * lambda_t = 0.                                                          */
/* ------------------------------------------------------------------------ */
static int is_reset(const uint8_t* reset, int64_t bi, int64_t t, int64_t T) {
    return reset != NULL && reset[(size_t)bi * (size_t)T + (size_t)t] != 0;
}

/* ------------------------------------------------------------------------ */
/* Forward: h_{-1} = h0 (zero when h0 is NULL); h_t = a_t h_{t-1} + b_t.      */
/* out[b,t,d] = h_t; last[b,d] = h_{T-1}.                                    */
/* (_real_forward: zero state, one multiply-add per step, every state stored, */
/*  the final state stored separately.)                                       */
/* ------------------------------------------------------------------------ */
static void fwd_lanes(int64_t B, int64_t T, int64_t D, int64_t lane0, int64_t lane1,
                      const double* a, const double* b, const double* h0,
                      const uint8_t* reset, double* out, double* last) {
    (void)B;
    for (int64_t lane = lane0; lane < lane1; ++lane) {
        int64_t bi = lane / D, d = lane % D;
        double h = h0 ? h0[lane] : 0.0;
        for (int64_t t = 0; t < T; ++t) {
            size_t i = idx3(bi, t, d, T, D);
            double at = is_reset(reset, bi, t, T) ? 0.0 : a[i];
            h = at * h + b[i];
            if (out) out[i] = h;
        }
        if (last) last[lane] = h;
    }
}

void oracle_scan_fwd(int64_t B, int64_t T, int64_t D, const double* a, const double* b,
                     const double* h0, const uint8_t* reset, double* out, double* last) {
    fwd_lanes(B, T, D, 0, B * D, a, b, h0, reset, out, last);
}

/* ------------------------------------------------------------------------ */
/* Backward of L = <grad_out, out> + <grad_last, last>.                      */
/* The adjoint lambda_t = dL/dh_t obeys                                       */
/*   lambda_{T-1} = g_{T-1} + grad_last,  lambda_t = g_t + a_{t+1} lambda_{t+1} */
/* and                                                                        */
/*   grad_b_t = lambda_t,   grad_a_t = lambda_t * h_{t-1}  (h_{-1} = h0 or 0), */
/*   grad_h0  = a_0 * lambda_0.                                               */
/* (_real_backward: walk time in reverse, add the direct gradient, emit       */
/*  grad_a from the previous state and grad_b from the adjoint, then carry    */
/*  the adjoint back through a_t.)                                            */
/* `h` holds the forward states h_t (the forward's `out`).                    */
/* ------------------------------------------------------------------------ */
static void bwd_lanes(int64_t B, int64_t T, int64_t D, int64_t lane0, int64_t lane1,
                      const double* a, const double* h, const double* g,
                      const double* h0, const double* grad_last, const uint8_t* reset,
                      double* grad_a, double* grad_b, double* grad_h0) {
    (void)B;
    for (int64_t lane = lane0; lane < lane1; ++lane) {
        int64_t bi = lane / D, d = lane % D;
        double carry = grad_last ? grad_last[lane] : 0.0; /* a_{t+1} lambda_{t+1} */
        for (int64_t t = T - 1; t >= 0; --t) {
            size_t i = idx3(bi, t, d, T, D);
            int r = is_reset(reset, bi, t, T);
            double lam = g[i] + carry;
            double h_prev = (t > 0) ? h[idx3(bi, t - 1, d, T, D)] : (h0 ? h0[lane] : 0.0);
            grad_b[i] = lam;
            grad_a[i] = r ? 0.0 : lam * h_prev;
            carry = (r ? 0.0 : a[i]) * lam;
        }
        if (grad_h0) grad_h0[lane] = carry;
    }
}

void oracle_scan_bwd(int64_t B, int64_t T, int64_t D, const double* a, const double* h,
                     const double* g, const double* h0, const double* grad_last,
                     const uint8_t* reset, double* grad_a, double* grad_b, double* grad_h0) {
    bwd_lanes(B, T, D, 0, B * D, a, h, g, h0, grad_last, reset, grad_a, grad_b, grad_h0);
}

/* ------------------------------------------------------------------------ */
/* Chunk summary (_real_chunk_summary): each chunk k of C steps, rows        */
/* [kC, min(kC+C, T)), is the affine map h -> P_k h + Q_k with               */
/*   P_k = product of a_t over the chunk,                                     */
/*   Q_k = the chunk scanned from a zero state.                               */
/* Rows past T do not exist; they contribute the identity step.               */
/* ------------------------------------------------------------------------ */
void oracle_chunk_summary(int64_t B, int64_t T, int64_t D, int64_t C, const double* a,
                          const double* b, double* P, double* Q) {
    int64_t NC = (T + C - 1) / C;
    for (int64_t bi = 0; bi < B; ++bi)
        for (int64_t k = 0; k < NC; ++k)
            for (int64_t d = 0; d < D; ++d) {
                double p = 1.0, q = 0.0;
                for (int64_t t = k * C; t < k * C + C && t < T; ++t) {
                    size_t i = idx3(bi, t, d, T, D);
                    p = a[i] * p;
                    q = a[i] * q + b[i];
                }
                P[idx3(bi, k, d, NC, D)] = p;
                Q[idx3(bi, k, d, NC, D)] = q;
            }
}

/* Chunk prefix (_real_chunk_prefix): exclusive scan over the chunk maps.     */
/*   chunk_in_0 = h0 (or 0),  chunk_in_{k+1} = P_k chunk_in_k + Q_k.          */
/* If `last` is given it receives P_{NC-1} chunk_in_{NC-1} + Q_{NC-1}.         */
void oracle_chunk_prefix(int64_t B, int64_t NC, int64_t D, const double* P, const double* Q,
                         const double* h0, double* chunk_in, double* last) {
    for (int64_t bi = 0; bi < B; ++bi)
        for (int64_t d = 0; d < D; ++d) {
            double s = h0 ? h0[bi * D + d] : 0.0;
            for (int64_t k = 0; k < NC; ++k) {
                size_t i = idx3(bi, k, d, NC, D);
                chunk_in[i] = s;
                s = P[i] * s + Q[i];
            }
            if (last) last[bi * D + d] = s;
        }
}

/* Chunk replay (_real_chunk_replay): rescan every chunk from chunk_in_k.     */
/* The final chunk's end state is the sequence's last state.                  */
void oracle_chunk_replay(int64_t B, int64_t T, int64_t D, int64_t C, const double* a,
                         const double* b, const double* chunk_in, double* out, double* last) {
    int64_t NC = (T + C - 1) / C;
    for (int64_t bi = 0; bi < B; ++bi)
        for (int64_t k = 0; k < NC; ++k)
            for (int64_t d = 0; d < D; ++d) {
                double h = chunk_in[idx3(bi, k, d, NC, D)];
                for (int64_t t = k * C; t < k * C + C && t < T; ++t) {
                    size_t i = idx3(bi, t, d, T, D);
                    h = a[i] * h + b[i];
                    out[i] = h;
                }
                if (last && k == NC - 1) last[bi * D + d] = h;
            }
}

/* ------------------------------------------------------------------------ */
/* Reverse chunk summary (_real_reverse_chunk_summary).  Let mu_t = a_t       */
/* lambda_t be the carry that leaves step t towards the left.  Inside a chunk */
/* walking t from its last row down to its first:                            */
/*   mu_t = a_t (g_t + mu_{t+1}),                                             */
/* so the chunk maps the carry entering from the right to the carry leaving  */
/* on the left by mu -> P_k mu + Q_k with                                     */
/*   P_k = product of a_t over the chunk,  Q <- a_t Q + a_t g_t from Q = 0.   */
/* ------------------------------------------------------------------------ */
void oracle_reverse_chunk_summary(int64_t B, int64_t T, int64_t D, int64_t C, const double* a,
                                  const double* g, double* P, double* Q) {
    int64_t NC = (T + C - 1) / C;
    for (int64_t bi = 0; bi < B; ++bi)
        for (int64_t k = 0; k < NC; ++k)
            for (int64_t d = 0; d < D; ++d) {
                double p = 1.0, q = 0.0;
                int64_t end = (k * C + C < T) ? k * C + C : T;
                for (int64_t t = end - 1; t >= k * C; --t) {
                    size_t i = idx3(bi, t, d, T, D);
                    p = a[i] * p;
                    q = a[i] * q + a[i] * g[i];
                }
                P[idx3(bi, k, d, NC, D)] = p;
                Q[idx3(bi, k, d, NC, D)] = q;
            }
}

/* Reverse chunk prefix (_real_reverse_chunk_prefix): exclusive scan from the */
/* right.  future_{NC-1} = grad_last (or 0); future_{k-1} = P_k future_k + Q_k. */
/* If `grad_h0` is given it receives P_0 future_0 + Q_0 (= a_0 lambda_0).     */
void oracle_reverse_chunk_prefix(int64_t B, int64_t NC, int64_t D, const double* P,
                                 const double* Q, const double* grad_last, double* future,
                                 double* grad_h0) {
    for (int64_t bi = 0; bi < B; ++bi)
        for (int64_t d = 0; d < D; ++d) {
            double s = grad_last ? grad_last[bi * D + d] : 0.0;
            for (int64_t k = NC - 1; k >= 0; --k) {
                size_t i = idx3(bi, k, d, NC, D);
                future[i] = s;
                s = P[i] * s + Q[i];
            }
            if (grad_h0) grad_h0[bi * D + d] = s;
        }
}

/* Reverse chunk replay (_real_reverse_chunk_replay): start each chunk from   */
/* its future carry and walk it backwards exactly as the sequential backward; */
/* h_{t-1} at the chunk's first row is the previous chunk's last state.       */
void oracle_reverse_chunk_replay(int64_t B, int64_t T, int64_t D, int64_t C, const double* a,
                                 const double* h, const double* g, const double* future,
                                 const double* h0, double* grad_a, double* grad_b) {
    int64_t NC = (T + C - 1) / C;
    for (int64_t bi = 0; bi < B; ++bi)
        for (int64_t k = 0; k < NC; ++k)
            for (int64_t d = 0; d < D; ++d) {
                double carry = future[idx3(bi, k, d, NC, D)];
                int64_t end = (k * C + C < T) ? k * C + C : T;
                for (int64_t t = end - 1; t >= k * C; --t) {
                    size_t i = idx3(bi, t, d, T, D);
                    double lam = g[i] + carry;
                    double h_prev = (t > 0) ? h[idx3(bi, t - 1, d, T, D)]
                                            : (h0 ? h0[bi * D + d] : 0.0);
                    grad_b[i] = lam;
                    grad_a[i] = lam * h_prev;
                    carry = a[i] * lam;
                }
            }
}

/* ------------------------------------------------------------------------ */
/* Multi-threaded drivers for the CPU baseline: split the independent lanes  */
/* (b, d) into contiguous ranges, one per thread, and run the same workers.  */
/* ------------------------------------------------------------------------ */
typedef struct {
    int dir; /* 0 forward, 1 backward */
    int64_t B, T, D, lane0, lane1;
    const double *a, *b, *h, *g, *h0, *grad_last;
    const uint8_t* reset;
    double *out, *last, *grad_a, *grad_b, *grad_h0;
} job_t;

static void* run_job(void* p) {
    job_t* j = (job_t*)p;
    if (j->dir == 0)
        fwd_lanes(j->B, j->T, j->D, j->lane0, j->lane1, j->a, j->b, j->h0, j->reset, j->out,
                  j->last);
    else
        bwd_lanes(j->B, j->T, j->D, j->lane0, j->lane1, j->a, j->h, j->g, j->h0, j->grad_last,
                  j->reset, j->grad_a, j->grad_b, j->grad_h0);
    return NULL;
}

static int run_parallel(job_t proto, int threads) {
    int64_t lanes = proto.B * proto.D;
    if (threads < 1) threads = 1;
    if (threads > lanes) threads = (int)lanes;
    if (threads < 1) return 0;
    job_t* jobs = (job_t*)calloc((size_t)threads, sizeof(job_t));
    pthread_t* tid = (pthread_t*)calloc((size_t)threads, sizeof(pthread_t));
    if (!jobs || !tid) { free(jobs); free(tid); return -1; }
    int started = 0, rc = 0;
    for (int i = 0; i < threads; ++i) {
        jobs[i] = proto;
        jobs[i].lane0 = lanes * i / threads;
        jobs[i].lane1 = lanes * (i + 1) / threads;
        if (pthread_create(&tid[i], NULL, run_job, &jobs[i]) != 0) { rc = -1; break; }
        ++started;
    }
    for (int i = 0; i < started; ++i) pthread_join(tid[i], NULL);
    free(jobs);
    free(tid);
    return rc;
}

int oracle_parallel_fwd(int64_t B, int64_t T, int64_t D, const double* a, const double* b,
                        const double* h0, const uint8_t* reset, double* out, double* last,
                        int threads) {
    job_t j = {0};
    j.dir = 0; j.B = B; j.T = T; j.D = D; j.a = a; j.b = b; j.h0 = h0; j.reset = reset;
    j.out = out; j.last = last;
    return run_parallel(j, threads);
}

int oracle_parallel_bwd(int64_t B, int64_t T, int64_t D, const double* a, const double* h,
                        const double* g, const double* h0, const double* grad_last,
                        const uint8_t* reset, double* grad_a, double* grad_b, double* grad_h0,
                        int threads) {
    job_t j = {0};
    j.dir = 1; j.B = B; j.T = T; j.D = D; j.a = a; j.h = h; j.g = g; j.h0 = h0; j.reset = reset;
    j.grad_last = grad_last; j.grad_a = grad_a; j.grad_b = grad_b; j.grad_h0 = grad_h0;
    return run_parallel(j, threads);
}
