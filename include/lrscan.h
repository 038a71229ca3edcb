/*
 * lrscan.h -- C ABI of the MI355X (gfx950) diagonal affine recurrence scan.
 *
 * The operation (page "triton_training_scan.py", botwwt.github.io/SAMU_GPU/
 * benchmark, kernels _real_forward and _real_backward, and the autograd
 * classes _RealScan / _RealChunkScan and the function real_scan_with_last):
 *
 *   forward   h_{-1} = h0 (zero unless given),  h_t = a_t * h_{t-1} + b_t,
 *             out[b,t,d] = h_t,  last[b,d] = h_{T-1}
 *   backward  the gradient of  L = <grad_out, out> + <grad_last, last>:
 *             lambda_{T-1} = grad_out_{T-1} + grad_last,
 *             lambda_t     = grad_out_t + a_{t+1} * lambda_{t+1},
 *             grad_b_t = lambda_t,  grad_a_t = lambda_t * h_{t-1},
 *             grad_h0  = a_0 * lambda_0
 *
 * Conventions shared by every entry point:
 *
 *  - Pointers are device pointers on the current HIP device, except `opts`,
 *    which is a host pointer.  The caller owns every buffer; the library never
 *    frees caller memory.
 *  - [B, T, D] tensors are contiguous, row-major, D fastest: element (b,t,d)
 *    is at (b*T + t)*D + d.  [B, D] tensors (h0, last, grad_last, grad_h0) are
 *    fp32 at b*D + d.  Chunk tensors are fp32 [B, NC, D], NC = ceil(T / chunk).
 *  - `dtype` (LRSCAN_F32 or LRSCAN_BF16) is the storage type of a, b, out,
 *    grad_out, grad_a and grad_b.  Loads are widened to fp32, all arithmetic
 *    and every carried state is fp32, and stores to bf16 round to nearest
 *    even.  last, h0, grad_last, grad_h0 and all chunk tensors are fp32.
 *  - `stream` is a hipStream_t (NULL for the default stream).  Work is
 *    enqueued asynchronously on it.  Argument errors are found before any
 *    work is enqueued and return a negative status.
 *  - Inputs and outputs must not alias each other.
 *  - Results are deterministic: the same call on the same data gives the same
 *    bits every time.
 *  - Calls that share one workspace (the library's own per-stream workspace,
 *    or one passed in opts) must be ordered on one stream.
 *  - Graph capture.  While `stream` is capturing a HIP graph, the library
 *    allocates, frees and initialises nothing.  A call that needs the
 *    library's workspace (opts->workspace NULL) then uses the one this stream
 *    already has, which an eager call of at least the same size on the same
 *    stream must have set up first; otherwise it returns LRSCAN_ERR_CAPTURE
 *    and enqueues nothing.  The captured graph keeps using that buffer on
 *    every replay: the library never frees a buffer a capture was given (a
 *    later, larger eager call on the stream gets a new one), and replays must
 *    be ordered with the other calls on that stream.  A caller workspace
 *    (opts->workspace) is initialised inside each captured call instead.
 */
#ifndef LRSCAN_H
#define LRSCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LRSCAN_API __attribute__((visibility("default")))

/* storage types */
enum { LRSCAN_F32 = 0, LRSCAN_BF16 = 1 };

/* status codes */
enum {
    LRSCAN_OK = 0,
    LRSCAN_ERR_NULL = -1,      /* a required pointer is NULL */
    LRSCAN_ERR_DIM = -2,       /* B, T or D < 1, or a size overflows */
    LRSCAN_ERR_DTYPE = -3,     /* dtype is not LRSCAN_F32 / LRSCAN_BF16 */
    LRSCAN_ERR_CHUNK = -4,     /* chunk length not supported by the chosen algorithm */
    LRSCAN_ERR_WORKSPACE = -5, /* workspace given but smaller than scan_workspace_bytes() */
    LRSCAN_ERR_HIP = -6,       /* the HIP runtime reported an error (launch or allocation) */
    LRSCAN_ERR_ALGO = -7,      /* unknown algorithm */
    LRSCAN_ERR_CAPTURE = -8,   /* the stream is capturing a graph and its library workspace is
                                  missing or too small (see "Graph capture" above) */
    LRSCAN_ERR_TOO_BIG = -9    /* scan_fwd_noalloc: the call needs more scratch than its static
                                  buffer holds */
};

/* Bytes of the static device scratch of scan_fwd_noalloc (per device). */
#define LRSCAN_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/* algorithms */
enum {
    LRSCAN_ALGO_AUTO = 0,    /* the library picks: SEQ for sequences of at most 8 steps (bf16:
                                16) over at least 2^20 lanes (rows that are not 16-byte
                                aligned: at most 32 steps, fp32 128, over at least 2^18
                                lanes), CHUNKED for sequences of at least 2^20 steps over
                                one or two 128-byte lane blocks in all, else FUSED with a measured tile
                                shape, or CHUNKED (complex scan: SEQ) where a tile would exceed
                                the fused form's 32-bit in-tile offsets (rows of hundreds of MB).
                                Complex scan: SEQ for T <= 16, and from 2^18 lanes for T <= 32
                                (bf16 forward: T <= 64), else FUSED */
    LRSCAN_ALGO_SEQ = 1,     /* one thread walks all T steps of its lanes */
    LRSCAN_ALGO_CHUNKED = 2, /* three launches: chunk summary, chunk prefix, chunk replay */
    LRSCAN_ALGO_FUSED = 3    /* one launch: tile summary, look-back prefix, replay from registers */
};

typedef struct {
    int algo;               /* LRSCAN_ALGO_* */
    int chunk;              /* 0: the algorithm's default.  CHUNKED: a power of two in [16, 1024].
                               FUSED: rows per tile (see `width`).  SEQ: ignored. */
    int width;              /* FUSED only: threads of 16 bytes per tile row (8, 16 or 32; a
                               tile row is 128, 256 or 512 contiguous bytes); 0: default.
                               Supported (width, chunk): forward (8,256) (8,512) (16,128)
                               (16,256) (32,32) (32,64) (32,128); backward (8,256) (8,128) (16,128)
                               (32,64) (32,32).  Rows that are not 16-byte aligned
                               (D * elem_bytes % 16 != 0 or an unaligned pointer) support
                               (8,256) (16,128) (32,64), and backward (8,128). */
    void* workspace;        /* device scratch, or NULL for the library's own per-stream cache */
    size_t workspace_bytes; /* size of `workspace` */
    const float* h0;        /* [B, D] initial state, or NULL for zero (forward and backward) */
    float* grad_h0;         /* [B, D] output of the backward, or NULL */
    int polls;              /* FUSED only: times a tile polls for its predecessors' published
                               results before it stops waiting and derives the missing ones
                               from the inputs itself; <= 0: the library default.  Results
                               are bitwise the same for every value (1 exercises the
                               derivation path). */
    const uint8_t* reset;   /* [B, T] bytes (b*T + t), or NULL.  Nonzero marks step t of batch
                               row b as the first step of a new segment: the state entering it
                               is dropped (the step's transition is taken as 0, so
                               h_t = b_t).  Forward and backward take the same mask; the
                               backward then gives grad_a_t = 0 at such a step (a_t is not
                               used), carries no adjoint past it, and grad_h0 = 0 for a row
                               whose step 0 is marked (page "triton_training_scan.py",
                               _samu_tiled_serial_forward/_backward: a step at segment
                               position 0 forces the decay to 0).  Every algorithm. */
} lrscan_opts;

/*
 * scan_fwd: out = every state of the scan of (a, b); last = the final state.
 *   a, b  [B,T,D] dtype, read only.     out  [B,T,D] dtype, written; may be NULL
 *   when last is given (a state-only forward, e.g. a prefill that keeps only
 *   the final state: no [B,T,D] output is written, and last is bitwise the
 *   one the full forward gives).
 *   last  [B,D] fp32, written; may be NULL when out is given.
 * Returns LRSCAN_OK or a negative status (LRSCAN_ERR_NULL if both are NULL).
 */
LRSCAN_API int scan_fwd(const void* a, const void* b, void* out, float* last, int64_t B, int64_t T,
                        int64_t D, int dtype, void* stream);

/*
 * scan_bwd: gradients of <grad_out, out> + <grad_last, last> with respect to
 * a and b.  `out` is the forward's output (h_{t-1} is read from it).
 *   a, out, grad_out [B,T,D] dtype, read only.   grad_last [B,D] fp32 or NULL.
 *   grad_a, grad_b   [B,T,D] dtype, written.
 */
LRSCAN_API int scan_bwd(const void* a, const void* out, const void* grad_out,
                        const float* grad_last, void* grad_a, void* grad_b, int64_t B, int64_t T,
                        int64_t D, int dtype, void* stream);

/* As above, with options (algorithm, chunk, workspace, initial state).  opts may be NULL. */
LRSCAN_API int scan_fwd_ex(const void* a, const void* b, void* out, float* last, int64_t B,
                           int64_t T, int64_t D, int dtype, void* stream, const lrscan_opts* opts);
LRSCAN_API int scan_bwd_ex(const void* a, const void* out, const void* grad_out,
                           const float* grad_last, void* grad_a, void* grad_b, int64_t B,
                           int64_t T, int64_t D, int dtype, void* stream, const lrscan_opts* opts);

/*
 * scan_fwd_noalloc: scan_fwd_ex that allocates nothing, for callers that
 * cannot call hipMalloc (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and algorithm
 * choice as scan_fwd_ex; the caller still passes every input and output.
 * Scratch comes from a static device array of LRSCAN_NOALLOC_SCRATCH_BYTES
 * (16 MiB) that each device holds for the life of the process; the part a
 * call uses is initialised by a kernel inside the call.
 *   opts->workspace must be NULL (else LRSCAN_ERR_WORKSPACE).  A call that
 *   needs more scratch than the array holds returns LRSCAN_ERR_TOO_BIG and
 *   enqueues nothing (scan_workspace_bytes gives a shape's need; the per-lane
 *   walk, LRSCAN_ALGO_SEQ, needs none).
 *   Every call on a device shares that device's array: calls that overlap in
 *   time on one device (on different streams, or from different threads
 *   without ordering) race and give wrong results.
 */
LRSCAN_API int scan_fwd_noalloc(const void* a, const void* b, void* out, float* last, int64_t B,
                                int64_t T, int64_t D, int dtype, void* stream,
                                const lrscan_opts* opts);

/*
 * scan_step: one time step of the recurrence on [B, D] lanes, for decoding
 * token by token from a carried fp32 state (page "triton_training_scan.py",
 * real_scan_with_last returns that fp32 final state for inference, and
 * _samu_decode updates the state one token at a time in one launch):
 *   h = a * state_in + b   (state_in NULL: zero;  reset[b] != 0: the state is
 *                            dropped for batch row b, so h = b)
 *   a, b       [B, D] dtype, read only (one step of the [B,T,D] inputs).
 *   state_in   [B, D] fp32 or NULL.       reset  [B] bytes or NULL.
 *   out        [B, D] dtype, written (h rounded to dtype); may be NULL.
 *   state_out  [B, D] fp32, written (h); may be NULL; may equal state_in
 *              (an in-place update).  At least one of out, state_out.
 * Chaining T calls from a zero state gives bitwise the states and outputs of
 * scan_fwd with LRSCAN_ALGO_SEQ.  Returns LRSCAN_OK or a negative status.
 */
LRSCAN_API int scan_step(const void* a, const void* b, const float* state_in,
                         const uint8_t* reset, void* out, float* state_out, int64_t B, int64_t D,
                         int dtype, void* stream);

/* ------------------------------------------------------------------------
 * Complex diagonal scan, planar storage (page "triton_training_scan.py":
 * _complex_forward, _complex_backward, complex_scan, complex_scan_with_last):
 *   h_{-1} = h0 (zero unless given),  h_t = a_t * h_{t-1} + b_t  (complex).
 * Real and imaginary parts are separate [B, T, M] arrays of `dtype` (M modes,
 * layout as above); states are pairs of fp32 [B, M] arrays.  Every (re, im)
 * pair of pointers is given whole or NULL whole (else LRSCAN_ERR_NULL).
 * The backward is the gradient of the real loss
 *   L = sum Re(conj(grad_out) * out) + Re(conj(grad_last) * last),
 * written as dL/dRe + i dL/dIm:
 *   lambda_{T-1} = grad_out_{T-1} + grad_last,
 *   lambda_t = grad_out_t + conj(a_{t+1}) * lambda_{t+1},
 *   grad_b_t = lambda_t,  grad_a_t = lambda_t * conj(h_{t-1}),
 *   grad_h0 = conj(a_0) * lambda_0.
 * opts: algo AUTO, FUSED (the library's tile shapes: chunk and width must be
 * 0, else LRSCAN_ERR_CHUNK) or SEQ (CHUNKED returns LRSCAN_ERR_ALGO); workspace,
 * polls and reset as for the real scan; opts->h0 and opts->grad_h0 are not
 * used (the states are the explicit arguments).
 * ------------------------------------------------------------------------ */
/*   ar, ai, br, bi  read.   out_r, out_i written (NULL pair: state-only
 *   forward, then last is required).   last_r, last_i written (nullable pair).
 *   h0_r, h0_i (nullable pair). */
LRSCAN_API int scan_complex_fwd(const void* ar, const void* ai, const void* br, const void* bi,
                                void* out_r, void* out_i, float* last_r, float* last_i,
                                const float* h0_r, const float* h0_i, int64_t B, int64_t T,
                                int64_t M, int dtype, void* stream, const lrscan_opts* opts);
/*   out_r, out_i: the forward's outputs (h_{t-1} is read from them).
 *   grad_last_*, h0_*, grad_h0_*: nullable pairs.  grad_ar .. grad_bi written. */
LRSCAN_API int scan_complex_bwd(const void* ar, const void* ai, const void* out_r,
                                const void* out_i, const void* grad_out_r, const void* grad_out_i,
                                const float* grad_last_r, const float* grad_last_i,
                                const float* h0_r, const float* h0_i, void* grad_ar,
                                void* grad_ai, void* grad_br, void* grad_bi, float* grad_h0_r,
                                float* grad_h0_i, int64_t B, int64_t T, int64_t M, int dtype,
                                void* stream, const lrscan_opts* opts);
/* Bytes of caller workspace a complex call with these arguments needs (0 if none). */
LRSCAN_API size_t scan_complex_workspace_bytes(int64_t B, int64_t T, int64_t M, int dtype,
                                               const lrscan_opts* opts);

/* ------------------------------------------------------------------------
 * Fused-transition complex scan, SAMU form (page "triton_training_scan.py":
 * _samu_forward, _samu_backward, _SAMUScan).  The transition is not an input:
 * for batch b, step t and mode m it is rebuilt inside the kernels from
 * per-token controls eta, delta ([B, T], `dtype`) and per-mode parameters
 * nu_log, theta_log ([M], fp32):
 *   a = exp(-e^{nu_log[m]} * e^{eta[b,t]}) * exp(i (e^{theta_log[m]} + delta[b,t])),
 *   h_t = a_t * h_{t-1} + b_t   (complex, planar b / out as for scan_complex_*).
 * The backward is the gradient of the same real loss as scan_complex_bwd;
 * with grad_a_t = lambda_t * conj(h_{t-1}), w = conj(a) * grad_a:
 *   grad_eta[b,t]     = sum_m -e^{nu_log} e^{eta} Re(w),
 *   grad_delta[b,t]   = sum_m Im(w),
 *   grad_nu_log[m]    = sum_{b,t} -e^{nu_log} e^{eta} Re(w),
 *   grad_theta_log[m] = sum_{b,t} e^{theta_log} Im(w),
 * all fp32; grad_b and grad_h0 as for scan_complex_bwd.  The sums are taken in
 * a fixed order (results do not depend on scheduling).  At a reset step
 * (opts->reset) the transition is 0 and contributes nothing to the four
 * parameter gradients.
 * opts: algo AUTO, FUSED or SEQ (a per-lane walk; CHUNKED returns
 * LRSCAN_ERR_ALGO) with chunk and width 0: the tile shapes are the library's
 * (else LRSCAN_ERR_CHUNK); AUTO walks sequences of at most 16 steps (bf16:
 * 64) over at least 2^18 lanes and tiles the rest; workspace, polls and reset as for the
 * real scan.  A caller workspace must hold scan_samu_workspace_bytes() (the
 * same for every algorithm); its contents are overwritten by every call.
 * ------------------------------------------------------------------------ */
/*   eta, delta, nu_log, theta_log, br, bi read.  out_r, out_i written (NULL
 *   pair: state-only forward, then last is required).  last_r, last_i written
 *   (nullable pair).  h0_r, h0_i (nullable pair). */
LRSCAN_API int scan_samu_fwd(const void* eta, const void* delta, const float* nu_log,
                             const float* theta_log, const void* br, const void* bi, void* out_r,
                             void* out_i, float* last_r, float* last_i, const float* h0_r,
                             const float* h0_i, int64_t B, int64_t T, int64_t M, int dtype,
                             void* stream, const lrscan_opts* opts);
/*   out_r, out_i: the forward's outputs.  grad_last_*, h0_*, grad_h0_*:
 *   nullable pairs.  grad_eta, grad_delta ([B, T]), grad_nu_log,
 *   grad_theta_log ([M]): each nullable (not computed when NULL).
 *   grad_br, grad_bi ([B, T, M], dtype) written. */
LRSCAN_API int scan_samu_bwd(const void* eta, const void* delta, const float* nu_log,
                             const float* theta_log, const void* out_r, const void* out_i,
                             const void* grad_out_r, const void* grad_out_i,
                             const float* grad_last_r, const float* grad_last_i,
                             const float* h0_r, const float* h0_i, float* grad_eta,
                             float* grad_delta, float* grad_nu_log, float* grad_theta_log,
                             void* grad_br, void* grad_bi, float* grad_h0_r, float* grad_h0_i,
                             int64_t B, int64_t T, int64_t M, int dtype, void* stream,
                             const lrscan_opts* opts);
/* Bytes of caller workspace a fused-transition call needs (0 for invalid arguments). */
LRSCAN_API size_t scan_samu_workspace_bytes(int64_t B, int64_t T, int64_t M, int dtype,
                                            const lrscan_opts* opts);

/* Bytes of workspace the call with these arguments needs (0 if none).
 * Returns 0 for invalid arguments. */
LRSCAN_API size_t scan_workspace_bytes(int64_t B, int64_t T, int64_t D, int dtype,
                                       const lrscan_opts* opts);

/* A static string naming a status code. */
LRSCAN_API const char* scan_status_string(int status);

/* The algorithm LRSCAN_ALGO_AUTO picks for this shape with 16-byte aligned pointers (forward
 * if dir == 0, else backward), and through *chunk and *width (both nullable) its chunk or tile
 * length and tile width.  Returns the algorithm, or a negative status on bad arguments. */
LRSCAN_API int scan_auto_algo(int64_t B, int64_t T, int64_t D, int dtype, int dir, int* chunk,
                              int* width);

/* ------------------------------------------------------------------------
 * The steps of the chunked form, one entry point each (page
 * "triton_training_scan.py": _real_chunk_summary, _real_chunk_prefix,
 * _real_chunk_replay and the _real_reverse_chunk_* trio).  NC = ceil(T/chunk);
 * chunk is a power of two in [16, 1024].  Steps past T inside the final chunk
 * are identity steps (a = 1, b = 0, grad_out = 0).
 * ------------------------------------------------------------------------ */

/* P[b,k,d] = product of a over chunk k;  Q[b,k,d] = chunk k scanned from a zero state. */
LRSCAN_API int scan_chunk_summary(const void* a, const void* b, float* P, float* Q, int64_t B,
                                  int64_t T, int64_t D, int chunk, int dtype, void* stream);

/* Exclusive scan over the chunk maps: chunk_in[:,0] = h0 (or 0),
 * chunk_in[:,k+1] = P[:,k] * chunk_in[:,k] + Q[:,k].  last (nullable) receives
 * the state after the final chunk.  h0 may be NULL. */
LRSCAN_API int scan_chunk_prefix(const float* P, const float* Q, const float* h0, float* chunk_in,
                                 float* last, int64_t B, int64_t NC, int64_t D, void* stream);

/* Rescan every chunk from chunk_in and write out (dtype); last (nullable) gets
 * the final state of the final chunk. */
LRSCAN_API int scan_chunk_replay(const void* a, const void* b, const float* chunk_in, void* out,
                                 float* last, int64_t B, int64_t T, int64_t D, int chunk,
                                 int dtype, void* stream);

/* Reverse summary: walking chunk k backwards, P = product of a,
 * Q <- a_t * (Q + grad_out_t) from Q = 0: the map from the carry entering the
 * chunk on the right to the carry a_s * lambda_s leaving its first row s. */
LRSCAN_API int scan_reverse_chunk_summary(const void* a, const void* grad_out, float* P, float* Q,
                                          int64_t B, int64_t T, int64_t D, int chunk, int dtype,
                                          void* stream);

/* Exclusive right-to-left scan: future[:,NC-1] = grad_last (or 0),
 * future[:,k-1] = P[:,k] * future[:,k] + Q[:,k];  grad_h0 (nullable) receives
 * P[:,0] * future[:,0] + Q[:,0].  grad_last may be NULL. */
LRSCAN_API int scan_reverse_chunk_prefix(const float* P, const float* Q, const float* grad_last,
                                         float* future, float* grad_h0, int64_t B, int64_t NC,
                                         int64_t D, void* stream);

/* Walk every chunk backwards from its future carry, writing grad_a and grad_b
 * (dtype).  h_{t-1} comes from out (and from h0, or zero, at t = 0). */
LRSCAN_API int scan_reverse_chunk_replay(const void* a, const void* out, const void* grad_out,
                                         const float* future, const float* h0, void* grad_a,
                                         void* grad_b, int64_t B, int64_t T, int64_t D, int chunk,
                                         int dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LRSCAN_H */
