// launch.hpp -- host-side launchers of the scan kernels (internal to liblrscan).
//
// Every launcher enqueues on `stream` and returns hipSuccess or the error the
// runtime reported for the launch.  Arguments have been validated by the
// C-ABI layer; the launchers only check what the kernels themselves assume.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lrscan {

struct Shape {
    int64_t B, T, D;
    int dtype;  // DT_F32 / DT_BF16
};

// True when every [B,T,D] row starts 16-byte aligned for these base pointers
// (D * elem_bytes % 16 == 0 and each pointer 16-byte aligned).
bool rows_aligned(const Shape& s, const void* const* ptrs, int n);

// ---- per-lane sequential walk ---------------------------------------------
// `reset` ([B, T] bytes, or NULL) marks segment starts, where the step's
// transition is taken as 0 (every launcher below that takes it).
hipError_t launch_seq_fwd(const Shape& s, const void* a, const void* b, void* out, float* last,
                          const float* h0, const uint8_t* reset, hipStream_t st);
hipError_t launch_seq_bwd(const Shape& s, const void* a, const void* out, const void* g,
                          const float* grad_last, const float* h0, const uint8_t* reset,
                          void* grad_a, void* grad_b, float* grad_h0, hipStream_t st);

// ---- three-launch chunked form ----------------------------------------------
hipError_t launch_chunk_summary(const Shape& s, int chunk, const void* a, const void* b,
                                const uint8_t* reset, float* P, float* Q, hipStream_t st);
hipError_t launch_chunk_prefix(int64_t B, int64_t NC, int64_t D, const float* P, const float* Q,
                               const float* h0, float* chunk_in, float* last, hipStream_t st);
hipError_t launch_chunk_replay(const Shape& s, int chunk, const void* a, const void* b,
                               const uint8_t* reset, const float* chunk_in, void* out, float* last,
                               hipStream_t st);
hipError_t launch_reverse_chunk_summary(const Shape& s, int chunk, const void* a, const void* g,
                                        const uint8_t* reset, float* P, float* Q, hipStream_t st);
hipError_t launch_reverse_chunk_prefix(int64_t B, int64_t NC, int64_t D, const float* P,
                                       const float* Q, const float* grad_last, float* future,
                                       float* grad_h0, hipStream_t st);
hipError_t launch_reverse_chunk_replay(const Shape& s, int chunk, const void* a, const void* out,
                                       const void* g, const uint8_t* reset, const float* future,
                                       const float* h0, void* grad_a, void* grad_b,
                                       hipStream_t st);

// ---- one time step on [B, D] lanes (decoding) --------------------------------
hipError_t launch_step(int64_t B, int64_t D, int dtype, const void* a, const void* b,
                       const float* state_in, const uint8_t* reset, void* out, float* state_out,
                       hipStream_t st);

// ---- single-launch fused form ----------------------------------------------
// A configuration is (width, tile): width threads of 16 bytes cover one row of
// a tile (8, 16 or 32) and a tile spans `tile` rows.  Unaligned rows support
// only width 8, tile 256.
bool fused_cfg_supported(const Shape& s, int dir, int width, int tile, bool aligned);
void fused_default_cfg(const Shape& s, int dir, bool aligned, int* width, int* tile);
size_t fused_workspace_bytes(const Shape& s, int width, int tile);
// `ws` holds the fused form's header and two scratch regions; `init` must be
// true the first time a buffer is used (and whenever its contents were
// disturbed): the launcher then enqueues one initialisation kernel first.
// Every launch on a buffer must use the same `ws_bytes`.  `polls` (<= 0: the
// default) bounds how often a tile polls for its predecessors before it
// derives their missing maps itself; results are bitwise the same either way.
hipError_t launch_fused_fwd(const Shape& s, int width, int tile, const void* a, const void* b,
                            void* out, float* last, const float* h0, const uint8_t* reset,
                            void* ws, size_t ws_bytes, bool init, int polls, hipStream_t st);
hipError_t launch_fused_bwd(const Shape& s, int width, int tile, const void* a, const void* out,
                            const void* g, const float* grad_last, const float* h0,
                            const uint8_t* reset, void* grad_a, void* grad_b, float* grad_h0,
                            void* ws, size_t ws_bytes, bool init, int polls, hipStream_t st);

// ---- complex diagonal scan (planar real / imaginary arrays) ----------------
// [B, T, M] arrays of one storage type; states [B, M] fp32.  NULL h0 / last /
// grad_last / grad_h0 pairs mean "zero" / "not wanted".
struct CxFwdPtrs {
    const void *ar, *ai, *br, *bi;
    void *out_r, *out_i;         // NULL pair: state-only forward
    float *last_r, *last_i;
    const float *h0r, *h0i;
    const uint8_t* reset;
};
struct CxBwdPtrs {
    const void *ar, *ai, *hr, *hi, *gr, *gi;  // h = the forward's out
    const float *glr, *gli, *h0r, *h0i;
    const uint8_t* reset;
    void *gar, *gai, *gbr, *gbi;
    float *gh0r, *gh0i;
};
hipError_t launch_complex_seq_fwd(const Shape& s, const CxFwdPtrs& p, hipStream_t st);
hipError_t launch_complex_seq_bwd(const Shape& s, const CxBwdPtrs& p, hipStream_t st);
// The fused complex form has fixed tile shapes per direction; its workspace
// follows the fused conventions.
bool complex_fused_supported(const Shape& s);
size_t complex_fused_workspace_bytes(const Shape& s);
hipError_t launch_complex_fused_fwd(const Shape& s, const CxFwdPtrs& p, void* ws, size_t ws_bytes,
                                    bool init, int polls, hipStream_t st);
hipError_t launch_complex_fused_bwd(const Shape& s, const CxBwdPtrs& p, void* ws, size_t ws_bytes,
                                    bool init, int polls, hipStream_t st);

// ---- fused-transition (SAMU-form) complex scan ------------------------------
// The transition is rebuilt from per-token controls eta, delta ([B, T], I/O
// type) and per-mode parameters nu_log, theta_log ([M], fp32).
struct SamuFwdPtrs {
    const void *eta, *delta;
    const float *nu_log, *theta_log;
    const void *br, *bi;
    void *out_r, *out_i;  // NULL pair: state-only forward
    float *last_r, *last_i;
    const float *h0r, *h0i;
    const uint8_t* reset;
};
struct SamuBwdPtrs {
    const void *eta, *delta;
    const float *nu_log, *theta_log;
    const void *hr, *hi, *gr, *gi;  // h = the forward's out
    const float *glr, *gli, *h0r, *h0i;
    const uint8_t* reset;
    float *grad_eta, *grad_delta, *grad_nu_log, *grad_theta_log;
    void *gbr, *gbi;
    float *gh0r, *gh0i;
};
bool samu_supported(const Shape& s);
// Two buffers: `ws` is the fused scratch (conventions of the fused form,
// samu_scratch_bytes); `aux` (256-byte aligned, samu_aux_bytes) holds the
// per-call transition factor tables and the backward's partial sums, and is
// overwritten by every call.
size_t samu_scratch_bytes(const Shape& s);
size_t samu_aux_bytes(const Shape& s);
hipError_t launch_samu_fwd(const Shape& s, const SamuFwdPtrs& p, void* ws, size_t ws_bytes,
                           bool init, void* aux, int polls, hipStream_t st);
hipError_t launch_samu_bwd(const Shape& s, const SamuBwdPtrs& p, void* ws, size_t ws_bytes,
                           bool init, void* aux, int polls, hipStream_t st);
// The per-lane walk of the same scan (no fused scratch; `aux` as above).
hipError_t launch_samu_seq_fwd(const Shape& s, const SamuFwdPtrs& p, void* aux, hipStream_t st);
hipError_t launch_samu_seq_bwd(const Shape& s, const SamuBwdPtrs& p, void* aux, hipStream_t st);

}  // namespace lrscan
