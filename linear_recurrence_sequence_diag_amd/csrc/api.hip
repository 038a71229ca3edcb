// api.hip -- the C ABI of liblrscan (declared in include/lrscan.h): argument
// validation, the algorithm choice, workspace handling, and the calls into
// the kernel launchers.  No torch type crosses this boundary.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <tuple>
#include <utility>
#include <vector>

#include "../../include/lrscan.h"
#include "device.hpp"
#include "launch.hpp"

using namespace lrscan;

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 40;  // generous bound that keeps size_t math exact

bool dims_ok(int64_t B, int64_t T, int64_t D) {
    if (B < 1 || T < 1 || D < 1) return false;
    if (B > kMaxElems || T > kMaxElems || D > kMaxElems) return false;
    if (B * D > kMaxElems / T) return false;
    return true;
}

bool dtype_ok(int dt) { return dt == LRSCAN_F32 || dt == LRSCAN_BF16; }

bool chunk_ok(int chunk) { return chunk >= 16 && chunk <= 1024 && (chunk & (chunk - 1)) == 0; }

constexpr int kDefaultChunk = 64;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---- library-owned workspaces, one per (device, stream, kind) ----------------
// Kind 0 holds the chunked form's P, Q and entering states; kind 1 holds the
// fused form's self-cleaning scratch, which must not be shared with anything
// else and is initialised once per allocation; kind 2 holds the
// fused-transition scan's factor tables and partial sums.
//
// Graph capture.  A call captured into a HIP graph bakes the workspace
// address into the graph's kernel arguments, and every replay uses it.  So
// while a stream is capturing, the library neither allocates, frees nor
// initialises: it hands out the stream's buffer only if that buffer is
// already big enough and initialised (an eager call of at least this size
// ran on the stream before), and marks it as captured.  A captured buffer is
// never freed: when a later eager call needs a bigger one, it is retired
// (kept for the life of the process) and a new one is allocated.
struct CachedWs {
    void* ptr = nullptr;
    size_t bytes = 0;
    bool fresh = false;     // not yet initialised for the fused form
    bool captured = false;  // handed to a call under capture: a graph may hold it
};
std::mutex g_ws_mutex;
std::map<std::tuple<int, void*, int>, CachedWs> g_ws;
std::vector<void*> g_retired;  // superseded captured buffers (never freed)

struct Workspace {
    void* ptr = nullptr;
    size_t bytes = 0;
    bool init = false;     // the fused form must initialise it before use
    bool library = false;  // one of the library's per-stream buffers
};

// Whether `st` is capturing into a graph (an invalidated capture counts).
hipError_t stream_capturing(hipStream_t st, bool* capturing) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    const hipError_t e = hipStreamIsCapturing(st, &cs);
    *capturing = cs != hipStreamCaptureStatusNone;
    return e;
}

// A device buffer of at least `bytes` owned by the library, ordered on `st`.
int library_workspace(size_t bytes, int kind, hipStream_t st, Workspace* out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return LRSCAN_ERR_HIP;
    bool capturing = false;
    if (stream_capturing(st, &capturing) != hipSuccess) return LRSCAN_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    CachedWs& c = g_ws[std::make_tuple(dev, (void*)st, kind)];
    if (capturing) {
        if (!c.ptr || c.bytes < bytes || c.fresh) return LRSCAN_ERR_CAPTURE;
        c.captured = true;
    } else if (c.bytes < bytes) {
        if (c.ptr) {
            if (c.captured) {
                g_retired.push_back(c.ptr);
            } else if (hipFreeAsync(c.ptr, st) != hipSuccess) {
                return LRSCAN_ERR_HIP;
            }
            c = CachedWs{};
        }
        const size_t want = align_up(bytes + bytes / 4, 1 << 20);
        if (hipMallocAsync(&c.ptr, want, st) != hipSuccess) {
            c = CachedWs{};
            return LRSCAN_ERR_HIP;
        }
        c.bytes = want;
        c.fresh = kind == 1;  // only the fused scratch has an initial state
    }
    out->ptr = c.ptr;
    out->bytes = c.bytes;
    out->init = c.fresh;
    out->library = true;
    return LRSCAN_OK;
}

// Called after a launch that initialised the library's fused workspace was
// enqueued successfully.
void workspace_initialised(hipStream_t st) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return;
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    auto it = g_ws.find(std::make_tuple(dev, (void*)st, 1));
    if (it != g_ws.end()) it->second.fresh = false;
}

int fused_status(hipError_t e, const Workspace& ws, hipStream_t st) {
    if (e != hipSuccess) return LRSCAN_ERR_HIP;
    if (ws.init && ws.library) workspace_initialised(st);
    return LRSCAN_OK;
}

struct Resolved {
    int algo;
    int chunk;
    int width;
};

// Whether rows of this shape can be 16-byte aligned at all (pointers are
// checked separately at launch time).
bool shape_aligned(const Shape& s) { return (s.D * (s.dtype == LRSCAN_F32 ? 4 : 2)) % 16 == 0; }

// The per-lane walk when the sequences are short and B*D alone fills the GPU
// many times over: every tile of the fused form would be mostly idle rows,
// while each lane's walk is a few steps of plain streaming.  Measured on
// MI355X with 10M-42M lanes (D = 2560): T = 8 5.6-5.8 TB/s against 3.4-3.6
// for the best tile shape (32 rows of 512-byte lane blocks); bf16 T = 16
// 5.3 against 3.7 (forward) and 4.9 (backward).  fp32 T = 16 is the other
// way round (the tile 5.6 / 5.5 against 5.3 / 5.4), and from T = 32 the tile
// wins for both types; below about 1M lanes the walk has too few threads in
// flight to be competitive.
bool prefer_seq(const Shape& s) {
    return (s.T <= 8 || (s.T <= 16 && s.dtype == LRSCAN_BF16)) &&
           s.B * s.D >= ((int64_t)1 << 20);
}

// Rows that are not 16-byte aligned have one tile shape (256 rows of 128-byte
// rows), so short sequences leave most of every tile idle there; from 2^18
// lanes the walk is faster up to 64 steps (fp32: 128).  Measured on MI355X
// (D = 2559, caches flushed, forward / backward TB/s, tile against walk):
// bf16 T = 32 0.42 / 0.29 against 1.6 / 1.3, T = 64 0.79 / 0.56 against 1.5
// / 1.1, T = 128 1.4 / 1.0 against 0.95 / 0.98; fp32 T = 64 0.84 / 0.62
// against 2.6 / 2.6, T = 128 1.5 / 1.1 against 2.4 / 2.4, T = 256 2.0 / 1.5
// against 1.6 / 1.5.
//
// With 16-byte accesses at element-aligned addresses and 64-row tiles of
// 512-byte blocks for sequences of at most 64 steps, the tiles took bf16 T =
// 64 (3.7 / 3.7 against 2.2 / 2.2 for the walk, [692, 64, 2559]) and tie at
// T = 32 (2.5 / 2.6 against 2.5 / 2.4); the fp32 walk still leads up to 128
// steps (T = 128: 4.1 / 3.9 against 4.1 / 3.7).  Rows too short for 512-byte
// blocks keep the walk up to 64 steps.
bool prefer_seq_unaligned(const Shape& s) {
    if (s.B * s.D < ((int64_t)1 << 18)) return false;
    if (s.dtype == LRSCAN_F32) return s.T <= 128;
    return s.T <= 32 || (s.T <= 64 && s.D * 2 < 512);
}

// The three-launch form for long sequences over one or two 128-byte lane
// blocks in all: the fused form's tiles then form one or two chains, whose
// states advance by one look-back window per publication round trip, while
// the three-launch form summarises every chunk in parallel once there are
// thousands of chunks.  Measured on MI355X (caches flushed, forward /
// backward TB/s, fused -> chunks of 256 / of 1024 rows): one chain, bf16
// D = 64: T = 256K 1.0 / 1.0 -> 0.8 / 0.4 (fused ahead), T = 1M 1.2 / 1.0 ->
// 1.9 / 1.3, T = 4M 1.2 / 1.0 -> 1.8 / 1.9 and 2.5 / 1.3, T = 8M 1.2 / 1.0 ->
// 1.6 / 1.9 and 2.6 / 2.4; two chains, bf16 D = 128: T = 1M 2.4 / 2.0 ->
// 2.5 / 2.1, T = 2M 2.4 / 2.1 -> 2.3 / 2.6 and 2.8 / 1.4; fp32 D = 64: T = 2M
// 2.4 / 2.1 -> 2.3 / 2.7 and 2.8 / 1.5.  From four chains the fused form is
// ahead (bf16 D = 256, T = 1M: 4.4 / 3.9 against 2.6 / 2.6).  Returns the
// chunk length, or 0 for the other forms.
// The best chunk grows with T: about T / 4096 rows forward and T / 8192
// backward (one chain, bf16: T = 1M forward 256 rows 1.9 TB/s against 1.5
// at 128, backward 128 rows 1.7 against 1.2 at 256), so that there are some
// thousands of chunks.
int chunk_for(int64_t T, int64_t per, int lo) {
    int c = lo;
    while (c < 1024 && (int64_t)c * 2 * per <= T) c *= 2;
    return c;
}
int prefer_chunked(const Shape& s, int dir) {
    if (s.T < ((int64_t)1 << 20)) return 0;
    const int64_t eb = s.dtype == LRSCAN_F32 ? 4 : 2;
    const int64_t chains = s.B * ((s.D * eb + 127) / 128);
    if (chains > 2) return 0;
    if (dir == 1) return chunk_for(s.T, 8192, 128);
    if (chains == 1 || s.T >= ((int64_t)1 << 21)) return chunk_for(s.T, 4096, 256);
    return 0;
}

// The automatic choice: the per-lane walk for short sequences over many
// lanes (prefer_seq, and prefer_seq_unaligned for rows that are not 16-byte
// aligned); the three-launch form for long sequences over one or
// two lane blocks (prefer_chunked); otherwise the single-launch fused form,
// which reads every input once and was the fastest form on every other
// measured shape, with its tile shape from fused_default_cfg; the
// three-launch form past the fused form's index limits.
Resolved resolve(const Shape& s, int dir, const lrscan_opts* o, bool aligned) {
    Resolved r;
    r.algo = o ? o->algo : LRSCAN_ALGO_AUTO;
    r.chunk = o ? o->chunk : 0;
    r.width = o ? o->width : 0;
    if (r.algo == LRSCAN_ALGO_AUTO && (prefer_seq(s) || (!aligned && prefer_seq_unaligned(s)))) {
        r.algo = LRSCAN_ALGO_SEQ;
        r.chunk = 0;
        r.width = 0;
        return r;
    }
    if (r.algo == LRSCAN_ALGO_AUTO && prefer_chunked(s, dir) > 0) {
        r.algo = LRSCAN_ALGO_CHUNKED;
        r.chunk = prefer_chunked(s, dir);
        r.width = 0;
        return r;
    }
    if (r.algo == LRSCAN_ALGO_AUTO) {
        int w = 0, t = 0;
        fused_default_cfg(s, dir, aligned, &w, &t);
        if (fused_cfg_supported(s, dir, w, t, aligned)) {
            r.algo = LRSCAN_ALGO_FUSED;
            r.width = w;
            r.chunk = t;
        } else {
            // past the tiled form's 32-bit in-tile offsets (a tile of rows of
            // more than about 2 GB / tile bytes): the three-launch form
            r.algo = LRSCAN_ALGO_CHUNKED;
            r.chunk = kDefaultChunk;
            r.width = 0;
        }
        return r;
    }
    if (r.algo == LRSCAN_ALGO_CHUNKED && r.chunk == 0) r.chunk = kDefaultChunk;
    if (r.algo == LRSCAN_ALGO_FUSED && (r.chunk == 0 || r.width == 0)) {
        int w = 0, t = 0;
        fused_default_cfg(s, dir, aligned, &w, &t);
        if (r.width == 0) r.width = w;
        if (r.chunk == 0) r.chunk = t;
    }
    return r;
}

int validate_algo(const Shape& s, int dir, const Resolved& r, bool aligned) {
    switch (r.algo) {
        case LRSCAN_ALGO_SEQ: return LRSCAN_OK;
        case LRSCAN_ALGO_CHUNKED: return chunk_ok(r.chunk) ? LRSCAN_OK : LRSCAN_ERR_CHUNK;
        case LRSCAN_ALGO_FUSED:
            return fused_cfg_supported(s, dir, r.width, r.chunk, aligned) ? LRSCAN_OK
                                                                            : LRSCAN_ERR_CHUNK;
    }
    return LRSCAN_ERR_ALGO;
}

size_t chunked_bytes(const Shape& s, int chunk) {
    const size_t nc = (size_t)((s.T + chunk - 1) / chunk);
    return 3 * align_up(nc * (size_t)s.B * (size_t)s.D * 4, 256);
}

size_t needed_bytes(const Shape& s, const Resolved& r) {
    switch (r.algo) {
        case LRSCAN_ALGO_CHUNKED: return chunked_bytes(s, r.chunk);
        case LRSCAN_ALGO_FUSED: return fused_workspace_bytes(s, r.width, r.chunk);
    }
    return 0;
}

// Workspace for a call: the caller's (checked; the fused form initialises it
// on every call, since the library cannot know what the caller did with it
// in between) or the library's.
int get_workspace(const Shape& s, const Resolved& r, const lrscan_opts* o, hipStream_t st,
                  Workspace* ws) {
    const size_t need = needed_bytes(s, r);
    *ws = Workspace{};
    if (need == 0) return LRSCAN_OK;
    if (o && o->workspace) {
        if (o->workspace_bytes < need) return LRSCAN_ERR_WORKSPACE;
        if (reinterpret_cast<uintptr_t>(o->workspace) % 256 != 0) return LRSCAN_ERR_WORKSPACE;
        ws->ptr = o->workspace;
        ws->bytes = need;  // initialised on every call: only what this call uses
        ws->init = true;
        return LRSCAN_OK;
    }
    const int kind = r.algo == LRSCAN_ALGO_FUSED ? 1 : 0;
    return library_workspace(need, kind, st, ws);
}

int hip_status(hipError_t e) { return e == hipSuccess ? LRSCAN_OK : LRSCAN_ERR_HIP; }

// ---- complex scan helpers ----

bool pair_ok(const void* re, const void* im) { return (re == nullptr) == (im == nullptr); }

// The per-lane walk for short complex sequences, whose 128-row tiles would
// be mostly idle rows.  Measured on MI355X (M = 2560, caches flushed before
// each call): for T <= 16 the walk is as fast at 20K lanes and 4-8x faster
// from 330K lanes (bf16 T = 8 over 1.3M lanes: 4.0 / 4.9 against 0.6 / 0.9
// TB/s forward / backward); for T <= 32 from 262K lanes (bf16, 330K lanes:
// 4.0 / 4.4 against 2.0 / 2.9; at 82K lanes the tiles are faster); the bf16
// forward also up to T = 64 from 262K lanes (1.3M lanes: 4.9 against 3.9),
// while its backward and the fp32 scan at T = 64 are even or faster tiled.
bool complex_prefer_seq(const Shape& s, int dir) {
    if (s.T <= 16) return true;
    if (s.B * s.D < ((int64_t)1 << 18)) return false;
    if (s.T <= 32) return true;
    return dir == 0 && s.dtype == LRSCAN_BF16 && s.T <= 64;
}

// AUTO -> SEQ for short sequences (complex_prefer_seq, per direction) and
// past the tiled form's index limits, else FUSED; FUSED takes the library's
// tile shapes (chunk and width 0); CHUNKED is not provided.
int complex_algo(const Shape& s, int dir, const lrscan_opts* o, int* algo) {
    const int a = o ? o->algo : LRSCAN_ALGO_AUTO;
    if (a == LRSCAN_ALGO_AUTO || a == LRSCAN_ALGO_FUSED) {
        if (o && (o->chunk != 0 || o->width != 0)) return LRSCAN_ERR_CHUNK;
        const bool seq = a == LRSCAN_ALGO_AUTO &&
                         (!complex_fused_supported(s) || complex_prefer_seq(s, dir));
        *algo = seq ? LRSCAN_ALGO_SEQ : LRSCAN_ALGO_FUSED;
        return LRSCAN_OK;
    }
    if (a == LRSCAN_ALGO_SEQ) {
        *algo = a;
        return LRSCAN_OK;
    }
    return LRSCAN_ERR_ALGO;
}

int complex_workspace(const Shape& s, int algo, const lrscan_opts* o, hipStream_t st,
                      Workspace* ws) {
    *ws = Workspace{};
    if (algo != LRSCAN_ALGO_FUSED) return LRSCAN_OK;
    if (!complex_fused_supported(s)) return LRSCAN_ERR_DIM;
    const size_t need = complex_fused_workspace_bytes(s);
    if (o && o->workspace) {
        if (o->workspace_bytes < need) return LRSCAN_ERR_WORKSPACE;
        if (reinterpret_cast<uintptr_t>(o->workspace) % 256 != 0) return LRSCAN_ERR_WORKSPACE;
        ws->ptr = o->workspace;
        ws->bytes = need;
        ws->init = true;
        return LRSCAN_OK;
    }
    return library_workspace(need, 1, st, ws);
}

// ---- fused-transition scan helpers ----

// The per-lane walk of the fused-transition scan for short sequences over
// at least 2^18 lanes, where even tiles as short as the sequence spend much
// of their time on fixed costs.  Measured on MI355X (M = 2560, B*T*M fixed,
// caches flushed, forward / backward TB/s, tiles against walk): bf16 T = 8
// 1.2 / 1.1 against 3.9 / 2.9, T = 32 3.5 / 3.0 against 4.6 / 4.1, T = 64
// 4.3 / 3.9 against 4.5 / 4.2; fp32 T = 16 4.6 / 4.1 against 5.1 / 4.4,
// T = 32 5.1 / 4.8 against 4.8 / 4.5.
bool samu_prefer_seq(const Shape& s) {
    if (s.B * s.D < ((int64_t)1 << 18)) return false;
    return s.T <= 16 || (s.dtype == LRSCAN_BF16 && s.T <= 64);
}

// AUTO (SEQ for short sequences, else FUSED), FUSED with the library's tile
// shapes (chunk and width 0) or SEQ; CHUNKED is not provided.
int samu_algo(const Shape& s, const lrscan_opts* o, int* algo) {
    const int a = o ? o->algo : LRSCAN_ALGO_AUTO;
    if (a != LRSCAN_ALGO_AUTO && a != LRSCAN_ALGO_FUSED && a != LRSCAN_ALGO_SEQ)
        return LRSCAN_ERR_ALGO;
    if (o && (o->chunk != 0 || o->width != 0)) return LRSCAN_ERR_CHUNK;
    *algo = a == LRSCAN_ALGO_AUTO ? (samu_prefer_seq(s) ? LRSCAN_ALGO_SEQ : LRSCAN_ALGO_FUSED) : a;
    return LRSCAN_OK;
}

size_t samu_need(const Shape& s) { return align_up(samu_scratch_bytes(s), 256) + samu_aux_bytes(s); }

// The fused scratch (library kind 1, or the head of the caller's buffer) and
// the auxiliary tables (library kind 2, or the caller's buffer after it).
int samu_workspace(const Shape& s, const lrscan_opts* o, hipStream_t st, Workspace* ws,
                   void** aux) {
    *ws = Workspace{};
    if (!samu_supported(s)) return LRSCAN_ERR_DIM;
    if (o && o->workspace) {
        if (o->workspace_bytes < samu_need(s)) return LRSCAN_ERR_WORKSPACE;
        if (reinterpret_cast<uintptr_t>(o->workspace) % 256 != 0) return LRSCAN_ERR_WORKSPACE;
        ws->ptr = o->workspace;
        ws->bytes = samu_scratch_bytes(s);
        ws->init = true;
        *aux = static_cast<char*>(o->workspace) + align_up(samu_scratch_bytes(s), 256);
        return LRSCAN_OK;
    }
    int rc = library_workspace(samu_scratch_bytes(s), 1, st, ws);
    if (rc != LRSCAN_OK) return rc;
    Workspace a;
    rc = library_workspace(samu_aux_bytes(s), 2, st, &a);
    if (rc != LRSCAN_OK) return rc;
    *aux = a.ptr;
    return LRSCAN_OK;
}

// ---- the forward, shared by scan_fwd_ex and scan_fwd_noalloc ----

struct FwdCall {
    const void* a;
    const void* b;
    void* out;
    float* last;
    Shape s;
    hipStream_t hs;
    const lrscan_opts* o;
};

// Argument checks and the algorithm choice of a forward call.
int check_fwd(const FwdCall& c, Resolved* r) {
    if (!c.a || !c.b || (!c.out && !c.last)) return LRSCAN_ERR_NULL;
    if (!dims_ok(c.s.B, c.s.T, c.s.D)) return LRSCAN_ERR_DIM;
    if (!dtype_ok(c.s.dtype)) return LRSCAN_ERR_DTYPE;
    const void* ptrs[3] = {c.a, c.b, c.out};
    const bool aligned = rows_aligned(c.s, ptrs, 3);
    *r = resolve(c.s, 0, c.o, aligned);
    return validate_algo(c.s, 0, *r, aligned);
}

// Enqueue a checked forward call on workspace `ws`.
int run_fwd(const FwdCall& c, const Resolved& r, const Workspace& ws) {
    const Shape& s = c.s;
    const float* h0 = c.o ? c.o->h0 : nullptr;
    const uint8_t* reset = c.o ? c.o->reset : nullptr;
    switch (r.algo) {
        case LRSCAN_ALGO_SEQ:
            return hip_status(launch_seq_fwd(s, c.a, c.b, c.out, c.last, h0, reset, c.hs));
        case LRSCAN_ALGO_CHUNKED: {
            const int64_t NC = (s.T + r.chunk - 1) / r.chunk;
            const size_t part = align_up((size_t)NC * s.B * s.D * 4, 256);
            float* P = static_cast<float*>(ws.ptr);
            float* Q = reinterpret_cast<float*>(static_cast<char*>(ws.ptr) + part);
            float* cin = reinterpret_cast<float*>(static_cast<char*>(ws.ptr) + 2 * part);
            hipError_t e = launch_chunk_summary(s, r.chunk, c.a, c.b, reset, P, Q, c.hs);
            if (e == hipSuccess) e = launch_chunk_prefix(s.B, NC, s.D, P, Q, h0, cin, nullptr, c.hs);
            if (e == hipSuccess)
                e = launch_chunk_replay(s, r.chunk, c.a, c.b, reset, cin, c.out, c.last, c.hs);
            return hip_status(e);
        }
        case LRSCAN_ALGO_FUSED:
            return fused_status(launch_fused_fwd(s, r.width, r.chunk, c.a, c.b, c.out, c.last, h0,
                                                 reset, ws.ptr, ws.bytes, ws.init,
                                                 c.o ? c.o->polls : 0, c.hs),
                                ws, c.hs);
    }
    return LRSCAN_ERR_ALGO;
}

}  // namespace

namespace lrscan {

// A forward call whose scratch comes from a fixed buffer of `cap` bytes that
// `acquire` supplies (only when the chosen algorithm needs scratch): no
// allocation, and the buffer is initialised inside the call.
int fwd_on_fixed_scratch(const void* a, const void* b, void* out, float* last, int64_t B,
                         int64_t T, int64_t D, int dtype, void* stream, const lrscan_opts* opts,
                         size_t cap, int (*acquire)(void**)) {
    if (opts && opts->workspace) return LRSCAN_ERR_WORKSPACE;
    const FwdCall c{a, b, out, last, Shape{B, T, D, dtype}, static_cast<hipStream_t>(stream), opts};
    Resolved r;
    int st = check_fwd(c, &r);
    if (st != LRSCAN_OK) return st;
    const size_t need = needed_bytes(c.s, r);
    if (need > cap) return LRSCAN_ERR_TOO_BIG;
    Workspace ws;
    if (need > 0) {
        st = acquire(&ws.ptr);
        if (st != LRSCAN_OK) return st;
        ws.bytes = need;
        ws.init = true;  // nothing carries over from the previous user of the buffer
    }
    return run_fwd(c, r, ws);
}

}  // namespace lrscan

extern "C" {

LRSCAN_API const char* scan_status_string(int status) {
    switch (status) {
        case LRSCAN_OK: return "ok";
        case LRSCAN_ERR_NULL: return "a required pointer is NULL";
        case LRSCAN_ERR_DIM: return "B, T and D must be >= 1 and their product must fit";
        case LRSCAN_ERR_DTYPE: return "dtype must be LRSCAN_F32 or LRSCAN_BF16";
        case LRSCAN_ERR_CHUNK: return "chunk / tile length not supported by the algorithm";
        case LRSCAN_ERR_WORKSPACE: return "workspace smaller than scan_workspace_bytes() or not 256-byte aligned";
        case LRSCAN_ERR_HIP: return "the HIP runtime reported an error";
        case LRSCAN_ERR_ALGO: return "unknown algorithm";
        case LRSCAN_ERR_TOO_BIG:
            return "the call needs more scratch than the static buffer of scan_fwd_noalloc "
                   "(LRSCAN_NOALLOC_SCRATCH_BYTES) holds";
        case LRSCAN_ERR_CAPTURE:
            return "the stream is capturing a graph and has no library workspace of this size yet "
                   "(make one eager call of at least this size on the stream first, or pass "
                   "opts->workspace)";
    }
    return "unknown status";
}

LRSCAN_API int scan_auto_algo(int64_t B, int64_t T, int64_t D, int dtype, int dir, int* chunk,
                              int* width) {
    if (!dims_ok(B, T, D)) return LRSCAN_ERR_DIM;
    if (!dtype_ok(dtype)) return LRSCAN_ERR_DTYPE;
    const Shape s{B, T, D, dtype};
    const Resolved r = resolve(s, dir, nullptr, shape_aligned(s));
    if (chunk) *chunk = r.chunk;
    if (width) *width = r.width;
    return r.algo;
}

// The largest need over both directions and both pointer alignments (a call
// with unaligned pointers falls back to the narrowest fused tile).
LRSCAN_API size_t scan_workspace_bytes(int64_t B, int64_t T, int64_t D, int dtype,
                                       const lrscan_opts* opts) {
    if (!dims_ok(B, T, D) || !dtype_ok(dtype)) return 0;
    const Shape s{B, T, D, dtype};
    size_t need = 0;
    for (int dir = 0; dir < 2; ++dir)
        for (int al = 0; al < 2; ++al) {
            if (al && !shape_aligned(s)) continue;
            const Resolved r = resolve(s, dir, opts, al != 0);
            if (validate_algo(s, dir, r, al != 0) != LRSCAN_OK) continue;
            const size_t n = needed_bytes(s, r);
            if (n > need) need = n;
        }
    return need;
}

LRSCAN_API int scan_fwd_ex(const void* a, const void* b, void* out, float* last, int64_t B,
                           int64_t T, int64_t D, int dtype, void* stream, const lrscan_opts* opts) {
    const FwdCall c{a, b, out, last, Shape{B, T, D, dtype}, static_cast<hipStream_t>(stream), opts};
    Resolved r;
    int st = check_fwd(c, &r);
    if (st != LRSCAN_OK) return st;
    Workspace ws;
    st = get_workspace(c.s, r, opts, c.hs, &ws);
    if (st != LRSCAN_OK) return st;
    return run_fwd(c, r, ws);
}

LRSCAN_API int scan_bwd_ex(const void* a, const void* out, const void* grad_out,
                           const float* grad_last, void* grad_a, void* grad_b, int64_t B,
                           int64_t T, int64_t D, int dtype, void* stream, const lrscan_opts* opts) {
    if (!a || !out || !grad_out || !grad_a || !grad_b) return LRSCAN_ERR_NULL;
    if (!dims_ok(B, T, D)) return LRSCAN_ERR_DIM;
    if (!dtype_ok(dtype)) return LRSCAN_ERR_DTYPE;
    const Shape s{B, T, D, dtype};
    const void* ptrs[5] = {a, out, grad_out, grad_a, grad_b};
    const bool aligned = rows_aligned(s, ptrs, 5);
    const Resolved r = resolve(s, 1, opts, aligned);
    int st = validate_algo(s, 1, r, aligned);
    if (st != LRSCAN_OK) return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const float* h0 = opts ? opts->h0 : nullptr;
    float* grad_h0 = opts ? opts->grad_h0 : nullptr;
    const uint8_t* reset = opts ? opts->reset : nullptr;
    Workspace ws;
    st = get_workspace(s, r, opts, hs, &ws);
    if (st != LRSCAN_OK) return st;
    switch (r.algo) {
        case LRSCAN_ALGO_SEQ:
            return hip_status(launch_seq_bwd(s, a, out, grad_out, grad_last, h0, reset, grad_a, grad_b,
                                             grad_h0, hs));
        case LRSCAN_ALGO_CHUNKED: {
            const int64_t NC = (T + r.chunk - 1) / r.chunk;
            const size_t part = align_up((size_t)NC * B * D * 4, 256);
            float* P = static_cast<float*>(ws.ptr);
            float* Q = reinterpret_cast<float*>(static_cast<char*>(ws.ptr) + part);
            float* fut = reinterpret_cast<float*>(static_cast<char*>(ws.ptr) + 2 * part);
            hipError_t e = launch_reverse_chunk_summary(s, r.chunk, a, grad_out, reset, P, Q, hs);
            if (e == hipSuccess)
                e = launch_reverse_chunk_prefix(B, NC, D, P, Q, grad_last, fut, grad_h0, hs);
            if (e == hipSuccess)
                e = launch_reverse_chunk_replay(s, r.chunk, a, out, grad_out, reset, fut, h0, grad_a,
                                                grad_b, hs);
            return hip_status(e);
        }
        case LRSCAN_ALGO_FUSED:
            return fused_status(launch_fused_bwd(s, r.width, r.chunk, a, out, grad_out, grad_last,
                                                 h0, reset, grad_a, grad_b, grad_h0, ws.ptr, ws.bytes,
                                                 ws.init, opts ? opts->polls : 0, hs),
                                ws, hs);
    }
    return LRSCAN_ERR_ALGO;
}

LRSCAN_API int scan_fwd(const void* a, const void* b, void* out, float* last, int64_t B, int64_t T,
                        int64_t D, int dtype, void* stream) {
    return scan_fwd_ex(a, b, out, last, B, T, D, dtype, stream, nullptr);
}

LRSCAN_API int scan_bwd(const void* a, const void* out, const void* grad_out,
                        const float* grad_last, void* grad_a, void* grad_b, int64_t B, int64_t T,
                        int64_t D, int dtype, void* stream) {
    return scan_bwd_ex(a, out, grad_out, grad_last, grad_a, grad_b, B, T, D, dtype, stream,
                       nullptr);
}

LRSCAN_API int scan_step(const void* a, const void* b, const float* state_in,
                         const uint8_t* reset, void* out, float* state_out, int64_t B, int64_t D,
                         int dtype, void* stream) {
    if (!a || !b || (!out && !state_out)) return LRSCAN_ERR_NULL;
    if (!dims_ok(B, 1, D)) return LRSCAN_ERR_DIM;
    if (!dtype_ok(dtype)) return LRSCAN_ERR_DTYPE;
    return hip_status(launch_step(B, D, dtype, a, b, state_in, reset, out, state_out,
                                  static_cast<hipStream_t>(stream)));
}

// ---- complex diagonal scan --------------------------------------------------------

LRSCAN_API int scan_complex_fwd(const void* ar, const void* ai, const void* br, const void* bi,
                                void* out_r, void* out_i, float* last_r, float* last_i,
                                const float* h0_r, const float* h0_i, int64_t B, int64_t T,
                                int64_t M, int dtype, void* stream, const lrscan_opts* opts) {
    if (!ar || !ai || !br || !bi) return LRSCAN_ERR_NULL;
    if (!pair_ok(out_r, out_i) || !pair_ok(last_r, last_i) || !pair_ok(h0_r, h0_i))
        return LRSCAN_ERR_NULL;
    if (!out_r && !last_r) return LRSCAN_ERR_NULL;
    if (!dims_ok(B, T, M)) return LRSCAN_ERR_DIM;
    if (!dtype_ok(dtype)) return LRSCAN_ERR_DTYPE;
    int algo = 0;
    const Shape s{B, T, M, dtype};
    int st = complex_algo(s, 0, opts, &algo);
    if (st != LRSCAN_OK) return st;
    const CxFwdPtrs p{ar, ai, br, bi, out_r, out_i, last_r, last_i, h0_r, h0_i,
                      opts ? opts->reset : nullptr};
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (algo == LRSCAN_ALGO_SEQ) return hip_status(launch_complex_seq_fwd(s, p, hs));
    Workspace ws;
    st = complex_workspace(s, algo, opts, hs, &ws);
    if (st != LRSCAN_OK) return st;
    return fused_status(launch_complex_fused_fwd(s, p, ws.ptr, ws.bytes, ws.init,
                                                 opts ? opts->polls : 0, hs),
                        ws, hs);
}

LRSCAN_API int scan_complex_bwd(const void* ar, const void* ai, const void* out_r,
                                const void* out_i, const void* grad_out_r, const void* grad_out_i,
                                const float* grad_last_r, const float* grad_last_i,
                                const float* h0_r, const float* h0_i, void* grad_ar,
                                void* grad_ai, void* grad_br, void* grad_bi, float* grad_h0_r,
                                float* grad_h0_i, int64_t B, int64_t T, int64_t M, int dtype,
                                void* stream, const lrscan_opts* opts) {
    if (!ar || !ai || !out_r || !out_i || !grad_out_r || !grad_out_i || !grad_ar || !grad_ai ||
        !grad_br || !grad_bi)
        return LRSCAN_ERR_NULL;
    if (!pair_ok(grad_last_r, grad_last_i) || !pair_ok(h0_r, h0_i) ||
        !pair_ok(grad_h0_r, grad_h0_i))
        return LRSCAN_ERR_NULL;
    if (!dims_ok(B, T, M)) return LRSCAN_ERR_DIM;
    if (!dtype_ok(dtype)) return LRSCAN_ERR_DTYPE;
    int algo = 0;
    const Shape s{B, T, M, dtype};
    int st = complex_algo(s, 1, opts, &algo);
    if (st != LRSCAN_OK) return st;
    const CxBwdPtrs p{ar, ai, out_r, out_i, grad_out_r, grad_out_i, grad_last_r, grad_last_i,
                      h0_r, h0_i, opts ? opts->reset : nullptr, grad_ar, grad_ai, grad_br,
                      grad_bi, grad_h0_r, grad_h0_i};
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (algo == LRSCAN_ALGO_SEQ) return hip_status(launch_complex_seq_bwd(s, p, hs));
    Workspace ws;
    st = complex_workspace(s, algo, opts, hs, &ws);
    if (st != LRSCAN_OK) return st;
    return fused_status(launch_complex_fused_bwd(s, p, ws.ptr, ws.bytes, ws.init,
                                                 opts ? opts->polls : 0, hs),
                        ws, hs);
}

LRSCAN_API size_t scan_complex_workspace_bytes(int64_t B, int64_t T, int64_t M, int dtype,
                                               const lrscan_opts* opts) {
    if (!dims_ok(B, T, M) || !dtype_ok(dtype)) return 0;
    const Shape s{B, T, M, dtype};
    // the tiled form's scratch if either direction takes it
    bool fused = false;
    for (int dir = 0; dir < 2; ++dir) {
        int algo = 0;
        if (complex_algo(s, dir, opts, &algo) != LRSCAN_OK) return 0;
        fused = fused || algo == LRSCAN_ALGO_FUSED;
    }
    return fused && complex_fused_supported(s) ? complex_fused_workspace_bytes(s) : 0;
}

// ---- fused-transition (SAMU-form) complex scan ---------------------------------------

LRSCAN_API int scan_samu_fwd(const void* eta, const void* delta, const float* nu_log,
                             const float* theta_log, const void* br, const void* bi, void* out_r,
                             void* out_i, float* last_r, float* last_i, const float* h0_r,
                             const float* h0_i, int64_t B, int64_t T, int64_t M, int dtype,
                             void* stream, const lrscan_opts* opts) {
    if (!eta || !delta || !nu_log || !theta_log || !br || !bi) return LRSCAN_ERR_NULL;
    if (!pair_ok(out_r, out_i) || !pair_ok(last_r, last_i) || !pair_ok(h0_r, h0_i))
        return LRSCAN_ERR_NULL;
    if (!out_r && !last_r) return LRSCAN_ERR_NULL;
    if (!dims_ok(B, T, M)) return LRSCAN_ERR_DIM;
    if (!dtype_ok(dtype)) return LRSCAN_ERR_DTYPE;
    const Shape s{B, T, M, dtype};
    int algo = 0;
    int st = samu_algo(s, opts, &algo);
    if (st != LRSCAN_OK) return st;
    const SamuFwdPtrs p{eta,    delta,  nu_log, theta_log, br,   bi,  out_r,
                        out_i,  last_r, last_i, h0_r,      h0_i, opts ? opts->reset : nullptr};
    hipStream_t hs = static_cast<hipStream_t>(stream);
    Workspace ws;
    void* aux = nullptr;
    st = samu_workspace(s, opts, hs, &ws, &aux);
    if (st != LRSCAN_OK) return st;
    // the walk leaves the fused scratch untouched (not initialised by it)
    if (algo == LRSCAN_ALGO_SEQ) return hip_status(launch_samu_seq_fwd(s, p, aux, hs));
    return fused_status(
        launch_samu_fwd(s, p, ws.ptr, ws.bytes, ws.init, aux, opts ? opts->polls : 0, hs),
        ws, hs);
}

LRSCAN_API int scan_samu_bwd(const void* eta, const void* delta, const float* nu_log,
                             const float* theta_log, const void* out_r, const void* out_i,
                             const void* grad_out_r, const void* grad_out_i,
                             const float* grad_last_r, const float* grad_last_i,
                             const float* h0_r, const float* h0_i, float* grad_eta,
                             float* grad_delta, float* grad_nu_log, float* grad_theta_log,
                             void* grad_br, void* grad_bi, float* grad_h0_r, float* grad_h0_i,
                             int64_t B, int64_t T, int64_t M, int dtype, void* stream,
                             const lrscan_opts* opts) {
    if (!eta || !delta || !nu_log || !theta_log || !out_r || !out_i || !grad_out_r ||
        !grad_out_i || !grad_br || !grad_bi)
        return LRSCAN_ERR_NULL;
    if (!pair_ok(grad_last_r, grad_last_i) || !pair_ok(h0_r, h0_i) ||
        !pair_ok(grad_h0_r, grad_h0_i))
        return LRSCAN_ERR_NULL;
    if (!dims_ok(B, T, M)) return LRSCAN_ERR_DIM;
    if (!dtype_ok(dtype)) return LRSCAN_ERR_DTYPE;
    const Shape s{B, T, M, dtype};
    int algo = 0;
    int st = samu_algo(s, opts, &algo);
    if (st != LRSCAN_OK) return st;
    SamuBwdPtrs p;
    p.eta = eta;
    p.delta = delta;
    p.nu_log = nu_log;
    p.theta_log = theta_log;
    p.hr = out_r;
    p.hi = out_i;
    p.gr = grad_out_r;
    p.gi = grad_out_i;
    p.glr = grad_last_r;
    p.gli = grad_last_i;
    p.h0r = h0_r;
    p.h0i = h0_i;
    p.reset = opts ? opts->reset : nullptr;
    p.grad_eta = grad_eta;
    p.grad_delta = grad_delta;
    p.grad_nu_log = grad_nu_log;
    p.grad_theta_log = grad_theta_log;
    p.gbr = grad_br;
    p.gbi = grad_bi;
    p.gh0r = grad_h0_r;
    p.gh0i = grad_h0_i;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    Workspace ws;
    void* aux = nullptr;
    st = samu_workspace(s, opts, hs, &ws, &aux);
    if (st != LRSCAN_OK) return st;
    if (algo == LRSCAN_ALGO_SEQ) return hip_status(launch_samu_seq_bwd(s, p, aux, hs));
    return fused_status(
        launch_samu_bwd(s, p, ws.ptr, ws.bytes, ws.init, aux, opts ? opts->polls : 0, hs),
        ws, hs);
}

LRSCAN_API size_t scan_samu_workspace_bytes(int64_t B, int64_t T, int64_t M, int dtype,
                                            const lrscan_opts* opts) {
    if (!dims_ok(B, T, M) || !dtype_ok(dtype)) return 0;
    const Shape s{B, T, M, dtype};
    int algo = 0;
    if (samu_algo(s, opts, &algo) != LRSCAN_OK) return 0;
    // the walk uses the same buffer (its tables and partial sums in the part
    // after the fused scratch), so the need is the same for every algorithm
    return samu_supported(s) ? samu_need(s) : 0;
}

// ---- the chunked form, step by step ---------------------------------------------
LRSCAN_API int scan_chunk_summary(const void* a, const void* b, float* P, float* Q, int64_t B,
                                  int64_t T, int64_t D, int chunk, int dtype, void* stream) {
    if (!a || !b || !P || !Q) return LRSCAN_ERR_NULL;
    if (!dims_ok(B, T, D)) return LRSCAN_ERR_DIM;
    if (!dtype_ok(dtype)) return LRSCAN_ERR_DTYPE;
    if (!chunk_ok(chunk)) return LRSCAN_ERR_CHUNK;
    return hip_status(launch_chunk_summary(Shape{B, T, D, dtype}, chunk, a, b, nullptr, P, Q,
                                           static_cast<hipStream_t>(stream)));
}

LRSCAN_API int scan_chunk_prefix(const float* P, const float* Q, const float* h0, float* chunk_in,
                                 float* last, int64_t B, int64_t NC, int64_t D, void* stream) {
    if (!P || !Q || !chunk_in) return LRSCAN_ERR_NULL;
    if (!dims_ok(B, NC, D)) return LRSCAN_ERR_DIM;
    return hip_status(launch_chunk_prefix(B, NC, D, P, Q, h0, chunk_in, last,
                                          static_cast<hipStream_t>(stream)));
}

LRSCAN_API int scan_chunk_replay(const void* a, const void* b, const float* chunk_in, void* out,
                                 float* last, int64_t B, int64_t T, int64_t D, int chunk,
                                 int dtype, void* stream) {
    if (!a || !b || !chunk_in || !out) return LRSCAN_ERR_NULL;
    if (!dims_ok(B, T, D)) return LRSCAN_ERR_DIM;
    if (!dtype_ok(dtype)) return LRSCAN_ERR_DTYPE;
    if (!chunk_ok(chunk)) return LRSCAN_ERR_CHUNK;
    return hip_status(launch_chunk_replay(Shape{B, T, D, dtype}, chunk, a, b, nullptr, chunk_in, out, last,
                                          static_cast<hipStream_t>(stream)));
}

LRSCAN_API int scan_reverse_chunk_summary(const void* a, const void* grad_out, float* P, float* Q,
                                          int64_t B, int64_t T, int64_t D, int chunk, int dtype,
                                          void* stream) {
    if (!a || !grad_out || !P || !Q) return LRSCAN_ERR_NULL;
    if (!dims_ok(B, T, D)) return LRSCAN_ERR_DIM;
    if (!dtype_ok(dtype)) return LRSCAN_ERR_DTYPE;
    if (!chunk_ok(chunk)) return LRSCAN_ERR_CHUNK;
    return hip_status(launch_reverse_chunk_summary(Shape{B, T, D, dtype}, chunk, a, grad_out, nullptr, P, Q,
                                                   static_cast<hipStream_t>(stream)));
}

LRSCAN_API int scan_reverse_chunk_prefix(const float* P, const float* Q, const float* grad_last,
                                         float* future, float* grad_h0, int64_t B, int64_t NC,
                                         int64_t D, void* stream) {
    if (!P || !Q || !future) return LRSCAN_ERR_NULL;
    if (!dims_ok(B, NC, D)) return LRSCAN_ERR_DIM;
    return hip_status(launch_reverse_chunk_prefix(B, NC, D, P, Q, grad_last, future, grad_h0,
                                                  static_cast<hipStream_t>(stream)));
}

LRSCAN_API int scan_reverse_chunk_replay(const void* a, const void* out, const void* grad_out,
                                         const float* future, const float* h0, void* grad_a,
                                         void* grad_b, int64_t B, int64_t T, int64_t D, int chunk,
                                         int dtype, void* stream) {
    if (!a || !out || !grad_out || !future || !grad_a || !grad_b) return LRSCAN_ERR_NULL;
    if (!dims_ok(B, T, D)) return LRSCAN_ERR_DIM;
    if (!dtype_ok(dtype)) return LRSCAN_ERR_DTYPE;
    if (!chunk_ok(chunk)) return LRSCAN_ERR_CHUNK;
    return hip_status(launch_reverse_chunk_replay(Shape{B, T, D, dtype}, chunk, a, out, grad_out, nullptr,
                                                  future, h0, grad_a, grad_b,
                                                  static_cast<hipStream_t>(stream)));
}

}  // extern "C"
