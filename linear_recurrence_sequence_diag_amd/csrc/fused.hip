// fused.hip -- the single-launch chunked scan (forward and reverse time).
//
// The three steps of the chunked form (page "triton_training_scan.py":
// chunk summary, prefix over the chunk maps, replay) run inside one launch,
// and every input byte is read from HBM once:
//
//  * A tile is CT = SEGS*NR consecutive steps of W lanes of one batch row
//    (W = 8 x 16 bytes: 64 bf16 or 32 fp32 lanes, one 128-byte line per row).
//    A workgroup of WAVES wavefronts loads its tile into registers: lane l of
//    a wavefront owns the 16-byte vector (l % 8) of rows of segment
//    seg = wave*8 + l/8, NR consecutive rows each.  Each instruction thus
//    reads 8 full 128-byte lines, and every load of the tile is issued before
//    the first is used.
//  * Summary: each thread folds its NR rows into one affine map per lane;
//    the 8 segments of a wavefront are scanned with an in-wavefront scan, the
//    wavefronts through LDS, giving the tile's map (P, Q) per lane.
//  * Prefix: tiles of one lane block form a chain.  Tiles take tickets from
//    an atomic counter in chain order (all tiles of chunk k before any tile of
//    chunk k+1), publish (P, Q) as soon as the summary is done, then look back
//    over up to LB predecessors for the nearest published inclusive state H
//    and apply the predecessors' maps to it, oldest first, before publishing
//    their own H.  This is the decoupled look-back of Merrill & Garland
//    ("Single-pass Parallel Prefix Scan with Decoupled Look-back", 2016),
//    made deterministic: every H equals the plain chained value
//    H_k = fma(P_k, H_{k-1}, Q_k) whatever the timing, so results do not
//    depend on scheduling.  A tile only waits on tiles with smaller tickets,
//    which are already resident or finished, so the chain always drains.
//  * Replay: each thread rescans its rows from registers, starting from the
//    state entering its segment, and writes the outputs once.
//
// Published words are single 32- or 64-bit device-scope atomic stores;
// every word starts as the all-ones pattern, which no published value takes,
// so readers need no separate flag or fence.  The reverse-time kernel is the
// mirror image: tickets run from the last chunk to the first and carries flow
// from later rows to earlier ones.
#include <algorithm>
#include <cstddef>

#include "device.hpp"
#include "launch.hpp"

namespace lrscan {

namespace {

constexpr int kCG = 8;           // threads per row (8 x 16 B = 128 B)
constexpr int kRG = kWave / kCG;  // row groups (segments) per wavefront
constexpr int kLB = 8;           // look-back window
constexpr uint32_t kSpinLimit = 1u << 20;

// Workspace of the fused form.  A 256-byte header, then two regions of equal
// size.  A launch publishes into region `phase`, which is all-ones wherever it
// will write; it clears the words the previous launch dirtied in the other
// region, and the workgroup that takes the last ticket resets the other
// region's ticket counter, records how many words this launch dirties and
// flips the phase.  Every workgroup has read the phase before the last ticket
// is taken, so back-to-back launches on one stream need no separate
// initialisation step.
// The ticket counters live in their own 128-byte line: every workgroup reads
// the phase word, and sharing its line with the atomically updated counters
// slowed the launch down several-fold on MI355X.
struct Header {
    uint32_t phase;
    uint32_t reserved;
    unsigned long long dirty[2];  // words the last user of each region wrote
    uint32_t pad[26];
    uint32_t ctr[2];              // ticket counters (all-ones: no ticket taken yet)
};
static_assert(offsetof(Header, ctr) == 128, "ticket counters start a new cache line");

struct Scratch {
    Header* hdr;
    uint32_t* region[2];
    unsigned long long entries;  // NK * nS * W published entries (3 words each)
    uint32_t total_tiles;
};

constexpr int kHeaderBytes = 256;

struct TileTicket {
    uint32_t ticket;
    uint32_t phase;
    unsigned long long nclear;
};

__device__ __forceinline__ void header_update(const Scratch& sc, uint32_t p) {
    publish_u32(&sc.hdr->ctr[p ^ 1u], kEmpty);
    publish_u64(&sc.hdr->dirty[p], 3ull * sc.entries);
    publish_u32(&sc.hdr->phase, p ^ 1u);
}

// Restore the all-ones state of the words the previous launch wrote in the
// region this launch does not use (spread over all workgroups).
__device__ __forceinline__ void clear_other_region(const Scratch& sc, const TileTicket& tt,
                                                   int nthreads) {
    uint32_t* other = sc.region[tt.phase ^ 1u];
    const unsigned long long stride = (unsigned long long)sc.total_tiles * nthreads;
    for (unsigned long long i = (unsigned long long)tt.ticket * nthreads + threadIdx.x; i < tt.nclear;
         i += stride)
        other[i] = kEmpty;
}

__device__ __forceinline__ unsigned long long pack_aff(Aff m) {
    return (unsigned long long)publishable(m.p) | ((unsigned long long)publishable(m.q) << 32);
}
__device__ __forceinline__ Aff unpack_aff(unsigned long long w) {
    return Aff{__uint_as_float((uint32_t)w), __uint_as_float((uint32_t)(w >> 32))};
}

// Carry entering tile k of a chain (forward: DIR = -1 looks at k-1, k-2, ...;
// reverse: DIR = +1 looks at k+1, k+2, ...).  `base0` is the carry entering the
// chain (h0 forward, grad_last reverse).  Returns the chained value; NaN if
// the wait ever exceeded the spin limit (then every output of the tile is NaN).
template <int DIR>
__device__ float look_back(const unsigned long long* pqs, const uint32_t* hs, int64_t k, int64_t NK,
                           int64_t nS, int64_t s, int W, int c, float base0) {
    const int64_t span = DIR < 0 ? k : (NK - 1 - k);  // predecessors in the chain
    if (span == 0) return base0;
    for (uint32_t spin = 0;; ++spin) {
        uint32_t hw[kLB];
        unsigned long long pq[kLB];
#pragma unroll
        for (int i = 0; i < kLB; ++i) {
            const int64_t j = k + DIR * (1 + i);
            if (i < span) {
                const size_t o = ((size_t)j * nS + s) * W + c;
                hw[i] = peek_u32(hs + o);
                pq[i] = peek_u64(pqs + o);
            } else {
                hw[i] = kEmpty;
                pq[i] = ~0ull;
            }
        }
        int depth = -1;
        bool stop = false;
        float base = base0;
#pragma unroll
        for (int i = 0; i < kLB; ++i) {
            if (depth < 0 && !stop) {
                if (i >= span) {
                    depth = i;  // reached the start of the chain
                } else if (hw[i] != kEmpty) {
                    depth = i;
                    base = __uint_as_float(hw[i]);
                } else if ((uint32_t)pq[i] == kEmpty) {
                    stop = true;
                }
            }
        }
        if (depth < 0 && !stop && span == kLB) depth = kLB;  // chain start just past the window
        if (depth >= 0) {
            float x = base;
#pragma unroll
            for (int i = kLB - 1; i >= 0; --i)
                if (i < depth) x = aff_apply(unpack_aff(pq[i]), x);
            return x;
        }
        if (spin >= kSpinLimit) return __uint_as_float(0x7fc00000u);
        __builtin_amdgcn_s_sleep(1);
    }
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
template <int DT, bool ALIGNED, int NR, int WAVES>
__global__ __launch_bounds__(WAVES* kWave) void fused_fwd_kernel(
    const void* __restrict__ a, const void* __restrict__ b, void* __restrict__ out,
    float* __restrict__ last, const float* __restrict__ h0, Scratch sc, int64_t T, int64_t D,
    int64_t nW, int64_t nS, int64_t NK) {
    constexpr int V = Elem<DT>::V;
    constexpr int EB = Elem<DT>::bytes;
    constexpr int W = kCG * V;
    constexpr int SEGS = WAVES * kRG;
    constexpr int64_t CT = (int64_t)SEGS * NR;

    __shared__ TileTicket s_tt;
    __shared__ Aff s_excl[WAVES][V][kWave];
    __shared__ Aff s_wtot[WAVES][W];
    __shared__ float s_hin[W];

    const int tid = threadIdx.x;
    const int wave = uniform((int)(threadIdx.x / kWave));
    const int l = tid % kWave;
    const int rg = l / kCG;
    const int cg = l % kCG;
    if (tid == 0) {
        const uint32_t p = peek_u32(&sc.hdr->phase);
        s_tt.phase = p;
        s_tt.ticket = atomicAdd(&sc.hdr->ctr[p], 1u) + 1u;
        s_tt.nclear = sc.hdr->dirty[p ^ 1u];
        if (s_tt.ticket == sc.total_tiles - 1) header_update(sc, p);
    }
    __syncthreads();
    const TileTicket tt = s_tt;
    const int64_t ticket = uniform(tt.ticket);
    const uint32_t phase = uniform(tt.phase);
    const unsigned long long* pqs = reinterpret_cast<const unsigned long long*>(sc.region[phase]);
    const uint32_t* hs = sc.region[phase] + 2 * sc.entries;
    const int64_t k = ticket / nS;
    const int64_t s = ticket - k * nS;
    const int64_t bi = s / nW;
    const int64_t dcol0 = (s - bi * nW) * W;
    const int64_t d0 = dcol0 + cg * V;
    const int nvalid = d0 >= D ? 0 : (int)((D - d0) < V ? (D - d0) : V);
    const int64_t trow0 = k * CT;                                         // first row of the tile
    const int64_t row0 = trow0 + (int64_t)(wave * kRG + rg) * NR;          // first row of this thread
    const int64_t rowbytes = D * EB;
    const size_t tbase = (((size_t)bi * T + trow0) * D + dcol0) * EB;     // wave-uniform
    // lanes past D read a valid column and are then replaced by identity steps
    const uint32_t coff = (uint32_t)((nvalid > 0 ? cg * V : 0) * EB);
    const char* pa = static_cast<const char*>(a) + tbase;
    const char* pb = static_cast<const char*>(b) + tbase;
    char* po = static_cast<char*>(out) + tbase;

    // every load is issued unconditionally (rows past T read row T-1) so that
    // all of them are in flight together; invalid rows become identity steps
    RowVec<DT> ra[NR], rb[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const int64_t row = row0 + i;
        const int64_t rc = row < T ? row : T - 1;
        const uint32_t off = (uint32_t)(rc - trow0) * (uint32_t)rowbytes + coff;
        const RowVec<DT> xa = load_vec<DT, ALIGNED>(pa, off, nvalid, 1.0f);
        const RowVec<DT> xb = load_vec<DT, ALIGNED>(pb, off, nvalid, 0.0f);
        const bool ok = row < T && nvalid > 0;
        ra[i] = ok ? xa : RowVec<DT>::splat(1.0f);
        rb[i] = ok ? xb : RowVec<DT>::splat(0.0f);
    }
    clear_other_region(sc, tt, WAVES * kWave);

    // summary of this thread's segment, per lane, then the wavefront scan
#pragma unroll
    for (int j = 0; j < V; ++j) {
        Aff m = aff_identity();
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const float at = ra[i].get(j);
            m.p = at * m.p;
            m.q = fmaf(at, m.q, rb[i].get(j));
        }
        const Aff inc = wave_scan_up<kCG>(m);
        Aff ex;
        ex.p = shfl_up_f(inc.p, kCG);
        ex.q = shfl_up_f(inc.q, kCG);
        if (rg == 0) ex = aff_identity();
        s_excl[wave][j][l] = ex;
        if (rg == kRG - 1) s_wtot[wave][cg * V + j] = inc;
    }
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        opaque(ra[i]);
        opaque(rb[i]);
    }
    __syncthreads();

    // tile map, publication, look-back (one lane per column in wavefront 0)
    if (wave == 0 && l < W) {
        const int c = l;
        Aff A = aff_identity();
#pragma unroll
        for (int w = 0; w < WAVES; ++w) A = aff_then(A, s_wtot[w][c]);
        const size_t o = ((size_t)k * nS + s) * W + c;
        const bool more = k + 1 < NK;
        if (more) publish_u64(const_cast<unsigned long long*>(pqs) + o, pack_aff(A));
        const int64_t dl = dcol0 + c;
        const float base0 = (h0 && dl < D) ? h0[bi * D + dl] : 0.0f;
        const float hin = look_back<-1>(pqs, hs, k, NK, nS, s, W, c, base0);
        if (more) publish_u32(const_cast<uint32_t*>(hs) + o, publishable(aff_apply(A, hin)));
        s_hin[c] = hin;
    }
    __syncthreads();

    // replay from registers
    float h[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
        const int col = cg * V + j;
        float x = s_hin[col];
        for (int w = 0; w < wave; ++w) x = aff_apply(s_wtot[w][col], x);
        h[j] = aff_apply(s_excl[wave][j][l], x);
    }
    if (nvalid > 0) {
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            if (row0 + i < T) {
                RowOut<DT> o;
#pragma unroll
                for (int j = 0; j < V; ++j) {
                    h[j] = fmaf(ra[i].get(j), h[j], rb[i].get(j));
                    o.v[j] = h[j];
                }
                store_vec<DT, ALIGNED>(po, (uint32_t)(row0 + i - trow0) * (uint32_t)rowbytes + coff,
                                       nvalid, o);
            }
        }
        if (last && row0 <= T - 1 && T - 1 < row0 + NR) {
#pragma unroll
            for (int j = 0; j < V; ++j)
                if (j < nvalid) last[bi * D + d0 + j] = h[j];
        }
    }
}

// ---------------------------------------------------------------------------
// reverse time (backward)
// ---------------------------------------------------------------------------
template <int DT, bool ALIGNED, int NR, int WAVES>
__global__ __launch_bounds__(WAVES* kWave) void fused_bwd_kernel(
    const void* __restrict__ a, const void* __restrict__ out, const void* __restrict__ g,
    const float* __restrict__ grad_last, const float* __restrict__ h0, void* __restrict__ grad_a,
    void* __restrict__ grad_b, float* __restrict__ grad_h0, Scratch sc, int64_t T, int64_t D,
    int64_t nW, int64_t nS, int64_t NK) {
    constexpr int V = Elem<DT>::V;
    constexpr int EB = Elem<DT>::bytes;
    constexpr int W = kCG * V;
    constexpr int SEGS = WAVES * kRG;
    constexpr int64_t CT = (int64_t)SEGS * NR;

    __shared__ TileTicket s_tt;
    __shared__ Aff s_excl[WAVES][V][kWave];
    __shared__ Aff s_wtot[WAVES][W];
    __shared__ float s_cin[W];

    const int tid = threadIdx.x;
    const int wave = uniform((int)(threadIdx.x / kWave));
    const int l = tid % kWave;
    const int rg = l / kCG;
    const int cg = l % kCG;
    if (tid == 0) {
        const uint32_t p = peek_u32(&sc.hdr->phase);
        s_tt.phase = p;
        s_tt.ticket = atomicAdd(&sc.hdr->ctr[p], 1u) + 1u;
        s_tt.nclear = sc.hdr->dirty[p ^ 1u];
        if (s_tt.ticket == sc.total_tiles - 1) header_update(sc, p);
    }
    __syncthreads();
    const TileTicket tt = s_tt;
    const int64_t ticket = uniform(tt.ticket);
    const uint32_t phase = uniform(tt.phase);
    const unsigned long long* pqs = reinterpret_cast<const unsigned long long*>(sc.region[phase]);
    const uint32_t* hs = sc.region[phase] + 2 * sc.entries;
    const int64_t kr = ticket / nS;
    const int64_t s = ticket - kr * nS;
    const int64_t k = NK - 1 - kr;
    const int64_t bi = s / nW;
    const int64_t dcol0 = (s - bi * nW) * W;
    const int64_t d0 = dcol0 + cg * V;
    const int nvalid = d0 >= D ? 0 : (int)((D - d0) < V ? (D - d0) : V);
    const int64_t trow0 = k * CT;
    const int64_t row0 = trow0 + (int64_t)(wave * kRG + rg) * NR;
    const int64_t rowbytes = D * EB;
    const size_t tbase = (((size_t)bi * T + trow0) * D + dcol0) * EB;
    const int64_t hrow0 = trow0 > 0 ? trow0 - 1 : 0;  // first row of `out` the tile reads
    const size_t hbase = (((size_t)bi * T + hrow0) * D + dcol0) * EB;
    const uint32_t coff = (uint32_t)((nvalid > 0 ? cg * V : 0) * EB);
    const char* pa = static_cast<const char*>(a) + tbase;
    const char* pg = static_cast<const char*>(g) + tbase;
    const char* ph = static_cast<const char*>(out) + hbase;
    char* pga = static_cast<char*>(grad_a) + tbase;
    char* pgb = static_cast<char*>(grad_b) + tbase;

    RowVec<DT> ra[NR], rg_[NR], rh[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const int64_t row = row0 + i;
        const int64_t rc = row < T ? row : T - 1;
        const int64_t hr = rc >= 1 ? rc - 1 : 0;  // h_{t-1} lives in row t-1 of out
        const uint32_t off = (uint32_t)(rc - trow0) * (uint32_t)rowbytes + coff;
        const uint32_t hoff = (uint32_t)(hr - hrow0) * (uint32_t)rowbytes + coff;
        const RowVec<DT> xa = load_vec<DT, ALIGNED>(pa, off, nvalid, 1.0f);
        const RowVec<DT> xg = load_vec<DT, ALIGNED>(pg, off, nvalid, 0.0f);
        const RowVec<DT> xh = load_vec<DT, ALIGNED>(ph, hoff, nvalid, 0.0f);
        const bool ok = row < T && nvalid > 0;
        ra[i] = ok ? xa : RowVec<DT>::splat(1.0f);
        rg_[i] = ok ? xg : RowVec<DT>::splat(0.0f);
        rh[i] = (ok && row >= 1) ? xh : RowVec<DT>::splat(0.0f);
    }
    clear_other_region(sc, tt, WAVES * kWave);

    // reverse summary: the map from the carry entering the segment on the
    // right to the carry a_s*lambda_s leaving its first row s
#pragma unroll
    for (int j = 0; j < V; ++j) {
        Aff m = aff_identity();
#pragma unroll
        for (int i = NR - 1; i >= 0; --i) {
            const float at = ra[i].get(j);
            m.p = at * m.p;
            m.q = at * (m.q + rg_[i].get(j));
        }
        const Aff inc = wave_scan_down<kCG>(m);
        Aff ex;
        ex.p = shfl_down_f(inc.p, kCG);
        ex.q = shfl_down_f(inc.q, kCG);
        if (rg == kRG - 1) ex = aff_identity();
        s_excl[wave][j][l] = ex;
        if (rg == 0) s_wtot[wave][cg * V + j] = inc;
    }
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        opaque(ra[i]);
        opaque(rg_[i]);
    }
    __syncthreads();

    if (wave == 0 && l < W) {
        const int c = l;
        Aff A = aff_identity();
#pragma unroll
        for (int w = WAVES - 1; w >= 0; --w) A = aff_then(A, s_wtot[w][c]);
        const size_t o = ((size_t)k * nS + s) * W + c;
        const bool more = k > 0;
        if (more) publish_u64(const_cast<unsigned long long*>(pqs) + o, pack_aff(A));
        const int64_t dl = dcol0 + c;
        const float base0 = (grad_last && dl < D) ? grad_last[bi * D + dl] : 0.0f;
        const float cin = look_back<+1>(pqs, hs, k, NK, nS, s, W, c, base0);
        if (more) publish_u32(const_cast<uint32_t*>(hs) + o, publishable(aff_apply(A, cin)));
        s_cin[c] = cin;
    }
    __syncthreads();

    float carry[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
        const int col = cg * V + j;
        float x = s_cin[col];
        for (int w = WAVES - 1; w > wave; --w) x = aff_apply(s_wtot[w][col], x);
        carry[j] = aff_apply(s_excl[wave][j][l], x);
    }
    if (nvalid > 0) {
#pragma unroll
        for (int i = NR - 1; i >= 0; --i) {
            const int64_t row = row0 + i;
            if (row < T) {
                RowOut<DT> oa, ob;
#pragma unroll
                for (int j = 0; j < V; ++j) {
                    const float lam = rg_[i].get(j) + carry[j];
                    float hp = rh[i].get(j);
                    if (row == 0) hp = (h0 && j < nvalid) ? h0[bi * D + d0 + j] : 0.0f;
                    ob.v[j] = lam;
                    oa.v[j] = lam * hp;
                    carry[j] = ra[i].get(j) * lam;
                }
                const uint32_t off = (uint32_t)(row - trow0) * (uint32_t)rowbytes + coff;
                store_vec<DT, ALIGNED>(pga, off, nvalid, oa);
                store_vec<DT, ALIGNED>(pgb, off, nvalid, ob);
            }
        }
        if (grad_h0 && row0 == 0) {
#pragma unroll
            for (int j = 0; j < V; ++j)
                if (j < nvalid) grad_h0[bi * D + d0 + j] = carry[j];
        }
    }
}

// Workspace initialisation: header (phase 0, both counters unused, nothing
// dirty) and both regions all-ones.
__global__ void scratch_init_kernel(uint32_t* __restrict__ p, size_t words) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
         i += (size_t)gridDim.x * blockDim.x) {
        uint32_t v = kEmpty;
        if (i < kHeaderBytes / 4) v = (i == 32 || i == 33) ? kEmpty : 0u;  // Header::ctr
        p[i] = v;
    }
}

// ---------------------------------------------------------------------------
// tile configurations: tile length -> (rows per thread, wavefronts)
// ---------------------------------------------------------------------------
struct TileCfg {
    int tile, nr, waves;
};
constexpr TileCfg kFwdTiles[] = {{256, 8, 4}, {512, 16, 4}, {1024, 16, 8}};
constexpr TileCfg kBwdTiles[] = {{256, 8, 4}, {512, 8, 8}};

int64_t series_width(int dtype) {
    return kCG * (dtype == DT_F32 ? Elem<DT_F32>::V : Elem<DT_BF16>::V);
}

struct Layout {
    int64_t nW, nS, NK, W;
    unsigned long long entries;
};

Layout layout_of(const Shape& s, int tile) {
    Layout L;
    L.W = series_width(s.dtype);
    L.nW = (s.D + L.W - 1) / L.W;
    L.nS = s.B * L.nW;
    L.NK = (s.T + tile - 1) / tile;
    L.entries = (unsigned long long)L.NK * L.nS * L.W;
    return L;
}

size_t region_bytes_for(const Layout& L) { return (L.entries * 12 + 255) / 256 * 256; }

// Region size implied by a workspace size (the same for every call on one buffer).
size_t region_bytes_of(size_t ws_bytes) {
    return ws_bytes < (size_t)kHeaderBytes ? 0 : (ws_bytes - kHeaderBytes) / 2 / 256 * 256;
}

hipError_t prepare(void* ws, size_t ws_bytes, bool init, const Layout& L, hipStream_t st,
                   Scratch* sc) {
    const size_t rb = region_bytes_of(ws_bytes);
    if (rb < region_bytes_for(L)) return hipErrorInvalidValue;
    if ((unsigned long long)L.NK * L.nS >= 0xffffffffull) return hipErrorInvalidValue;
    char* base = static_cast<char*>(ws);
    if (init) {
        const size_t words = (kHeaderBytes + 2 * rb) / 4;
        const unsigned blocks = (unsigned)std::min<size_t>((words + 255) / 256, 8192);
        hipLaunchKernelGGL(scratch_init_kernel, dim3(blocks), dim3(256), 0, st,
                           reinterpret_cast<uint32_t*>(base), words);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    sc->hdr = reinterpret_cast<Header*>(base);
    sc->region[0] = reinterpret_cast<uint32_t*>(base + kHeaderBytes);
    sc->region[1] = reinterpret_cast<uint32_t*>(base + kHeaderBytes + rb);
    sc->entries = L.entries;
    sc->total_tiles = (uint32_t)(L.NK * L.nS);
    return hipSuccess;
}

template <int DT, bool AL, int NR, int WAVES>
void fwd_launch(const Shape& s, const Layout& L, const void* a, const void* b, void* out,
                float* last, const float* h0, const Scratch& sc, hipStream_t st) {
    const dim3 grid((unsigned)(L.NK * L.nS));
    hipLaunchKernelGGL((fused_fwd_kernel<DT, AL, NR, WAVES>), grid, dim3(WAVES * kWave), 0, st, a,
                       b, out, last, h0, sc, s.T, s.D, L.nW, L.nS, L.NK);
}

template <int DT, bool AL, int NR, int WAVES>
void bwd_launch(const Shape& s, const Layout& L, const void* a, const void* out, const void* g,
                const float* gl, const float* h0, void* ga, void* gb, float* gh0,
                const Scratch& sc, hipStream_t st) {
    const dim3 grid((unsigned)(L.NK * L.nS));
    hipLaunchKernelGGL((fused_bwd_kernel<DT, AL, NR, WAVES>), grid, dim3(WAVES * kWave), 0, st, a,
                       out, g, gl, h0, ga, gb, gh0, sc, s.T, s.D, L.nW, L.nS, L.NK);
}

template <int DT, bool AL>
bool fwd_dispatch(int tile, const Shape& s, const Layout& L, const void* a, const void* b,
                  void* out, float* last, const float* h0, const Scratch& sc, hipStream_t st) {
    switch (tile) {
        case 256: fwd_launch<DT, AL, 8, 4>(s, L, a, b, out, last, h0, sc, st); return true;
        case 512: fwd_launch<DT, AL, 16, 4>(s, L, a, b, out, last, h0, sc, st); return true;
        case 1024: fwd_launch<DT, AL, 16, 8>(s, L, a, b, out, last, h0, sc, st); return true;
    }
    return false;
}

template <int DT, bool AL>
bool bwd_dispatch(int tile, const Shape& s, const Layout& L, const void* a, const void* out,
                  const void* g, const float* gl, const float* h0, void* ga, void* gb, float* gh0,
                  const Scratch& sc, hipStream_t st) {
    switch (tile) {
        case 256: bwd_launch<DT, AL, 8, 4>(s, L, a, out, g, gl, h0, ga, gb, gh0, sc, st); return true;
        case 512: bwd_launch<DT, AL, 8, 8>(s, L, a, out, g, gl, h0, ga, gb, gh0, sc, st); return true;
    }
    return false;
}

}  // namespace

bool fused_tile_supported(const Shape& s, int dir, int tile) {
    // per-lane row offsets inside a tile are 32-bit
    const int64_t eb = s.dtype == DT_F32 ? 4 : 2;
    if ((int64_t)tile * s.D * eb >= ((int64_t)1 << 31)) return false;
    if (dir == 0) {
        for (const auto& c : kFwdTiles)
            if (c.tile == tile) return true;
    } else {
        for (const auto& c : kBwdTiles)
            if (c.tile == tile) return true;
    }
    return false;
}

int fused_default_tile(const Shape& s, int dir) {
    (void)s;
    return dir == 0 ? 512 : 256;
}

size_t fused_workspace_bytes(const Shape& s, int tile) {
    return kHeaderBytes + 2 * region_bytes_for(layout_of(s, tile));
}

hipError_t launch_fused_fwd(const Shape& s, int tile, const void* a, const void* b, void* out,
                            float* last, const float* h0, void* ws, size_t ws_bytes, bool init,
                            hipStream_t st) {
    const Layout L = layout_of(s, tile);
    Scratch sc;
    hipError_t e = prepare(ws, ws_bytes, init, L, st, &sc);
    if (e != hipSuccess) return e;
    const void* ptrs[3] = {a, b, out};
    const bool al = rows_aligned(s, ptrs, 3);
    bool ok;
    if (s.dtype == DT_F32)
        ok = al ? fwd_dispatch<DT_F32, true>(tile, s, L, a, b, out, last, h0, sc, st)
                : fwd_dispatch<DT_F32, false>(tile, s, L, a, b, out, last, h0, sc, st);
    else
        ok = al ? fwd_dispatch<DT_BF16, true>(tile, s, L, a, b, out, last, h0, sc, st)
                : fwd_dispatch<DT_BF16, false>(tile, s, L, a, b, out, last, h0, sc, st);
    if (!ok) return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_fused_bwd(const Shape& s, int tile, const void* a, const void* out,
                            const void* g, const float* grad_last, const float* h0, void* grad_a,
                            void* grad_b, float* grad_h0, void* ws, size_t ws_bytes, bool init,
                            hipStream_t st) {
    const Layout L = layout_of(s, tile);
    Scratch sc;
    hipError_t e = prepare(ws, ws_bytes, init, L, st, &sc);
    if (e != hipSuccess) return e;
    const void* ptrs[5] = {a, out, g, grad_a, grad_b};
    const bool al = rows_aligned(s, ptrs, 5);
    bool ok;
    if (s.dtype == DT_F32)
        ok = al ? bwd_dispatch<DT_F32, true>(tile, s, L, a, out, g, grad_last, h0, grad_a, grad_b,
                                             grad_h0, sc, st)
                : bwd_dispatch<DT_F32, false>(tile, s, L, a, out, g, grad_last, h0, grad_a,
                                              grad_b, grad_h0, sc, st);
    else
        ok = al ? bwd_dispatch<DT_BF16, true>(tile, s, L, a, out, g, grad_last, h0, grad_a, grad_b,
                                              grad_h0, sc, st)
                : bwd_dispatch<DT_BF16, false>(tile, s, L, a, out, g, grad_last, h0, grad_a,
                                               grad_b, grad_h0, sc, st);
    if (!ok) return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace lrscan
