// fused_common.hpp -- machinery shared by the single-launch (fused) scans,
// real (fused.hip) and complex (complex.hip): the self-cleaning workspace
// with its spread ticket counters, the tile geometry, the look-back with its
// bounded waiting, and the workspace layout.  Internal to liblrscan; every
// translation unit that includes it gets its own copy (anonymous namespace).
#pragma once

#include <algorithm>
#include <cstddef>

#include "device.hpp"
#include "launch.hpp"

namespace lrscan {

namespace {

// Look-back polls before a tile stops waiting and derives the predecessor
// maps it is missing (normal waits take a few polls; this bound only matters
// when a predecessor's workgroup is descheduled for a long time).
constexpr uint32_t kDefaultPolls = 1024;


// Workspace of the fused form: a header, the ticket counters, then two
// regions of equal size.  A region holds the published tile maps (P, Q), then
// the published inclusive states H (3 words per entry for a real scan, 6 for
// a complex one).  A launch uses region `phase`, which is all-ones wherever it
// will write, and clears the words the previous launch dirtied in the other
// region (the header records how many, per region), so back-to-back launches
// on one stream (or replays of a captured graph) need no separate
// initialisation step.
//
// Tickets.  Same-address atomics serialise (about 11.5 ns each on MI355X: one
// counter for 2560 workgroups costs 30 us), so tickets come from nC counters,
// nC a divisor of the number of series nS.  Counter c hands out local indices
// i = 0, 1, ... in arrival order, and the tile is t = i*nC + c, taken in the
// chain-major order k = t / nS, s = t % nS.  Because nC divides nS, every
// predecessor t - j*nS of a tile comes from the same counter with a smaller
// index, so it was taken by a workgroup that is already running: the chain
// always drains.  Workgroups are spread over counters so that each counter is
// fed from all XCDs and the counters advance together, which keeps the rows
// in flight close to each other (this matters for DRAM locality).
//
// A counter is one 64-bit word: the launches it has served (its epoch) in
// the high half, the tickets taken in the current launch in the low half, so
// the one atomic increment that takes a ticket also says which region this
// launch uses (the epoch's parity).  The taker of a counter's last ticket
// moves it to the next epoch with its count back at zero, and also moves on
// the counters this launch leaves unused, so that every counter's epoch
// counts every launch on the workspace.  (Reading a separate phase word
// before the increment cost a second round trip, about 1 us of the 2 us a
// tile spent getting its ticket.)
struct Header {
    unsigned long long dirty[2];  // words the last launch using each region wrote there
    uint32_t pad[60];
};
static_assert(sizeof(Header) == 256, "header size");

constexpr int kCtrStride = 16;  // 64-bit words between ticket counters (one 128-byte line each)
constexpr int kMaxCounters = 64;
constexpr int kHeaderBytes = (int)sizeof(Header) + kMaxCounters * kCtrStride * 8;

struct Scratch {
    Header* hdr;
    unsigned long long* ctr;       // kMaxCounters counters, kCtrStride words apart
    uint32_t* region[2];
    unsigned long long entries;    // NK * nS * W published entries
    uint32_t words;                // 32-bit words each entry publishes (map + state)
    uint32_t total_tiles;
    uint32_t nC;                   // ticket counters (divides nS)
    uint32_t quota;                // tickets per counter = total_tiles / nC
};

// ---------------------------------------------------------------------------
// tile configuration
//
// TPR threads (16-byte vectors) cover one row of a tile: W = TPR*V lanes,
// TPR*16 contiguous bytes per row.  A wavefront holds RG = 64/TPR row groups,
// each thread NR consecutive rows; a workgroup of WAVES wavefronts covers
// CT = WAVES*RG*NR rows.  LB is the look-back window.
// ---------------------------------------------------------------------------
template <int DT_, int TPR_, int NR_, int WAVES_, int LB_>
struct Cfg {
    static constexpr int DT = DT_, TPR = TPR_, NR = NR_, WAVES = WAVES_, LB = LB_;
    static constexpr int V = Elem<DT>::V;
    static constexpr int EB = Elem<DT>::bytes;
    static constexpr int RG = kWave / TPR;
    static constexpr int W = TPR * V;
    static constexpr int NT = WAVES * kWave;
    static constexpr int CT = WAVES * RG * NR;
    static constexpr int EW = 1;  // predecessors the look-back reads early (measured: 1 beats 2 and 4)
    static_assert(TPR == 8 || TPR == 16 || TPR == 32, "row width");
    static_assert(W <= NT, "one look-back column per thread");
    // waves per SIMD the register budget is held to (the forward keeps two
    // input arrays of NR rows in registers through the look-back, the
    // backward three)
    static constexpr int OCC_F = NR <= 8 ? 3 : 2;
    static constexpr int OCC_B = NR <= 4 ? (TPR > 8 ? 4 : 3) : (NR <= 8 && TPR > 8 ? 3 : 2);
};

struct Dims {
    int T, D, nW, nS, NK;
};

// One thread's view of its tile.
struct Geo {
    int k, s, bi, dcol0, d0, trow0, row0;
    int nvalid;     // lanes of this thread's vector that exist (0..V)
    int nrows;      // rows of this thread's segment that exist (0..NR)
    size_t tbase;   // byte offset of (batch bi, row trow0, lane dcol0)
    uint32_t coff;  // this thread's byte offset inside a row
};

template <class C, bool REV>
__device__ __forceinline__ Geo tile_geo(uint32_t ticket, const Dims& d, int wave, int rg, int cg) {
    Geo g;
    const int kk = (int)(ticket / (uint32_t)d.nS);
    g.s = (int)ticket - kk * d.nS;
    g.k = REV ? d.NK - 1 - kk : kk;
    g.bi = g.s / d.nW;
    g.dcol0 = (g.s - g.bi * d.nW) * C::W;
    g.d0 = g.dcol0 + cg * C::V;
    g.nvalid = g.d0 >= d.D ? 0 : ((d.D - g.d0) < C::V ? (d.D - g.d0) : C::V);
    g.trow0 = g.k * C::CT;
    g.row0 = g.trow0 + (wave * C::RG + rg) * C::NR;
    const int left = d.T - g.row0;
    g.nrows = g.nvalid == 0 ? 0 : (left <= 0 ? 0 : (left < C::NR ? left : C::NR));
    g.tbase = (((size_t)g.bi * d.T + g.trow0) * d.D + g.dcol0) * C::EB;
    // lanes past D read a valid column (their values are never used)
    g.coff = (uint32_t)((g.nvalid > 0 ? cg * C::V : 0) * C::EB);
    return g;
}

// Byte offset, from the tile base, of row `row` of this thread's column,
// clamped to a row that exists (rows past T are read but never used).
__device__ __forceinline__ uint32_t row_off(const Geo& g, int row, int T, uint32_t rowbytes) {
    const int rc = row < T ? row : T - 1;
    return (uint32_t)(rc - g.trow0) * rowbytes + g.coff;
}

// Segment-start byte of row i of this thread's segment (rows past T read the
// last row; their steps are identity steps anyway).
__device__ __forceinline__ uint32_t reset_byte(const uint8_t* reset, const Geo& g, int i, int T) {
    const int row = g.row0 + i;
    const int rc = row < T ? row : T - 1;
    return reset[(size_t)g.bi * T + rc];
}

// Ticket, phase and the number of words to clear, read once per workgroup.
struct Ticket {
    uint32_t ticket, phase;
    unsigned long long nclear;
};

// Thread 0: the ticket, the region of this launch and the number of words to
// clear, in one round trip (the header's two counts are read beside the
// increment and the one for the other region kept).
__device__ __forceinline__ Ticket take_ticket(const Scratch& sc) {
    __shared__ Ticket s_t;
    if (threadIdx.x == 0) {
        const uint32_t b = blockIdx.x;
        const uint32_t c = (b % sc.nC + b / sc.nC) % sc.nC;  // a permutation within each row of nC
        const unsigned long long d0 = peek_u64(&sc.hdr->dirty[0]);
        const unsigned long long d1 = peek_u64(&sc.hdr->dirty[1]);
        unsigned long long* w = sc.ctr + (size_t)c * kCtrStride;
        const unsigned long long v = atomicAdd(w, 1ull);
        const uint32_t i = (uint32_t)v;
        const uint32_t p = (uint32_t)(v >> 32) & 1u;
        s_t.phase = p;
        s_t.ticket = i * sc.nC + c;
        s_t.nclear = p ? d0 : d1;
        if (i == sc.quota - 1) {
            // the counter's last ticket of this launch: next epoch, count 0;
            // the same for the counters this launch leaves unused
            atomicAdd(w, (1ull << 32) - sc.quota);
            for (uint32_t u = c + sc.nC; u < (uint32_t)kMaxCounters; u += sc.nC)
                atomicAdd(sc.ctr + (size_t)u * kCtrStride, 1ull << 32);
        }
        if (i == 0 && c == 0)
            publish_u64(&sc.hdr->dirty[p], (unsigned long long)sc.words * sc.entries);
    }
    __syncthreads();
    Ticket t;
    t.ticket = uniform(s_t.ticket);
    t.phase = uniform(s_t.phase);
    t.nclear = (unsigned long long)uniform64((int64_t)s_t.nclear);
    return t;
}

// Restore the all-ones state of this ticket's share of the words the
// previous launch wrote in the region this launch does not use.
__device__ __forceinline__ void clear_share(const Scratch& sc, uint32_t phase,
                                            unsigned long long nclear, int nthreads, uint32_t ticket) {
    uint32_t* other = sc.region[phase ^ 1u];
    const unsigned long long stride = (unsigned long long)sc.total_tiles * nthreads;
    for (unsigned long long i = (unsigned long long)ticket * nthreads + threadIdx.x; i < nclear;
         i += stride)
        other[i] = kEmpty;
}

// Largest `v` over the active lanes of the wavefront (wave-uniform result).
__device__ __forceinline__ int wave_max_active(int v) {
    unsigned long long act = __ballot(1);
    int r = 0;
    while (act) {
        const int lane = __builtin_ctzll(act);
        const int u = __shfl(v, lane, kWave);
        r = u > r ? u : r;
        act &= act - 1;
    }
    return uniform(r);
}

// One reading of N predecessors' words (index 0 the nearest), `rem` of which
// exist before the chain start: the depth of the nearest published state (its
// value in *base) or of the chain start (base0), N + 1 when every map of the
// window is published and neither lies within it, or -1 when a map is missing
// first.
template <class Link, int N>
__device__ __forceinline__ int scan_window(const typename Link::HRaw (&hw)[N],
                                           const typename Link::MRaw (&mw)[N], int rem,
                                           typename Link::S base0, typename Link::S* base) {
    int depth = -1;
    bool stop = false;
    *base = base0;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        if (depth < 0 && !stop) {
            if (i >= rem) {
                depth = i;  // reached the start of the chain
            } else if (Link::ready_h(hw[i])) {
                depth = i;
                *base = Link::state(hw[i]);
            } else if (!Link::ready_m(mw[i])) {
                stop = true;
            }
        }
    }
    if (depth < 0 && !stop) depth = rem == N ? N : N + 1;  // chain start just past the window
    return depth;
}

// Carry from one reading of the N nearest predecessors' words (index 0 the
// nearest): the nearest published inclusive state, with the maps of the tiles
// in between applied to it oldest first, or the chain start when it lies
// within reach and every map up to it is published.  False if the reading
// does not decide the carry yet.
template <class Link, int N>
__device__ __forceinline__ bool resolve_window(const typename Link::HRaw (&hw)[N],
                                               const typename Link::MRaw (&mw)[N], int span,
                                               typename Link::S base0, typename Link::S* out) {
    using S = typename Link::S;
    S base;
    const int depth = scan_window<Link, N>(hw, mw, span, base0, &base);
    if (depth < 0 || depth > N) return false;
    S x = base;
#pragma unroll
    for (int i = N - 1; i >= 0; --i)
        if (i < depth) x = Link::apply(Link::map(mw[i]), x);
    *out = x;
    return true;
}

// An early reading of the N nearest predecessors' words, taken while the
// tile's own summary is still being combined, so that the look-back can
// often finish without a further round trip.
template <class Link, int N>
struct EarlyWindow {
    typename Link::HRaw hw[N];
    typename Link::MRaw mw[N];
    template <int DIR>
    __device__ __forceinline__ void take(const Link& lk, int k, int NK) {
        const int span = DIR < 0 ? k : (NK - 1 - k);
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const bool have = i < span;
            hw[i] = have ? lk.load_h(k + DIR * (1 + i)) : Link::empty_h();
            mw[i] = have ? lk.load_m(k + DIR * (1 + i)) : Link::empty_m();
        }
    }
    template <int DIR>
    __device__ __forceinline__ bool resolve(int k, int NK, typename Link::S base0,
                                            typename Link::S* out) const {
        const int span = DIR < 0 ? k : (NK - 1 - k);
        if (span == 0) {
            *out = base0;
            return true;
        }
        return resolve_window<Link, N>(hw, mw, span, base0, out);
    }
};

// Carry entering tile k of a chain (forward: DIR = -1 looks at k-1, k-2, ...;
// reverse: DIR = +1 looks at k+1, k+2, ...).  `base0` is the carry entering the
// chain (h0 forward, grad_last reverse).  The nearest published inclusive
// state within a window of LB predecessors is taken and the maps of the tiles
// in between are applied to it oldest first, so the result is the plain
// chained value.
//
// The window is polled up to `polls` times.  After that the tile stops
// waiting: it finds the nearest published state at any distance, and derives
// every map in between that is not yet published itself, with `map_of(j)`,
// from the inputs and bitwise equal to what tile j publishes.  So no tile
// ever waits on a workgroup that has not started, whatever order the
// hardware starts workgroups in, and results do not depend on which path
// was taken.
//
// `Link` reads one lane's published words of chunk j (load_h / load_m, each
// a single atomic load per word), says whether they are published
// (ready_h / ready_m), decodes them (state / map) and applies a map to a
// state; it fixes the value types (real or complex).
template <class Link, int DIR, int LB, class MapOf>
__device__ typename Link::S look_back(const Link& lk, int k, int NK, typename Link::S base0,
                                      uint32_t polls, MapOf&& map_of) {
    using S = typename Link::S;
    using M = typename Link::M;
    const int span = DIR < 0 ? k : (NK - 1 - k);  // predecessors in the chain
    if (span == 0) return base0;
    auto chunk = [&](int i) { return k + DIR * (1 + i); };  // predecessor i (0: the nearest)
    for (uint32_t spin = 0; spin < polls; ++spin) {
        typename Link::HRaw hw[LB];
        typename Link::MRaw mw[LB];
#pragma unroll
        for (int i = 0; i < LB; ++i) {
            if (i < span) {
                hw[i] = lk.load_h(chunk(i));
                mw[i] = lk.load_m(chunk(i));
            } else {
                hw[i] = Link::empty_h();
                mw[i] = Link::empty_m();
            }
        }
        S x;
        if (resolve_window<Link, LB>(hw, mw, span, base0, &x)) return x;
        __builtin_amdgcn_s_sleep(1);
    }
    // nearest published state at any distance (or the chain start) ...
    int m = span;
    S base = base0;
    for (int i0 = 0; i0 < span && m == span; i0 += LB) {
        typename Link::HRaw hw[LB];
#pragma unroll
        for (int i = 0; i < LB; ++i)
            hw[i] = i0 + i < span ? lk.load_h(chunk(i0 + i)) : Link::empty_h();
#pragma unroll
        for (int i = 0; i < LB; ++i) {
            if (m == span && Link::ready_h(hw[i])) {
                m = i0 + i;
                base = Link::state(hw[i]);
            }
        }
    }
    // ... then the m maps in between, oldest first, published or derived.
    // The walk is wave-uniform, so a map that some lane has to derive is
    // derived for the same tile in every lane at once (each for its own lane
    // of the block), with wave-uniform row addresses.
    S x = base;
    const int m_max = wave_max_active(m);
#pragma unroll 1
    for (int i = m_max - 1; i >= 0; --i) {
        const bool mine = i < m;
        const typename Link::MRaw w = mine ? lk.load_m(chunk(i)) : Link::empty_m();
        const bool need = mine && !Link::ready_m(w);
        M a = Link::map(w);
        if (__any(need)) {
            const M dm = map_of(chunk(i));
            if (need) a = dm;
        }
        if (mine) x = Link::apply(a, x);
    }
    return x;
}

// First level of a tile's fold, per wavefront and lane, right after the
// wavefront has written its segments' maps to s_seg: the wavefront's RG
// segments are folded in order (REV: from the last), each replaced by the
// composition of the wavefront's segments before it (an exclusive prefix),
// and the total goes to s_wav.  All wavefronts do this at once; the
// look-back wavefront then folds only the WAVES totals, which shortens the
// serial fold before a tile's map is published from WAVES*RG steps to
// RG + WAVES.  Lane c of a row is folded by lane c % 64 of the wavefront
// (W / 64 lanes each, or one by each of the first W lanes when W < 64).
// Then::then(e, l) is the composition "l after e".
template <class C, bool REV, class Then, class M>
__device__ __forceinline__ void fold_wave_segments(M (&s_seg)[C::WAVES * C::RG][C::W],
                                                   M (&s_wav)[C::WAVES][C::W], int wave, int l,
                                                   M identity) {
    constexpr int RG = C::RG, W = C::W;
    // the wavefront's own writes above, visible to all of its lanes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int q = 0; q < (W + kWave - 1) / kWave; ++q) {
        const int c = q * kWave + l;
        if (W < kWave && c >= W) break;
        M A = identity;
#pragma unroll
        for (int r0 = 0; r0 < RG; ++r0) {
            const int r = REV ? RG - 1 - r0 : r0;
            const M t = s_seg[wave * RG + r][c];
            s_seg[wave * RG + r][c] = A;
            A = Then::then(A, t);
        }
        s_wav[wave][c] = A;
    }
}

// Workspace initialisation: header and counters zero (nothing dirty, epoch
// 0, no tickets taken) and both regions all-ones.
__global__ void scratch_init_kernel(uint32_t* __restrict__ p, size_t words) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = i < (size_t)kHeaderBytes / 4 ? 0u : kEmpty;
}

struct Layout {
    int nW, nS, NK, W;
    unsigned long long entries;
};

Layout layout_of(const Shape& s, int width, int tile) {
    Layout L;
    L.W = width * (s.dtype == DT_F32 ? Elem<DT_F32>::V : Elem<DT_BF16>::V);
    L.nW = (int)((s.D + L.W - 1) / L.W);
    L.nS = (int)(s.B * L.nW);
    L.NK = (int)((s.T + tile - 1) / tile);
    L.entries = (unsigned long long)L.NK * L.nS * L.W;
    return L;
}

// A launch of one workgroup of `nt` threads per tile stays within the 32-bit
// count of work-items of a grid dimension.
bool grid_fits(const Layout& L, int nt) {
    return (unsigned long long)L.NK * (unsigned long long)L.nS * (unsigned long long)nt <
           (1ull << 32);
}

// Ticket counters: the largest power of two up to kMaxCounters dividing nS.
int counters_of(const Layout& L) {
    int c = 1;
    while (c < kMaxCounters && L.nS % (2 * c) == 0) c *= 2;
    return c;
}

// Bytes of one region for `words` 32-bit words per published entry.
size_t region_bytes_for(const Layout& L, int words) {
    return ((unsigned long long)words * L.entries * 4 + 255) / 256 * 256;
}

// Region size implied by a workspace size (the same for every call on one buffer).
size_t region_bytes_of(size_t ws_bytes) {
    return ws_bytes < (size_t)kHeaderBytes ? 0 : (ws_bytes - kHeaderBytes) / 2 / 256 * 256;
}

hipError_t prepare(void* ws, size_t ws_bytes, bool init, const Layout& L, int words,
                   hipStream_t st, Scratch* sc) {
    const size_t rb = region_bytes_of(ws_bytes);
    if (rb < region_bytes_for(L, words)) return hipErrorInvalidValue;
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
    sc->ctr = reinterpret_cast<unsigned long long*>(base + sizeof(Header));
    sc->region[0] = reinterpret_cast<uint32_t*>(base + kHeaderBytes);
    sc->region[1] = reinterpret_cast<uint32_t*>(base + kHeaderBytes + rb);
    sc->entries = L.entries;
    sc->words = (uint32_t)words;
    sc->total_tiles = (uint32_t)((unsigned long long)L.NK * L.nS);
    sc->nC = (uint32_t)counters_of(L);
    sc->quota = sc->total_tiles / sc->nC;
    return hipSuccess;
}

}  // namespace

}  // namespace lrscan
