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
//  * Summary: each thread folds its NR rows (its segment) into one affine
//    map per lane and writes it to LDS.  One wavefront then folds the
//    segments of each lane in order, giving the tile's map (P, Q) per lane,
//    and leaves in LDS, in place of each segment's map, the composition of
//    the segments before it (an exclusive prefix).  (Folding in LDS rather
//    than scanning across the lanes of a wavefront keeps the registers free
//    for the tile itself.)
//  * Prefix: tiles of one lane block form a chain.  Tiles take tickets from
//    an atomic counter in chain order (all tiles of chunk k before any tile of
//    chunk k+1), publish (P, Q) as soon as the summary is done, then look back
//    over up to LB predecessors for the nearest published inclusive state H
//    and apply the predecessors' maps to it, oldest first, before publishing
//    their own H.  This is the decoupled look-back of Merrill & Garland
//    ("Single-pass Parallel Prefix Scan with Decoupled Look-back", 2016),
//    made deterministic: every H equals the plain chained value
//    H_k = fma(P_k, H_{k-1}, Q_k) whatever the timing, so results do not
//    depend on scheduling.  The nearest predecessor's words are read once
//    already before the summary barrier (as soon as the tile's own rows have
//    arrived), so a tile whose predecessor has published by then needs no
//    further round trip.  A tile only waits on tiles with smaller tickets,
//    which are already resident or finished, so the chain always drains; and
//    a tile that has polled long enough derives the maps it is missing from
//    the inputs itself (bitwise the values their owners publish), so no wait
//    is unbounded and no result depends on which path was taken.
//  * Replay: each thread applies its segment's exclusive prefix to the
//    carry entering the tile, then rescans its rows from registers and
//    writes the outputs once.
//
// Published words are single 32- or 64-bit device-scope atomic stores;
// every word starts as the all-ones pattern, which no published value takes,
// so readers need no separate flag or fence.  The reverse-time kernel is the
// mirror image: tickets run from the last chunk to the first and carries flow
// from later rows to earlier ones.
#include "fused_common.hpp"

namespace lrscan {

namespace {

__device__ __forceinline__ unsigned long long pack_aff(Aff m) {
    return (unsigned long long)publishable(m.p) | ((unsigned long long)publishable(m.q) << 32);
}
__device__ __forceinline__ Aff unpack_aff(unsigned long long w) {
    return Aff{__uint_as_float((uint32_t)w), __uint_as_float((uint32_t)(w >> 32))};
}

// A real entry: (P, Q) in one 64-bit word, H in one 32-bit word.
struct RealLink {
    using S = float;
    using M = Aff;
    using HRaw = uint32_t;
    using MRaw = unsigned long long;
    const uint32_t* hs;
    const unsigned long long* pqs;
    int nS, s, W, c;
    __device__ size_t entry(int j) const { return ((size_t)j * (size_t)nS + (size_t)s) * W + c; }
    __device__ HRaw load_h(int j) const { return peek_u32(hs + entry(j)); }
    __device__ MRaw load_m(int j) const { return peek_u64(pqs + entry(j)); }
    __device__ static HRaw empty_h() { return kEmpty; }
    __device__ static MRaw empty_m() { return ~0ull; }
    __device__ static bool ready_h(HRaw w) { return w != kEmpty; }
    __device__ static bool ready_m(MRaw w) { return (uint32_t)w != kEmpty; }
    __device__ static S state(HRaw w) { return __uint_as_float(w); }
    __device__ static M map(MRaw w) { return unpack_aff(w); }
    __device__ static S apply(M m, S x) { return aff_apply(m, x); }
};

// Words per published entry: (P, Q) and H.
constexpr int kRealWords = 3;

struct AffThen {
    __device__ static Aff then(Aff earlier, Aff later) { return aff_then(earlier, later); }
};

struct FwdArgs {
    const void* a;
    const void* b;
    void* out;
    float* last;
    const float* h0;
    const uint8_t* reset;  // [B, T] segment starts, or NULL
    Scratch sc;
    Dims d;
    uint32_t polls;
};

struct BwdArgs {
    const void* a;
    const void* out;
    const void* g;
    const float* grad_last;
    const float* h0;
    const uint8_t* reset;  // [B, T] segment starts, or NULL
    void* grad_a;
    void* grad_b;
    float* grad_h0;
    Scratch sc;
    Dims d;
    uint32_t polls;
};

// Map of tile j of series (bi, lane block) for lane `col`, derived from the
// inputs in exactly the order the workgroup owning tile j computes it: each
// segment of NR rows folded from the identity, then the segments folded in
// order.  Lanes past D are the identity.
template <class C>
__device__ Aff fwd_tile_map(const FwdArgs& x, int j, int bi, int col) {
    constexpr int NR = C::NR, RG = C::RG, SEGS = C::WAVES * C::RG;
    Aff A = aff_identity(), Wv = aff_identity();
    if (col >= x.d.D) return A;
    // wave-uniform row addresses, one 32-bit lane offset
    const size_t rowbytes = (size_t)x.d.D * C::EB;
    const char* a0 = static_cast<const char*>(x.a) + (size_t)bi * x.d.T * rowbytes;
    const char* b0 = static_cast<const char*>(x.b) + (size_t)bi * x.d.T * rowbytes;
    const uint32_t coff = (uint32_t)col * C::EB;
#pragma unroll 1
    for (int sg = 0; sg < SEGS; ++sg) {
        Aff t = aff_identity();
        const int r0 = j * C::CT + sg * NR;
#pragma unroll 1
        for (int i = 0; i < NR; ++i) {
            const int r = r0 + i;
            float at = 1.0f, bt = 0.0f;
            if (r < x.d.T) {
                const size_t ro = (size_t)uniform64((int64_t)r * (int64_t)rowbytes);  // same tile in every lane
                at = Elem<C::DT>::load1(a0 + ro + coff, 0);
                bt = Elem<C::DT>::load1(b0 + ro + coff, 0);
                if (x.reset && x.reset[(size_t)bi * x.d.T + r]) at = 0.0f;
            }
            t.p = at * t.p;
            t.q = fmaf(at, t.q, bt);
        }
        Wv = aff_then(Wv, t);
        if (sg % RG == RG - 1) {  // a wavefront's segments, then the wavefronts in order
            A = aff_then(A, Wv);
            Wv = aff_identity();
        }
    }
    return unpack_aff(pack_aff(A));
}

// Reverse-time counterpart: rows in decreasing order, segments from the last
// to the first.
template <class C>
__device__ Aff bwd_tile_map(const BwdArgs& x, int j, int bi, int col) {
    constexpr int NR = C::NR, RG = C::RG, SEGS = C::WAVES * C::RG;
    Aff A = aff_identity(), Wv = aff_identity();
    if (col >= x.d.D) return A;
    const size_t rowbytes = (size_t)x.d.D * C::EB;
    const char* a0 = static_cast<const char*>(x.a) + (size_t)bi * x.d.T * rowbytes;
    const char* g0 = static_cast<const char*>(x.g) + (size_t)bi * x.d.T * rowbytes;
    const uint32_t coff = (uint32_t)col * C::EB;
#pragma unroll 1
    for (int sg = SEGS - 1; sg >= 0; --sg) {
        Aff t = aff_identity();
        const int r0 = j * C::CT + sg * NR;
#pragma unroll 1
        for (int i = NR - 1; i >= 0; --i) {
            const int r = r0 + i;
            float at = 1.0f, gt = 0.0f;
            if (r < x.d.T) {
                const size_t ro = (size_t)uniform64((int64_t)r * (int64_t)rowbytes);  // same tile in every lane
                at = Elem<C::DT>::load1(a0 + ro + coff, 0);
                gt = Elem<C::DT>::load1(g0 + ro + coff, 0);
                if (x.reset && x.reset[(size_t)bi * x.d.T + r]) at = 0.0f;
            }
            t.p = at * t.p;
            t.q = at * (t.q + gt);
        }
        Wv = aff_then(Wv, t);
        if (sg % RG == 0) {  // a wavefront's segments (last first), then the wavefronts
            A = aff_then(A, Wv);
            Wv = aff_identity();
        }
    }
    return unpack_aff(pack_aff(A));
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
// OUT = false: state-only forward (no `out`): only the thread holding row T-1
// of a lane replays, to write `last` exactly as the full forward does.
template <class C, bool ALIGNED, bool RST, bool OUT>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::OCC_F)))
void fused_fwd_kernel(FwdArgs x) {
    constexpr int V = C::V, W = C::W, RG = C::RG, NR = C::NR, TPR = C::TPR;
    constexpr int SEGS = C::WAVES * RG;
    __shared__ Aff s_seg[SEGS][W];  // each segment's map, then its wavefront's maps before it composed
    __shared__ Aff s_wav[C::WAVES][W];  // each wavefront's map, then the wavefronts' before it composed
    __shared__ float s_hin[W];      // the state entering the tile, per lane

    const Dims d = x.d;
    const int tid = threadIdx.x;
    const int wave = uniform((int)(threadIdx.x / kWave));
    const int l = tid % kWave;
    const int rg = l / TPR;
    const int cg = l % TPR;
    const Ticket tk = take_ticket(x.sc);
    const Geo g = tile_geo<C, false>(tk.ticket, d, wave, rg, cg);
    const uint32_t rowbytes = (uint32_t)d.D * C::EB;
    const char* pa = static_cast<const char*>(x.a) + g.tbase;
    const char* pb = static_cast<const char*>(x.b) + g.tbase;
    char* po = static_cast<char*>(x.out) + g.tbase;

    // every load is issued before any is used; rows past T and lanes past D
    // are read from valid addresses and replaced by identity steps below
    uint32_t rs[NR];
    if constexpr (RST) {
#pragma unroll
        for (int i = 0; i < NR; ++i) rs[i] = reset_byte(x.reset, g, i, d.T);
    }
    RowVec<C::DT> ra[NR], rb[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const uint32_t off = row_off(g, g.row0 + i, d.T, rowbytes);
        ra[i] = load_vec<C::DT, ALIGNED, false>(pa, off, g.nvalid, 1.0f);
        rb[i] = load_vec<C::DT, ALIGNED, true>(pb, off, g.nvalid, 0.0f);
    }
    if constexpr (RST) {
        // a segment start drops the entering state: its transition becomes 0
#pragma unroll
        for (int i = 0; i < NR; ++i)
            if (rs[i]) ra[i] = RowVec<C::DT>::splat(0.0f);
    }
    // rows past T (and every row of a thread whose lanes lie past D) become
    // identity steps, once per row here rather than per element in the
    // summary; a tile whose rows and lanes all exist (wave-uniform, and every
    // tile when T and D are multiples of the tile) skips this
    const bool full = g.trow0 + C::CT <= d.T && g.dcol0 + W <= d.D;
    if (!full) {
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            if (i >= g.nrows) {
                ra[i] = RowVec<C::DT>::splat(1.0f);
                rb[i] = RowVec<C::DT>::splat(0.0f);
            }
        }
    }

    // summary of this thread's rows, per lane (rows outer, so only one row
    // is widened to fp32 at a time), then the wavefront scan over its RG
    // row groups
    Aff m[V];
#pragma unroll
    for (int j = 0; j < V; ++j) m[j] = aff_identity();
#pragma unroll
    for (int i = 0; i < NR; ++i) {
#pragma unroll
        for (int j = 0; j < V; ++j) {
            const float at = ra[i].get(j);
            m[j].p = at * m[j].p;
            m[j].q = fmaf(at, m[j].q, rb[i].get(j));
        }
    }
    const int seg = wave * RG + rg;
#pragma unroll
    for (int j = 0; j < V; ++j) s_seg[seg][cg * V + j] = m[j];
    fold_wave_segments<C, false, AffThen>(s_seg, s_wav, wave, l, aff_identity());
    const uint32_t phase = tk.phase;
    const unsigned long long* pqs =
        reinterpret_cast<const unsigned long long*>(x.sc.region[phase]);
    const uint32_t* hs = x.sc.region[phase] + 2 * x.sc.entries;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        opaque(ra[i]);
        opaque(rb[i]);
    }
    // early reading of the look-back window, issued once this thread's rows
    // have arrived (the summary above consumed them)
    EarlyWindow<RealLink, C::EW> early;
    if (tid < W) {
        int z = 0;
#pragma unroll
        for (int j = 0; j < V; ++j) z += zero_after(m[j].q);
        early.template take<-1>(RealLink{hs, pqs, d.nS, g.s, W, tid + z}, g.k, d.NK);
    }
    __syncthreads();

    // exclusive prefixes and tile map, publication, look-back: one lane per thread
    if (tid < W) {
        const int c = tid;
        Aff A = aff_identity();
#pragma unroll
        for (int w = 0; w < C::WAVES; ++w) {
            const Aff t = s_wav[w][c];
            s_wav[w][c] = A;
            A = aff_then(A, t);
        }
        const size_t o = ((size_t)g.k * (size_t)d.nS + (size_t)g.s) * W + c;
        const bool more = g.k + 1 < d.NK;
        if (more) publish_u64(const_cast<unsigned long long*>(pqs) + o, pack_aff(A));
        const int dl = g.dcol0 + c;
        const float base0 = (x.h0 && dl < d.D) ? x.h0[(size_t)g.bi * d.D + dl] : 0.0f;
        const RealLink lk{hs, pqs, d.nS, g.s, W, c};
        float hin;
        if (!early.template resolve<-1>(g.k, d.NK, base0, &hin))
            hin = look_back<RealLink, -1, C::LB>(
                lk, g.k, d.NK, base0, x.polls, [&](int j) { return fwd_tile_map<C>(x, j, g.bi, dl); });
        if (more) publish_u32(const_cast<uint32_t*>(hs) + o, publishable(aff_apply(A, hin)));
        s_hin[c] = hin;
    }
    __syncthreads();
    // this tile's share of clearing the other region (here, not before the
    // summary: a loop of stores there would make the summary wait for every load)
    clear_share(x.sc, tk.phase, tk.nclear, C::NT, tk.ticket);

    const bool ends = g.nrows > 0 && g.row0 + g.nrows == d.T;  // holds row T-1
    if constexpr (!OUT) {
        if (!(x.last && ends)) return;
    }

    // replay from registers
    float h[V];
#pragma unroll
    for (int j = 0; j < V; ++j)
        h[j] = aff_apply(s_seg[seg][cg * V + j], aff_apply(s_wav[wave][cg * V + j], s_hin[cg * V + j]));
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        if (full || i < g.nrows) {
            RowOut<C::DT> o;
#pragma unroll
            for (int j = 0; j < V; ++j) {
                h[j] = fmaf(ra[i].get(j), h[j], rb[i].get(j));
                o.v[j] = h[j];
            }
            if constexpr (OUT)
                store_vec<C::DT, ALIGNED>(po, row_off(g, g.row0 + i, d.T, rowbytes), g.nvalid, o);
        }
    }
    if (x.last && ends) {
#pragma unroll
        for (int j = 0; j < V; ++j)
            if (j < g.nvalid) x.last[(size_t)g.bi * d.D + g.d0 + j] = h[j];
    }
}

// ---------------------------------------------------------------------------
// reverse time (backward)
// ---------------------------------------------------------------------------
template <class C, bool ALIGNED, bool RST>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::OCC_B)))
void fused_bwd_kernel(BwdArgs x) {
    constexpr int V = C::V, W = C::W, RG = C::RG, NR = C::NR, TPR = C::TPR;
    constexpr int SEGS = C::WAVES * RG;
    __shared__ Aff s_seg[SEGS][W];  // each segment's reverse map, then its wavefront's maps after it composed
    __shared__ Aff s_wav[C::WAVES][W];  // each wavefront's reverse map, then the wavefronts' after it composed
    __shared__ float s_cin[W];      // the carry entering the tile from the right, per lane

    const Dims d = x.d;
    const int tid = threadIdx.x;
    const int wave = uniform((int)(threadIdx.x / kWave));
    const int l = tid % kWave;
    const int rg = l / TPR;
    const int cg = l % TPR;
    const Ticket tk = take_ticket(x.sc);
    const Geo g = tile_geo<C, true>(tk.ticket, d, wave, rg, cg);
    const uint32_t rowbytes = (uint32_t)d.D * C::EB;
    const char* pa = static_cast<const char*>(x.a) + g.tbase;
    const char* pg = static_cast<const char*>(x.g) + g.tbase;
    // h_{t-1} lives in row t-1 of `out`: its offsets count from the row the
    // tile's reads of `out` start at (one before the tile, or row 0)
    const int hrow0 = g.trow0 > 0 ? g.trow0 - 1 : 0;
    const char* ph = static_cast<const char*>(x.out) + g.tbase - (size_t)(g.trow0 - hrow0) * rowbytes;
    char* pga = static_cast<char*>(x.grad_a) + g.tbase;
    char* pgb = static_cast<char*>(x.grad_b) + g.tbase;

    uint32_t rs[NR];
    if constexpr (RST) {
#pragma unroll
        for (int i = 0; i < NR; ++i) rs[i] = reset_byte(x.reset, g, i, d.T);
    }
    // a and grad_out first, last row first (the order the reverse summary
    // uses them), then `out`: the summary and the look-back proceed while the
    // rows of `out` (used only by the replay) arrive.  The scheduling
    // barriers keep the compiler from reordering or sinking the loads.
    RowVec<C::DT> ra[NR], rg_[NR], rh[NR];
#pragma unroll
    for (int i = NR - 1; i >= 0; --i) {
        const uint32_t off = row_off(g, g.row0 + i, d.T, rowbytes);
        ra[i] = load_vec<C::DT, ALIGNED, true>(pa, off, g.nvalid, 1.0f);
        rg_[i] = load_vec<C::DT, ALIGNED, true>(pg, off, g.nvalid, 0.0f);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const int row = g.row0 + i;
        const int rc = row < d.T ? row : d.T - 1;
        const int hr = rc >= 1 ? rc - 1 : 0;
        const uint32_t hoff = (uint32_t)(hr - hrow0) * rowbytes + g.coff;
        rh[i] = load_vec<C::DT, ALIGNED, true>(ph, hoff, g.nvalid, 0.0f);
    }
    __builtin_amdgcn_sched_barrier(0);
    // at a segment start a_t is not used: its transition is 0 (no adjoint
    // crosses it) and grad_a_t = 0 (the previous state is taken as 0)
    uint32_t rbits = 0;
    if constexpr (RST) {
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            if (rs[i]) {
                ra[i] = RowVec<C::DT>::splat(0.0f);
                rh[i] = RowVec<C::DT>::splat(0.0f);
                rbits |= 1u << i;
            }
        }
    }
    // rows past T (and every row of a thread whose lanes lie past D) become
    // identity steps (wave-uniform skip for a tile whose rows and lanes all exist)
    const bool full = g.trow0 + C::CT <= d.T && g.dcol0 + W <= d.D;
    if (!full) {
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            if (i >= g.nrows) {
                ra[i] = RowVec<C::DT>::splat(1.0f);
                rg_[i] = RowVec<C::DT>::splat(0.0f);
            }
        }
    }

    // reverse summary: the map from the carry entering the segment on the
    // right to the carry a_s*lambda_s leaving its first row s
    Aff m[V];
#pragma unroll
    for (int j = 0; j < V; ++j) m[j] = aff_identity();
#pragma unroll
    for (int i = NR - 1; i >= 0; --i) {
#pragma unroll
        for (int j = 0; j < V; ++j) {
            const float at = ra[i].get(j);
            m[j].p = at * m[j].p;
            m[j].q = at * (m[j].q + rg_[i].get(j));
        }
    }
    const int seg = wave * RG + rg;
#pragma unroll
    for (int j = 0; j < V; ++j) s_seg[seg][cg * V + j] = m[j];
    fold_wave_segments<C, true, AffThen>(s_seg, s_wav, wave, l, aff_identity());
    const uint32_t phase = tk.phase;
    const unsigned long long* pqs =
        reinterpret_cast<const unsigned long long*>(x.sc.region[phase]);
    const uint32_t* hs = x.sc.region[phase] + 2 * x.sc.entries;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        opaque(ra[i]);
        opaque(rg_[i]);
    }
    EarlyWindow<RealLink, C::EW> early;
    if (tid < W) {
        int z = 0;
#pragma unroll
        for (int j = 0; j < V; ++j) z += zero_after(m[j].q);
        early.template take<+1>(RealLink{hs, pqs, d.nS, g.s, W, tid + z}, g.k, d.NK);
    }
    __syncthreads();

    if (tid < W) {
        const int c = tid;
        Aff A = aff_identity();
#pragma unroll
        for (int w = C::WAVES - 1; w >= 0; --w) {
            const Aff t = s_wav[w][c];
            s_wav[w][c] = A;
            A = aff_then(A, t);
        }
        const size_t o = ((size_t)g.k * (size_t)d.nS + (size_t)g.s) * W + c;
        const bool more = g.k > 0;
        if (more) publish_u64(const_cast<unsigned long long*>(pqs) + o, pack_aff(A));
        const int dl = g.dcol0 + c;
        const float base0 = (x.grad_last && dl < d.D) ? x.grad_last[(size_t)g.bi * d.D + dl] : 0.0f;
        const RealLink lk{hs, pqs, d.nS, g.s, W, c};
        float cin;
        if (!early.template resolve<+1>(g.k, d.NK, base0, &cin))
            cin = look_back<RealLink, +1, C::LB>(
                lk, g.k, d.NK, base0, x.polls, [&](int j) { return bwd_tile_map<C>(x, j, g.bi, dl); });
        if (more) publish_u32(const_cast<uint32_t*>(hs) + o, publishable(aff_apply(A, cin)));
        s_cin[c] = cin;
    }
    __syncthreads();
    // this tile's share of clearing the other region (here, not before the
    // summary: a loop of stores there would make the summary wait for every load)
    clear_share(x.sc, tk.phase, tk.nclear, C::NT, tk.ticket);

    // lam[j] starts as the carry a_{s+1}*lambda_{s+1} entering this thread's
    // last row from the right; each row then takes
    // lambda_t = g_t + a_{t+1}*lambda_{t+1} as one fma with the a of the row
    // after it (the carry itself for the first row processed)
    float lam[V];
#pragma unroll
    for (int j = 0; j < V; ++j)
        lam[j] = aff_apply(s_seg[seg][cg * V + j], aff_apply(s_wav[wave][cg * V + j], s_cin[cg * V + j]));
#pragma unroll
    for (int i = NR - 1; i >= 0; --i) {
        if (full || i < g.nrows) {
            const int row = g.row0 + i;
            const bool after = i + 1 < NR && (full || i + 1 < g.nrows);  // row t+1 is in this segment
            RowOut<C::DT> oa, ob;
#pragma unroll
            for (int j = 0; j < V; ++j) {
                const float an = (i + 1 < NR && after) ? ra[i + 1 < NR ? i + 1 : i].get(j) : 1.0f;
                lam[j] = fmaf(an, lam[j], rg_[i].get(j));
                float hp = rh[i].get(j);
                if (i == 0 && g.row0 == 0 && !((rbits >> i) & 1u))  // row 0: h0, or 0
                    hp = (x.h0 && j < g.nvalid) ? x.h0[(size_t)g.bi * d.D + g.d0 + j] : 0.0f;
                ob.v[j] = lam[j];
                oa.v[j] = lam[j] * hp;
            }
            const uint32_t off = row_off(g, row, d.T, rowbytes);
            store_vec<C::DT, ALIGNED>(pga, off, g.nvalid, oa);
            store_vec<C::DT, ALIGNED>(pgb, off, g.nvalid, ob);
        }
    }
    if (x.grad_h0 && g.nrows > 0 && g.row0 == 0) {
#pragma unroll
        for (int j = 0; j < V; ++j)
            if (j < g.nvalid) x.grad_h0[(size_t)g.bi * d.D + g.d0 + j] = ra[0].get(j) * lam[j];
    }
}

// ---------------------------------------------------------------------------
// host side: configurations, layout, launch
// ---------------------------------------------------------------------------
// (width = threads per row, tile = rows per tile) -> kernel parameters
struct TileCfg {
    int width, tile, nr, waves, lb;
};
constexpr TileCfg kFwdCfgs[] = {
    {8, 256, 8, 4, 8}, {8, 512, 16, 4, 8}, {16, 128, 8, 4, 4},
    {16, 256, 16, 4, 4}, {32, 32, 4, 4, 4}, {32, 64, 8, 4, 4}, {32, 128, 16, 4, 4},
};
constexpr TileCfg kBwdCfgs[] = {
    {8, 256, 8, 4, 8}, {8, 128, 4, 4, 8}, {16, 128, 8, 4, 4},
    {32, 64, 8, 4, 4}, {32, 32, 4, 4, 4},
};

const TileCfg* find_cfg(int dir, int width, int tile) {
    if (dir == 0) {
        for (const auto& c : kFwdCfgs)
            if (c.width == width && c.tile == tile) return &c;
    } else {
        for (const auto& c : kBwdCfgs)
            if (c.width == width && c.tile == tile) return &c;
    }
    return nullptr;
}

template <int DT, int TPR, int NR, int WAVES, int LB, bool AL>
void launch_fwd_cfg(const FwdArgs& x0, hipStream_t st) {
    using C = Cfg<DT, TPR, NR, WAVES, LB>;
    const dim3 grid(x0.sc.total_tiles), block(C::NT);
    if (x0.out) {
        if (x0.reset) hipLaunchKernelGGL((fused_fwd_kernel<C, AL, true, true>), grid, block, 0, st, x0);
        else hipLaunchKernelGGL((fused_fwd_kernel<C, AL, false, true>), grid, block, 0, st, x0);
    } else {
        if (x0.reset) hipLaunchKernelGGL((fused_fwd_kernel<C, AL, true, false>), grid, block, 0, st, x0);
        else hipLaunchKernelGGL((fused_fwd_kernel<C, AL, false, false>), grid, block, 0, st, x0);
    }
}

template <int DT, int TPR, int NR, int WAVES, int LB, bool AL>
void launch_bwd_cfg(const BwdArgs& x, hipStream_t st) {
    using C = Cfg<DT, TPR, NR, WAVES, LB>;
    if (x.reset)
        hipLaunchKernelGGL((fused_bwd_kernel<C, AL, true>), dim3(x.sc.total_tiles), dim3(C::NT), 0, st, x);
    else
        hipLaunchKernelGGL((fused_bwd_kernel<C, AL, false>), dim3(x.sc.total_tiles), dim3(C::NT), 0, st, x);
}

// Unaligned rows (D * elem_bytes not a multiple of 16, or unaligned pointers)
// use 16-byte accesses at element-aligned addresses, in the shapes
// unaligned_cfg accepts.
template <int DT>
bool fwd_dispatch(const TileCfg& c, bool al, const FwdArgs& x, hipStream_t st) {
    if (!al) {
        if (c.width == 8 && c.tile == 256) launch_fwd_cfg<DT, 8, 8, 4, 8, false>(x, st);
        else if (c.width == 16 && c.tile == 128) launch_fwd_cfg<DT, 16, 8, 4, 4, false>(x, st);
        else if (c.width == 32 && c.tile == 64) launch_fwd_cfg<DT, 32, 8, 4, 4, false>(x, st);
        else return false;
        return true;
    }
    if (c.width == 8 && c.tile == 256) launch_fwd_cfg<DT, 8, 8, 4, 8, true>(x, st);
    else if (c.width == 8 && c.tile == 512) launch_fwd_cfg<DT, 8, 16, 4, 8, true>(x, st);
    else if (c.width == 16 && c.tile == 128) launch_fwd_cfg<DT, 16, 8, 4, 4, true>(x, st);
    else if (c.width == 16 && c.tile == 256) launch_fwd_cfg<DT, 16, 16, 4, 4, true>(x, st);
    else if (c.width == 32 && c.tile == 32) launch_fwd_cfg<DT, 32, 4, 4, 4, true>(x, st);
    else if (c.width == 32 && c.tile == 64) launch_fwd_cfg<DT, 32, 8, 4, 4, true>(x, st);
    else if (c.width == 32 && c.tile == 128) launch_fwd_cfg<DT, 32, 16, 4, 4, true>(x, st);
    else return false;
    return true;
}

template <int DT>
bool bwd_dispatch(const TileCfg& c, bool al, const BwdArgs& x, hipStream_t st) {
    if (!al) {
        if (c.width == 8 && c.tile == 256) launch_bwd_cfg<DT, 8, 8, 4, 8, false>(x, st);
        else if (c.width == 8 && c.tile == 128) launch_bwd_cfg<DT, 8, 4, 4, 8, false>(x, st);
        else if (c.width == 16 && c.tile == 128) launch_bwd_cfg<DT, 16, 8, 4, 4, false>(x, st);
        else if (c.width == 32 && c.tile == 64) launch_bwd_cfg<DT, 32, 8, 4, 4, false>(x, st);
        else return false;
        return true;
    }
    // At most eight chains: a look-back window of 16 tiles.  The backward
    // holds two waves per SIMD at either window, and with few chains the
    // walk back over published tiles is the critical path (measured: one
    // to four chains 16-25% faster, eight 2%, sixteen or more unchanged).
    if (c.width == 8 && c.tile == 256 && x.d.nS <= 8) launch_bwd_cfg<DT, 8, 8, 4, 16, true>(x, st);
    else if (c.width == 8 && c.tile == 256) launch_bwd_cfg<DT, 8, 8, 4, 8, true>(x, st);
    else if (c.width == 8 && c.tile == 128) launch_bwd_cfg<DT, 8, 4, 4, 8, true>(x, st);
    else if (c.width == 16 && c.tile == 128) launch_bwd_cfg<DT, 16, 8, 4, 4, true>(x, st);
    else if (c.width == 32 && c.tile == 64) launch_bwd_cfg<DT, 32, 8, 4, 4, true>(x, st);
    else if (c.width == 32 && c.tile == 32) launch_bwd_cfg<DT, 32, 4, 4, 4, true>(x, st);
    else return false;
    return true;
}

// Tile shapes for rows that are not 16-byte aligned: 128-byte rows x 256 (x
// 128 backward), 256-byte rows x 128 and 512-byte rows x 64.
bool unaligned_cfg(int dir, int width, int tile) {
    return (width == 8 && tile == 256) || (width == 16 && tile == 128) ||
           (width == 32 && tile == 64) || (dir == 1 && width == 8 && tile == 128);
}

}  // namespace

bool fused_cfg_supported(const Shape& s, int dir, int width, int tile, bool aligned) {
    if (!find_cfg(dir, width, tile)) return false;
    if (!aligned && !unaligned_cfg(dir, width, tile)) return false;
    // 32-bit row offsets inside a tile, 32-bit lane and row indices, 32-bit tickets
    const int64_t eb = s.dtype == DT_F32 ? 4 : 2;
    if ((int64_t)(tile + 1) * s.D * eb >= ((int64_t)1 << 31)) return false;
    if (s.T >= ((int64_t)1 << 31) - tile || s.D >= ((int64_t)1 << 30)) return false;
    const Layout L = layout_of(s, width, tile);
    if ((unsigned long long)L.NK * L.nS >= 0xffffffffull) return false;
    if (!grid_fits(L, find_cfg(dir, width, tile)->waves * kWave)) return false;
    if (s.B * (int64_t)L.nW >= ((int64_t)1 << 31)) return false;
    return true;
}

// Default tile shape, from measurements on MI355X (kernel time with the caches
// flushed before each launch; [B,T,D] bf16 and fp32 from [8,2048,2560] and
// [16,4096,2560] to [1,131072,1024], and short sequences T = 8 .. 1024 at
// about 340M elements).  A tile should not be much taller than the sequence:
// its rows past T are idle threads.
//
// Forward: 32 rows of 512-byte lane blocks for T <= 32 ([4150,32,2560] bf16
// 5.5 against 4.7 TB/s at 64 rows and 1.7 at 256); 64 rows of them for bf16
// T <= 64; 128 rows of 256-byte blocks for T <= 128 (bf16 T = 128: 6.0
// against 4.9 TB/s at 64 rows of 512 bytes) and for fp32 T <= 64 ([1038,64,
// 2560]: 6.0 against 5.9); else 128-byte blocks: 512 rows for 256 < T <= 512,
// so that a chain is one tile with no look-back and no mostly idle second
// tile ([461,288,2560] bf16 5.1 against 4.5 TB/s at 256 rows, T = 512 5.6
// against 5.5), 512 rows also when there are fewer than 64 chains of
// 128-byte lane blocks and T >= 4096, where consecutive tiles of a chain
// start so close together that each waits on its predecessor ([1,131072,
// 1024]: 152.4 -> 147.7 us), else 256 rows.
//
// Backward: 32 rows of 512-byte blocks for T <= 32, 64 rows for T <= 64, 128
// rows of 128-byte blocks for T <= 128, else 256 rows of 128-byte blocks (T
// of 256..512 over many lane blocks: 5.8 against 5.2 TB/s).  128 rows of
// 256-byte blocks are within 3% of it either way on [8,2048,2560] and
// [16,4096,2560] bf16 (which one leads changes from one GPU to another), but
// 20% slower on [16,2048,4096] and 5-8% on [8,2048,8192], [32,2048,2048]
// and [64,1024,1024] (13% faster only on [16,4096,2048]).
//
// Rows that are not 16-byte aligned: 64 rows of 512-byte blocks for T <= 64
// (bf16 [692,64,2559] 3.7 / 3.7 TB/s, against 2.6 / 2.7 at 128 rows of
// 256-byte blocks); otherwise 128 rows of 256-byte blocks when there
// are at least 128 chains of them (fewer shared 128-byte lines between tiles:
// bf16 [8,2048,2559] 2.8 / 2.9 -> 3.2 / 3.4 TB/s forward / backward), for
// fp32 64 rows of 512-byte blocks ([2,4096,4097] 3.1 / 3.2 -> 3.8 / 4.2,
// against 3.4 / 4.0 at 256 bytes; bf16 is 4-6% slower at 512 bytes), else
// 256 rows of 128-byte blocks (few chains: [1,131072,1023] bf16 3.1 / 3.1
// against 2.2 / 3.0 at 256 bytes).
//
// A lane block wider than the row (D smaller than the block) would leave
// lanes idle, so the widths fall back to narrower rows.
void fused_default_cfg(const Shape& s, int dir, bool aligned, int* width, int* tile) {
    *width = 8;
    *tile = 256;
    const int64_t row_bytes = s.D * (s.dtype == DT_F32 ? 4 : 2);
    const auto fits = [&](int w) { return row_bytes >= (int64_t)w * 16; };
    if (!aligned) {
        if (s.T <= 64 && fits(32)) {
            *width = 32;
            *tile = 64;
        } else if (fits(16) && s.B * ((row_bytes + 255) / 256) >= 128) {
            const bool w32 = s.dtype == DT_F32 && fits(32);
            *width = w32 ? 32 : 16;
            *tile = w32 ? 64 : 128;
        }
        return;
    }
    if (dir == 0) {
        if (s.T <= 32 && fits(32)) {
            *width = 32;
            *tile = 32;
        } else if (s.T <= 64 && s.dtype == DT_BF16 && fits(32)) {
            *width = 32;
            *tile = 64;
        } else if (s.T <= 128 && fits(16)) {
            *width = 16;
            *tile = 128;
        } else {
            const int64_t lanes8 = 8 * (s.dtype == DT_F32 ? Elem<DT_F32>::V : Elem<DT_BF16>::V);
            const int64_t chains8 = s.B * ((s.D + lanes8 - 1) / lanes8);
            if ((s.T > 256 && s.T <= 512) || (s.T >= 8 * 512 && chains8 < 64)) *tile = 512;
        }
        return;
    }
    if (s.T <= 32 && fits(32)) {
        *width = 32;
        *tile = 32;
    } else if (s.T <= 64 && fits(32)) {
        *width = 32;
        *tile = 64;
    } else if (s.T <= 128) {
        *tile = 128;
    }
}

size_t fused_workspace_bytes(const Shape& s, int width, int tile) {
    return kHeaderBytes + 2 * region_bytes_for(layout_of(s, width, tile), kRealWords);
}

hipError_t launch_fused_fwd(const Shape& s, int width, int tile, const void* a, const void* b,
                            void* out, float* last, const float* h0, const uint8_t* reset,
                            void* ws, size_t ws_bytes, bool init, int polls, hipStream_t st) {
    const TileCfg* c = find_cfg(0, width, tile);
    if (!c) return hipErrorInvalidValue;
    const Layout L = layout_of(s, width, tile);
    FwdArgs x;
    hipError_t e = prepare(ws, ws_bytes, init, L, kRealWords, st, &x.sc);
    if (e != hipSuccess) return e;
    x.a = a;
    x.b = b;
    x.out = out;
    x.last = last;
    x.h0 = h0;
    x.reset = reset;
    x.d = Dims{(int)s.T, (int)s.D, L.nW, L.nS, L.NK};
    x.polls = polls > 0 ? (uint32_t)polls : kDefaultPolls;
    const void* ptrs[3] = {a, b, out};
    const bool al = rows_aligned(s, ptrs, 3);
    const bool ok = s.dtype == DT_F32 ? fwd_dispatch<DT_F32>(*c, al, x, st)
                                      : fwd_dispatch<DT_BF16>(*c, al, x, st);
    if (!ok) return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_fused_bwd(const Shape& s, int width, int tile, const void* a, const void* out,
                            const void* g, const float* grad_last, const float* h0,
                            const uint8_t* reset, void* grad_a, void* grad_b, float* grad_h0,
                            void* ws, size_t ws_bytes, bool init, int polls, hipStream_t st) {
    const TileCfg* c = find_cfg(1, width, tile);
    if (!c) return hipErrorInvalidValue;
    const Layout L = layout_of(s, width, tile);
    BwdArgs x;
    hipError_t e = prepare(ws, ws_bytes, init, L, kRealWords, st, &x.sc);
    if (e != hipSuccess) return e;
    x.a = a;
    x.out = out;
    x.g = g;
    x.grad_last = grad_last;
    x.h0 = h0;
    x.reset = reset;
    x.grad_a = grad_a;
    x.grad_b = grad_b;
    x.grad_h0 = grad_h0;
    x.d = Dims{(int)s.T, (int)s.D, L.nW, L.nS, L.NK};
    x.polls = polls > 0 ? (uint32_t)polls : kDefaultPolls;
    const void* ptrs[5] = {a, out, g, grad_a, grad_b};
    const bool al = rows_aligned(s, ptrs, 5);
    const bool ok = s.dtype == DT_F32 ? bwd_dispatch<DT_F32>(*c, al, x, st)
                                      : bwd_dispatch<DT_BF16>(*c, al, x, st);
    if (!ok) return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace lrscan
