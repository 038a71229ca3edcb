// complex.hip -- the complex diagonal scan  h_t = a_t * h_{t-1} + b_t  with
// complex a, b, h (page "triton_training_scan.py": _complex_forward,
// _complex_backward and _ComplexScan), forward and reverse time.
//
// Storage is planar, as on the page: the real and imaginary parts of a, b,
// out and of every gradient are separate [B, T, M] arrays of one storage
// type; states (h0, last, grad_last, grad_h0) are pairs of fp32 [B, M]
// arrays.  The adjoint is that of the real loss
//   L = sum Re(conj(g_t) h_t) + Re(conj(g_last) h_{T-1}),
// with gradients written as dL/dRe + i dL/dIm:
//   lambda_t = g_t + conj(a_{t+1}) lambda_{t+1},  grad_b = lambda,
//   grad_a_t = lambda_t conj(h_{t-1}),  grad_h0 = conj(a_0) lambda_0.
//
// Two forms:
//  * the per-lane walk (one thread owns 16 bytes of each array, i.e. V
//    complex lanes, and walks all T steps);
//  * the single-launch tiled form of fused.hip with complex affine maps
//    (P, Q complex): tickets, summary (segment maps folded in LDS by one
//    wavefront, which leaves each segment's exclusive prefix), deterministic
//    look-back with bounded waiting, replay from registers.  A published
//    entry is three 64-bit words (P, Q and the inclusive state H, each a
//    (re, im) pair).
// All complex products are spelled out with explicit fmas, identically on
// every path that must agree bit for bit.
#include <type_traits>

#include "complex_math.hpp"

namespace lrscan {

namespace {

// ---------------------------------------------------------------------------
// arguments and derived tile maps (the look-back's derivation path)
// ---------------------------------------------------------------------------
struct CxFwdArgs {
    CxFwdPtrs p;
    Scratch sc;
    Dims d;
    uint32_t polls;
};
struct CxBwdArgs {
    CxBwdPtrs p;
    Scratch sc;
    Dims d;
    uint32_t polls;
};


// Map of tile j of series (bi, lane block) for lane `col`, derived from the
// inputs in the owning workgroup's exact operation order: each segment of NR
// rows folded from the identity, then the segments folded in order.
template <class C>
__device__ CAff cx_fwd_tile_map(const CxFwdArgs& x, int j, int bi, int col) {
    constexpr int NR = C::NR, SEGS = C::WAVES * C::RG;
    CAff A = caff_identity(), Wv = caff_identity();
    if (col >= x.d.D) return A;
    const size_t rowbytes = (size_t)x.d.D * C::EB;
    const size_t b0 = (size_t)bi * x.d.T * rowbytes;
    const char* ar = static_cast<const char*>(x.p.ar) + b0;
    const char* ai = static_cast<const char*>(x.p.ai) + b0;
    const char* br = static_cast<const char*>(x.p.br) + b0;
    const char* bim = static_cast<const char*>(x.p.bi) + b0;
    const uint32_t coff = (uint32_t)col * C::EB;
#pragma unroll 1
    for (int sg = 0; sg < SEGS; ++sg) {
        CAff t = caff_identity();
        const int r0 = j * C::CT + sg * NR;
#pragma unroll 1
        for (int i = 0; i < NR; ++i) {
            const int r = r0 + i;
            Cx at{1.0f, 0.0f}, bt{0.0f, 0.0f};
            if (r < x.d.T) {
                const size_t ro = (size_t)uniform64((int64_t)r * (int64_t)rowbytes) + coff;
                at = load_cx<C::DT>(ar, ai, ro);
                bt = load_cx<C::DT>(br, bim, ro);
                if (x.p.reset && x.p.reset[(size_t)bi * x.d.T + r]) at = Cx{0.0f, 0.0f};
            }
            t = caff_then(t, fwd_step(at, bt));
        }
        Wv = caff_then(Wv, t);
        if (sg % C::RG == C::RG - 1) {  // a wavefront's segments, then the wavefronts in order
            A = caff_then(A, Wv);
            Wv = caff_identity();
        }
    }
    return CAff{unpack_cx(pack_cx(A.p)), unpack_cx(pack_cx(A.q))};
}

// Reverse-time counterpart: rows in decreasing order, segments from the last
// to the first.
template <class C>
__device__ CAff cx_bwd_tile_map(const CxBwdArgs& x, int j, int bi, int col) {
    constexpr int NR = C::NR, SEGS = C::WAVES * C::RG;
    CAff A = caff_identity();
    if (col >= x.d.D) return A;
    const size_t rowbytes = (size_t)x.d.D * C::EB;
    const size_t b0 = (size_t)bi * x.d.T * rowbytes;
    const char* ar = static_cast<const char*>(x.p.ar) + b0;
    const char* ai = static_cast<const char*>(x.p.ai) + b0;
    const char* gr = static_cast<const char*>(x.p.gr) + b0;
    const char* gi = static_cast<const char*>(x.p.gi) + b0;
    const uint32_t coff = (uint32_t)col * C::EB;
#pragma unroll 1
    for (int sg = SEGS - 1; sg >= 0; --sg) {
        CAff t = caff_identity();
        const int r0 = j * C::CT + sg * NR;
#pragma unroll 1
        for (int i = NR - 1; i >= 0; --i) {
            const int r = r0 + i;
            Cx at{1.0f, 0.0f}, gt{0.0f, 0.0f};
            if (r < x.d.T) {
                const size_t ro = (size_t)uniform64((int64_t)r * (int64_t)rowbytes) + coff;
                at = load_cx<C::DT>(ar, ai, ro);
                gt = load_cx<C::DT>(gr, gi, ro);
                if (x.p.reset && x.p.reset[(size_t)bi * x.d.T + r]) at = Cx{0.0f, 0.0f};
            }
            t = rev_fold(t, at, gt);
        }
        A = caff_then(A, t);
    }
    return CAff{unpack_cx(pack_cx(A.p)), unpack_cx(pack_cx(A.q))};
}


// ---------------------------------------------------------------------------
// forward, tiled single launch
// ---------------------------------------------------------------------------
template <class C, bool ALIGNED, bool RST, bool OUT>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(2)))
void cx_fused_fwd_kernel(CxFwdArgs x) {
    constexpr int V = C::V, W = C::W, RG = C::RG, NR = C::NR, TPR = C::TPR;
    constexpr int SEGS = C::WAVES * RG;
    __shared__ CAff s_seg[SEGS][W];  // each segment's map, then its wavefront's maps before it composed
    __shared__ CAff s_wav[C::WAVES][W];  // each wavefront's map, then the wavefronts' before it composed
    __shared__ Cx s_hin[W];          // the state entering the tile, per lane

    const Dims d = x.d;
    const int tid = threadIdx.x;
    const int wave = uniform((int)(threadIdx.x / kWave));
    const int l = tid % kWave;
    const int rg = l / TPR;
    const int cg = l % TPR;
    const int seg = wave * RG + rg;
    const Ticket tk = take_ticket(x.sc);
    const Geo g = tile_geo<C, false>(tk.ticket, d, wave, rg, cg);
    const uint32_t rowbytes = (uint32_t)d.D * C::EB;
    const char* par = static_cast<const char*>(x.p.ar) + g.tbase;
    const char* pai = static_cast<const char*>(x.p.ai) + g.tbase;
    const char* pbr = static_cast<const char*>(x.p.br) + g.tbase;
    const char* pbi = static_cast<const char*>(x.p.bi) + g.tbase;

    uint32_t rs[NR];
    if constexpr (RST) {
#pragma unroll
        for (int i = 0; i < NR; ++i) rs[i] = reset_byte(x.p.reset, g, i, d.T);
    }
    RowVec<C::DT> ar[NR], ai[NR], br[NR], bi[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const uint32_t off = row_off(g, g.row0 + i, d.T, rowbytes);
        ar[i] = load_vec<C::DT, ALIGNED>(par, off, g.nvalid, 1.0f);
        ai[i] = load_vec<C::DT, ALIGNED>(pai, off, g.nvalid, 0.0f);
        br[i] = load_vec<C::DT, ALIGNED, true>(pbr, off, g.nvalid, 0.0f);
        bi[i] = load_vec<C::DT, ALIGNED, true>(pbi, off, g.nvalid, 0.0f);
    }
    if constexpr (RST) {
#pragma unroll
        for (int i = 0; i < NR; ++i)
            if (rs[i]) {
                ar[i] = RowVec<C::DT>::splat(0.0f);
                ai[i] = RowVec<C::DT>::splat(0.0f);
            }
    }
    // rows past T (and every row of a thread whose lanes lie past D) become
    // identity steps, once here (skipped by a tile whose rows and lanes all exist)
    const bool full = g.trow0 + C::CT <= d.T && g.dcol0 + W <= d.D;
    if (!full) {
#pragma unroll
        for (int i = 0; i < NR; ++i)
            if (i >= g.nrows) {
                ar[i] = RowVec<C::DT>::splat(1.0f);
                ai[i] = RowVec<C::DT>::splat(0.0f);
                br[i] = RowVec<C::DT>::splat(0.0f);
                bi[i] = RowVec<C::DT>::splat(0.0f);
            }
    }

    // summary of this thread's rows per lane, into LDS
#pragma unroll
    for (int j = 0; j < V; ++j) {
        CAff m = caff_identity();
#pragma unroll
        for (int i = 0; i < NR; ++i) m = caff_then(m, fwd_step(vget(ar[i], ai[i], j), vget(br[i], bi[i], j)));
        s_seg[seg][cg * V + j] = m;
    }
    fold_wave_segments<C, false, CAffThen>(s_seg, s_wav, seg / C::RG, (int)threadIdx.x % kWave,
                                           caff_identity());
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        opaque(ar[i]);
        opaque(ai[i]);
        opaque(br[i]);
        opaque(bi[i]);
    }
    // early reading of the look-back window, issued once this thread's last
    // row has arrived
    EarlyWindow<ComplexLink, C::EW> early;
    if (tid < W) {
        const CxWords we = cx_words(x.sc, tk.phase);
        const int z = zero_after_row(bi[NR - 1]);
        early.template take<-1>(ComplexLink{we.ps, we.qs, we.hs, d.nS, g.s, W, tid + z}, g.k, d.NK);
    }
    __syncthreads();

    // exclusive prefixes and tile map, publication, look-back: one lane per thread
    if (tid < W) {
        const int c = tid;
        const CxWords wd = cx_words(x.sc, tk.phase);
        CAff A = caff_identity();
#pragma unroll
        for (int w = 0; w < C::WAVES; ++w) {
            const CAff t = s_wav[w][c];
            s_wav[w][c] = A;
            A = caff_then(A, t);
        }
        const size_t o = ((size_t)g.k * (size_t)d.nS + (size_t)g.s) * W + c;
        const bool more = g.k + 1 < d.NK;
        if (more) {
            publish_u64(wd.ps + o, pack_cx(A.p));
            publish_u64(wd.qs + o, pack_cx(A.q));
        }
        const int dl = g.dcol0 + c;
        Cx base0{0.0f, 0.0f};
        if (x.p.h0r && dl < d.D)
            base0 = Cx{x.p.h0r[(size_t)g.bi * d.D + dl], x.p.h0i[(size_t)g.bi * d.D + dl]};
        const ComplexLink lk{wd.ps, wd.qs, wd.hs, d.nS, g.s, W, c};
        Cx hin;
        if (!early.template resolve<-1>(g.k, d.NK, base0, &hin))
            hin = look_back<ComplexLink, -1, C::LB>(
                lk, g.k, d.NK, base0, x.polls, [&](int j) { return cx_fwd_tile_map<C>(x, j, g.bi, dl); });
        if (more) publish_u64(wd.hs + o, pack_cx(caff_apply(A, hin)));
        s_hin[c] = hin;
    }
    __syncthreads();
    // this tile's share of clearing the other region (here, not before the
    // summary: a loop of stores there would make the summary wait for every load)
    clear_share(x.sc, tk.phase, tk.nclear, C::NT, tk.ticket);

    const bool ends = g.nrows > 0 && g.row0 + g.nrows == d.T;
    if constexpr (!OUT) {
        if (!(x.p.last_r && ends)) return;
    }
    char* por = static_cast<char*>(x.p.out_r) + g.tbase;
    char* poi = static_cast<char*>(x.p.out_i) + g.tbase;
    Cx h[V];
#pragma unroll
    for (int j = 0; j < V; ++j) h[j] = caff_apply(s_seg[seg][cg * V + j],
                          caff_apply(s_wav[seg / C::RG][cg * V + j], s_hin[cg * V + j]));
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        if (full || i < g.nrows) {
            RowOut<C::DT> orr, oii;
#pragma unroll
            for (int j = 0; j < V; ++j) {
                h[j] = cfma(vget(ar[i], ai[i], j), h[j], vget(br[i], bi[i], j));
                orr.v[j] = h[j].r;
                oii.v[j] = h[j].i;
            }
            if constexpr (OUT) {
                const uint32_t off = row_off(g, g.row0 + i, d.T, rowbytes);
                store_vec<C::DT, ALIGNED>(por, off, g.nvalid, orr);
                store_vec<C::DT, ALIGNED>(poi, off, g.nvalid, oii);
            }
        }
    }
    if (x.p.last_r && ends) {
#pragma unroll
        for (int j = 0; j < V; ++j)
            if (j < g.nvalid) {
                x.p.last_r[(size_t)g.bi * d.D + g.d0 + j] = h[j].r;
                x.p.last_i[(size_t)g.bi * d.D + g.d0 + j] = h[j].i;
            }
    }
}

// ---------------------------------------------------------------------------
// reverse time, tiled single launch
// ---------------------------------------------------------------------------
template <class C, bool ALIGNED, bool RST>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(3)))
void cx_fused_bwd_kernel(CxBwdArgs x) {
    constexpr int V = C::V, W = C::W, RG = C::RG, NR = C::NR, TPR = C::TPR;
    constexpr int SEGS = C::WAVES * RG;
    __shared__ CAff s_seg[SEGS][W];  // each segment's reverse map, then the maps after it composed
    __shared__ Cx s_cin[W];          // the carry entering the tile from the right, per lane

    const Dims d = x.d;
    const int tid = threadIdx.x;
    const int wave = uniform((int)(threadIdx.x / kWave));
    const int l = tid % kWave;
    const int rg = l / TPR;
    const int cg = l % TPR;
    const int seg = wave * RG + rg;
    const Ticket tk = take_ticket(x.sc);
    const Geo g = tile_geo<C, true>(tk.ticket, d, wave, rg, cg);
    const uint32_t rowbytes = (uint32_t)d.D * C::EB;
    const char* par = static_cast<const char*>(x.p.ar) + g.tbase;
    const char* pai = static_cast<const char*>(x.p.ai) + g.tbase;
    const char* pgr = static_cast<const char*>(x.p.gr) + g.tbase;
    const char* pgi = static_cast<const char*>(x.p.gi) + g.tbase;
    // h_{t-1} lives in row t-1 of out: offsets count from the row the tile's
    // reads of out start at (one before the tile, or row 0)
    const int hrow0 = g.trow0 > 0 ? g.trow0 - 1 : 0;
    const size_t hback = (size_t)(g.trow0 - hrow0) * rowbytes;
    const char* phr = static_cast<const char*>(x.p.hr) + g.tbase - hback;
    const char* phi = static_cast<const char*>(x.p.hi) + g.tbase - hback;

    uint32_t rs[NR];
    if constexpr (RST) {
#pragma unroll
        for (int i = 0; i < NR; ++i) rs[i] = reset_byte(x.p.reset, g, i, d.T);
    }
    RowVec<C::DT> ar[NR], ai[NR], gr[NR], gi[NR], hr[NR], hi[NR];
#pragma unroll
    for (int i = NR - 1; i >= 0; --i) {  // last row first: the reverse summary's order
        const uint32_t off = row_off(g, g.row0 + i, d.T, rowbytes);
        ar[i] = load_vec<C::DT, ALIGNED, true>(par, off, g.nvalid, 1.0f);
        ai[i] = load_vec<C::DT, ALIGNED, true>(pai, off, g.nvalid, 0.0f);
        gr[i] = load_vec<C::DT, ALIGNED, true>(pgr, off, g.nvalid, 0.0f);
        gi[i] = load_vec<C::DT, ALIGNED, true>(pgi, off, g.nvalid, 0.0f);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the load order as written
    // the rows of `out` last: only the replay uses them
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const int row = g.row0 + i;
        const int rc = row < d.T ? row : d.T - 1;
        const int hrw = rc >= 1 ? rc - 1 : 0;
        const uint32_t hoff = (uint32_t)(hrw - hrow0) * rowbytes + g.coff;
        hr[i] = load_vec<C::DT, ALIGNED, true>(phr, hoff, g.nvalid, 0.0f);
        hi[i] = load_vec<C::DT, ALIGNED, true>(phi, hoff, g.nvalid, 0.0f);
    }
    __builtin_amdgcn_sched_barrier(0);
    // at a segment start a_t is not used: transition 0, grad_a_t = 0
    uint32_t rbits = 0;
    if constexpr (RST) {
#pragma unroll
        for (int i = 0; i < NR; ++i)
            if (rs[i]) {
                ar[i] = RowVec<C::DT>::splat(0.0f);
                ai[i] = RowVec<C::DT>::splat(0.0f);
                hr[i] = RowVec<C::DT>::splat(0.0f);
                hi[i] = RowVec<C::DT>::splat(0.0f);
                rbits |= 1u << i;
            }
    }
    // rows past T (and every row of a thread whose lanes lie past D) become
    // identity steps (skipped by a tile whose rows and lanes all exist)
    const bool full = g.trow0 + C::CT <= d.T && g.dcol0 + W <= d.D;
    if (!full) {
#pragma unroll
        for (int i = 0; i < NR; ++i)
            if (i >= g.nrows) {
                ar[i] = RowVec<C::DT>::splat(1.0f);
                ai[i] = RowVec<C::DT>::splat(0.0f);
                gr[i] = RowVec<C::DT>::splat(0.0f);
                gi[i] = RowVec<C::DT>::splat(0.0f);
            }
    }

    // reverse summary, into LDS: the map from the carry entering on the right
    // to the carry conj(a_s) lambda_s leaving the segment's first row s
#pragma unroll
    for (int j = 0; j < V; ++j) {
        CAff m = caff_identity();
#pragma unroll
        for (int i = NR - 1; i >= 0; --i) m = rev_fold(m, vget(ar[i], ai[i], j), vget(gr[i], gi[i], j));
        s_seg[seg][cg * V + j] = m;
    }
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        opaque(ar[i]);
        opaque(ai[i]);
        opaque(gr[i]);
        opaque(gi[i]);
    }
    // early reading of the look-back window, issued once this thread's last
    // row has arrived
    EarlyWindow<ComplexLink, C::EW> early;
    if (tid < W) {
        const CxWords we = cx_words(x.sc, tk.phase);
        const int z = zero_after_row(gi[NR - 1]);
        early.template take<+1>(ComplexLink{we.ps, we.qs, we.hs, d.nS, g.s, W, tid + z}, g.k, d.NK);
    }
    __syncthreads();

    if (tid < W) {
        const int c = tid;
        const CxWords wd = cx_words(x.sc, tk.phase);
        CAff A = caff_identity();
#pragma unroll 4
        for (int sg = SEGS - 1; sg >= 0; --sg) {
            const CAff t = s_seg[sg][c];
            s_seg[sg][c] = A;
            A = caff_then(A, t);
        }
        const size_t o = ((size_t)g.k * (size_t)d.nS + (size_t)g.s) * W + c;
        const bool more = g.k > 0;
        if (more) {
            publish_u64(wd.ps + o, pack_cx(A.p));
            publish_u64(wd.qs + o, pack_cx(A.q));
        }
        const int dl = g.dcol0 + c;
        Cx base0{0.0f, 0.0f};
        if (x.p.glr && dl < d.D)
            base0 = Cx{x.p.glr[(size_t)g.bi * d.D + dl], x.p.gli[(size_t)g.bi * d.D + dl]};
        const ComplexLink lk{wd.ps, wd.qs, wd.hs, d.nS, g.s, W, c};
        Cx cin;
        if (!early.template resolve<+1>(g.k, d.NK, base0, &cin))
            cin = look_back<ComplexLink, +1, C::LB>(
                lk, g.k, d.NK, base0, x.polls, [&](int j) { return cx_bwd_tile_map<C>(x, j, g.bi, dl); });
        if (more) publish_u64(wd.hs + o, pack_cx(caff_apply(A, cin)));
        s_cin[c] = cin;
    }
    __syncthreads();
    // this tile's share of clearing the other region (here, not before the
    // summary: a loop of stores there would make the summary wait for every load)
    clear_share(x.sc, tk.phase, tk.nclear, C::NT, tk.ticket);

    char* pgar = static_cast<char*>(x.p.gar) + g.tbase;
    char* pgai = static_cast<char*>(x.p.gai) + g.tbase;
    char* pgbr = static_cast<char*>(x.p.gbr) + g.tbase;
    char* pgbi = static_cast<char*>(x.p.gbi) + g.tbase;
    Cx carry[V];
#pragma unroll
    for (int j = 0; j < V; ++j) carry[j] = caff_apply(s_seg[seg][cg * V + j], s_cin[cg * V + j]);
#pragma unroll
    for (int i = NR - 1; i >= 0; --i) {
        if (full || i < g.nrows) {
            const int row = g.row0 + i;
            RowOut<C::DT> oar, oai, obr, obi;
#pragma unroll
            for (int j = 0; j < V; ++j) {
                const Cx lam = cadd(vget(gr[i], gi[i], j), carry[j]);
                Cx hp = vget(hr[i], hi[i], j);
                if (i == 0 && g.row0 == 0 && !((rbits >> i) & 1u)) {  // row 0: h0, or 0
                    hp = Cx{0.0f, 0.0f};
                    if (x.p.h0r && j < g.nvalid)
                        hp = Cx{x.p.h0r[(size_t)g.bi * d.D + g.d0 + j],
                                x.p.h0i[(size_t)g.bi * d.D + g.d0 + j]};
                }
                const Cx ga = cmul(lam, cconj(hp));
                oar.v[j] = ga.r;
                oai.v[j] = ga.i;
                obr.v[j] = lam.r;
                obi.v[j] = lam.i;
                carry[j] = cmul(cconj(vget(ar[i], ai[i], j)), lam);
            }
            const uint32_t off = row_off(g, row, d.T, rowbytes);
            store_vec<C::DT, ALIGNED>(pgar, off, g.nvalid, oar);
            store_vec<C::DT, ALIGNED>(pgai, off, g.nvalid, oai);
            store_vec<C::DT, ALIGNED>(pgbr, off, g.nvalid, obr);
            store_vec<C::DT, ALIGNED>(pgbi, off, g.nvalid, obi);
        }
    }
    if (x.p.gh0r && g.nrows > 0 && g.row0 == 0) {
#pragma unroll
        for (int j = 0; j < V; ++j)
            if (j < g.nvalid) {
                x.p.gh0r[(size_t)g.bi * d.D + g.d0 + j] = carry[j].r;
                x.p.gh0i[(size_t)g.bi * d.D + g.d0 + j] = carry[j].i;
            }
    }
}

// ---------------------------------------------------------------------------
// per-lane walk
// ---------------------------------------------------------------------------
constexpr int kCxSeqBlock = 256;
constexpr int kCxSeqU = 4;  // rows loaded ahead

template <int DT, bool ALIGNED, bool RST>
__global__ __launch_bounds__(kCxSeqBlock) void cx_seq_fwd_kernel(CxFwdPtrs p, int64_t B, int64_t T,
                                                                 int64_t D, int64_t vpr) {
    constexpr int V = Elem<DT>::V;
    constexpr int U = kCxSeqU;
    const int64_t gid = (int64_t)blockIdx.x * kCxSeqBlock + threadIdx.x;
    const int64_t bi = gid / vpr;
    if (bi >= B) return;
    const int64_t d0 = (gid - bi * vpr) * V;
    const int nvalid = (int)((D - d0) < V ? (D - d0) : V);
    const size_t base = (size_t)bi * (size_t)T * (size_t)D + (size_t)d0;
    Cx h[V];
#pragma unroll
    for (int j = 0; j < V; ++j)
        h[j] = (p.h0r && j < nvalid) ? Cx{p.h0r[bi * D + d0 + j], p.h0i[bi * D + d0 + j]}
                                     : Cx{0.0f, 0.0f};
    for (int64_t t0 = 0; t0 < T; t0 += U) {
        RowVec<DT> ar[U], ai[U], br[U], bi_[U];
        uint32_t rr[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (t0 + u < T) {
                const size_t e = base + (size_t)(t0 + u) * D;
                ar[u] = load_row<DT, ALIGNED>(p.ar, e, nvalid, 1.0f);
                ai[u] = load_row<DT, ALIGNED>(p.ai, e, nvalid, 0.0f);
                br[u] = load_row<DT, ALIGNED>(p.br, e, nvalid, 0.0f);
                bi_[u] = load_row<DT, ALIGNED>(p.bi, e, nvalid, 0.0f);
                if (RST) rr[u] = p.reset[(size_t)bi * T + t0 + u];
            }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (t0 + u < T) {
                RowOut<DT> orr, oii;
#pragma unroll
                for (int j = 0; j < V; ++j) {
                    const Cx at = (RST && rr[u]) ? Cx{0.0f, 0.0f} : vget(ar[u], ai[u], j);
                    h[j] = cfma(at, h[j], vget(br[u], bi_[u], j));
                    orr.v[j] = h[j].r;
                    oii.v[j] = h[j].i;
                }
                if (p.out_r) {
                    const size_t e = base + (size_t)(t0 + u) * D;
                    store_row<DT, ALIGNED>(p.out_r, e, nvalid, orr);
                    store_row<DT, ALIGNED>(p.out_i, e, nvalid, oii);
                }
            }
    }
    if (p.last_r) {
#pragma unroll
        for (int j = 0; j < V; ++j)
            if (j < nvalid) {
                p.last_r[bi * D + d0 + j] = h[j].r;
                p.last_i[bi * D + d0 + j] = h[j].i;
            }
    }
}

template <int DT, bool ALIGNED, bool RST>
__global__ __launch_bounds__(kCxSeqBlock) void cx_seq_bwd_kernel(CxBwdPtrs p, int64_t B, int64_t T,
                                                                 int64_t D, int64_t vpr) {
    constexpr int V = Elem<DT>::V;
    constexpr int U = kCxSeqU;
    const int64_t gid = (int64_t)blockIdx.x * kCxSeqBlock + threadIdx.x;
    const int64_t bi = gid / vpr;
    if (bi >= B) return;
    const int64_t d0 = (gid - bi * vpr) * V;
    const int nvalid = (int)((D - d0) < V ? (D - d0) : V);
    const size_t base = (size_t)bi * (size_t)T * (size_t)D + (size_t)d0;
    Cx carry[V];
#pragma unroll
    for (int j = 0; j < V; ++j)
        carry[j] = (p.glr && j < nvalid) ? Cx{p.glr[bi * D + d0 + j], p.gli[bi * D + d0 + j]}
                                         : Cx{0.0f, 0.0f};
    for (int64_t top = T - 1; top >= 0; top -= U) {
        RowVec<DT> ar[U], ai[U], gr[U], gi[U], hr[U], hi[U];
        uint32_t rr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t t = top - u;
            if (t >= 0) {
                const size_t e = base + (size_t)t * D;
                ar[u] = load_row<DT, ALIGNED>(p.ar, e, nvalid, 1.0f);
                ai[u] = load_row<DT, ALIGNED>(p.ai, e, nvalid, 0.0f);
                gr[u] = load_row<DT, ALIGNED>(p.gr, e, nvalid, 0.0f);
                gi[u] = load_row<DT, ALIGNED>(p.gi, e, nvalid, 0.0f);
                if (t >= 1) {
                    hr[u] = load_row<DT, ALIGNED>(p.hr, e - D, nvalid, 0.0f);
                    hi[u] = load_row<DT, ALIGNED>(p.hi, e - D, nvalid, 0.0f);
                }
                if (RST) rr[u] = p.reset[(size_t)bi * T + t];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t t = top - u;
            if (t >= 0) {
                const bool rs = RST && rr[u];
                RowOut<DT> oar, oai, obr, obi;
#pragma unroll
                for (int j = 0; j < V; ++j) {
                    const Cx lam = cadd(vget(gr[u], gi[u], j), carry[j]);
                    Cx hp{0.0f, 0.0f};
                    if (!rs) {
                        if (t >= 1)
                            hp = vget(hr[u], hi[u], j);
                        else if (p.h0r && j < nvalid)
                            hp = Cx{p.h0r[bi * D + d0 + j], p.h0i[bi * D + d0 + j]};
                    }
                    const Cx ga = cmul(lam, cconj(hp));
                    oar.v[j] = ga.r;
                    oai.v[j] = ga.i;
                    obr.v[j] = lam.r;
                    obi.v[j] = lam.i;
                    const Cx at = rs ? Cx{0.0f, 0.0f} : vget(ar[u], ai[u], j);
                    carry[j] = cmul(cconj(at), lam);
                }
                const size_t e = base + (size_t)t * D;
                store_row<DT, ALIGNED>(p.gar, e, nvalid, oar);
                store_row<DT, ALIGNED>(p.gai, e, nvalid, oai);
                store_row<DT, ALIGNED>(p.gbr, e, nvalid, obr);
                store_row<DT, ALIGNED>(p.gbi, e, nvalid, obi);
            }
        }
    }
    if (p.gh0r) {
#pragma unroll
        for (int j = 0; j < V; ++j)
            if (j < nvalid) {
                p.gh0r[bi * D + d0 + j] = carry[j].r;
                p.gh0i[bi * D + d0 + j] = carry[j].i;
            }
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
template <class F>
void dispatch2(bool al, bool rst, F&& f) {
    if (al && rst) f(std::true_type{}, std::true_type{});
    else if (al) f(std::true_type{}, std::false_type{});
    else if (rst) f(std::false_type{}, std::true_type{});
    else f(std::false_type{}, std::false_type{});
}

// Tile shapes of the two directions: Cfg<type, threads of 16 bytes per row,
// rows per thread, wavefronts, look-back window>.  128 rows of 128-byte rows
// per array; measured on MI355X (bf16 B8 T2048 M2560), 256-row tiles (8 rows
// per thread, or 8 wavefronts) were no faster forward and 14-17% slower
// backward, where six arrays of 8 rows no longer fit in registers.  The
// backward folds its segments in one level (the forward's two levels,
// wavefront segments first, raised it to 168 registers with 8 spilled:
// 145.3 -> 152.7 us) and looks back over 2 tiles, not 4: the window's words
// are what kept it at 173 registers and 2 waves per SIMD; at 160 it runs 3
// (155.6 -> 145.5 us with the caches flushed; a window of 2 in the forward,
// at 3 or 4 waves, changed nothing measurable).
template <int DT>
using CxFwdCfg = Cfg<DT, 8, 4, 4, 4>;
template <int DT>
using CxBwdCfg = Cfg<DT, 8, 4, 4, 2>;

Layout cx_fwd_layout(const Shape& s) {
    return layout_of(s, CxFwdCfg<DT_F32>::TPR, CxFwdCfg<DT_F32>::CT);
}
Layout cx_bwd_layout(const Shape& s) {
    return layout_of(s, CxBwdCfg<DT_F32>::TPR, CxBwdCfg<DT_F32>::CT);
}

bool fwd_aligned(const Shape& s, const CxFwdPtrs& p) {
    const void* ptrs[6] = {p.ar, p.ai, p.br, p.bi, p.out_r, p.out_i};
    return rows_aligned(s, ptrs, 6);
}
bool bwd_aligned(const Shape& s, const CxBwdPtrs& p) {
    const void* ptrs[10] = {p.ar, p.ai, p.hr, p.hi, p.gr, p.gi, p.gar, p.gai, p.gbr, p.gbi};
    return rows_aligned(s, ptrs, 10);
}

template <int DT>
hipError_t cx_seq_fwd_t(const Shape& s, const CxFwdPtrs& p, hipStream_t st) {
    const int64_t vpr = (s.D + Elem<DT>::V - 1) / Elem<DT>::V;
    const dim3 grid((unsigned)((s.B * vpr + kCxSeqBlock - 1) / kCxSeqBlock));
    dispatch2(fwd_aligned(s, p), p.reset != nullptr, [&](auto AL, auto RS) {
        hipLaunchKernelGGL((cx_seq_fwd_kernel<DT, decltype(AL)::value, decltype(RS)::value>), grid,
                           dim3(kCxSeqBlock), 0, st, p, s.B, s.T, s.D, vpr);
    });
    return hipGetLastError();
}

template <int DT>
hipError_t cx_seq_bwd_t(const Shape& s, const CxBwdPtrs& p, hipStream_t st) {
    const int64_t vpr = (s.D + Elem<DT>::V - 1) / Elem<DT>::V;
    const dim3 grid((unsigned)((s.B * vpr + kCxSeqBlock - 1) / kCxSeqBlock));
    dispatch2(bwd_aligned(s, p), p.reset != nullptr, [&](auto AL, auto RS) {
        hipLaunchKernelGGL((cx_seq_bwd_kernel<DT, decltype(AL)::value, decltype(RS)::value>), grid,
                           dim3(kCxSeqBlock), 0, st, p, s.B, s.T, s.D, vpr);
    });
    return hipGetLastError();
}

template <int DT>
hipError_t cx_fused_fwd_t(const Shape& s, const CxFwdPtrs& p, void* ws, size_t ws_bytes, bool init,
                          int polls, hipStream_t st) {
    using C = CxFwdCfg<DT>;
    const Layout L = cx_fwd_layout(s);
    CxFwdArgs x;
    x.p = p;
    hipError_t e = prepare(ws, ws_bytes, init, L, kComplexWords, st, &x.sc);
    if (e != hipSuccess) return e;
    x.d = Dims{(int)s.T, (int)s.D, L.nW, L.nS, L.NK};
    x.polls = polls > 0 ? (uint32_t)polls : kDefaultPolls;
    const dim3 grid(x.sc.total_tiles), block(C::NT);
    const bool out = p.out_r != nullptr;
    dispatch2(fwd_aligned(s, p), p.reset != nullptr, [&](auto AL, auto RS) {
        constexpr bool al = decltype(AL)::value, rs = decltype(RS)::value;
        if (out) hipLaunchKernelGGL((cx_fused_fwd_kernel<C, al, rs, true>), grid, block, 0, st, x);
        else hipLaunchKernelGGL((cx_fused_fwd_kernel<C, al, rs, false>), grid, block, 0, st, x);
    });
    return hipGetLastError();
}

template <int DT>
hipError_t cx_fused_bwd_t(const Shape& s, const CxBwdPtrs& p, void* ws, size_t ws_bytes, bool init,
                          int polls, hipStream_t st) {
    using C = CxBwdCfg<DT>;
    const Layout L = cx_bwd_layout(s);
    CxBwdArgs x;
    x.p = p;
    hipError_t e = prepare(ws, ws_bytes, init, L, kComplexWords, st, &x.sc);
    if (e != hipSuccess) return e;
    x.d = Dims{(int)s.T, (int)s.D, L.nW, L.nS, L.NK};
    x.polls = polls > 0 ? (uint32_t)polls : kDefaultPolls;
    const dim3 grid(x.sc.total_tiles), block(C::NT);
    dispatch2(bwd_aligned(s, p), p.reset != nullptr, [&](auto AL, auto RS) {
        hipLaunchKernelGGL((cx_fused_bwd_kernel<C, decltype(AL)::value, decltype(RS)::value>), grid,
                           block, 0, st, x);
    });
    return hipGetLastError();
}

}  // namespace

hipError_t launch_complex_seq_fwd(const Shape& s, const CxFwdPtrs& p, hipStream_t st) {
    return s.dtype == DT_F32 ? cx_seq_fwd_t<DT_F32>(s, p, st) : cx_seq_fwd_t<DT_BF16>(s, p, st);
}

hipError_t launch_complex_seq_bwd(const Shape& s, const CxBwdPtrs& p, hipStream_t st) {
    return s.dtype == DT_F32 ? cx_seq_bwd_t<DT_F32>(s, p, st) : cx_seq_bwd_t<DT_BF16>(s, p, st);
}

bool complex_fused_supported(const Shape& s) {
    return tiled_layout_ok(s, CxFwdCfg<DT_F32>::CT, CxFwdCfg<DT_F32>::NT, cx_fwd_layout(s)) &&
           tiled_layout_ok(s, CxBwdCfg<DT_F32>::CT, CxBwdCfg<DT_F32>::NT, cx_bwd_layout(s));
}

size_t complex_fused_workspace_bytes(const Shape& s) {
    return kHeaderBytes + 2 * std::max(region_bytes_for(cx_fwd_layout(s), kComplexWords),
                                       region_bytes_for(cx_bwd_layout(s), kComplexWords));
}

hipError_t launch_complex_fused_fwd(const Shape& s, const CxFwdPtrs& p, void* ws, size_t ws_bytes,
                                    bool init, int polls, hipStream_t st) {
    return s.dtype == DT_F32 ? cx_fused_fwd_t<DT_F32>(s, p, ws, ws_bytes, init, polls, st)
                             : cx_fused_fwd_t<DT_BF16>(s, p, ws, ws_bytes, init, polls, st);
}

hipError_t launch_complex_fused_bwd(const Shape& s, const CxBwdPtrs& p, void* ws, size_t ws_bytes,
                                    bool init, int polls, hipStream_t st) {
    return s.dtype == DT_F32 ? cx_fused_bwd_t<DT_F32>(s, p, ws, ws_bytes, init, polls, st)
                             : cx_fused_bwd_t<DT_BF16>(s, p, ws, ws_bytes, init, polls, st);
}

}  // namespace lrscan
