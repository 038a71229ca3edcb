// samu.hip -- the fused-transition complex scan (page "triton_training_scan.py",
// _samu_forward and _samu_backward): the transition of every (token, mode)
// is rebuilt inside the kernel from per-token controls and per-mode
// parameters instead of being read from HBM,
//   nu = e^{nu_log[m]},  theta = e^{theta_log[m]},
//   a  = exp(-nu e^{eta[b,t]}) * (cos(theta + delta[b,t]), sin(theta + delta[b,t])),
// and then h_t = a_t h_{t-1} + b_t over complex values (planar storage of b,
// out and grad_b, as in complex.hip).  Trigonometry of theta is taken once per
// mode and of delta once per token; the angle-addition identity combines
// them, as the page does, so each (token, mode) costs one exponential.
//
// The kernels are the tiled single-launch form of complex.hip with the
// transition computed in registers.  The backward also forms the page's
//   radial = -nu e^eta Re(conj(a) grad_a),  phase = Im(conj(a) grad_a)
// per element and reduces them deterministically: over the lanes of a tile
// row into one partial per (token, lane block), and over the rows of a tile
// into one partial per (tile, mode); a small second kernel sums the partials
// in a fixed order into grad_eta, grad_delta (per token) and grad_nu_log,
// grad_theta_log (per mode).
#include <type_traits>

#include "complex_math.hpp"

namespace lrscan {

namespace {

// Per-mode and per-token factors of the transition, computed once per call by
// samu_factor_kernel into two small tables that every tile reads.
struct SamuLane {
    float nu2, th, ct, st;  // nu log2(e), theta, cos theta, sin theta
};
struct SamuTok {
    float e, cd, sd;  // e^eta, cos delta, sin delta
};

__device__ __forceinline__ SamuLane samu_lane(const float4* mode_tab, int m) {
    const float4 v = mode_tab[m];
    return SamuLane{v.x, v.y, v.z, v.w};
}

__device__ __forceinline__ SamuTok samu_tok(const float4* tok_tab, size_t t) {
    const float4 v = tok_tab[t];
    return SamuTok{v.x, v.y, v.z};
}

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.693147180559945309417f;

template <int DT>
__global__ void samu_factor_kernel(const void* __restrict__ eta, const void* __restrict__ delta,
                                   const float* __restrict__ nu_log,
                                   const float* __restrict__ theta_log, int64_t tokens, int64_t M,
                                   float4* __restrict__ tok_tab, float4* __restrict__ mode_tab) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < tokens) {
        float sd, cd;
        sincosf(Elem<DT>::load1(delta, (size_t)i), &sd, &cd);
        tok_tab[i] = make_float4(expf(Elem<DT>::load1(eta, (size_t)i)), cd, sd, 0.0f);
    }
    if (i < M) {
        const float th = expf(theta_log[i]);
        float st, ct;
        sincosf(th, &st, &ct);
        mode_tab[i] = make_float4(expf(nu_log[i]) * kLog2e, th, ct, st);
    }
}

// a = exp(-nu e^eta) e^{i (theta + delta)}: the decay as 2^{-x2} with
// x2 = nu log2(e) e^eta (one hardware exp2), the rotation by angle addition.
__device__ __forceinline__ float samu_x2(const SamuLane& L, const SamuTok& k) { return L.nu2 * k.e; }
__device__ __forceinline__ Cx samu_a_of(const SamuLane& L, const SamuTok& k, float x2) {
    const float cosine = fmaf(L.ct, k.cd, -(L.st * k.sd));
    const float sine = fmaf(L.st, k.cd, L.ct * k.sd);
    const float rho = __builtin_amdgcn_exp2f(-x2);
    return Cx{rho * cosine, rho * sine};
}
__device__ __forceinline__ Cx samu_a(const SamuLane& L, const SamuTok& k) {
    return samu_a_of(L, k, samu_x2(L, k));
}

// Make the compiler forget the factors after the summary, so that the
// replay recomputes each transition instead of keeping the summary's copies
// of all of them alive across the look-back.
__device__ __forceinline__ void opaque(SamuTok& k) { asm volatile("" : "+v"(k.e), "+v"(k.cd), "+v"(k.sd)); }
__device__ __forceinline__ void opaque(SamuLane& L) { asm volatile("" : "+v"(L.nu2), "+v"(L.ct), "+v"(L.st)); }

struct SamuFwdArgs {
    SamuFwdPtrs p;
    const float4 *tok_tab, *mode_tab;
    Scratch sc;
    Dims d;
    uint32_t polls;
};
struct SamuBwdArgs {
    SamuBwdPtrs p;
    const float4 *tok_tab, *mode_tab;
    Scratch sc;
    Dims d;
    uint32_t polls;
    size_t tokens;                // B * T
    float *tok_eta, *tok_delta;   // [nW, B*T] partial sums over a tile row's lanes
    float *mode_nu, *mode_theta;  // [NK, B, M] partial sums over a tile's rows
};

// Derived tile maps for the look-back, in the owners' operation order: each
// segment of NR rows folded from the identity, then the segments folded in
// order (forward) or in reverse order (backward).
template <class C>
__device__ CAff samu_fwd_tile_map(const SamuFwdArgs& x, int j, int bi, int col) {
    constexpr int NR = C::NR, SEGS = C::WAVES * C::RG;
    CAff A = caff_identity(), Wv = caff_identity();
    if (col >= x.d.D) return A;
    const SamuLane L = samu_lane(x.mode_tab, col);
    const size_t rowbytes = (size_t)x.d.D * C::EB;
    const size_t b0 = (size_t)bi * x.d.T * rowbytes;
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
                const size_t tok = (size_t)bi * x.d.T + r;
                const size_t ro = (size_t)uniform64((int64_t)r * (int64_t)rowbytes) + coff;
                at = samu_a(L, samu_tok(x.tok_tab, tok));
                bt = load_cx<C::DT>(br, bim, ro);
                if (x.p.reset && x.p.reset[tok]) at = Cx{0.0f, 0.0f};
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

template <class C>
__device__ CAff samu_bwd_tile_map(const SamuBwdArgs& x, int j, int bi, int col) {
    constexpr int NR = C::NR, SEGS = C::WAVES * C::RG;
    CAff A = caff_identity(), Wv = caff_identity();
    if (col >= x.d.D) return A;
    const SamuLane L = samu_lane(x.mode_tab, col);
    const size_t rowbytes = (size_t)x.d.D * C::EB;
    const size_t b0 = (size_t)bi * x.d.T * rowbytes;
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
                const size_t tok = (size_t)bi * x.d.T + r;
                const size_t ro = (size_t)uniform64((int64_t)r * (int64_t)rowbytes) + coff;
                at = samu_a(L, samu_tok(x.tok_tab, tok));
                gt = load_cx<C::DT>(gr, gi, ro);
                if (x.p.reset && x.p.reset[tok]) at = Cx{0.0f, 0.0f};
            }
            t = rev_fold(t, at, gt);
        }
        Wv = caff_then(Wv, t);
        if (sg % C::RG == 0) {  // a wavefront's segments (last first), then the wavefronts
            A = caff_then(A, Wv);
            Wv = caff_identity();
        }
    }
    return CAff{unpack_cx(pack_cx(A.p)), unpack_cx(pack_cx(A.q))};
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
// Distinct empty statements at the top of the two versions of a tile body:
// without them the compiler hoists the identical start of both versions
// above the branch, and the registers that the hoisted part keeps alive into
// both made the pair spill where each version alone does not.
template <bool FULL>
__device__ __forceinline__ void tile_marker() {
    if constexpr (FULL) asm volatile("; full tile");
    else asm volatile("; partial tile");
}

// One tile of the forward.  FULL: every row and lane of the tile exists
// (wave-uniform, and every tile when T and M are multiples of the tile), so
// the tile runs without the per-element guards that rows past T and lanes
// past M need.
template <class C, bool ALIGNED, bool RST, bool OUT, bool FULL>
__device__ __forceinline__ void samu_fwd_tile(const SamuFwdArgs& x, const Ticket& tk, const Geo& g,
                                              int seg, int cg, CAff (&s_seg)[C::WAVES * C::RG][C::W],
                                              CAff (&s_wav)[C::WAVES][C::W], Cx (&s_hin)[C::W]) {
    constexpr int V = C::V, W = C::W, NR = C::NR, SEGS = C::WAVES * C::RG;
    tile_marker<FULL>();
    const Dims d = x.d;
    const int tid = threadIdx.x;
    const uint32_t rowbytes = (uint32_t)d.D * C::EB;
    const char* pbr = static_cast<const char*>(x.p.br) + g.tbase;
    const char* pbi = static_cast<const char*>(x.p.bi) + g.tbase;

    RowVec<C::DT> br[NR], bi[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const uint32_t off = row_off(g, g.row0 + i, d.T, rowbytes);
        br[i] = load_vec<C::DT, ALIGNED, true>(pbr, off, g.nvalid, 0.0f);
        bi[i] = load_vec<C::DT, ALIGNED, true>(pbi, off, g.nvalid, 0.0f);
    }
    // per-token and per-mode factors of this thread's rows and lanes (rows
    // past T and lanes past M read the last valid one; never used)
    SamuTok tok[NR];
    uint32_t rbits = 0;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const int row = g.row0 + i;
        const size_t t = (size_t)g.bi * d.T + (FULL || row < d.T ? row : d.T - 1);
        tok[i] = samu_tok(x.tok_tab, t);
        if constexpr (RST) rbits |= (x.p.reset[t] ? 1u : 0u) << i;
    }
    SamuLane ln[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
        const int m = FULL || g.d0 + j < d.D ? g.d0 + j : d.D - 1;
        ln[j] = samu_lane(x.mode_tab, m);
    }
    // lanes past M step with the identity, as the derived maps assume
    auto trans = [&](int i, int j) -> Cx {
        if (!FULL && j >= g.nvalid) return Cx{1.0f, 0.0f};
        if (RST && ((rbits >> i) & 1u)) return Cx{0.0f, 0.0f};
        return samu_a(ln[j], tok[i]);
    };

#pragma unroll
    for (int j = 0; j < V; ++j) {
        CAff m = caff_identity();
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const bool ok = FULL || i < g.nrows;
            const Cx at = ok ? trans(i, j) : Cx{1.0f, 0.0f};
            const Cx bt = ok ? vget(br[i], bi[i], j) : Cx{0.0f, 0.0f};
            m = caff_then(m, fwd_step(at, bt));
        }
        s_seg[seg][cg * V + j] = m;
    }
    fold_wave_segments<C, false, CAffThen>(s_seg, s_wav, seg / C::RG, (int)threadIdx.x % kWave,
                                           caff_identity());
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        opaque(br[i]);
        opaque(bi[i]);
        opaque(tok[i]);
    }
#pragma unroll
    for (int j = 0; j < V; ++j) opaque(ln[j]);
    // early reading of the look-back window, issued once this thread's last
    // row has arrived
    EarlyWindow<ComplexLink, C::EW> early;
    if (tid < W) {
        const CxWords we = cx_words(x.sc, tk.phase);
        const int z = zero_after_row(bi[NR - 1]);
        early.template take<-1>(ComplexLink{we.ps, we.qs, we.hs, d.nS, g.s, W, tid + z}, g.k, d.NK);
    }
    __syncthreads();

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
                lk, g.k, d.NK, base0, x.polls, [&](int j) { return samu_fwd_tile_map<C>(x, j, g.bi, dl); });
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
        if (FULL || i < g.nrows) {
            RowOut<C::DT> orr, oii;
#pragma unroll
            for (int j = 0; j < V; ++j) {
                h[j] = cfma(trans(i, j), h[j], vget(br[i], bi[i], j));
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
            if (FULL || j < g.nvalid) {
                x.p.last_r[(size_t)g.bi * d.D + g.d0 + j] = h[j].r;
                x.p.last_i[(size_t)g.bi * d.D + g.d0 + j] = h[j].i;
            }
    }
}

template <class C, bool ALIGNED, bool RST, bool OUT>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(2)))
void samu_fwd_kernel(SamuFwdArgs x) {
    constexpr int W = C::W, RG = C::RG, TPR = C::TPR;
    constexpr int SEGS = C::WAVES * RG;
    __shared__ CAff s_seg[SEGS][W];  // each segment's map, then its wavefront's maps before it composed
    __shared__ CAff s_wav[C::WAVES][W];  // each wavefront's map, then the wavefronts' before it composed
    __shared__ Cx s_hin[W];          // the state entering the tile, per lane

    const int tid = threadIdx.x;
    const int wave = uniform((int)(threadIdx.x / kWave));
    const int l = tid % kWave;
    const int rg = l / TPR;
    const int cg = l % TPR;
    const int seg = wave * RG + rg;
    const Ticket tk = take_ticket(x.sc);
    const Geo g = tile_geo<C, false>(tk.ticket, x.d, wave, rg, cg);
    if (g.trow0 + C::CT <= x.d.T && g.dcol0 + W <= x.d.D)
        samu_fwd_tile<C, ALIGNED, RST, OUT, true>(x, tk, g, seg, cg, s_seg, s_wav, s_hin);
    else
        samu_fwd_tile<C, ALIGNED, RST, OUT, false>(x, tk, g, seg, cg, s_seg, s_wav, s_hin);
}

// Transposing sum of N values per lane over the lanes {l ^ o}, o running
// over the powers of two from O down to LAST.  While a lane holds more than
// one value, each stage halves them: the lane whose offset bit is clear keeps
// the lower half, its partner the upper half, and each adds the partner's
// copy of the half it keeps; once one value is left the remaining stages are
// plain butterfly sums.  Afterwards a lane holds K = max(1, N / G) values (G
// the number of lanes in the group), value q being the total of index
//   q + K * (g / max(1, G / N)),   g = the lane's position in its group,
// and lanes with the same g / max(1, G / N) hold the same totals.  The order of
// the additions is fixed, so the sums are deterministic, and a stage costs
// max(1, N / 2^k) shuffles instead of N.
template <int N, int O, int LAST>
__device__ __forceinline__ void tsum(float* v, int lane) {
    if constexpr (N >= 2) {
        constexpr int H = N / 2;
        const bool up = (lane & O) != 0;
#pragma unroll
        for (int q = 0; q < H; ++q) {
            const float mine = up ? v[H + q] : v[q];
            const float give = up ? v[q] : v[H + q];
            v[q] = mine + __shfl_xor(give, O, kWave);
        }
        if constexpr (O > LAST) tsum<H, O / 2, LAST>(v, lane);
    } else {
        v[0] += __shfl_xor(v[0], O, kWave);
        if constexpr (O > LAST) tsum<1, O / 2, LAST>(v, lane);
    }
}

// ---------------------------------------------------------------------------
// reverse time
// ---------------------------------------------------------------------------
// One tile of the backward.  (Unlike the forward it has one body for all
// tiles: a separate unguarded body for complete tiles raised its register
// count past the budget and spilled.)
template <class C, bool ALIGNED, bool RST>
__device__ __forceinline__ void samu_bwd_tile(const SamuBwdArgs& x, const Ticket& tk, const Geo& g,
                                              int wave, int seg, int rg, int cg,
                                              CAff (&s_seg)[C::WAVES * C::RG][C::W],
                                              CAff (&s_wav)[C::WAVES][C::W], Cx (&s_cin)[C::W],
                                              float (&s_acc)[2][C::WAVES][C::W]) {
    constexpr int V = C::V, W = C::W, RG = C::RG, NR = C::NR, WAVES = C::WAVES, TPR = C::TPR;
    constexpr int SEGS = WAVES * RG;
    const Dims d = x.d;
    const int tid = threadIdx.x;
    const int l = tid % kWave;
    const uint32_t rowbytes = (uint32_t)d.D * C::EB;
    const char* pgr = static_cast<const char*>(x.p.gr) + g.tbase;
    const char* pgi = static_cast<const char*>(x.p.gi) + g.tbase;
    const int hrow0 = g.trow0 > 0 ? g.trow0 - 1 : 0;
    const size_t hback = (size_t)(g.trow0 - hrow0) * rowbytes;
    const char* phr = static_cast<const char*>(x.p.hr) + g.tbase - hback;
    const char* phi = static_cast<const char*>(x.p.hi) + g.tbase - hback;

    RowVec<C::DT> gr[NR], gi[NR], hr[NR], hi[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const uint32_t off = row_off(g, g.row0 + i, d.T, rowbytes);
        gr[i] = load_vec<C::DT, ALIGNED, true>(pgr, off, g.nvalid, 0.0f);
        gi[i] = load_vec<C::DT, ALIGNED, true>(pgi, off, g.nvalid, 0.0f);
    }
    // The rows of `out` last, as only the replay uses them; the later half
    // now, the earlier half during the replay (the replay walks the rows
    // from the last), so that the two halves never hold registers at once.
    // With fewer than 4 rows per thread every row is loaded now.
    auto load_h = [&](int i, int z) {
        const int row = g.row0 + i;
        const int rc = row < d.T ? row : d.T - 1;
        const int hrw = rc >= 1 ? rc - 1 : 0;
        const uint32_t hoff = (uint32_t)(hrw - hrow0) * rowbytes + g.coff + (uint32_t)z;
        hr[i] = load_vec<C::DT, ALIGNED, true>(phr, hoff, g.nvalid, 0.0f);
        hi[i] = load_vec<C::DT, ALIGNED, true>(phi, hoff, g.nvalid, 0.0f);
    };
    constexpr int kHLate = NR >= 4 ? NR / 2 : 0;  // rows of `out` loaded during the replay
#pragma unroll
    for (int i = kHLate; i < NR; ++i) load_h(i, 0);
    SamuTok tok[NR];
    uint32_t rbits = 0;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const int row = g.row0 + i;
        const size_t t = (size_t)g.bi * d.T + (row < d.T ? row : d.T - 1);
        tok[i] = samu_tok(x.tok_tab, t);
        if constexpr (RST) rbits |= (x.p.reset[t] ? 1u : 0u) << i;
    }
    SamuLane ln[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
        const int m = g.d0 + j < d.D ? g.d0 + j : d.D - 1;
        ln[j] = samu_lane(x.mode_tab, m);
    }
    // lanes past M step with the identity, as the derived maps assume
    auto trans = [&](int i, int j) -> Cx {
        if (j >= g.nvalid) return Cx{1.0f, 0.0f};
        if (RST && ((rbits >> i) & 1u)) return Cx{0.0f, 0.0f};
        return samu_a(ln[j], tok[i]);
    };

#pragma unroll
    for (int j = 0; j < V; ++j) {
        CAff m = caff_identity();
#pragma unroll
        for (int i = NR - 1; i >= 0; --i) {
            const bool ok = i < g.nrows;
            const Cx at = ok ? trans(i, j) : Cx{1.0f, 0.0f};
            const Cx gt = ok ? vget(gr[i], gi[i], j) : Cx{0.0f, 0.0f};
            m = rev_fold(m, at, gt);
        }
        s_seg[seg][cg * V + j] = m;
    }
    fold_wave_segments<C, true, CAffThen>(s_seg, s_wav, seg / C::RG, (int)threadIdx.x % kWave,
                                          caff_identity());
#pragma unroll
    for (int i = 0; i < NR; ++i) {
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
#pragma unroll
        for (int w = C::WAVES - 1; w >= 0; --w) {
            const CAff t = s_wav[w][c];
            s_wav[w][c] = A;
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
                lk, g.k, d.NK, base0, x.polls, [&](int j) { return samu_bwd_tile_map<C>(x, j, g.bi, dl); });
        if (more) publish_u64(wd.hs + o, pack_cx(caff_apply(A, cin)));
        s_cin[c] = cin;
    }
    __syncthreads();
    // this tile's share of clearing the other region (here, not before the
    // summary: a loop of stores there would make the summary wait for every load)
    clear_share(x.sc, tk.phase, tk.nclear, C::NT, tk.ticket);

    char* pgbr = static_cast<char*>(x.p.gbr) + g.tbase;
    char* pgbi = static_cast<char*>(x.p.gbi) + g.tbase;
    Cx carry[V];
    // With w = conj(a) grad_a per element, the radial term is
    // -nu e^eta Re(w) = -ln2 * nu2_j * e_t * Re(w) and the phase term Im(w).
    // acc[2j], acc[2j+1]: this thread's sums over its rows of lane j's
    // e_t Re(w) and Im(w) (the factor -ln2 nu2_j and theta are applied once
    // per tile and lane); tsum_[2i], [2i+1]: row i's sums over this thread's
    // lanes of nu2_j Re(w) and Im(w) (the factor -ln2 e_t once per row).
    float acc[2 * V], tsum_[2 * NR];
#pragma unroll
    for (int j = 0; j < V; ++j) {
        carry[j] = caff_apply(s_seg[seg][cg * V + j],
                              caff_apply(s_wav[seg / C::RG][cg * V + j], s_cin[cg * V + j]));
        acc[2 * j] = 0.0f;
        acc[2 * j + 1] = 0.0f;
    }
    const int lb = g.s - g.bi * d.nW;  // lane block of this tile
#pragma unroll
    for (int i = NR - 1; i >= 0; --i) {
        const int row = g.row0 + i;
        if (kHLate > 0 && i == NR - 3) {
            // the earlier half of `out`, once two rows have freed their
            // registers (addressed with a zero that depends on the carry,
            // so the loads cannot be issued sooner)
            const int z = zero_after(carry[0].r);
#pragma unroll
            for (int r = 0; r < kHLate; ++r) load_h(r, z);
        }
        tsum_[2 * i] = 0.0f;
        tsum_[2 * i + 1] = 0.0f;
        if (row < d.T) {  // the same for every lane of a row group
            RowOut<C::DT> obr, obi;
            float rsum = 0.0f, psum = 0.0f;
#pragma unroll
            for (int j = 0; j < V; ++j) {
                const Cx at = trans(i, j);
                const Cx lam = cadd(vget(gr[i], gi[i], j), carry[j]);
                Cx hp = vget(hr[i], hi[i], j);
                if (i == 0 && g.row0 == 0) {  // row 0: the state before it is h0, or 0
                    hp = Cx{0.0f, 0.0f};
                    if (x.p.h0r && (j < g.nvalid))
                        hp = Cx{x.p.h0r[(size_t)g.bi * d.D + g.d0 + j],
                                x.p.h0i[(size_t)g.bi * d.D + g.d0 + j]};
                }
                const bool rs = RST && ((rbits >> i) & 1u);
                // w = conj(a) grad_a = conj(a) lambda conj(h_{t-1}): the new
                // carry conj(a) lambda times conj(h_{t-1}), one product fewer
                carry[j] = cmul(cconj(at), lam);
                const Cx w = rs ? Cx{0.0f, 0.0f} : cmul(carry[j], cconj(hp));
                const bool live = j < g.nvalid;
                const float wr = live ? w.r : 0.0f;
                const float wi = live ? w.i : 0.0f;
                rsum = fmaf(ln[j].nu2, wr, rsum);
                psum += wi;
                acc[2 * j] = fmaf(tok[i].e, wr, acc[2 * j]);
                acc[2 * j + 1] += wi;
                obr.v[j] = lam.r;
                obi.v[j] = lam.i;
            }
            if (g.nvalid > 0) {
                const uint32_t off = row_off(g, row, d.T, rowbytes);
                store_vec<C::DT, ALIGNED>(pgbr, off, g.nvalid, obr);
                store_vec<C::DT, ALIGNED>(pgbi, off, g.nvalid, obi);
            }
            tsum_[2 * i] = rsum * -(tok[i].e * kLn2);
            tsum_[2 * i + 1] = psum;
        }
    }
#pragma unroll
    for (int j = 0; j < V; ++j) acc[2 * j] *= -(ln[j].nu2 * kLn2);
    // per-token partials over the row group's TPR lanes; value index 2i is
    // row i's radial sum, 2i + 1 its phase sum
    {
        constexpr int NV = 2 * NR;
        constexpr int KT = NV >= TPR ? NV / TPR : 1;
        constexpr int SP = NV >= TPR ? 1 : TPR / NV;
        tsum<NV, TPR / 2, 1>(tsum_, cg);
        if (cg % SP == 0) {
#pragma unroll
            for (int q = 0; q < KT; ++q) {
                const int idx = q + KT * (cg / SP);
                const int row = g.row0 + idx / 2;
                if (row < d.T) {
                    const size_t tp = (size_t)lb * x.tokens + (size_t)g.bi * d.T + row;
                    ((idx & 1) ? x.tok_delta : x.tok_eta)[tp] = tsum_[q];
                }
            }
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
    // per-mode partials of this tile: over the RG row groups, then over the
    // waves; value index 2j of acc is lane j's radial sum, 2j + 1 its phase sum
    {
        constexpr int NV = 2 * V;
        constexpr int KM = NV >= RG ? NV / RG : 1;
        constexpr int SP = NV >= RG ? 1 : RG / NV;
        tsum<NV, kWave / 2, TPR>(acc, l);
        if (rg % SP == 0) {
#pragma unroll
            for (int q = 0; q < KM; ++q) {
                const int idx = q + KM * (rg / SP);
                s_acc[idx & 1][wave][cg * V + idx / 2] = acc[q];
            }
        }
    }
    __syncthreads();
    if (tid < W) {
        const int dl = g.dcol0 + tid;
        if (dl < d.D) {
            float nu = 0.0f, th = 0.0f;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) {
                nu += s_acc[0][w][tid];
                th += s_acc[1][w][tid];
            }
            const size_t mp = ((size_t)g.k * (d.nS / d.nW) + g.bi) * d.D + dl;
            x.mode_nu[mp] = nu;
            x.mode_theta[mp] = th * x.mode_tab[dl].y;  // d/dtheta_log = theta d/dtheta
        }
    }
}

template <class C, bool ALIGNED, bool RST>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(2)))
void samu_bwd_kernel(SamuBwdArgs x) {
    constexpr int W = C::W, RG = C::RG, WAVES = C::WAVES, TPR = C::TPR;
    constexpr int SEGS = WAVES * RG;
    __shared__ CAff s_seg[SEGS][W];  // each segment's reverse map, then its wavefront's maps after it composed
    __shared__ CAff s_wav[C::WAVES][W];  // each wavefront's reverse map, then the wavefronts' after it composed
    __shared__ Cx s_cin[W];          // the carry entering the tile from the right, per lane
    __shared__ float s_acc[2][WAVES][W];

    const int tid = threadIdx.x;
    const int wave = uniform((int)(threadIdx.x / kWave));
    const int l = tid % kWave;
    const int rg = l / TPR;
    const int cg = l % TPR;
    const int seg = wave * RG + rg;
    const Ticket tk = take_ticket(x.sc);
    const Geo g = tile_geo<C, true>(tk.ticket, x.d, wave, rg, cg);
    samu_bwd_tile<C, ALIGNED, RST>(x, tk, g, wave, seg, rg, cg, s_seg, s_wav, s_cin, s_acc);
}

// The second pass: dst[i] = sum_k src[k n + i] over k < count, for two arrays
// at once.  A workgroup covers 64 consecutive i; its four wavefronts take the
// k of one residue mod 4 each, in increasing order, and the four partial sums
// are added in wavefront order: a fixed order, so results are deterministic.
struct SumJob {
    const float *src0, *src1;
    float *dst0, *dst1;
    int64_t n, count;
};
constexpr int kSumLanes = 64;
constexpr int kSumSlices = 4;

__global__ __launch_bounds__(kSumLanes* kSumSlices) void samu_reduce_kernel(SumJob a, SumJob b,
                                                                            unsigned blocks_a) {
    __shared__ float s_part[2][kSumSlices][kSumLanes];
    const bool first = blockIdx.x < blocks_a;
    const SumJob& j = first ? a : b;
    const int64_t blk = first ? blockIdx.x : blockIdx.x - blocks_a;
    const int lane = threadIdx.x % kSumLanes;
    const int slice = threadIdx.x / kSumLanes;
    const int64_t i = blk * kSumLanes + lane;
    float s0 = 0.0f, s1 = 0.0f;
    if (i < j.n) {
#pragma unroll 4
        for (int64_t k = slice; k < j.count; k += kSumSlices) {
            s0 += j.src0[k * j.n + i];
            s1 += j.src1[k * j.n + i];
        }
    }
    s_part[0][slice][lane] = s0;
    s_part[1][slice][lane] = s1;
    __syncthreads();
    if (slice == 0 && i < j.n) {
        float t0 = s_part[0][0][lane], t1 = s_part[1][0][lane];
#pragma unroll
        for (int q = 1; q < kSumSlices; ++q) {
            t0 += s_part[0][q][lane];
            t1 += s_part[1][q][lane];
        }
        if (j.dst0) j.dst0[i] = t0;
        if (j.dst1) j.dst1[i] = t1;
    }
}

template <class F>
void dispatch2(bool al, bool rst, F&& f) {
    if (al && rst) f(std::true_type{}, std::true_type{});
    else if (al) f(std::true_type{}, std::false_type{});
    else if (rst) f(std::false_type{}, std::true_type{});
    else f(std::false_type{}, std::false_type{});
}

// ---------------------------------------------------------------------------
// per-lane walk
// ---------------------------------------------------------------------------
// One thread per (batch row, 16-byte vector of modes) walks all T steps with
// each transition rebuilt in registers, as the complex scan's walk does with
// stored ones: for sequences too short for the tiles' fixed costs.  In the
// backward a row's vectors are padded to whole wavefronts (`tpr` threads per
// row, a multiple of 64), so that a wavefront sums each token's radial and
// phase terms over its lanes with butterfly shuffles and writes one partial
// per (wavefront of the row, token); each thread keeps its modes' sums over
// the row's tokens and writes one partial per (row, mode).  The reduction
// kernel adds the partials as for the tiles.
constexpr int kSamuSeqBlock = 256;
constexpr int kSamuSeqU = 4;  // rows loaded ahead

template <int DT, bool ALIGNED, bool RST>
__global__ __launch_bounds__(kSamuSeqBlock) void samu_seq_fwd_kernel(
    SamuFwdPtrs p, const float4* __restrict__ tok_tab, const float4* __restrict__ mode_tab,
    int64_t B, int64_t T, int64_t M, int64_t vpr) {
    constexpr int V = Elem<DT>::V;
    constexpr int U = kSamuSeqU;
    const int64_t gid = (int64_t)blockIdx.x * kSamuSeqBlock + threadIdx.x;
    const int64_t b = gid / vpr;
    if (b >= B) return;
    const int64_t d0 = (gid - b * vpr) * V;
    const int nvalid = (int)((M - d0) < V ? (M - d0) : V);
    const size_t base = (size_t)b * (size_t)T * (size_t)M + (size_t)d0;
    SamuLane ln[V];
#pragma unroll
    for (int j = 0; j < V; ++j) ln[j] = samu_lane(mode_tab, d0 + j < M ? (int)(d0 + j) : (int)(M - 1));
    Cx h[V];
#pragma unroll
    for (int j = 0; j < V; ++j)
        h[j] = (p.h0r && j < nvalid) ? Cx{p.h0r[b * M + d0 + j], p.h0i[b * M + d0 + j]}
                                     : Cx{0.0f, 0.0f};
    for (int64_t t0 = 0; t0 < T; t0 += U) {
        RowVec<DT> vr[U], vi[U];
        SamuTok tk[U];
        uint32_t rr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (t0 + u < T) {
                const size_t e = base + (size_t)(t0 + u) * M;
                vr[u] = load_row<DT, ALIGNED>(p.br, e, nvalid, 0.0f);
                vi[u] = load_row<DT, ALIGNED>(p.bi, e, nvalid, 0.0f);
                tk[u] = samu_tok(tok_tab, (size_t)b * T + t0 + u);
                if (RST) rr[u] = p.reset[(size_t)b * T + t0 + u];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (t0 + u < T) {
                RowOut<DT> orr, oii;
#pragma unroll
                for (int j = 0; j < V; ++j) {
                    const Cx at = (RST && rr[u]) ? Cx{0.0f, 0.0f} : samu_a(ln[j], tk[u]);
                    h[j] = cfma(at, h[j], vget(vr[u], vi[u], j));
                    orr.v[j] = h[j].r;
                    oii.v[j] = h[j].i;
                }
                if (p.out_r) {
                    const size_t e = base + (size_t)(t0 + u) * M;
                    store_row<DT, ALIGNED>(p.out_r, e, nvalid, orr);
                    store_row<DT, ALIGNED>(p.out_i, e, nvalid, oii);
                }
            }
        }
    }
    if (p.last_r) {
#pragma unroll
        for (int j = 0; j < V; ++j)
            if (j < nvalid) {
                p.last_r[b * M + d0 + j] = h[j].r;
                p.last_i[b * M + d0 + j] = h[j].i;
            }
    }
}

struct SamuSeqParts {
    float *tok_eta, *tok_delta;   // [tpr / 64, B*T]
    float *mode_nu, *mode_theta;  // [B, M]
};

template <int DT, bool ALIGNED, bool RST>
__global__ __launch_bounds__(kSamuSeqBlock) void samu_seq_bwd_kernel(
    SamuBwdPtrs p, const float4* __restrict__ tok_tab, const float4* __restrict__ mode_tab,
    SamuSeqParts q, int64_t B, int64_t T, int64_t M, int64_t tpr) {
    constexpr int V = Elem<DT>::V;
    constexpr int U = kSamuSeqU;
    const int64_t gid = (int64_t)blockIdx.x * kSamuSeqBlock + threadIdx.x;
    const int64_t b = gid / tpr;
    if (b >= B) return;  // whole wavefronts: tpr and the block are multiples of 64
    const int64_t col = gid - b * tpr;
    const int64_t d0 = col * V;
    const int nvalid = d0 >= M ? 0 : (int)((M - d0) < V ? (M - d0) : V);
    const int wrow = (int)(col / kWave);
    const int lane = (int)(threadIdx.x % kWave);
    const size_t tokens = (size_t)B * T;
    // padding threads (past M) read the row's first vector; their terms are 0
    const size_t base = (size_t)b * (size_t)T * (size_t)M + (size_t)(nvalid > 0 ? d0 : 0);
    SamuLane ln[V];
#pragma unroll
    for (int j = 0; j < V; ++j) ln[j] = samu_lane(mode_tab, d0 + j < M ? (int)(d0 + j) : (int)(M - 1));
    Cx carry[V];
#pragma unroll
    for (int j = 0; j < V; ++j)
        carry[j] = (p.glr && j < nvalid) ? Cx{p.glr[b * M + d0 + j], p.gli[b * M + d0 + j]}
                                         : Cx{0.0f, 0.0f};
    // acc[2j], acc[2j+1]: lane j's sums over the row's tokens of e_t Re(w) and Im(w)
    float acc[2 * V];
#pragma unroll
    for (int k = 0; k < 2 * V; ++k) acc[k] = 0.0f;
    for (int64_t top = T - 1; top >= 0; top -= U) {
        RowVec<DT> gr[U], gi[U], hr[U], hi[U];
        SamuTok tk[U];
        uint32_t rr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t t = top - u;
            if (t >= 0) {
                const size_t e = base + (size_t)t * M;
                gr[u] = load_row<DT, ALIGNED>(p.gr, e, nvalid, 0.0f);
                gi[u] = load_row<DT, ALIGNED>(p.gi, e, nvalid, 0.0f);
                if (t >= 1) {
                    hr[u] = load_row<DT, ALIGNED>(p.hr, e - M, nvalid, 0.0f);
                    hi[u] = load_row<DT, ALIGNED>(p.hi, e - M, nvalid, 0.0f);
                }
                tk[u] = samu_tok(tok_tab, (size_t)b * T + t);
                if (RST) rr[u] = p.reset[(size_t)b * T + t];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t t = top - u;
            if (t >= 0) {
                const bool rs = RST && rr[u];
                RowOut<DT> obr, obi;
                float rsum = 0.0f, psum = 0.0f;
#pragma unroll
                for (int j = 0; j < V; ++j) {
                    const Cx at = rs ? Cx{0.0f, 0.0f} : samu_a(ln[j], tk[u]);
                    const Cx lam = cadd(vget(gr[u], gi[u], j), carry[j]);
                    Cx hp{0.0f, 0.0f};
                    if (t >= 1)
                        hp = vget(hr[u], hi[u], j);
                    else if (p.h0r && j < nvalid)
                        hp = Cx{p.h0r[b * M + d0 + j], p.h0i[b * M + d0 + j]};
                    // w = conj(a) grad_a = conj(a) lambda conj(h_{t-1}): the new
                    // carry conj(a) lambda times conj(h_{t-1})
                    carry[j] = cmul(cconj(at), lam);
                    const Cx w = rs ? Cx{0.0f, 0.0f} : cmul(carry[j], cconj(hp));
                    const bool live = j < nvalid;
                    const float wr = live ? w.r : 0.0f;
                    const float wi = live ? w.i : 0.0f;
                    rsum = fmaf(ln[j].nu2, wr, rsum);
                    psum += wi;
                    acc[2 * j] = fmaf(tk[u].e, wr, acc[2 * j]);
                    acc[2 * j + 1] += wi;
                    obr.v[j] = lam.r;
                    obi.v[j] = lam.i;
                }
                if (nvalid > 0) {
                    const size_t e = base + (size_t)t * M;
                    store_row<DT, ALIGNED>(p.gbr, e, nvalid, obr);
                    store_row<DT, ALIGNED>(p.gbi, e, nvalid, obi);
                }
                // the token's sums over this wavefront's lanes, in a fixed order
#pragma unroll
                for (int o = kWave / 2; o >= 1; o >>= 1) {
                    rsum += __shfl_xor(rsum, o, kWave);
                    psum += __shfl_xor(psum, o, kWave);
                }
                if (lane == 0) {
                    const size_t tp = (size_t)wrow * tokens + (size_t)b * T + t;
                    q.tok_eta[tp] = rsum * -(tk[u].e * kLn2);
                    q.tok_delta[tp] = psum;
                }
            }
        }
    }
#pragma unroll
    for (int j = 0; j < V; ++j)
        if (j < nvalid) {
            if (p.gh0r) {
                p.gh0r[b * M + d0 + j] = carry[j].r;
                p.gh0i[b * M + d0 + j] = carry[j].i;
            }
            const size_t mp = (size_t)b * M + d0 + j;
            q.mode_nu[mp] = acc[2 * j] * -(ln[j].nu2 * kLn2);
            q.mode_theta[mp] = acc[2 * j + 1] * ln[j].th;  // d/dtheta_log = theta d/dtheta
        }
}

// Tile shapes: Cfg<type, threads of 16 bytes per row, rows per thread,
// wavefronts, look-back window>.  Long sequences: 256 rows of 128-byte rows
// per array; measured on MI355X (bf16 B8 T2048 M2560) against 128 rows and
// 256-byte rows (8 or 4 rows per thread, 4 or 8 wavefronts), this shape was
// the fastest in both directions; the tile's fixed costs (ticket, look-back,
// barriers) dominate smaller tiles, whose bytes per tile are fewer than the
// real scan's because the transitions are not read.  The backward looks back
// over 2 tiles: with a window of 4 its registers spilled (144.7 -> 142.6 us).
// Short sequences: a tile no taller than the sequence, with wider rows to
// keep the bytes per tile up, as in the real scan -- 32 rows of 512-byte rows
// for T <= 32, 64 of them for T <= 64, 128 rows of 256-byte rows for
// T <= 128 (a 256-row tile over an 8-step sequence is 97% idle rows).
enum SamuShape { kSamuLong = 0, kSamuT32 = 1, kSamuT64 = 2, kSamuT128 = 3, kSamuT8 = 4, kSamuT16 = 5 };
template <int DT, int SH>
struct SamuShapeCfg;
template <int DT>
struct SamuShapeCfg<DT, kSamuLong> {
    using Fwd = Cfg<DT, 8, 8, 4, 4>;
    using Bwd = Cfg<DT, 8, 8, 4, 2>;
};
template <int DT>
struct SamuShapeCfg<DT, kSamuT8> {
    using Fwd = Cfg<DT, 32, 1, 4, 4>;
    using Bwd = Cfg<DT, 32, 1, 4, 2>;
};
template <int DT>
struct SamuShapeCfg<DT, kSamuT16> {
    using Fwd = Cfg<DT, 32, 2, 4, 4>;
    using Bwd = Cfg<DT, 32, 2, 4, 2>;
};
template <int DT>
struct SamuShapeCfg<DT, kSamuT32> {
    using Fwd = Cfg<DT, 32, 4, 4, 4>;
    using Bwd = Cfg<DT, 32, 4, 4, 2>;
};
template <int DT>
struct SamuShapeCfg<DT, kSamuT64> {
    using Fwd = Cfg<DT, 32, 8, 4, 4>;
    using Bwd = Cfg<DT, 32, 8, 4, 2>;
};
template <int DT>
struct SamuShapeCfg<DT, kSamuT128> {
    using Fwd = Cfg<DT, 16, 8, 4, 4>;
    using Bwd = Cfg<DT, 16, 8, 4, 2>;
};

// The shape for a problem (the same in both directions, so that the
// workspace and the partial sums are sized from the shape alone).  A row of
// lanes narrower than a wide tile row keeps the long shape.
int samu_shape(const Shape& s) {
    const int64_t row_bytes = s.D * (s.dtype == DT_F32 ? 4 : 2);
    if (s.T <= 8 && row_bytes >= 512) return kSamuT8;
    if (s.T <= 16 && row_bytes >= 512) return kSamuT16;
    if (s.T <= 32 && row_bytes >= 512) return kSamuT32;
    if (s.T <= 64 && row_bytes >= 512) return kSamuT64;
    if (s.T <= 128 && row_bytes >= 256) return kSamuT128;
    return kSamuLong;
}
// tiles of the shape: threads of 16 bytes per row and rows per tile
void samu_tile(int sh, int* tpr, int* ct) {
    switch (sh) {
        case kSamuT8: *tpr = 32; *ct = 8; return;
        case kSamuT16: *tpr = 32; *ct = 16; return;
        case kSamuT32: *tpr = 32; *ct = 32; return;
        case kSamuT64: *tpr = 32; *ct = 64; return;
        case kSamuT128: *tpr = 16; *ct = 128; return;
        default: *tpr = 8; *ct = 256; return;
    }
}
static_assert(SamuShapeCfg<DT_F32, kSamuT8>::Fwd::CT == 8 &&
                  SamuShapeCfg<DT_F32, kSamuT16>::Fwd::CT == 16 &&
                  SamuShapeCfg<DT_F32, kSamuT32>::Fwd::CT == 32 &&
                  SamuShapeCfg<DT_F32, kSamuT64>::Fwd::CT == 64 &&
                  SamuShapeCfg<DT_F32, kSamuT128>::Fwd::CT == 128 &&
                  SamuShapeCfg<DT_F32, kSamuLong>::Fwd::CT == 256,
              "tile heights");

// Both directions use the same rows per tile and row width.
Layout samu_layout(const Shape& s) {
    int tpr = 0, ct = 0;
    samu_tile(samu_shape(s), &tpr, &ct);
    return layout_of(s, tpr, ct);
}

// The auxiliary buffer: the mode table [M] and token table [B*T] (float4
// each), then, for the backward, the partial sums.
struct AuxLayout {
    size_t mode, tok, tok_part, mode_part, total;
};
size_t up256(size_t x) { return (x + 255) / 256 * 256; }
AuxLayout aux_layout(const Shape& s) {
    const Layout L = samu_layout(s);
    const size_t tokens = (size_t)s.B * s.T;
    AuxLayout a;
    a.mode = 0;
    a.tok = up256((size_t)s.D * 16);
    a.tok_part = a.tok + up256(tokens * 16);
    a.mode_part = a.tok_part + up256(2 * tokens * L.nW * 4);
    a.total = a.mode_part + up256(2 * (size_t)L.NK * s.B * s.D * 4);
    return a;
}

template <int DT>
hipError_t samu_factors(const Shape& s, const void* eta, const void* delta, const float* nu_log,
                        const float* theta_log, char* aux, hipStream_t st) {
    const AuxLayout a = aux_layout(s);
    const int64_t tokens = s.B * s.T;
    const int64_t n = std::max<int64_t>(tokens, s.D);
    hipLaunchKernelGGL((samu_factor_kernel<DT>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       st, eta, delta, nu_log, theta_log, tokens, s.D,
                       reinterpret_cast<float4*>(aux + a.tok),
                       reinterpret_cast<float4*>(aux + a.mode));
    return hipGetLastError();
}

template <int DT, class C>
hipError_t samu_fwd_t(const Shape& s, const SamuFwdPtrs& p, void* ws, size_t ws_bytes, bool init,
                      void* auxp, int polls, hipStream_t st) {
    const Layout L = samu_layout(s);
    char* aux = static_cast<char*>(auxp);
    const AuxLayout a = aux_layout(s);
    SamuFwdArgs x;
    x.p = p;
    x.mode_tab = reinterpret_cast<const float4*>(aux + a.mode);
    x.tok_tab = reinterpret_cast<const float4*>(aux + a.tok);
    hipError_t e = samu_factors<DT>(s, p.eta, p.delta, p.nu_log, p.theta_log, aux, st);
    if (e != hipSuccess) return e;
    e = prepare(ws, ws_bytes, init, L, kComplexWords, st, &x.sc);
    if (e != hipSuccess) return e;
    x.d = Dims{(int)s.T, (int)s.D, L.nW, L.nS, L.NK};
    x.polls = polls > 0 ? (uint32_t)polls : kDefaultPolls;
    const void* ptrs[4] = {p.br, p.bi, p.out_r, p.out_i};
    const bool al = rows_aligned(s, ptrs, 4);
    const dim3 grid(x.sc.total_tiles), block(C::NT);
    const bool out = p.out_r != nullptr;
    dispatch2(al, p.reset != nullptr, [&](auto AL, auto RS) {
        constexpr bool a_ = decltype(AL)::value, r_ = decltype(RS)::value;
        if (out) hipLaunchKernelGGL((samu_fwd_kernel<C, a_, r_, true>), grid, block, 0, st, x);
        else hipLaunchKernelGGL((samu_fwd_kernel<C, a_, r_, false>), grid, block, 0, st, x);
    });
    return hipGetLastError();
}

template <int DT, class C>
hipError_t samu_bwd_t(const Shape& s, const SamuBwdPtrs& p, void* ws, size_t ws_bytes, bool init,
                      void* auxp, int polls, hipStream_t st) {
    const Layout L = samu_layout(s);
    char* aux = static_cast<char*>(auxp);
    const AuxLayout a = aux_layout(s);
    SamuBwdArgs x;
    x.p = p;
    x.mode_tab = reinterpret_cast<const float4*>(aux + a.mode);
    x.tok_tab = reinterpret_cast<const float4*>(aux + a.tok);
    hipError_t e = samu_factors<DT>(s, p.eta, p.delta, p.nu_log, p.theta_log, aux, st);
    if (e != hipSuccess) return e;
    e = prepare(ws, ws_bytes, init, L, kComplexWords, st, &x.sc);
    if (e != hipSuccess) return e;
    x.d = Dims{(int)s.T, (int)s.D, L.nW, L.nS, L.NK};
    x.polls = polls > 0 ? (uint32_t)polls : kDefaultPolls;
    const size_t tokens = (size_t)s.B * s.T;
    const size_t nmode = (size_t)L.NK * s.B * s.D;
    x.tokens = tokens;
    x.tok_eta = reinterpret_cast<float*>(aux + a.tok_part);
    x.tok_delta = x.tok_eta + tokens * L.nW;
    x.mode_nu = reinterpret_cast<float*>(aux + a.mode_part);
    x.mode_theta = x.mode_nu + nmode;
    const void* ptrs[6] = {p.hr, p.hi, p.gr, p.gi, p.gbr, p.gbi};
    const bool al = rows_aligned(s, ptrs, 6);
    dispatch2(al, p.reset != nullptr, [&](auto AL, auto RS) {
        hipLaunchKernelGGL((samu_bwd_kernel<C, decltype(AL)::value, decltype(RS)::value>),
                           dim3(x.sc.total_tiles), dim3(C::NT), 0, st, x);
    });
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // grad_eta / grad_delta: a token's nW lane-block partials; grad_nu_log /
    // grad_theta_log: a mode's NK*B tile partials
    const SumJob jt{x.tok_eta, x.tok_delta, p.grad_eta, p.grad_delta, (int64_t)tokens,
                    (int64_t)L.nW};
    const SumJob jm{x.mode_nu, x.mode_theta, p.grad_nu_log, p.grad_theta_log, s.D,
                    (int64_t)L.NK * s.B};
    const unsigned bt = (unsigned)((tokens + kSumLanes - 1) / kSumLanes);
    const unsigned bm = (unsigned)((s.D + kSumLanes - 1) / kSumLanes);
    hipLaunchKernelGGL(samu_reduce_kernel, dim3(bt + bm), dim3(kSumLanes * kSumSlices), 0, st, jt,
                       jm, bt);
    return hipGetLastError();
}

template <int DT>
hipError_t samu_seq_fwd_t(const Shape& s, const SamuFwdPtrs& p, void* auxp, hipStream_t st) {
    char* aux = static_cast<char*>(auxp);
    const AuxLayout a = aux_layout(s);
    hipError_t e = samu_factors<DT>(s, p.eta, p.delta, p.nu_log, p.theta_log, aux, st);
    if (e != hipSuccess) return e;
    const float4* mode_tab = reinterpret_cast<const float4*>(aux + a.mode);
    const float4* tok_tab = reinterpret_cast<const float4*>(aux + a.tok);
    const int64_t vpr = (s.D + Elem<DT>::V - 1) / Elem<DT>::V;
    const int64_t blocks = (s.B * vpr + kSamuSeqBlock - 1) / kSamuSeqBlock;
    if (blocks >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    const void* ptrs[4] = {p.br, p.bi, p.out_r, p.out_i};
    const bool al = rows_aligned(s, ptrs, 4);
    dispatch2(al, p.reset != nullptr, [&](auto AL, auto RS) {
        hipLaunchKernelGGL((samu_seq_fwd_kernel<DT, decltype(AL)::value, decltype(RS)::value>),
                           dim3((unsigned)blocks), dim3(kSamuSeqBlock), 0, st, p, tok_tab,
                           mode_tab, s.B, s.T, s.D, vpr);
    });
    return hipGetLastError();
}

template <int DT>
hipError_t samu_seq_bwd_t(const Shape& s, const SamuBwdPtrs& p, void* auxp, hipStream_t st) {
    char* aux = static_cast<char*>(auxp);
    const AuxLayout a = aux_layout(s);
    hipError_t e = samu_factors<DT>(s, p.eta, p.delta, p.nu_log, p.theta_log, aux, st);
    if (e != hipSuccess) return e;
    const float4* mode_tab = reinterpret_cast<const float4*>(aux + a.mode);
    const float4* tok_tab = reinterpret_cast<const float4*>(aux + a.tok);
    const int64_t vpr = (s.D + Elem<DT>::V - 1) / Elem<DT>::V;
    const int64_t tpr = (vpr + kWave - 1) / kWave * kWave;  // a row's threads, whole wavefronts
    const int64_t nww = tpr / kWave;
    // the partial sums fit where the tiles keep theirs: at most as many
    // per-token slots (wavefronts of 64 vectors against tile rows of at most
    // 32) and per-mode slots (B against tiles * B)
    const Layout L = samu_layout(s);
    if (nww > L.nW) return hipErrorInvalidValue;
    const int64_t blocks = (s.B * tpr + kSamuSeqBlock - 1) / kSamuSeqBlock;
    if (blocks >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    const size_t tokens = (size_t)s.B * s.T;
    SamuSeqParts q;
    q.tok_eta = reinterpret_cast<float*>(aux + a.tok_part);
    q.tok_delta = q.tok_eta + tokens * nww;
    q.mode_nu = reinterpret_cast<float*>(aux + a.mode_part);
    q.mode_theta = q.mode_nu + (size_t)s.B * s.D;
    const void* ptrs[6] = {p.hr, p.hi, p.gr, p.gi, p.gbr, p.gbi};
    const bool al = rows_aligned(s, ptrs, 6);
    dispatch2(al, p.reset != nullptr, [&](auto AL, auto RS) {
        hipLaunchKernelGGL((samu_seq_bwd_kernel<DT, decltype(AL)::value, decltype(RS)::value>),
                           dim3((unsigned)blocks), dim3(kSamuSeqBlock), 0, st, p, tok_tab,
                           mode_tab, q, s.B, s.T, s.D, tpr);
    });
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // grad_eta / grad_delta: a token's partials over the row's wavefronts;
    // grad_nu_log / grad_theta_log: a mode's partials over the batch rows
    const SumJob jt{q.tok_eta, q.tok_delta, p.grad_eta, p.grad_delta, (int64_t)tokens, nww};
    const SumJob jm{q.mode_nu, q.mode_theta, p.grad_nu_log, p.grad_theta_log, s.D, s.B};
    const unsigned bt = (unsigned)((tokens + kSumLanes - 1) / kSumLanes);
    const unsigned bm = (unsigned)((s.D + kSumLanes - 1) / kSumLanes);
    hipLaunchKernelGGL(samu_reduce_kernel, dim3(bt + bm), dim3(kSumLanes * kSumSlices), 0, st, jt,
                       jm, bt);
    return hipGetLastError();
}

}  // namespace

bool samu_supported(const Shape& s) {
    int tpr = 0, ct = 0;
    samu_tile(samu_shape(s), &tpr, &ct);
    return tiled_layout_ok(s, ct, 4 * kWave, samu_layout(s));
}

size_t samu_scratch_bytes(const Shape& s) {
    return kHeaderBytes + 2 * region_bytes_for(samu_layout(s), kComplexWords);
}

size_t samu_aux_bytes(const Shape& s) { return aux_layout(s).total; }

namespace {
template <int DT>
hipError_t samu_fwd_shape(const Shape& s, const SamuFwdPtrs& p, void* ws, size_t ws_bytes,
                          bool init, void* aux, int polls, hipStream_t st) {
    switch (samu_shape(s)) {
        case kSamuT8:
            return samu_fwd_t<DT, typename SamuShapeCfg<DT, kSamuT8>::Fwd>(s, p, ws, ws_bytes,
                                                                           init, aux, polls, st);
        case kSamuT16:
            return samu_fwd_t<DT, typename SamuShapeCfg<DT, kSamuT16>::Fwd>(s, p, ws, ws_bytes,
                                                                            init, aux, polls, st);
        case kSamuT32:
            return samu_fwd_t<DT, typename SamuShapeCfg<DT, kSamuT32>::Fwd>(s, p, ws, ws_bytes,
                                                                            init, aux, polls, st);
        case kSamuT64:
            return samu_fwd_t<DT, typename SamuShapeCfg<DT, kSamuT64>::Fwd>(s, p, ws, ws_bytes,
                                                                            init, aux, polls, st);
        case kSamuT128:
            return samu_fwd_t<DT, typename SamuShapeCfg<DT, kSamuT128>::Fwd>(s, p, ws, ws_bytes,
                                                                             init, aux, polls, st);
        default:
            return samu_fwd_t<DT, typename SamuShapeCfg<DT, kSamuLong>::Fwd>(s, p, ws, ws_bytes,
                                                                             init, aux, polls, st);
    }
}
template <int DT>
hipError_t samu_bwd_shape(const Shape& s, const SamuBwdPtrs& p, void* ws, size_t ws_bytes,
                          bool init, void* aux, int polls, hipStream_t st) {
    switch (samu_shape(s)) {
        case kSamuT8:
            return samu_bwd_t<DT, typename SamuShapeCfg<DT, kSamuT8>::Bwd>(s, p, ws, ws_bytes,
                                                                           init, aux, polls, st);
        case kSamuT16:
            return samu_bwd_t<DT, typename SamuShapeCfg<DT, kSamuT16>::Bwd>(s, p, ws, ws_bytes,
                                                                            init, aux, polls, st);
        case kSamuT32:
            return samu_bwd_t<DT, typename SamuShapeCfg<DT, kSamuT32>::Bwd>(s, p, ws, ws_bytes,
                                                                            init, aux, polls, st);
        case kSamuT64:
            return samu_bwd_t<DT, typename SamuShapeCfg<DT, kSamuT64>::Bwd>(s, p, ws, ws_bytes,
                                                                            init, aux, polls, st);
        case kSamuT128:
            return samu_bwd_t<DT, typename SamuShapeCfg<DT, kSamuT128>::Bwd>(s, p, ws, ws_bytes,
                                                                             init, aux, polls, st);
        default:
            return samu_bwd_t<DT, typename SamuShapeCfg<DT, kSamuLong>::Bwd>(s, p, ws, ws_bytes,
                                                                             init, aux, polls, st);
    }
}
}  // namespace

hipError_t launch_samu_fwd(const Shape& s, const SamuFwdPtrs& p, void* ws, size_t ws_bytes,
                           bool init, void* aux, int polls, hipStream_t st) {
    return s.dtype == DT_F32 ? samu_fwd_shape<DT_F32>(s, p, ws, ws_bytes, init, aux, polls, st)
                             : samu_fwd_shape<DT_BF16>(s, p, ws, ws_bytes, init, aux, polls, st);
}

hipError_t launch_samu_bwd(const Shape& s, const SamuBwdPtrs& p, void* ws, size_t ws_bytes,
                           bool init, void* aux, int polls, hipStream_t st) {
    return s.dtype == DT_F32 ? samu_bwd_shape<DT_F32>(s, p, ws, ws_bytes, init, aux, polls, st)
                             : samu_bwd_shape<DT_BF16>(s, p, ws, ws_bytes, init, aux, polls, st);
}

hipError_t launch_samu_seq_fwd(const Shape& s, const SamuFwdPtrs& p, void* aux, hipStream_t st) {
    return s.dtype == DT_F32 ? samu_seq_fwd_t<DT_F32>(s, p, aux, st)
                             : samu_seq_fwd_t<DT_BF16>(s, p, aux, st);
}

hipError_t launch_samu_seq_bwd(const Shape& s, const SamuBwdPtrs& p, void* aux, hipStream_t st) {
    return s.dtype == DT_F32 ? samu_seq_bwd_t<DT_F32>(s, p, aux, st)
                             : samu_seq_bwd_t<DT_BF16>(s, p, aux, st);
}

}  // namespace lrscan
