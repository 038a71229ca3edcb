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
    float nu, th, ct, st;  // nu, theta, cos theta, sin theta
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
        mode_tab[i] = make_float4(expf(nu_log[i]), th, ct, st);
    }
}

// a = exp(-nu e^eta) e^{i (theta + delta)}, by angle addition.
__device__ __forceinline__ Cx samu_a(const SamuLane& L, const SamuTok& k) {
    const float cosine = fmaf(L.ct, k.cd, -(L.st * k.sd));
    const float sine = fmaf(L.st, k.cd, L.ct * k.sd);
    const float rho = expf(-(L.nu * k.e));
    return Cx{rho * cosine, rho * sine};
}

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

// Derived tile maps for the look-back (same operation order as the owners).
template <class C>
__device__ CAff samu_fwd_tile_map(const SamuFwdArgs& x, int j, int bi, int col) {
    constexpr int RG = C::RG, NR = C::NR;
    CAff A = caff_identity();
    if (col >= x.d.D) return A;
    const SamuLane L = samu_lane(x.mode_tab, col);
    const size_t rowbytes = (size_t)x.d.D * C::EB;
    const size_t b0 = (size_t)bi * x.d.T * rowbytes;
    const char* br = static_cast<const char*>(x.p.br) + b0;
    const char* bim = static_cast<const char*>(x.p.bi) + b0;
    const uint32_t coff = (uint32_t)col * C::EB;
#pragma unroll 1
    for (int w = 0; w < C::WAVES; ++w) {
        TreeFold<RG, CAff, CAffThen> tree;
#pragma unroll
        for (int g = 0; g < RG; ++g) {
            CAff t = caff_identity();
            const int r0 = j * C::CT + (w * RG + g) * NR;
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
            tree.push(g, t);
        }
        A = caff_then(A, tree.total());
    }
    return CAff{unpack_cx(pack_cx(A.p)), unpack_cx(pack_cx(A.q))};
}

template <class C>
__device__ CAff samu_bwd_tile_map(const SamuBwdArgs& x, int j, int bi, int col) {
    constexpr int RG = C::RG, NR = C::NR;
    CAff A = caff_identity();
    if (col >= x.d.D) return A;
    const SamuLane L = samu_lane(x.mode_tab, col);
    const size_t rowbytes = (size_t)x.d.D * C::EB;
    const size_t b0 = (size_t)bi * x.d.T * rowbytes;
    const char* gr = static_cast<const char*>(x.p.gr) + b0;
    const char* gi = static_cast<const char*>(x.p.gi) + b0;
    const uint32_t coff = (uint32_t)col * C::EB;
#pragma unroll 1
    for (int w = C::WAVES - 1; w >= 0; --w) {
        TreeFold<RG, CAff, CAffThen> tree;
#pragma unroll
        for (int g = RG - 1; g >= 0; --g) {
            CAff t = caff_identity();
            const int r0 = j * C::CT + (w * RG + g) * NR;
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
            tree.push(RG - 1 - g, t);
        }
        A = caff_then(A, tree.total());
    }
    return CAff{unpack_cx(pack_cx(A.p)), unpack_cx(pack_cx(A.q))};
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
template <class C, bool ALIGNED, bool RST, bool OUT>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(2)))
void samu_fwd_kernel(SamuFwdArgs x) {
    constexpr int V = C::V, W = C::W, RG = C::RG, NR = C::NR, WAVES = C::WAVES, TPR = C::TPR;
    __shared__ CAff s_excl[WAVES][V][kWave];
    __shared__ CAff s_wtot[WAVES][W];
    __shared__ Cx s_hin[W];

    const Dims d = x.d;
    const int tid = threadIdx.x;
    const int wave = uniform((int)(threadIdx.x / kWave));
    const int l = tid % kWave;
    const int rg = l / TPR;
    const int cg = l % TPR;
    const Ticket tk = take_ticket(x.sc);
    const Geo g = tile_geo<C, false>(tk.ticket, d, wave, rg, cg);
    const uint32_t rowbytes = (uint32_t)d.D * C::EB;
    const char* pbr = static_cast<const char*>(x.p.br) + g.tbase;
    const char* pbi = static_cast<const char*>(x.p.bi) + g.tbase;

    RowVec<C::DT> br[NR], bi[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const uint32_t off = row_off(g, g.row0 + i, d.T, rowbytes);
        br[i] = load_vec<C::DT, ALIGNED>(pbr, off, g.nvalid, 0.0f);
        bi[i] = load_vec<C::DT, ALIGNED>(pbi, off, g.nvalid, 0.0f);
    }
    // per-token and per-mode factors of this thread's rows and lanes (rows
    // past T and lanes past M read the last valid one; never used)
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
    clear_share(x.sc, tk.phase, tk.nclear, C::NT, tk.ticket);
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
        for (int i = 0; i < NR; ++i) {
            const bool ok = i < g.nrows;
            const Cx at = ok ? trans(i, j) : Cx{1.0f, 0.0f};
            const Cx bt = ok ? vget(br[i], bi[i], j) : Cx{0.0f, 0.0f};
            m = caff_then(m, fwd_step(at, bt));
        }
        const CAff inc = cwave_scan_up<TPR>(m);
        CAff ex = cshfl_up<TPR>(inc);
        if (rg == 0) ex = caff_identity();
        s_excl[wave][j][l] = ex;
        if (rg == RG - 1) s_wtot[wave][cg * V + j] = inc;
    }
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        opaque(br[i]);
        opaque(bi[i]);
    }
    __syncthreads();

    if (tid < W) {
        const int c = tid;
        const CxWords wd = cx_words(x.sc, tk.phase);
        CAff A = caff_identity();
#pragma unroll
        for (int w = 0; w < WAVES; ++w) A = caff_then(A, s_wtot[w][c]);
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
        const Cx hin = look_back<ComplexLink, -1, C::LB>(
            lk, g.k, d.NK, base0, x.polls, [&](int j) { return samu_fwd_tile_map<C>(x, j, g.bi, dl); });
        if (more) publish_u64(wd.hs + o, pack_cx(caff_apply(A, hin)));
        s_hin[c] = hin;
    }
    __syncthreads();

    const bool ends = g.nrows > 0 && g.row0 + g.nrows == d.T;
    if constexpr (!OUT) {
        if (!(x.p.last_r && ends)) return;
    }
    char* por = static_cast<char*>(x.p.out_r) + g.tbase;
    char* poi = static_cast<char*>(x.p.out_i) + g.tbase;
    Cx h[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
        const int col = cg * V + j;
        Cx xv = s_hin[col];
        for (int w = 0; w < wave; ++w) xv = caff_apply(s_wtot[w][col], xv);
        h[j] = caff_apply(s_excl[wave][j][l], xv);
    }
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        if (i < g.nrows) {
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
            if (j < g.nvalid) {
                x.p.last_r[(size_t)g.bi * d.D + g.d0 + j] = h[j].r;
                x.p.last_i[(size_t)g.bi * d.D + g.d0 + j] = h[j].i;
            }
    }
}

// Sum over the TPR lanes of one row group (every lane gets the total; the
// butterfly has the same association in every lane).
template <int TPR>
__device__ __forceinline__ float row_sum(float v) {
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
// Sum over the row groups of a wavefront (lanes with the same column).
template <int TPR>
__device__ __forceinline__ float col_sum(float v) {
#pragma unroll
    for (int o = TPR; o < kWave; o <<= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// ---------------------------------------------------------------------------
// reverse time
// ---------------------------------------------------------------------------
template <class C, bool ALIGNED, bool RST>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(2)))
void samu_bwd_kernel(SamuBwdArgs x) {
    constexpr int V = C::V, W = C::W, RG = C::RG, NR = C::NR, WAVES = C::WAVES, TPR = C::TPR;
    __shared__ CAff s_excl[WAVES][V][kWave];
    __shared__ CAff s_wtot[WAVES][W];
    __shared__ Cx s_cin[W];
    __shared__ float s_acc[2][WAVES][W];

    const Dims d = x.d;
    const int tid = threadIdx.x;
    const int wave = uniform((int)(threadIdx.x / kWave));
    const int l = tid % kWave;
    const int rg = l / TPR;
    const int cg = l % TPR;
    const Ticket tk = take_ticket(x.sc);
    const Geo g = tile_geo<C, true>(tk.ticket, d, wave, rg, cg);
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
        const int row = g.row0 + i;
        const int rc = row < d.T ? row : d.T - 1;
        const int hrw = rc >= 1 ? rc - 1 : 0;
        const uint32_t off = (uint32_t)(rc - g.trow0) * rowbytes + g.coff;
        const uint32_t hoff = (uint32_t)(hrw - hrow0) * rowbytes + g.coff;
        gr[i] = load_vec<C::DT, ALIGNED>(pgr, off, g.nvalid, 0.0f);
        gi[i] = load_vec<C::DT, ALIGNED>(pgi, off, g.nvalid, 0.0f);
        hr[i] = load_vec<C::DT, ALIGNED>(phr, hoff, g.nvalid, 0.0f);
        hi[i] = load_vec<C::DT, ALIGNED>(phi, hoff, g.nvalid, 0.0f);
    }
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
    clear_share(x.sc, tk.phase, tk.nclear, C::NT, tk.ticket);
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
        const CAff inc = cwave_scan_down<TPR>(m);
        CAff ex = cshfl_down_n(inc, TPR);
        if (rg == RG - 1) ex = caff_identity();
        s_excl[wave][j][l] = ex;
        if (rg == 0) s_wtot[wave][cg * V + j] = inc;
    }
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        opaque(gr[i]);
        opaque(gi[i]);
    }
    __syncthreads();

    if (tid < W) {
        const int c = tid;
        const CxWords wd = cx_words(x.sc, tk.phase);
        CAff A = caff_identity();
#pragma unroll
        for (int w = WAVES - 1; w >= 0; --w) A = caff_then(A, s_wtot[w][c]);
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
        const Cx cin = look_back<ComplexLink, +1, C::LB>(
            lk, g.k, d.NK, base0, x.polls, [&](int j) { return samu_bwd_tile_map<C>(x, j, g.bi, dl); });
        if (more) publish_u64(wd.hs + o, pack_cx(caff_apply(A, cin)));
        s_cin[c] = cin;
    }
    __syncthreads();

    char* pgbr = static_cast<char*>(x.p.gbr) + g.tbase;
    char* pgbi = static_cast<char*>(x.p.gbi) + g.tbase;
    Cx carry[V];
    float acc_nu[V], acc_th[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
        const int col = cg * V + j;
        Cx xv = s_cin[col];
        for (int w = WAVES - 1; w > wave; --w) xv = caff_apply(s_wtot[w][col], xv);
        carry[j] = caff_apply(s_excl[wave][j][l], xv);
        acc_nu[j] = 0.0f;
        acc_th[j] = 0.0f;
    }
    const int lb = g.s - g.bi * d.nW;  // lane block of this tile
#pragma unroll
    for (int i = NR - 1; i >= 0; --i) {
        const int row = g.row0 + i;
        if (row < d.T) {  // the same for every lane of a row group
            RowOut<C::DT> obr, obi;
            float rsum = 0.0f, psum = 0.0f;
#pragma unroll
            for (int j = 0; j < V; ++j) {
                const Cx at = trans(i, j);
                const Cx lam = cadd(vget(gr[i], gi[i], j), carry[j]);
                Cx hp = vget(hr[i], hi[i], j);
                if (row == 0) {
                    hp = Cx{0.0f, 0.0f};
                    if (x.p.h0r && j < g.nvalid)
                        hp = Cx{x.p.h0r[(size_t)g.bi * d.D + g.d0 + j],
                                x.p.h0i[(size_t)g.bi * d.D + g.d0 + j]};
                }
                const bool rs = RST && ((rbits >> i) & 1u);
                const Cx ga = rs ? Cx{0.0f, 0.0f} : cmul(lam, cconj(hp));
                const Cx w = cmul(cconj(at), ga);
                const bool live = j < g.nvalid;
                const float radial = live ? -(ln[j].nu * tok[i].e) * w.r : 0.0f;
                const float phase = live ? w.i : 0.0f;
                rsum += radial;
                psum += phase;
                acc_nu[j] += radial;
                acc_th[j] += ln[j].th * phase;
                obr.v[j] = lam.r;
                obi.v[j] = lam.i;
                carry[j] = cmul(cconj(at), lam);
            }
            if (g.nvalid > 0) {
                const uint32_t off = row_off(g, row, d.T, rowbytes);
                store_vec<C::DT, ALIGNED>(pgbr, off, g.nvalid, obr);
                store_vec<C::DT, ALIGNED>(pgbi, off, g.nvalid, obi);
            }
            rsum = row_sum<TPR>(rsum);
            psum = row_sum<TPR>(psum);
            if (cg == 0) {
                const size_t tp = (size_t)lb * x.tokens + (size_t)g.bi * d.T + row;
                x.tok_eta[tp] = rsum;
                x.tok_delta[tp] = psum;
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
    // per-mode partials of this tile: over the row groups, then the waves
#pragma unroll
    for (int j = 0; j < V; ++j) {
        const float nu = col_sum<TPR>(acc_nu[j]);
        const float th = col_sum<TPR>(acc_th[j]);
        if (rg == 0) {
            s_acc[0][wave][cg * V + j] = nu;
            s_acc[1][wave][cg * V + j] = th;
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
            x.mode_theta[mp] = th;
        }
    }
}

// grad_eta / grad_delta: sum of a token's nW lane-block partials in order;
// grad_nu_log / grad_theta_log: sum of a mode's NK*B tile partials in order.
__global__ void samu_reduce_kernel(const float* __restrict__ tok_eta,
                                   const float* __restrict__ tok_delta,
                                   const float* __restrict__ mode_nu,
                                   const float* __restrict__ mode_theta, float* grad_eta,
                                   float* grad_delta, float* grad_nu_log, float* grad_theta_log,
                                   int64_t tokens, int nW, int64_t tiles, int64_t M) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < tokens) {
        float e = 0.0f, dl = 0.0f;
        for (int w = 0; w < nW; ++w) {
            e += tok_eta[(int64_t)w * tokens + i];
            dl += tok_delta[(int64_t)w * tokens + i];
        }
        if (grad_eta) grad_eta[i] = e;
        if (grad_delta) grad_delta[i] = dl;
    }
    if (i < M) {
        float n = 0.0f, t = 0.0f;
        for (int64_t k = 0; k < tiles; ++k) {
            n += mode_nu[k * M + i];
            t += mode_theta[k * M + i];
        }
        if (grad_nu_log) grad_nu_log[i] = n;
        if (grad_theta_log) grad_theta_log[i] = t;
    }
}

template <class F>
void dispatch2(bool al, bool rst, F&& f) {
    if (al && rst) f(std::true_type{}, std::true_type{});
    else if (al) f(std::true_type{}, std::false_type{});
    else if (rst) f(std::false_type{}, std::true_type{});
    else f(std::false_type{}, std::false_type{});
}

template <int DT>
using SamuCfg = Cfg<DT, kComplexWidth, 4, 4, 4>;  // 128 rows, as the complex form

Layout samu_layout(const Shape& s) { return layout_of(s, kComplexWidth, kComplexTile); }

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

template <int DT>
hipError_t samu_fwd_t(const Shape& s, const SamuFwdPtrs& p, void* ws, size_t ws_bytes, bool init,
                      void* auxp, int polls, hipStream_t st) {
    using C = SamuCfg<DT>;
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

template <int DT>
hipError_t samu_bwd_t(const Shape& s, const SamuBwdPtrs& p, void* ws, size_t ws_bytes, bool init,
                      void* auxp, int polls, hipStream_t st) {
    using C = SamuCfg<DT>;
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
    const int64_t n = std::max<int64_t>((int64_t)tokens, s.D);
    hipLaunchKernelGGL(samu_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       x.tok_eta, x.tok_delta, x.mode_nu, x.mode_theta, p.grad_eta, p.grad_delta,
                       p.grad_nu_log, p.grad_theta_log, (int64_t)tokens, L.nW,
                       (int64_t)L.NK * s.B, s.D);
    return hipGetLastError();
}

}  // namespace

bool samu_supported(const Shape& s) { return complex_fused_supported(s); }

size_t samu_scratch_bytes(const Shape& s) {
    return kHeaderBytes + 2 * region_bytes_for(samu_layout(s), kComplexWords);
}

size_t samu_aux_bytes(const Shape& s) { return aux_layout(s).total; }

hipError_t launch_samu_fwd(const Shape& s, const SamuFwdPtrs& p, void* ws, size_t ws_bytes,
                           bool init, void* aux, int polls, hipStream_t st) {
    return s.dtype == DT_F32 ? samu_fwd_t<DT_F32>(s, p, ws, ws_bytes, init, aux, polls, st)
                             : samu_fwd_t<DT_BF16>(s, p, ws, ws_bytes, init, aux, polls, st);
}

hipError_t launch_samu_bwd(const Shape& s, const SamuBwdPtrs& p, void* ws, size_t ws_bytes,
                           bool init, void* aux, int polls, hipStream_t st) {
    return s.dtype == DT_F32 ? samu_bwd_t<DT_F32>(s, p, ws, ws_bytes, init, aux, polls, st)
                             : samu_bwd_t<DT_BF16>(s, p, ws, ws_bytes, init, aux, polls, st);
}

}  // namespace lrscan
