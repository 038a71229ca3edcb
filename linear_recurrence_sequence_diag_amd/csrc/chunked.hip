// chunked.hip -- the three-launch chunked scan, forward and reverse time.
//
// Page "triton_training_scan.py": _real_chunk_summary / _real_chunk_prefix /
// _real_chunk_replay and the _real_reverse_chunk_* trio.  The sequence of
// every lane is cut into chunks of C steps; a chunk is summarised by the
// affine map h -> P h + Q (summary), the maps are scanned over the chunk axis
// into the state entering every chunk (prefix), and every chunk is rescanned
// from that state (replay).  The reverse-time trio does the same for the
// adjoint, whose carry flows from later chunks to earlier ones.
//
// Summary and replay: one thread per (batch row, chunk, 16-byte lane vector)
// walks the C steps of its chunk with all of the chunk's loads issued ahead
// (blocks of U rows).  Steps past T are identity steps (a = 1, b = 0, g = 0).
//
// Prefix: the chunk axis of 16 adjacent lanes is cut into 32 segments (4 per
// wavefront x 8 wavefronts); each thread folds its segment's maps, the
// segments of a wavefront are combined with an in-wavefront scan, the
// wavefronts through LDS, and every thread then rewalks its segment from the
// state entering it.
#include <type_traits>

#include "device.hpp"
#include "launch.hpp"

namespace lrscan {

namespace {

constexpr int kBlk = 256;
constexpr int kU = 16;  // rows loaded ahead per block

__device__ __forceinline__ void store_vecf(float* p, size_t off, int nvalid, const float* v, int V,
                                           bool aligned) {
    if (aligned) {
        for (int j = 0; j < V; j += 4)
            *reinterpret_cast<float4*>(p + off + j) = make_float4(v[j], v[j + 1], v[j + 2], v[j + 3]);
    } else {
        for (int j = 0; j < V; ++j)
            if (j < nvalid) p[off + j] = v[j];
    }
}

__device__ __forceinline__ void load_vecf(const float* p, size_t off, int nvalid, float* v, int V,
                                          bool aligned, float fill) {
    if (aligned) {
        for (int j = 0; j < V; j += 4) {
            const float4 x = *reinterpret_cast<const float4*>(p + off + j);
            v[j] = x.x;
            v[j + 1] = x.y;
            v[j + 2] = x.z;
            v[j + 3] = x.w;
        }
    } else {
        for (int j = 0; j < V; ++j) v[j] = (j < nvalid) ? p[off + j] : fill;
    }
}

struct ChunkIdx {
    int64_t bi, k, d0;
    int nvalid;
    bool ok;
};

template <int DT>
__device__ __forceinline__ ChunkIdx chunk_index(int64_t B, int64_t NC, int64_t D) {
    constexpr int V = Elem<DT>::V;
    const int64_t vpr = (D + V - 1) / V;
    const int64_t gid = (int64_t)blockIdx.x * kBlk + threadIdx.x;
    ChunkIdx c;
    const int64_t vi = gid % vpr;
    const int64_t rest = gid / vpr;
    c.k = rest % NC;
    c.bi = rest / NC;
    c.d0 = vi * V;
    c.nvalid = (int)((D - c.d0) < V ? (D - c.d0) : V);
    c.ok = c.bi < B;
    return c;
}

// ---------------------------------------------------------------------------
// forward summary: P = prod a, Q = chunk scanned from zero
// ---------------------------------------------------------------------------
// RST (every kernel below): `reset` ([B, T] bytes) marks segment starts,
// where the step's transition is taken as 0.
template <int DT, bool ALIGNED, bool RST>
__global__ __launch_bounds__(kBlk) void chunk_summary_kernel(const void* __restrict__ a,
                                                             const void* __restrict__ b,
                                                             const uint8_t* __restrict__ reset,
                                                             float* __restrict__ P,
                                                             float* __restrict__ Q, int64_t B,
                                                             int64_t T, int64_t D, int C) {
    constexpr int V = Elem<DT>::V;
    const int64_t NC = (T + C - 1) / C;
    const ChunkIdx ci = chunk_index<DT>(B, NC, D);
    if (!ci.ok) return;
    const size_t base = ((size_t)ci.bi * T) * D + ci.d0;
    float p[V], q[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
        p[j] = 1.0f;
        q[j] = 0.0f;
    }
    const int64_t t_begin = ci.k * C;
    const int64_t t_end = (t_begin + C < T) ? t_begin + C : T;
    const uint8_t* rrow = RST ? reset + (size_t)ci.bi * T : nullptr;
    for (int64_t t0 = t_begin; t0 < t_end; t0 += kU) {
        RowVec<DT> ra[kU], rb[kU];
        uint32_t rr[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u)
            if (t0 + u < t_end) {
                ra[u] = load_row<DT, ALIGNED>(a, base + (size_t)(t0 + u) * D, ci.nvalid, 1.0f);
                rb[u] = load_row<DT, ALIGNED>(b, base + (size_t)(t0 + u) * D, ci.nvalid, 0.0f);
                if (RST) rr[u] = rrow[t0 + u];
            }
#pragma unroll
        for (int u = 0; u < kU; ++u)
            if (t0 + u < t_end) {
#pragma unroll
                for (int j = 0; j < V; ++j) {
                    const float at = (RST && rr[u]) ? 0.0f : ra[u].get(j);
                    p[j] = at * p[j];
                    q[j] = fmaf(at, q[j], rb[u].get(j));
                }
            }
    }
    const size_t so = ((size_t)ci.bi * NC + ci.k) * D + ci.d0;
    store_vecf(P, so, ci.nvalid, p, V, ALIGNED);
    store_vecf(Q, so, ci.nvalid, q, V, ALIGNED);
}

// ---------------------------------------------------------------------------
// forward replay: rescan each chunk from chunk_in
// ---------------------------------------------------------------------------
template <int DT, bool ALIGNED, bool RST>
__global__ __launch_bounds__(kBlk) void chunk_replay_kernel(
    const void* __restrict__ a, const void* __restrict__ b, const uint8_t* __restrict__ reset,
    const float* __restrict__ chunk_in, void* __restrict__ out, float* __restrict__ last,
    int64_t B, int64_t T, int64_t D, int C) {
    constexpr int V = Elem<DT>::V;
    const int64_t NC = (T + C - 1) / C;
    const ChunkIdx ci = chunk_index<DT>(B, NC, D);
    if (!ci.ok) return;
    const size_t base = ((size_t)ci.bi * T) * D + ci.d0;
    float h[V];
    load_vecf(chunk_in, ((size_t)ci.bi * NC + ci.k) * D + ci.d0, ci.nvalid, h, V, ALIGNED, 0.0f);
    const int64_t t_begin = ci.k * C;
    const int64_t t_end = (t_begin + C < T) ? t_begin + C : T;
    const uint8_t* rrow = RST ? reset + (size_t)ci.bi * T : nullptr;
    for (int64_t t0 = t_begin; t0 < t_end; t0 += kU) {
        RowVec<DT> ra[kU], rb[kU];
        uint32_t rr[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u)
            if (t0 + u < t_end) {
                ra[u] = load_row<DT, ALIGNED>(a, base + (size_t)(t0 + u) * D, ci.nvalid, 1.0f);
                rb[u] = load_row<DT, ALIGNED>(b, base + (size_t)(t0 + u) * D, ci.nvalid, 0.0f);
                if (RST) rr[u] = rrow[t0 + u];
            }
#pragma unroll
        for (int u = 0; u < kU; ++u)
            if (t0 + u < t_end) {
                RowOut<DT> o;
#pragma unroll
                for (int j = 0; j < V; ++j) {
                    const float at = (RST && rr[u]) ? 0.0f : ra[u].get(j);
                    h[j] = fmaf(at, h[j], rb[u].get(j));
                    o.v[j] = h[j];
                }
                if (out) store_row<DT, ALIGNED>(out, base + (size_t)(t0 + u) * D, ci.nvalid, o);
            }
    }
    if (last && ci.k == NC - 1) {
#pragma unroll
        for (int j = 0; j < V; ++j)
            if (j < ci.nvalid) last[ci.bi * D + ci.d0 + j] = h[j];
    }
}

// ---------------------------------------------------------------------------
// reverse summary: walking the chunk backwards, P = prod a, Q <- a (Q + g)
// ---------------------------------------------------------------------------
template <int DT, bool ALIGNED, bool RST>
__global__ __launch_bounds__(kBlk) void reverse_chunk_summary_kernel(
    const void* __restrict__ a, const void* __restrict__ g, const uint8_t* __restrict__ reset,
    float* __restrict__ P, float* __restrict__ Q, int64_t B, int64_t T, int64_t D, int C) {
    constexpr int V = Elem<DT>::V;
    const int64_t NC = (T + C - 1) / C;
    const ChunkIdx ci = chunk_index<DT>(B, NC, D);
    if (!ci.ok) return;
    const size_t base = ((size_t)ci.bi * T) * D + ci.d0;
    float p[V], q[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
        p[j] = 1.0f;
        q[j] = 0.0f;
    }
    const int64_t t_begin = ci.k * C;
    const int64_t t_end = (t_begin + C < T) ? t_begin + C : T;
    const uint8_t* rrow = RST ? reset + (size_t)ci.bi * T : nullptr;
    for (int64_t top = t_end - 1; top >= t_begin; top -= kU) {
        RowVec<DT> ra[kU], rg[kU];
        uint32_t rr[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u)
            if (top - u >= t_begin) {
                ra[u] = load_row<DT, ALIGNED>(a, base + (size_t)(top - u) * D, ci.nvalid, 1.0f);
                rg[u] = load_row<DT, ALIGNED>(g, base + (size_t)(top - u) * D, ci.nvalid, 0.0f);
                if (RST) rr[u] = rrow[top - u];
            }
#pragma unroll
        for (int u = 0; u < kU; ++u)
            if (top - u >= t_begin) {
#pragma unroll
                for (int j = 0; j < V; ++j) {
                    const float at = (RST && rr[u]) ? 0.0f : ra[u].get(j);
                    p[j] = at * p[j];
                    q[j] = at * (q[j] + rg[u].get(j));
                }
            }
    }
    const size_t so = ((size_t)ci.bi * NC + ci.k) * D + ci.d0;
    store_vecf(P, so, ci.nvalid, p, V, ALIGNED);
    store_vecf(Q, so, ci.nvalid, q, V, ALIGNED);
}

// ---------------------------------------------------------------------------
// reverse replay: from the future carry, walk the chunk backwards
// ---------------------------------------------------------------------------
template <int DT, bool ALIGNED, bool RST>
__global__ __launch_bounds__(kBlk) void reverse_chunk_replay_kernel(
    const void* __restrict__ a, const void* __restrict__ out, const void* __restrict__ g,
    const uint8_t* __restrict__ reset, const float* __restrict__ future,
    const float* __restrict__ h0, void* __restrict__ grad_a, void* __restrict__ grad_b, int64_t B,
    int64_t T, int64_t D, int C) {
    constexpr int V = Elem<DT>::V;
    const int64_t NC = (T + C - 1) / C;
    const ChunkIdx ci = chunk_index<DT>(B, NC, D);
    if (!ci.ok) return;
    const size_t base = ((size_t)ci.bi * T) * D + ci.d0;
    float carry[V];
    load_vecf(future, ((size_t)ci.bi * NC + ci.k) * D + ci.d0, ci.nvalid, carry, V, ALIGNED, 0.0f);
    const int64_t t_begin = ci.k * C;
    const int64_t t_end = (t_begin + C < T) ? t_begin + C : T;
    const uint8_t* rrow = RST ? reset + (size_t)ci.bi * T : nullptr;
    for (int64_t top = t_end - 1; top >= t_begin; top -= kU) {
        RowVec<DT> ra[kU], rg[kU], rh[kU];
        uint32_t rr[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t t = top - u;
            if (t >= t_begin) {
                ra[u] = load_row<DT, ALIGNED>(a, base + (size_t)t * D, ci.nvalid, 1.0f);
                rg[u] = load_row<DT, ALIGNED>(g, base + (size_t)t * D, ci.nvalid, 0.0f);
                if (t >= 1) rh[u] = load_row<DT, ALIGNED>(out, base + (size_t)(t - 1) * D, ci.nvalid, 0.0f);
                if (RST) rr[u] = rrow[t];
            }
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t t = top - u;
            if (t >= t_begin) {
                RowOut<DT> oa, ob;
                // lambda_t = g_t + a_{t+1}*lambda_{t+1} as one fma inside a
                // block of rows; across blocks carry[] holds the product
                // a segment start uses no a_t: transition 0, grad_a_t = 0
                const int up = u > 0 ? u - 1 : 0;
                const bool rs = RST && rr[u];
#pragma unroll
                for (int j = 0; j < V; ++j) {
                    const float an = u > 0 ? ((RST && rr[up]) ? 0.0f : ra[up].get(j)) : 1.0f;
                    const float lam = fmaf(an, carry[j], rg[u].get(j));
                    float hp;
                    if (rs)
                        hp = 0.0f;
                    else if (t >= 1)
                        hp = rh[u].get(j);
                    else
                        hp = (h0 && j < ci.nvalid) ? h0[ci.bi * D + ci.d0 + j] : 0.0f;
                    ob.v[j] = lam;
                    oa.v[j] = lam * hp;
                    const float at = rs ? 0.0f : ra[u].get(j);
                    carry[j] = (u == kU - 1 || t == t_begin) ? at * lam : lam;
                }
                store_row<DT, ALIGNED>(grad_a, base + (size_t)t * D, ci.nvalid, oa);
                store_row<DT, ALIGNED>(grad_b, base + (size_t)t * D, ci.nvalid, ob);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// prefix over the chunk axis (forward: k increasing from h0; reverse: k
// decreasing from grad_last).  Block = 8 wavefronts; a wavefront holds 4
// segments x 16 adjacent lanes (lane = seg_in_wave * 16 + col).
// ---------------------------------------------------------------------------
constexpr int kPxCols = 16;
constexpr int kPxWaves = 8;
constexpr int kPxGroups = kWave / kPxCols;       // segments per wavefront
constexpr int kPxSegs = kPxWaves * kPxGroups;    // segments per block

template <bool REV>
__global__ __launch_bounds__(kPxWaves* kWave) void chunk_prefix_kernel(
    const float* __restrict__ P, const float* __restrict__ Q, const float* __restrict__ init,
    float* __restrict__ entering, float* __restrict__ final_state, int64_t B, int64_t NC,
    int64_t D) {
    __shared__ Aff s_tot[kPxWaves][kPxCols];
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int grp = lane / kPxCols;
    const int col = lane % kPxCols;
    const int64_t bi = blockIdx.y;
    const int64_t d = (int64_t)blockIdx.x * kPxCols + col;
    const bool dok = d < D;
    // segment in application order: forward = increasing k, reverse = decreasing k
    const int seg = wave * kPxGroups + grp;
    const int64_t L = (NC + kPxSegs - 1) / kPxSegs;
    const int64_t s_begin = seg * L < NC ? seg * L : NC;
    const int64_t s_end = (seg + 1) * L < NC ? (seg + 1) * L : NC;
    auto kidx = [&](int64_t i) { return REV ? (NC - 1 - i) : i; };
    auto at = [&](int64_t k) { return ((size_t)bi * NC + k) * D + d; };

    // 1. fold of the segment's maps, in application order
    Aff m = aff_identity();
    if (dok)
        for (int64_t i = s_begin; i < s_end; ++i) {
            const size_t o = at(kidx(i));
            m = aff_then(m, Aff{P[o], Q[o]});
        }
    // 2. in-wavefront scan over the 4 segments of this wavefront
    const Aff incl = wave_scan_up<kPxCols>(m);
    Aff excl;
    excl.p = shfl_up_f(incl.p, kPxCols);
    excl.q = shfl_up_f(incl.q, kPxCols);
    if (grp == 0) excl = aff_identity();
    if (grp == kPxGroups - 1) s_tot[wave][col] = incl;
    __syncthreads();
    // 3. state entering this wavefront, then this segment
    float s = (init && dok) ? init[bi * D + d] : 0.0f;
    for (int w = 0; w < wave; ++w) s = aff_apply(s_tot[w][col], s);
    s = aff_apply(excl, s);
    // 4. rewalk the segment writing the exclusive states
    if (dok) {
        for (int64_t i = s_begin; i < s_end; ++i) {
            const size_t o = at(kidx(i));
            entering[o] = s;
            s = fmaf(P[o], s, Q[o]);
        }
        if (final_state && s_begin < s_end && s_end == NC) final_state[bi * D + d] = s;
        if (final_state && NC == 0 && seg == 0) final_state[bi * D + d] = s;
    }
}

// Calls f(AL, RS) with both flags as std::integral_constant<bool>.
template <class F>
void dispatch2(bool al, bool rst, F&& f) {
    if (al && rst) f(std::true_type{}, std::true_type{});
    else if (al) f(std::true_type{}, std::false_type{});
    else if (rst) f(std::false_type{}, std::true_type{});
    else f(std::false_type{}, std::false_type{});
}

template <int DT>
hipError_t summary_t(const Shape& s, int C, const void* a, const void* b, const uint8_t* reset,
                     float* P, float* Q, bool reverse, hipStream_t st) {
    const int64_t NC = (s.T + C - 1) / C;
    const int64_t vpr = (s.D + Elem<DT>::V - 1) / Elem<DT>::V;
    const int64_t threads = s.B * NC * vpr;
    const dim3 grid((unsigned)((threads + kBlk - 1) / kBlk));
    const void* ptrs[2] = {a, b};
    const bool al = rows_aligned(s, ptrs, 2) && reinterpret_cast<uintptr_t>(P) % 16 == 0 &&
                    reinterpret_cast<uintptr_t>(Q) % 16 == 0;
    dispatch2(al, reset != nullptr, [&](auto AL, auto RS) {
        if (reverse)
            hipLaunchKernelGGL((reverse_chunk_summary_kernel<DT, decltype(AL)::value, decltype(RS)::value>),
                               grid, dim3(kBlk), 0, st, a, b, reset, P, Q, s.B, s.T, s.D, C);
        else
            hipLaunchKernelGGL((chunk_summary_kernel<DT, decltype(AL)::value, decltype(RS)::value>),
                               grid, dim3(kBlk), 0, st, a, b, reset, P, Q, s.B, s.T, s.D, C);
    });
    return hipGetLastError();
}

template <int DT>
hipError_t replay_t(const Shape& s, int C, const void* a, const void* b, const uint8_t* reset,
                    const float* cin, void* out, float* last, hipStream_t st) {
    const int64_t NC = (s.T + C - 1) / C;
    const int64_t vpr = (s.D + Elem<DT>::V - 1) / Elem<DT>::V;
    const int64_t threads = s.B * NC * vpr;
    const dim3 grid((unsigned)((threads + kBlk - 1) / kBlk));
    const void* ptrs[3] = {a, b, out};
    const bool al = rows_aligned(s, ptrs, 3) && reinterpret_cast<uintptr_t>(cin) % 16 == 0;
    dispatch2(al, reset != nullptr, [&](auto AL, auto RS) {
        hipLaunchKernelGGL((chunk_replay_kernel<DT, decltype(AL)::value, decltype(RS)::value>), grid,
                           dim3(kBlk), 0, st, a, b, reset, cin, out, last, s.B, s.T, s.D, C);
    });
    return hipGetLastError();
}

template <int DT>
hipError_t reverse_replay_t(const Shape& s, int C, const void* a, const void* out, const void* g,
                            const uint8_t* reset, const float* fut, const float* h0, void* ga,
                            void* gb, hipStream_t st) {
    const int64_t NC = (s.T + C - 1) / C;
    const int64_t vpr = (s.D + Elem<DT>::V - 1) / Elem<DT>::V;
    const int64_t threads = s.B * NC * vpr;
    const dim3 grid((unsigned)((threads + kBlk - 1) / kBlk));
    const void* ptrs[5] = {a, out, g, ga, gb};
    const bool al = rows_aligned(s, ptrs, 5) && reinterpret_cast<uintptr_t>(fut) % 16 == 0;
    dispatch2(al, reset != nullptr, [&](auto AL, auto RS) {
        hipLaunchKernelGGL((reverse_chunk_replay_kernel<DT, decltype(AL)::value, decltype(RS)::value>),
                           grid, dim3(kBlk), 0, st, a, out, g, reset, fut, h0, ga, gb, s.B, s.T,
                           s.D, C);
    });
    return hipGetLastError();
}

hipError_t prefix_t(bool rev, int64_t B, int64_t NC, int64_t D, const float* P, const float* Q,
                    const float* init, float* entering, float* final_state, hipStream_t st) {
    const dim3 grid((unsigned)((D + kPxCols - 1) / kPxCols), (unsigned)B);
    const dim3 block(kPxWaves * kWave);
    if (rev)
        hipLaunchKernelGGL((chunk_prefix_kernel<true>), grid, block, 0, st, P, Q, init, entering,
                           final_state, B, NC, D);
    else
        hipLaunchKernelGGL((chunk_prefix_kernel<false>), grid, block, 0, st, P, Q, init, entering,
                           final_state, B, NC, D);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_summary(const Shape& s, int chunk, const void* a, const void* b,
                                const uint8_t* reset, float* P, float* Q, hipStream_t st) {
    return s.dtype == DT_F32 ? summary_t<DT_F32>(s, chunk, a, b, reset, P, Q, false, st)
                             : summary_t<DT_BF16>(s, chunk, a, b, reset, P, Q, false, st);
}

hipError_t launch_chunk_prefix(int64_t B, int64_t NC, int64_t D, const float* P, const float* Q,
                               const float* h0, float* chunk_in, float* last, hipStream_t st) {
    return prefix_t(false, B, NC, D, P, Q, h0, chunk_in, last, st);
}

hipError_t launch_chunk_replay(const Shape& s, int chunk, const void* a, const void* b,
                               const uint8_t* reset, const float* chunk_in, void* out, float* last,
                               hipStream_t st) {
    return s.dtype == DT_F32 ? replay_t<DT_F32>(s, chunk, a, b, reset, chunk_in, out, last, st)
                             : replay_t<DT_BF16>(s, chunk, a, b, reset, chunk_in, out, last, st);
}

hipError_t launch_reverse_chunk_summary(const Shape& s, int chunk, const void* a, const void* g,
                                        const uint8_t* reset, float* P, float* Q, hipStream_t st) {
    return s.dtype == DT_F32 ? summary_t<DT_F32>(s, chunk, a, g, reset, P, Q, true, st)
                             : summary_t<DT_BF16>(s, chunk, a, g, reset, P, Q, true, st);
}

hipError_t launch_reverse_chunk_prefix(int64_t B, int64_t NC, int64_t D, const float* P,
                                       const float* Q, const float* grad_last, float* future,
                                       float* grad_h0, hipStream_t st) {
    return prefix_t(true, B, NC, D, P, Q, grad_last, future, grad_h0, st);
}

hipError_t launch_reverse_chunk_replay(const Shape& s, int chunk, const void* a, const void* out,
                                       const void* g, const uint8_t* reset, const float* future,
                                       const float* h0, void* grad_a, void* grad_b,
                                       hipStream_t st) {
    return s.dtype == DT_F32
               ? reverse_replay_t<DT_F32>(s, chunk, a, out, g, reset, future, h0, grad_a, grad_b, st)
               : reverse_replay_t<DT_BF16>(s, chunk, a, out, g, reset, future, h0, grad_a, grad_b, st);
}

}  // namespace lrscan
