// seq.hip -- the per-lane sequential scan (forward and backward).
//
// One thread owns V adjacent lanes (one 16-byte vector: 4 fp32 or 8 bf16) of
// one batch row and walks all T steps, keeping the fp32 state (forward) or the
// fp32 adjoint (backward) in registers, as the page "triton_training_scan.py"
// does in _real_forward and _real_backward.  On MI355X the walk is bound by
// memory latency unless B*D/V threads are many times the 256 CUs x 64 lanes:
// each thread keeps U rows of every input in flight (a register double
// buffer) to raise the bytes in flight per lane.
#include "device.hpp"
#include "launch.hpp"

namespace lrscan {

namespace {

constexpr int kSeqBlock = 256;
constexpr int kSeqU = 8;  // rows in flight per buffer

// RST: `reset` ([B, T] bytes) marks segment starts, where the step's
// transition is taken as 0 (the entering state is dropped).
template <int DT, bool ALIGNED, bool RST>
__global__ __launch_bounds__(kSeqBlock) void seq_fwd_kernel(const void* __restrict__ a,
                                                            const void* __restrict__ b,
                                                            void* __restrict__ out,
                                                            float* __restrict__ last,
                                                            const float* __restrict__ h0,
                                                            const uint8_t* __restrict__ reset,
                                                            int64_t B, int64_t T, int64_t D,
                                                            int64_t vpr) {
    constexpr int V = Elem<DT>::V;
    constexpr int U = kSeqU;
    const int64_t gid = (int64_t)blockIdx.x * kSeqBlock + threadIdx.x;
    const int64_t bi = gid / vpr;
    if (bi >= B) return;
    const int64_t d0 = (gid - bi * vpr) * V;
    const int nvalid = (int)((D - d0) < V ? (D - d0) : V);
    const size_t base = (size_t)bi * (size_t)T * (size_t)D + (size_t)d0;

    float h[V];
#pragma unroll
    for (int j = 0; j < V; ++j) h[j] = (h0 && j < nvalid) ? h0[bi * D + d0 + j] : 0.0f;

    const uint8_t* rrow = RST ? reset + (size_t)bi * (size_t)T : nullptr;
    RowVec<DT> ca[U], cb[U], na[U], nb[U];
    uint32_t cr[U], nr[U];  // segment-start bytes of the buffered rows (RST)
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (u < T) {
            ca[u] = load_row<DT, ALIGNED>(a, base + (size_t)u * D, nvalid, 1.0f);
            cb[u] = load_row<DT, ALIGNED>(b, base + (size_t)u * D, nvalid, 0.0f);
            if (RST) cr[u] = rrow[u];
        }
    }
    for (int64_t t0 = 0; t0 < T; t0 += U) {
        const int64_t tn = t0 + U;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (tn + u < T) {
                na[u] = load_row<DT, ALIGNED>(a, base + (size_t)(tn + u) * D, nvalid, 1.0f);
                nb[u] = load_row<DT, ALIGNED>(b, base + (size_t)(tn + u) * D, nvalid, 0.0f);
                if (RST) nr[u] = rrow[tn + u];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (t0 + u < T) {
                RowOut<DT> o;
#pragma unroll
                for (int j = 0; j < V; ++j) {
                    const float at = (RST && cr[u]) ? 0.0f : ca[u].get(j);
                    h[j] = fmaf(at, h[j], cb[u].get(j));
                    o.v[j] = h[j];
                }
                if (out) store_row<DT, ALIGNED>(out, base + (size_t)(t0 + u) * D, nvalid, o);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            ca[u] = na[u];
            cb[u] = nb[u];
            if (RST) cr[u] = nr[u];
        }
    }
    if (last) {
#pragma unroll
        for (int j = 0; j < V; ++j)
            if (j < nvalid) last[bi * D + d0 + j] = h[j];
    }
}

// RST: at a segment start a_t is not used (its transition is 0), so no
// adjoint crosses it and grad_a_t = 0.
template <int DT, bool ALIGNED, bool RST>
__global__ __launch_bounds__(kSeqBlock) void seq_bwd_kernel(
    const void* __restrict__ a, const void* __restrict__ out, const void* __restrict__ g,
    const float* __restrict__ grad_last, const float* __restrict__ h0,
    const uint8_t* __restrict__ reset, void* __restrict__ grad_a, void* __restrict__ grad_b,
    float* __restrict__ grad_h0, int64_t B, int64_t T, int64_t D, int64_t vpr) {
    constexpr int V = Elem<DT>::V;
    constexpr int U = kSeqU;
    const int64_t gid = (int64_t)blockIdx.x * kSeqBlock + threadIdx.x;
    const int64_t bi = gid / vpr;
    if (bi >= B) return;
    const int64_t d0 = (gid - bi * vpr) * V;
    const int nvalid = (int)((D - d0) < V ? (D - d0) : V);
    const size_t base = (size_t)bi * (size_t)T * (size_t)D + (size_t)d0;

    float carry[V], hinit[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
        carry[j] = (grad_last && j < nvalid) ? grad_last[bi * D + d0 + j] : 0.0f;
        hinit[j] = (h0 && j < nvalid) ? h0[bi * D + d0 + j] : 0.0f;
    }

    // block u of a buffer holds row t0 - u (walking down)
    const uint8_t* rrow = RST ? reset + (size_t)bi * (size_t)T : nullptr;
    RowVec<DT> ca[U], cg[U], ch[U], na[U], ng[U], nh[U];
    uint32_t cr[U], nr[U];  // segment-start bytes of the buffered rows (RST)
    auto load_block = [&](int64_t top, RowVec<DT>* ra, RowVec<DT>* rg, RowVec<DT>* rh,
                          uint32_t* rr) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t t = top - u;
            if (t >= 0) {
                ra[u] = load_row<DT, ALIGNED>(a, base + (size_t)t * D, nvalid, 1.0f);
                rg[u] = load_row<DT, ALIGNED>(g, base + (size_t)t * D, nvalid, 0.0f);
                if (t >= 1) rh[u] = load_row<DT, ALIGNED>(out, base + (size_t)(t - 1) * D, nvalid, 0.0f);
                if (RST) rr[u] = rrow[t];
            }
        }
    };
    load_block(T - 1, ca, cg, ch, cr);
    for (int64_t top = T - 1; top >= 0; top -= U) {
        if (top - U >= 0) load_block(top - U, na, ng, nh, nr);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t t = top - u;
            if (t >= 0) {
                RowOut<DT> oa, ob;
                // lambda_t = g_t + a_{t+1}*lambda_{t+1}: one fma with the a of
                // row t+1 inside a block; across blocks carry[] holds the
                // product a_{t+1}*lambda_{t+1}
                const int up = u > 0 ? u - 1 : 0;
                const bool rs = RST && cr[u];
#pragma unroll
                for (int j = 0; j < V; ++j) {
                    const float an = u > 0 ? ((RST && cr[up]) ? 0.0f : ca[up].get(j)) : 1.0f;
                    const float lam = fmaf(an, carry[j], cg[u].get(j));
                    const float hp = rs ? 0.0f : ((t >= 1) ? ch[u].get(j) : hinit[j]);
                    ob.v[j] = lam;
                    oa.v[j] = lam * hp;
                    const float at = rs ? 0.0f : ca[u].get(j);
                    carry[j] = (u == U - 1 || t == 0) ? at * lam : lam;
                }
                store_row<DT, ALIGNED>(grad_a, base + (size_t)t * D, nvalid, oa);
                store_row<DT, ALIGNED>(grad_b, base + (size_t)t * D, nvalid, ob);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            ca[u] = na[u];
            cg[u] = ng[u];
            ch[u] = nh[u];
            if (RST) cr[u] = nr[u];
        }
    }
    if (grad_h0) {
#pragma unroll
        for (int j = 0; j < V; ++j)
            if (j < nvalid) grad_h0[bi * D + d0 + j] = carry[j];
    }
}

template <int DT>
int64_t vecs_per_row(int64_t D) {
    return (D + Elem<DT>::V - 1) / Elem<DT>::V;
}

template <int DT, bool AL, bool RST>
void seq_fwd_launch(const Shape& s, dim3 grid, const void* a, const void* b, void* out,
                    float* last, const float* h0, const uint8_t* reset, int64_t vpr,
                    hipStream_t st) {
    hipLaunchKernelGGL((seq_fwd_kernel<DT, AL, RST>), grid, dim3(kSeqBlock), 0, st, a, b, out,
                       last, h0, reset, s.B, s.T, s.D, vpr);
}

template <int DT>
hipError_t seq_fwd_t(const Shape& s, const void* a, const void* b, void* out, float* last,
                     const float* h0, const uint8_t* reset, hipStream_t st) {
    const void* ptrs[3] = {a, b, out};
    const int64_t vpr = vecs_per_row<DT>(s.D);
    const int64_t threads = s.B * vpr;
    const dim3 grid((unsigned)((threads + kSeqBlock - 1) / kSeqBlock));
    const bool al = rows_aligned(s, ptrs, 3);
    if (al && reset) seq_fwd_launch<DT, true, true>(s, grid, a, b, out, last, h0, reset, vpr, st);
    else if (al) seq_fwd_launch<DT, true, false>(s, grid, a, b, out, last, h0, reset, vpr, st);
    else if (reset) seq_fwd_launch<DT, false, true>(s, grid, a, b, out, last, h0, reset, vpr, st);
    else seq_fwd_launch<DT, false, false>(s, grid, a, b, out, last, h0, reset, vpr, st);
    return hipGetLastError();
}

template <int DT, bool AL, bool RST>
void seq_bwd_launch(const Shape& s, dim3 grid, const void* a, const void* out, const void* g,
                    const float* grad_last, const float* h0, const uint8_t* reset, void* grad_a,
                    void* grad_b, float* grad_h0, int64_t vpr, hipStream_t st) {
    hipLaunchKernelGGL((seq_bwd_kernel<DT, AL, RST>), grid, dim3(kSeqBlock), 0, st, a, out, g,
                       grad_last, h0, reset, grad_a, grad_b, grad_h0, s.B, s.T, s.D, vpr);
}

template <int DT>
hipError_t seq_bwd_t(const Shape& s, const void* a, const void* out, const void* g,
                     const float* grad_last, const float* h0, const uint8_t* reset, void* grad_a,
                     void* grad_b, float* grad_h0, hipStream_t st) {
    const void* ptrs[5] = {a, out, g, grad_a, grad_b};
    const int64_t vpr = vecs_per_row<DT>(s.D);
    const int64_t threads = s.B * vpr;
    const dim3 grid((unsigned)((threads + kSeqBlock - 1) / kSeqBlock));
    const bool al = rows_aligned(s, ptrs, 5);
    if (al && reset)
        seq_bwd_launch<DT, true, true>(s, grid, a, out, g, grad_last, h0, reset, grad_a, grad_b, grad_h0, vpr, st);
    else if (al)
        seq_bwd_launch<DT, true, false>(s, grid, a, out, g, grad_last, h0, reset, grad_a, grad_b, grad_h0, vpr, st);
    else if (reset)
        seq_bwd_launch<DT, false, true>(s, grid, a, out, g, grad_last, h0, reset, grad_a, grad_b, grad_h0, vpr, st);
    else
        seq_bwd_launch<DT, false, false>(s, grid, a, out, g, grad_last, h0, reset, grad_a, grad_b, grad_h0, vpr, st);
    return hipGetLastError();
}

}  // namespace

bool rows_aligned(const Shape& s, const void* const* ptrs, int n) {
    const int eb = s.dtype == DT_F32 ? 4 : 2;
    if ((s.D * eb) % 16 != 0) return false;
    for (int i = 0; i < n; ++i)
        if (reinterpret_cast<uintptr_t>(ptrs[i]) % 16 != 0) return false;
    return true;
}

hipError_t launch_seq_fwd(const Shape& s, const void* a, const void* b, void* out, float* last,
                          const float* h0, const uint8_t* reset, hipStream_t st) {
    return s.dtype == DT_F32 ? seq_fwd_t<DT_F32>(s, a, b, out, last, h0, reset, st)
                             : seq_fwd_t<DT_BF16>(s, a, b, out, last, h0, reset, st);
}

hipError_t launch_seq_bwd(const Shape& s, const void* a, const void* out, const void* g,
                          const float* grad_last, const float* h0, const uint8_t* reset,
                          void* grad_a, void* grad_b, float* grad_h0, hipStream_t st) {
    return s.dtype == DT_F32
               ? seq_bwd_t<DT_F32>(s, a, out, g, grad_last, h0, reset, grad_a, grad_b, grad_h0, st)
               : seq_bwd_t<DT_BF16>(s, a, out, g, grad_last, h0, reset, grad_a, grad_b, grad_h0, st);
}

}  // namespace lrscan
