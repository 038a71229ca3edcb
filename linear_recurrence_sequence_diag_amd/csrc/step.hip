// step.hip -- one time step of the recurrence on [B, D] lanes (token-by-token
// decoding from a carried fp32 state).
//
// Each thread owns one 16-byte vector of a [B, D] row (4 fp32 or 8 bf16
// lanes): it reads a, b and the fp32 state, forms h = a*state + b with one
// fma per lane (the same operation the per-lane walk applies at every step,
// so chained steps reproduce it bit for bit), and writes h rounded to the
// I/O type and/or as the new fp32 state.  The state may be updated in place:
// every lane is read before it is written, by the same thread.
#include "device.hpp"
#include "launch.hpp"

namespace lrscan {

namespace {

constexpr int kStepBlock = 256;

template <int DT, bool ALIGNED>
__global__ __launch_bounds__(kStepBlock) void step_kernel(
    const void* __restrict__ a, const void* __restrict__ b, const float* state_in,
    const uint8_t* __restrict__ reset, void* __restrict__ out, float* state_out, int64_t B,
    int64_t D, int64_t vpr) {
    constexpr int V = Elem<DT>::V;
    const int64_t gid = (int64_t)blockIdx.x * kStepBlock + threadIdx.x;
    const int64_t bi = gid / vpr;
    if (bi >= B) return;
    const int64_t d0 = (gid - bi * vpr) * V;
    const int nvalid = (int)((D - d0) < V ? (D - d0) : V);
    const size_t e0 = (size_t)bi * (size_t)D + (size_t)d0;

    const RowVec<DT> av = load_row<DT, ALIGNED>(a, e0, nvalid, 1.0f);
    const RowVec<DT> bv = load_row<DT, ALIGNED>(b, e0, nvalid, 0.0f);
    float s[V];
    if (ALIGNED && state_in) {
#pragma unroll
        for (int q = 0; q < V / 4; ++q) {
            const float4 v = reinterpret_cast<const float4*>(state_in + e0)[q];
            s[4 * q] = v.x;
            s[4 * q + 1] = v.y;
            s[4 * q + 2] = v.z;
            s[4 * q + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < V; ++j) s[j] = (state_in && j < nvalid) ? state_in[e0 + j] : 0.0f;
    }
    const bool drop = reset && reset[bi];  // a segment starts here
    RowOut<DT> o;
#pragma unroll
    for (int j = 0; j < V; ++j) {
        const float at = drop ? 0.0f : av.get(j);
        o.v[j] = fmaf(at, s[j], bv.get(j));
    }
    if (out) store_row<DT, ALIGNED>(out, e0, nvalid, o);
    if (state_out) {
        if (ALIGNED) {
#pragma unroll
            for (int q = 0; q < V / 4; ++q)
                reinterpret_cast<float4*>(state_out + e0)[q] =
                    make_float4(o.v[4 * q], o.v[4 * q + 1], o.v[4 * q + 2], o.v[4 * q + 3]);
        } else {
#pragma unroll
            for (int j = 0; j < V; ++j)
                if (j < nvalid) state_out[e0 + j] = o.v[j];
        }
    }
}

template <int DT>
hipError_t step_t(int64_t B, int64_t D, const void* a, const void* b, const float* state_in,
                  const uint8_t* reset, void* out, float* state_out, hipStream_t st) {
    const Shape s{B, 1, D, DT};
    const void* ptrs[5] = {a, b, out, state_in, state_out};
    const int64_t vpr = (D + Elem<DT>::V - 1) / Elem<DT>::V;
    const dim3 grid((unsigned)((B * vpr + kStepBlock - 1) / kStepBlock));
    // fp32 state rows are 16-byte aligned whenever the I/O rows are (D is a
    // multiple of 4 lanes then); the pointers are checked with the others
    if (rows_aligned(s, ptrs, 5))
        hipLaunchKernelGGL((step_kernel<DT, true>), grid, dim3(kStepBlock), 0, st, a, b, state_in,
                           reset, out, state_out, B, D, vpr);
    else
        hipLaunchKernelGGL((step_kernel<DT, false>), grid, dim3(kStepBlock), 0, st, a, b,
                           state_in, reset, out, state_out, B, D, vpr);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_step(int64_t B, int64_t D, int dtype, const void* a, const void* b,
                       const float* state_in, const uint8_t* reset, void* out, float* state_out,
                       hipStream_t st) {
    return dtype == DT_F32 ? step_t<DT_F32>(B, D, a, b, state_in, reset, out, state_out, st)
                           : step_t<DT_BF16>(B, D, a, b, state_in, reset, out, state_out, st);
}

}  // namespace lrscan
