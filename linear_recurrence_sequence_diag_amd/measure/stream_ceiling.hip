// stream_ceiling.hip -- the achievable streaming bandwidth of MI355X for the
// scan's own access patterns, as a reference beside the scan's throughput
// (built into libstreamceil.so; only the benchmark loads it).
//
// Pattern 1 reads two arrays and writes one (the forward scan's traffic:
// a, b in; out); pattern 2 reads three and writes two (the backward's: a,
// out, grad_out in; grad_a, grad_b).  Every element is a 16-byte vector;
// a thread issues all U loads of its vectors before any store, consecutive
// threads touch consecutive vectors, and outputs are stored non-temporally,
// as the scan kernels store theirs (a normal store leaves dirty lines in the
// Infinity Cache that are written back after the kernel, outside any timing
// of it).  Each input can be loaded normally or non-temporally (bit i of
// `nt_mask` for input i), so the benchmark can take the best cache policy.
// The values written are a bitwise combination of the inputs: the
// measurement is of memory traffic alone.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void put(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }

template <bool NT>
__device__ __forceinline__ u32x4 get(const u32x4* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    return *p;
}

template <int U, int NIN, int NOUT, int NTM>
__global__ __launch_bounds__(kThreads) void stream_kernel(const u32x4* __restrict__ in0,
                                                         const u32x4* __restrict__ in1,
                                                         const u32x4* __restrict__ in2,
                                                         u32x4* __restrict__ out0,
                                                         u32x4* __restrict__ out1, size_t nvec) {
    const size_t base = (size_t)blockIdx.x * (kThreads * U) + threadIdx.x;
    u32x4 x0[U], x1[U], x2[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const size_t i = base + (size_t)u * kThreads;
        if (i < nvec) {
            x0[u] = get<(NTM & 1) != 0>(in0 + i);
            x1[u] = get<(NTM & 2) != 0>(in1 + i);
            if (NIN == 3) x2[u] = get<(NTM & 4) != 0>(in2 + i);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const size_t i = base + (size_t)u * kThreads;
        if (i < nvec) {
            put(out0 + i, x0[u] ^ x1[u]);
            if (NOUT == 2) put(out1 + i, (NIN == 3 ? x2[u] : x0[u]) ^ x1[u]);
        }
    }
}

template <int U, int NIN, int NOUT, int NTM>
hipError_t launch(const void* in0, const void* in1, const void* in2, void* out0, void* out1,
                  size_t nvec, hipStream_t st) {
    const size_t per_block = (size_t)kThreads * U;
    const size_t blocks = (nvec + per_block - 1) / per_block;
    if (blocks == 0 || blocks >= ((size_t)1 << 31) / kThreads) return hipErrorInvalidValue;
    hipLaunchKernelGGL((stream_kernel<U, NIN, NOUT, NTM>), dim3((unsigned)blocks), dim3(kThreads), 0,
                       st, static_cast<const u32x4*>(in0), static_cast<const u32x4*>(in1),
                       static_cast<const u32x4*>(in2), static_cast<u32x4*>(out0),
                       static_cast<u32x4*>(out1), nvec);
    return hipGetLastError();
}

template <int NIN, int NOUT, int NTM>
hipError_t by_unroll(int unroll, const void* in0, const void* in1, const void* in2, void* out0,
                     void* out1, size_t nvec, hipStream_t st) {
    switch (unroll) {
        case 1: return launch<1, NIN, NOUT, NTM>(in0, in1, in2, out0, out1, nvec, st);
        case 2: return launch<2, NIN, NOUT, NTM>(in0, in1, in2, out0, out1, nvec, st);
        case 4: return launch<4, NIN, NOUT, NTM>(in0, in1, in2, out0, out1, nvec, st);
    }
    return hipErrorInvalidValue;
}

template <int NIN, int NOUT>
hipError_t by_mask(int nt_mask, int unroll, const void* in0, const void* in1, const void* in2,
                   void* out0, void* out1, size_t nvec, hipStream_t st) {
    switch (nt_mask) {
        case 0: return by_unroll<NIN, NOUT, 0>(unroll, in0, in1, in2, out0, out1, nvec, st);
        case 2: return by_unroll<NIN, NOUT, 2>(unroll, in0, in1, in2, out0, out1, nvec, st);
        case 7: return by_unroll<NIN, NOUT, 7>(unroll, in0, in1, in2, out0, out1, nvec, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

// pattern 1: out0 = in0 ^ in1 (read 2, write 1); pattern 2: out0 = in0 ^ in1,
// out1 = in2 ^ in1 (read 3, write 2).  `bytes` per array, a multiple of 16;
// every pointer 16-byte aligned; `unroll` (vectors per thread) 1, 2 or 4;
// `nt_mask` 0 (every input loaded normally), 2 (input 1 non-temporally) or 7
// (every input non-temporally).  Returns 0, or -1 for bad arguments, -2 for a
// launch error.
extern "C" __attribute__((visibility("default"))) int stream_ceiling_run(
    int pattern, int unroll, int nt_mask, const void* in0, const void* in1, const void* in2,
    void* out0, void* out1, size_t bytes, void* stream) {
    if (bytes == 0 || bytes % 16 != 0 || !in0 || !in1 || !out0) return -1;
    const uintptr_t al = reinterpret_cast<uintptr_t>(in0) | reinterpret_cast<uintptr_t>(in1) |
                         reinterpret_cast<uintptr_t>(out0) | reinterpret_cast<uintptr_t>(in2) |
                         reinterpret_cast<uintptr_t>(out1);
    if (al % 16 != 0) return -1;
    if (pattern == 2 && (!in2 || !out1)) return -1;
    if (unroll != 1 && unroll != 2 && unroll != 4) return -1;
    if (nt_mask != 0 && nt_mask != 2 && nt_mask != 7) return -1;
    const size_t nvec = bytes / 16;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (pattern == 1) e = by_mask<2, 1>(nt_mask, unroll, in0, in1, nullptr, out0, nullptr, nvec, st);
    else if (pattern == 2) e = by_mask<3, 2>(nt_mask, unroll, in0, in1, in2, out0, out1, nvec, st);
    else return -1;
    return e == hipSuccess ? 0 : -2;
}
