// device.hpp -- device-side building blocks shared by the scan kernels (gfx950).
//
//  * storage types: fp32 and bf16 elements, widened to fp32 on load and
//    rounded to nearest even on store (bf16 via the gfx950 packed convert);
//  * 16-byte row vectors: one thread owns V = 16 / sizeof(elem) adjacent lanes
//    of a [B, T, D] row (4 fp32 or 8 bf16), loaded and stored with one
//    dwordx4 access (at an address aligned only to the element size when the
//    row is not 16-byte aligned; a row's last, partial vector lane by lane);
//  * the affine map h -> p*h + q that summarises a run of steps, and its
//    composition "later after earlier" (associative, not commutative; page
//    "triton_training_scan.py", the affine prefix kernels that compose the
//    current map with the accumulated one);
//  * cross-lane scans of such maps inside one 64-lane wavefront.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lrscan {

enum : int { DT_F32 = 0, DT_BF16 = 1 };

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// storage element conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Two floats -> two bf16 packed in one dword (lo in bits 0..15), RNE.  As a
// two-lane vector conversion this is one v_cvt_pk_bf16_f32 of both values
// (two scalar conversions cost that instruction twice plus a shift and an or).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    __bf16 v = (__bf16)x;
    return __builtin_bit_cast(uint16_t, v);
}

template <int DT>
struct Elem;

template <>
struct Elem<DT_F32> {
    using raw = float;
    static constexpr int bytes = 4;
    static constexpr int V = 4;  // lanes per 16-byte vector
    __device__ static float load1(const void* base, size_t i) {
        return reinterpret_cast<const float*>(base)[i];
    }
    __device__ static void store1(void* base, size_t i, float x) {
        __builtin_nontemporal_store(x, reinterpret_cast<float*>(base) + i);
    }
};

template <>
struct Elem<DT_BF16> {
    using raw = uint16_t;
    static constexpr int bytes = 2;
    static constexpr int V = 8;
    __device__ static float load1(const void* base, size_t i) {
        return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[i]);
    }
    __device__ static void store1(void* base, size_t i, float x) {
        __builtin_nontemporal_store(f32_to_bf16_bits(x), reinterpret_cast<uint16_t*>(base) + i);
    }
};

// ---------------------------------------------------------------------------
// 16-byte row vectors (raw storage kept packed in 4 dwords)
// ---------------------------------------------------------------------------
template <int DT>
struct RowVec {
    static constexpr int V = Elem<DT>::V;
    uint4 w;

    __device__ __forceinline__ float get(int j) const {
        if constexpr (DT == DT_F32) {
            const uint32_t x = (j == 0) ? w.x : (j == 1) ? w.y : (j == 2) ? w.z : w.w;
            return __uint_as_float(x);
        } else {
            const uint32_t x = (j >> 1 == 0) ? w.x : (j >> 1 == 1) ? w.y : (j >> 1 == 2) ? w.z : w.w;
            return (j & 1) ? __uint_as_float(x & 0xffff0000u) : __uint_as_float(x << 16);
        }
    }

    // identity row: every lane holds `v` (exact in both storage types for 0 and 1)
    __device__ __forceinline__ static RowVec splat(float v) {
        RowVec r;
        uint32_t x;
        if constexpr (DT == DT_F32) {
            x = __float_as_uint(v);
        } else {
            const uint32_t h = __float_as_uint(v) >> 16;
            x = h | (h << 16);
        }
        r.w = make_uint4(x, x, x, x);
        return r;
    }
};

// Outputs are written once and read by later launches only, so every output
// store is non-temporal: it does not displace data this launch still reads
// from the caches, and leaves fewer dirty lines for the end-of-launch
// write-back.  (Measured on MI355X: the backward on [8,2048,2560] bf16 went
// from 94 to 78 us; every other form gained 0-14%.)
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store16_nt(void* p, uint4 v) {
    const u32x4_nt w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4_nt*>(p));
}

// Output staging: V floats rounded into the storage type and written as one vector.
template <int DT>
struct RowOut {
    static constexpr int V = Elem<DT>::V;
    float v[V];
    __device__ __forceinline__ uint4 pack() const {
        if constexpr (DT == DT_F32) {
            return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                              __float_as_uint(v[3]));
        } else {
            return make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                              pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
        }
    }
};

// ---- rows that are not 16-byte aligned -------------------------------------
// A thread's 16 bytes [p, p + 16) then straddle two aligned blocks, sh = p mod
// 16 bytes (a multiple of the element size) into the first.  A row's last,
// partial vector is read as one or two aligned 16-byte loads and shifted, so
// that no read leaves the bytes of the row (element-wise accesses, eight
// 2-byte loads per bf16 vector, ran the scan about ten times slower).

// d[k + q] for q = 0..3, with no indexing of registers by a variable.
__device__ __forceinline__ uint32_t dword_at(const uint32_t (&d)[8], uint32_t q, int k) {
    return q == 0 ? d[k] : q == 1 ? d[k + 1] : q == 2 ? d[k + 2] : d[k + 3];
}

// The 16 bytes that start `sh` (0..15) bytes into the 32 bytes lo, hi.
__device__ __forceinline__ uint4 bytes16_at(uint4 lo, uint4 hi, uint32_t sh) {
    const uint32_t d[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    const uint32_t q = sh >> 2, r = sh & 3u;
    uint32_t e[5];
#pragma unroll
    for (int k = 0; k < 5; ++k) e[k] = dword_at(d, q, k);
    // alignbyte(hi, lo, r): bytes r .. r + 3 of the 64-bit value hi:lo
    return make_uint4(__builtin_amdgcn_alignbyte(e[1], e[0], r),
                      __builtin_amdgcn_alignbyte(e[2], e[1], r),
                      __builtin_amdgcn_alignbyte(e[3], e[2], r),
                      __builtin_amdgcn_alignbyte(e[4], e[3], r));
}

// 16 bytes at an address aligned only to the element size.  The compiler
// emits one 16-byte global access for it (gfx950 code objects for the HSA
// runtime run with unaligned accesses enabled); the hardware splits it at the
// cache-line boundaries.  It touches exactly those 16 bytes.  Measured on
// MI355X against per-block accesses with the neighbouring lanes' blocks
// shared (bf16 [8,2048,2559], forward / backward): 2117 / 1889 -> 2857 / 3016
// GB/s, the same bits out.
__device__ __forceinline__ uint4 load16_any(const void* p) {
    uint4 v;
    __builtin_memcpy(&v, p, 16);
    return v;
}
__device__ __forceinline__ void store16_any(void* p, uint4 v) { __builtin_memcpy(p, &v, 16); }

// Load a vector at an address that need not be 16-byte aligned.  A complete
// vector is one 16-byte access.  A row's last, partial vector reads the
// aligned block holding its first byte and, when lanes of the vector lie in
// it, the next block (each block read holds bytes of the vector, so no read
// reaches past memory the vector lies in; otherwise the first block is read
// twice), then shifted into place.  Lanes from `nvalid` on are `fill`.
template <int DT>
__device__ __forceinline__ RowVec<DT> load_vec_unaligned(const char* p, int nvalid, float fill) {
    constexpr int S = Elem<DT>::bytes;
    if (nvalid == Elem<DT>::V) {
        RowVec<DT> r;
        r.w = load16_any(p);
        return r;
    }
    const uintptr_t ua = reinterpret_cast<uintptr_t>(p);
    const uint32_t sh = (uint32_t)(ua & 15u);
    const uint4* blk = reinterpret_cast<const uint4*>(ua - sh);
    const bool straddles = (uint32_t)(nvalid * S) > 16u - sh;
    const uint4 lo = blk[0];
    const uint4 hi = blk[straddles ? 1 : 0];
    const uint4 w = bytes16_at(lo, hi, sh);
    // keep the bits of lanes below nvalid, `fill` elsewhere
    const uint4 f = RowVec<DT>::splat(fill).w;
    uint32_t m[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if constexpr (DT == DT_F32) {
            m[q] = q < nvalid ? 0xffffffffu : 0u;
        } else {
            m[q] = (2 * q < nvalid ? 0x0000ffffu : 0u) | (2 * q + 1 < nvalid ? 0xffff0000u : 0u);
        }
    }
    RowVec<DT> r;
    r.w = make_uint4((w.x & m[0]) | (f.x & ~m[0]), (w.y & m[1]) | (f.y & ~m[1]),
                     (w.z & m[2]) | (f.z & ~m[2]), (w.w & m[3]) | (f.w & ~m[3]));
    return r;
}

// Load V lanes starting at element offset `off` (lane d0 of a row), for the
// per-lane walk and the three-launch form.  ALIGNED: the whole vector is in
// range and 16-byte aligned.  Otherwise a complete vector is one 16-byte
// access at its own address, and a partial one (`nvalid` < V lanes) is read
// lane by lane, the rest `fill` (these kernels keep many rows of loads in
// flight per thread, and the two-block reads of a partial vector would
// double the registers that takes).
template <int DT, bool ALIGNED>
__device__ __forceinline__ RowVec<DT> load_row(const void* base, size_t off, int nvalid, float fill) {
    if constexpr (ALIGNED) {
        RowVec<DT> r;
        r.w = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(base) + off * Elem<DT>::bytes);
        return r;
    } else {
        if (nvalid == RowVec<DT>::V) {
            RowVec<DT> r;
            r.w = load16_any(reinterpret_cast<const char*>(base) + off * Elem<DT>::bytes);
            return r;
        }
        RowVec<DT> r = RowVec<DT>::splat(fill);
        uint32_t ws[4] = {r.w.x, r.w.y, r.w.z, r.w.w};
        const typename Elem<DT>::raw* p = reinterpret_cast<const typename Elem<DT>::raw*>(base) + off;
#pragma unroll
        for (int j = 0; j < RowVec<DT>::V; ++j) {
            if (j < nvalid) {
                if constexpr (DT == DT_F32) {
                    ws[j] = __float_as_uint(p[j]);
                } else {
                    const uint32_t h = p[j];
                    ws[j >> 1] = (j & 1) ? ((ws[j >> 1] & 0x0000ffffu) | (h << 16))
                                         : ((ws[j >> 1] & 0xffff0000u) | h);
                }
            }
        }
        r.w = make_uint4(ws[0], ws[1], ws[2], ws[3]);
        return r;
    }
}

template <int DT, bool ALIGNED>
__device__ __forceinline__ void store_row(void* base, size_t off, int nvalid, const RowOut<DT>& o) {
    if constexpr (ALIGNED) {
        store16_nt(reinterpret_cast<char*>(base) + off * Elem<DT>::bytes, o.pack());
    } else if (nvalid == RowOut<DT>::V) {
        store16_any(reinterpret_cast<char*>(base) + off * Elem<DT>::bytes, o.pack());
    } else {
#pragma unroll
        for (int j = 0; j < RowOut<DT>::V; ++j)
            if (j < nvalid) Elem<DT>::store1(base, off + j, o.v[j]);
    }
}

// Store a vector at an address that need not be 16-byte aligned: a complete
// vector is one 16-byte store at its own address, through the caches (a
// 128-byte line of such a row is written partly by each of two neighbouring
// tiles, and the caches merge the parts before the line reaches memory); a
// row's last, partial vector is written lane by lane.  Each thread writes
// exactly its own lanes.
template <int DT>
__device__ __forceinline__ void store_vec_unaligned(char* p, int nvalid, const RowOut<DT>& o) {
    if (nvalid == Elem<DT>::V) {
        store16_any(p, o.pack());
        return;
    }
#pragma unroll
    for (int j = 0; j < Elem<DT>::V; ++j)
        if (j < nvalid) Elem<DT>::store1(p, j, o.v[j]);
}

// Row vectors addressed as (wave-uniform row pointer) + (per-lane byte offset),
// so the compiler can keep the pointer in SGPRs and one 32-bit offset per lane
// in a VGPR for every row of a tile.
//
// NTL: a non-temporal load, for an input this launch reads for the last time
// in the step (the line is not kept in the caches, so it does not displace
// lines that a later read still wants).  An input that a later launch reads
// again is loaded normally, so part of it is still in the Infinity Cache
// then: the forward loads `a` normally and `b` non-temporally, the backward
// loads everything non-temporally.  Measured on MI355X, forward + backward
// with the caches flushed before each step: [16,4096,2560] bf16 5308 ->
// 5744 GB/s, [4,8192,4096] fp32 5809 -> 6303, [1,131072,1024] bf16 5194 ->
// 5424, [8,2048,2560] bf16 4762 -> 4965; loading `a` non-temporally in the
// forward as well was slower on every shape (the backward then misses it).
template <int DT, bool ALIGNED, bool NTL = false>
__device__ __forceinline__ RowVec<DT> load_vec(const char* row, uint32_t lane_off, int nvalid,
                                               float fill) {
    if constexpr (ALIGNED) {
        RowVec<DT> r;
        if constexpr (NTL) {
            const u32x4_nt w =
                __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(row + lane_off));
            r.w = make_uint4(w.x, w.y, w.z, w.w);
        } else {
            r.w = *reinterpret_cast<const uint4*>(row + lane_off);
        }
        return r;
    } else {
        return load_vec_unaligned<DT>(row + lane_off, nvalid, fill);
    }
}

// The store of one thread's vector of a tile row (`nvalid` lanes of it exist).
template <int DT, bool ALIGNED>
__device__ __forceinline__ void store_vec(char* row, uint32_t lane_off, int nvalid,
                                          const RowOut<DT>& o) {
    if constexpr (ALIGNED)
        store16_nt(row + lane_off, o.pack());
    else
        store_vec_unaligned<DT>(row + lane_off, nvalid, o);
}

// Make the compiler forget what it knows about a register-resident row, so it
// re-widens packed bf16 values where they are used again instead of keeping
// the widened copies alive (which would double the registers a tile needs).
template <int DT>
__device__ __forceinline__ void opaque(RowVec<DT>& r) {
    asm volatile("" : "+v"(r.w.x), "+v"(r.w.y), "+v"(r.w.z), "+v"(r.w.w));
}

// Zero that the compiler cannot see through and that depends on a row loaded
// into registers: loads addressed with it are issued after that row arrived.
template <int DT>
__device__ __forceinline__ int zero_after_row(const RowVec<DT>& r) {
    int z;
    asm volatile("" : "=v"(z) : "0"(0), "v"(r.w.x));
    return z;
}

// Zero that the compiler cannot see through and that depends on `v`: an
// address offset by it cannot be formed, nor its load issued, before `v` is.
__device__ __forceinline__ int zero_after(float v) {
    int z;
    asm volatile("" : "=v"(z) : "0"(0), "v"(v));
    return z;
}

template <typename T>
__device__ __forceinline__ T uniform(T x) {
    return __builtin_amdgcn_readfirstlane(x);
}
__device__ __forceinline__ int64_t uniform64(int64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// ---------------------------------------------------------------------------
// affine maps h -> p*h + q
// ---------------------------------------------------------------------------
struct Aff {
    float p, q;
};

__device__ __forceinline__ Aff aff_identity() { return Aff{1.0f, 0.0f}; }

// "later after earlier": h -> later.p*(earlier.p*h + earlier.q) + later.q
__device__ __forceinline__ Aff aff_then(Aff earlier, Aff later) {
    return Aff{later.p * earlier.p, fmaf(later.p, earlier.q, later.q)};
}

__device__ __forceinline__ float aff_apply(Aff m, float h) { return fmaf(m.p, h, m.q); }

// ---------------------------------------------------------------------------
// in-wavefront scans of affine maps
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ float shfl_up_f(float x, int delta) { return __shfl_up(x, delta, kWave); }

// Inclusive scan over the "group" index g = lane / STRIDE (groups of STRIDE
// adjacent lanes, G = 64 / STRIDE groups), in increasing g: on return lane
// (g, c) holds  m_g after m_{g-1} after ... after m_0  for its column c.
// Hillis-Steele: log2(G) steps, each a cross-lane move through the LDS
// crossbar (ds_bpermute; the offsets are multiples of STRIDE and cross the
// 16-lane DPP rows) and one compose.  The association order is fixed, so the
// result is deterministic.
template <int STRIDE>
__device__ __forceinline__ Aff wave_scan_up(Aff m) {
    const int g = lane_id() / STRIDE;
#pragma unroll
    for (int s = 1; s < kWave / STRIDE; s <<= 1) {
        Aff e;
        e.p = shfl_up_f(m.p, s * STRIDE);
        e.q = shfl_up_f(m.q, s * STRIDE);
        if (g >= s) m = aff_then(e, m);
    }
    return m;
}

// ---------------------------------------------------------------------------
// device-coherent single-word publication (look-back flags + values)
// ---------------------------------------------------------------------------
// A published float is never the all-ones pattern; scratch words start as it.
constexpr uint32_t kEmpty = 0xffffffffu;

__device__ __forceinline__ uint32_t publishable(float x) {
    const uint32_t u = __float_as_uint(x);
    return u == kEmpty ? 0x7fc00000u : u;  // an input NaN with that payload becomes the canonical NaN
}

__device__ __forceinline__ void publish_u32(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void publish_u64(unsigned long long* p, unsigned long long v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t peek_u32(const uint32_t* p) {
    return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long peek_u64(const unsigned long long* p) {
    return __hip_atomic_load(const_cast<unsigned long long*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace lrscan
