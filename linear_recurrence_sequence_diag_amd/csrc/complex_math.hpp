// complex_math.hpp -- complex fp32 arithmetic, complex affine maps, their
// in-wavefront scans and their publication words, shared by the complex
// scan (complex.hip) and the fused-transition scan (samu.hip).  Internal to
// liblrscan; each including translation unit gets its own copy.
#pragma once

#include "fused_common.hpp"

namespace lrscan {

namespace {

// The index limits of a tiled kernel (32-bit row offsets inside a tile,
// 32-bit lane and row indices, 32-bit tickets) for a tile of `tile` rows.
bool tiled_layout_ok(const Shape& s, int tile, int nt, const Layout& L) {
    const int64_t eb = s.dtype == DT_F32 ? 4 : 2;
    if ((int64_t)(tile + 1) * s.D * eb >= ((int64_t)1 << 31)) return false;
    if (s.T >= ((int64_t)1 << 31) - tile || s.D >= ((int64_t)1 << 30)) return false;
    if ((unsigned long long)L.NK * L.nS >= 0xffffffffull) return false;
    if (!grid_fits(L, nt)) return false;
    if (s.B * (int64_t)L.nW >= ((int64_t)1 << 31)) return false;
    return true;
}

// ---------------------------------------------------------------------------
// complex arithmetic (fp32)
// ---------------------------------------------------------------------------
struct Cx {
    float r, i;
};

__device__ __forceinline__ Cx cconj(Cx a) { return Cx{a.r, -a.i}; }
__device__ __forceinline__ Cx cadd(Cx a, Cx b) { return Cx{a.r + b.r, a.i + b.i}; }
// a * b
__device__ __forceinline__ Cx cmul(Cx a, Cx b) {
    return Cx{fmaf(a.r, b.r, -(a.i * b.i)), fmaf(a.r, b.i, a.i * b.r)};
}
// a * h + b
__device__ __forceinline__ Cx cfma(Cx a, Cx h, Cx b) {
    return Cx{fmaf(a.r, h.r, fmaf(-a.i, h.i, b.r)), fmaf(a.r, h.i, fmaf(a.i, h.r, b.i))};
}

// The affine map h -> p*h + q over complex values; "later after earlier".
struct CAff {
    Cx p, q;
};
__device__ __forceinline__ CAff caff_identity() { return CAff{Cx{1.0f, 0.0f}, Cx{0.0f, 0.0f}}; }
__device__ __forceinline__ CAff caff_then(CAff earlier, CAff later) {
    return CAff{cmul(later.p, earlier.p), cfma(later.p, earlier.q, later.q)};
}
__device__ __forceinline__ Cx caff_apply(CAff m, Cx h) { return cfma(m.p, h, m.q); }
struct CAffThen {
    __device__ static CAff then(CAff earlier, CAff later) { return caff_then(earlier, later); }
};

// One step of the forward as a map: h -> a*h + b.
__device__ __forceinline__ CAff fwd_step(Cx a, Cx b) { return CAff{a, b}; }
// One step of the reverse carry as a map: c -> conj(a)*(g + c).
__device__ __forceinline__ CAff rev_fold(CAff m, Cx a, Cx g) {
    const Cx ac = cconj(a);
    return CAff{cmul(ac, m.p), cmul(ac, cadd(m.q, g))};
}

// ---------------------------------------------------------------------------
// publication
// ---------------------------------------------------------------------------
__device__ __forceinline__ unsigned long long pack_cx(Cx z) {
    return (unsigned long long)publishable(z.r) | ((unsigned long long)publishable(z.i) << 32);
}
__device__ __forceinline__ Cx unpack_cx(unsigned long long w) {
    return Cx{__uint_as_float((uint32_t)w), __uint_as_float((uint32_t)(w >> 32))};
}

struct CxPair {
    unsigned long long p, q;
};

// A complex entry: P, Q and H, one 64-bit word each (6 words per entry).
constexpr int kComplexWords = 6;

struct ComplexLink {
    using S = Cx;
    using M = CAff;
    using HRaw = unsigned long long;
    using MRaw = CxPair;
    const unsigned long long* ps;
    const unsigned long long* qs;
    const unsigned long long* hs;
    int nS, s, W, c;
    __device__ size_t entry(int j) const { return ((size_t)j * (size_t)nS + (size_t)s) * W + c; }
    __device__ HRaw load_h(int j) const { return peek_u64(hs + entry(j)); }
    __device__ MRaw load_m(int j) const {
        const size_t e = entry(j);
        return CxPair{peek_u64(ps + e), peek_u64(qs + e)};
    }
    __device__ static HRaw empty_h() { return ~0ull; }
    __device__ static MRaw empty_m() { return CxPair{~0ull, ~0ull}; }
    __device__ static bool ready_h(HRaw w) { return (uint32_t)w != kEmpty; }
    __device__ static bool ready_m(MRaw w) {
        return (uint32_t)w.p != kEmpty && (uint32_t)w.q != kEmpty;
    }
    __device__ static S state(HRaw w) { return unpack_cx(w); }
    __device__ static M map(MRaw w) { return CAff{unpack_cx(w.p), unpack_cx(w.q)}; }
    __device__ static S apply(M m, S x) { return caff_apply(m, x); }
};

// Published words of region `phase`: P, Q, H arrays of `entries` words each.
struct CxWords {
    unsigned long long *ps, *qs, *hs;
};
__device__ __forceinline__ CxWords cx_words(const Scratch& sc, uint32_t phase) {
    unsigned long long* base =
        reinterpret_cast<unsigned long long*>(sc.region[phase]);
    return CxWords{base, base + sc.entries, base + 2 * sc.entries};
}

// One lane of a planar row pair, and one stored element pair.
template <int DT>
__device__ __forceinline__ Cx vget(const RowVec<DT>& re, const RowVec<DT>& im, int j) {
    return Cx{re.get(j), im.get(j)};
}

template <int DT>
__device__ __forceinline__ Cx load_cx(const char* re, const char* im, size_t off) {
    return Cx{Elem<DT>::load1(re + off, 0), Elem<DT>::load1(im + off, 0)};
}

}  // namespace

}  // namespace lrscan
