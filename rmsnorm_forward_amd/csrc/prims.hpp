// prims.hpp -- gfx950 device primitives for the row-wise norm kernels:
// storage-type conversion, 128-bit vector I/O, DPP wavefront reductions,
// and Chan's parallel merge of (n, mean, M2) partial statistics.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.hpp"

namespace mi355norm {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// --------------------------------------------------------------------------
// Storage types.  Each describes one I/O dtype: its storage word, how to
// widen an element to fp32 and how to round fp32 back (round-to-nearest-even,
// the hardware conversion's default mode).
// --------------------------------------------------------------------------

struct F32 {
    using storage = float;
    static constexpr int bytes = 4;
    __device__ static __forceinline__ float widen(float v) { return v; }
};

struct BF16 {
    using storage = uint16_t;
    static constexpr int bytes = 2;
    // bfloat16 is the high half of a binary32 word
    __device__ static __forceinline__ float widen(uint16_t b) {
        return __uint_as_float((unsigned)b << 16);
    }
    __device__ static __forceinline__ float lo(unsigned w) { return __uint_as_float(w << 16); }
    __device__ static __forceinline__ float hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }
    // v_cvt_pk_bf16_f32: two fp32 -> two bf16, RNE
    __device__ static __forceinline__ unsigned pack(float a, float b) {
        f32x2 v = {a, b};
        bf16x2 r = __builtin_convertvector(v, bf16x2);
        return __builtin_bit_cast(unsigned, r);
    }
    __device__ static __forceinline__ uint16_t narrow(float a) {
        return __builtin_bit_cast(uint16_t, (__bf16)a);
    }
};

struct F16 {
    using storage = uint16_t;
    static constexpr int bytes = 2;
    __device__ static __forceinline__ float widen(uint16_t h) {
        return (float)__builtin_bit_cast(_Float16, h);
    }
    __device__ static __forceinline__ float lo(unsigned w) { return widen((uint16_t)(w & 0xffffu)); }
    __device__ static __forceinline__ float hi(unsigned w) { return widen((uint16_t)(w >> 16)); }
    __device__ static __forceinline__ unsigned pack(float a, float b) {
        f32x2 v = {a, b};
        f16x2 r = __builtin_convertvector(v, f16x2);
        return __builtin_bit_cast(unsigned, r);
    }
    __device__ static __forceinline__ uint16_t narrow(float a) {
        return __builtin_bit_cast(uint16_t, (_Float16)a);
    }
};

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also
// waits for every global load and store in flight (s_waitcnt vmcnt(0)
// before s_barrier), which would stall the reductions on loads still in
// flight (the single passes' next row streaming into LDS, hoisted gamma
// loads) and on earlier stores (the previous row's y, the residual sum).
// Where it is used the wavefronts exchange only LDS values (partial sums,
// a row's statistics, a flag), so the LDS counter is all that must drain.
// The memory clobber keeps the compiler from moving memory accesses across
// it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// --------------------------------------------------------------------------
// Cache policy.  x is read exactly once and y written exactly once, so their
// accesses carry the nontemporal hint (streamed through the caches without
// being kept); gamma and beta are reused by every row and use ordinary loads.
// --------------------------------------------------------------------------

#ifndef MI355_NT_LOAD
#define MI355_NT_LOAD 1
#endif
#ifndef MI355_NT_STORE
#define MI355_NT_STORE 1
#endif

template <class P>
__device__ __forceinline__ P ld_stream(const P* p) {
    if constexpr (MI355_NT_LOAD) return __builtin_nontemporal_load(p);
    else return *p;
}
template <class P>
__device__ __forceinline__ void st_stream(P v, P* p) {
    if constexpr (MI355_NT_STORE) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// --------------------------------------------------------------------------
// A "vector" is the unit one lane moves with one memory instruction: 16 bytes
// (EPV = 16 / element size) on the aligned path, one element (EPV = 1) on the
// element-wise path.  Elements are widened to fp32 on access.
//   load()        cached load (gamma, beta)
//   load_stream() nontemporal load (x)
//   store()       nontemporal store (y)
//   set()         round fp32 values into the vector's storage (RNE)
//   put() / put_stream()   cached / nontemporal store of the vector as held
// --------------------------------------------------------------------------

template <class T, int EPV> struct Vec;

template <> struct Vec<F32, 4> {
    u32x4 w;
    __device__ __forceinline__ void opaque() { asm volatile("" : "+v"(w)); }
    __device__ __forceinline__ void load(const float* p) { w = *reinterpret_cast<const u32x4*>(p); }
    __device__ __forceinline__ void load_stream(const float* p) { w = ld_stream(reinterpret_cast<const u32x4*>(p)); }
    __device__ __forceinline__ void zero() { w = u32x4{0u, 0u, 0u, 0u}; }
    __device__ __forceinline__ float get(int k) const { return __uint_as_float(w[k]); }
    __device__ static __forceinline__ void store(float* p, const float (&v)[4]) {
        u32x4 o = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
        st_stream(o, reinterpret_cast<u32x4*>(p));
    }
    __device__ __forceinline__ void set(const float (&v)[4]) {
        w = u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
    }
    __device__ __forceinline__ void put(float* p) const { *reinterpret_cast<u32x4*>(p) = w; }
    __device__ __forceinline__ void put_stream(float* p) const { st_stream(w, reinterpret_cast<u32x4*>(p)); }
};

template <class H> struct VecHalf8 {
    u32x4 w;
    // Make the packed words opaque to the optimiser so that widened copies
    // made before this point cannot be reused after it (they are recomputed
    // from the packed registers instead of being kept live).
    __device__ __forceinline__ void opaque() { asm volatile("" : "+v"(w)); }
    __device__ __forceinline__ void load(const uint16_t* p) { w = *reinterpret_cast<const u32x4*>(p); }
    __device__ __forceinline__ void load_stream(const uint16_t* p) { w = ld_stream(reinterpret_cast<const u32x4*>(p)); }
    __device__ __forceinline__ void zero() { w = u32x4{0u, 0u, 0u, 0u}; }
    __device__ __forceinline__ float get(int k) const { return (k & 1) ? H::hi(w[k >> 1]) : H::lo(w[k >> 1]); }
    __device__ static __forceinline__ void store(uint16_t* p, const float (&v)[8]) {
        u32x4 o = {H::pack(v[0], v[1]), H::pack(v[2], v[3]), H::pack(v[4], v[5]), H::pack(v[6], v[7])};
        st_stream(o, reinterpret_cast<u32x4*>(p));
    }
    __device__ __forceinline__ void set(const float (&v)[8]) {
        w = u32x4{H::pack(v[0], v[1]), H::pack(v[2], v[3]), H::pack(v[4], v[5]), H::pack(v[6], v[7])};
    }
    __device__ __forceinline__ void put(uint16_t* p) const { *reinterpret_cast<u32x4*>(p) = w; }
    __device__ __forceinline__ void put_stream(uint16_t* p) const { st_stream(w, reinterpret_cast<u32x4*>(p)); }
};
template <> struct Vec<BF16, 8> : VecHalf8<BF16> {};
template <> struct Vec<F16, 8> : VecHalf8<F16> {};

template <class T> struct Vec<T, 1> {
    typename T::storage s;
    __device__ __forceinline__ void opaque() {}
    __device__ __forceinline__ void load(const typename T::storage* p) { s = *p; }
    __device__ __forceinline__ void load_stream(const typename T::storage* p) { s = ld_stream(p); }
    __device__ __forceinline__ void zero() { s = 0; }
    __device__ __forceinline__ float get(int) const { return T::widen(s); }
    __device__ static __forceinline__ void store(typename T::storage* p, const float (&v)[1]) {
        if constexpr (sizeof(typename T::storage) == 4) st_stream(v[0], p);
        else st_stream(T::narrow(v[0]), p);
    }
    __device__ __forceinline__ void set(const float (&v)[1]) {
        if constexpr (sizeof(typename T::storage) == 4) s = v[0];
        else s = T::narrow(v[0]);
    }
    __device__ __forceinline__ void put(typename T::storage* p) const { *p = s; }
    __device__ __forceinline__ void put_stream(typename T::storage* p) const { st_stream(s, p); }
};

// Residual add in the storage type: h = x + r rounded to T (RNE).  The fp32
// sum of two values of one of these formats rounds, if at all, only when the
// smaller is below half an ulp of the larger in T, so rounding the fp32 sum
// to T equals rounding the exact sum.
template <class T, int EPV>
__device__ __forceinline__ void add_into(Vec<T, EPV>& x, const Vec<T, EPV>& r) {
    float h[EPV];
#pragma unroll
    for (int k = 0; k < EPV; ++k) h[k] = x.get(k) + r.get(k);
    x.set(h);
}

// --------------------------------------------------------------------------
// FP8 output (OCP E4M3, the format gfx950's v_cvt_pk_fp8_f32 produces):
// values are saturated to +-448 first (the conversion itself turns anything
// that rounds past 448 into NaN), NaN passes through; rounding is to nearest
// even.  One vector of EPV results becomes EPV bytes, stored nontemporal.
// --------------------------------------------------------------------------

// v_med3_f32 clamps in one instruction but maps NaN to -448 on gfx950, so a
// NaN is put back with one compare and select (three instructions instead of
// the four of two compare-selects)
__device__ __forceinline__ float sat_e4m3(float v) {
    const float c = __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f);
    return __builtin_isnan(v) ? v : c;
}

__device__ __forceinline__ unsigned e4m3x4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(a), sat_e4m3(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(c), sat_e4m3(d), w, true);
    return (unsigned)w;
}

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

template <int EPV>
__device__ __forceinline__ void store_e4m3(uint8_t* p, const float (&v)[EPV]) {
    if constexpr (EPV == 8) {
        u32x2 w = {e4m3x4(v[0], v[1], v[2], v[3]), e4m3x4(v[4], v[5], v[6], v[7])};
        st_stream(w, reinterpret_cast<u32x2*>(p));
    } else if constexpr (EPV == 4) {
        st_stream(e4m3x4(v[0], v[1], v[2], v[3]), reinterpret_cast<unsigned*>(p));
    } else {
        static_assert(EPV == 1, "EPV");
        const int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(v[0]), 0.0f, 0, false);
        st_stream((uint8_t)(w & 0xff), p);
    }
}

// 1/sqrt(v) with the hardware reciprocal square root (v_rsq_f32, about one
// ulp): one instruction per row instead of a correctly rounded square root
// and divide.  rsq(0) = +inf as IEEE requires.
__device__ __forceinline__ float rsqrt_hw(float v) { return __builtin_amdgcn_rsqf(v); }

// --------------------------------------------------------------------------
// Cross-lane primitives (wave64).
// --------------------------------------------------------------------------

// DPP controls of the GFX9 family (gfx950 keeps them).
constexpr int DPP_QUAD_XOR1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;   // lane i <- lane 7-i within 8
constexpr int DPP_ROW_MIRROR = 0x140;        // lane i <- lane 15-i within 16

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_amdgcn_update_dpp(0.0f, v, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ float readlane(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// Sum over aligned groups of TEAM lanes (TEAM a power of two <= 64).  Every
// lane of a group ends with the bitwise-identical group total: each xor /
// mirror step adds a lane's value to its partner's, and IEEE addition is
// commutative, so both partners compute the same sum; the mirror steps pair
// quads (resp. 8-lane halves) only once those are already uniform.  All 64
// lanes must be active.
template <int TEAM>
__device__ __forceinline__ float team_sum(float v) {
    static_assert(TEAM >= 1 && TEAM <= 64 && (TEAM & (TEAM - 1)) == 0, "TEAM");
    if constexpr (TEAM >= 2) v += dpp<DPP_QUAD_XOR1>(v);
    if constexpr (TEAM >= 4) v += dpp<DPP_QUAD_XOR2>(v);
    if constexpr (TEAM >= 8) v += dpp<DPP_ROW_HALF_MIRROR>(v);
    if constexpr (TEAM >= 16) v += dpp<DPP_ROW_MIRROR>(v);
    if constexpr (TEAM == 32) {
        float a = readlane(v, 0), b = readlane(v, 16), c = readlane(v, 32), d = readlane(v, 48);
        v = (lane_id() < 32) ? (a + b) : (c + d);
    }
    if constexpr (TEAM == 64) {
        float a = readlane(v, 0), b = readlane(v, 16), c = readlane(v, 32), d = readlane(v, 48);
        v = (a + b) + (c + d);
    }
    return v;
}

// --------------------------------------------------------------------------
// Chan's parallel merge of partial statistics ("CUDA 算子工程" ch. 7,
// section 7.4.1): (na, ma, M2a) + (nb, mb, M2b) with n = na + nb,
// delta = mb - ma, mean = ma + delta * nb / n,
// M2 = M2a + M2b + delta^2 * na * nb / n.  Counts are fp32 (exact below 2^24).
// An empty operand returns the other one unchanged.
// --------------------------------------------------------------------------

struct Welford {
    float n, mean, m2;
};

__device__ __forceinline__ Welford chan_merge(Welford a, Welford b) {
    float n = a.n + b.n;
    float w = b.n / n;
    float d = b.mean - a.mean;
    Welford r;
    r.n = n;
    r.mean = a.mean + d * w;
    r.m2 = (a.m2 + b.m2) + (d * d) * (a.n * w);
    if (a.n == 0.0f) r = b;
    if (b.n == 0.0f) r = a;
    return r;
}

// Realigned loads of x (16-byte vectors when x alone is not 16-byte
// aligned, e.g. a view into a larger tensor, while y, gamma and beta are),
// used by the row and split-row kernels.  Each lane loads the aligned
// 16-byte block holding the start of its vector and takes the following
// block from the next lane (DPP wave_shl:1: lane l reads lane l + 1); a lane
// whose next block no lane of its wavefront and team holds (the team's and
// the wavefront's last lanes, and the row's last vector) loads it itself.
// Every block loaded holds at least one byte of the row, so no load leaves
// the row's pages.  `mb` is the row's byte misalignment (a multiple of the
// element size); the lane's vector is bytes [mb, mb + 16) of the 32 bytes
// cur:nxt.
template <bool UNIFORM>
__device__ __forceinline__ u32x4 realign_words(u32x4 cur, u32x4 nxt, unsigned mb) {
    const unsigned c0 = cur[0], c1 = cur[1], c2 = cur[2], c3 = cur[3];
    const unsigned c4 = nxt[0], c5 = nxt[1], c6 = nxt[2], c7 = nxt[3];
    const unsigned r = mb & 3u;
    auto shift = [r](unsigned lo, unsigned hi) { return __builtin_amdgcn_alignbyte(hi, lo, r); };
    const unsigned q = mb >> 2;
    if constexpr (UNIFORM) {
        // q is the same for the whole wavefront: one scalar branch
        switch (q) {
        case 0: return u32x4{shift(c0, c1), shift(c1, c2), shift(c2, c3), shift(c3, c4)};
        case 1: return u32x4{shift(c1, c2), shift(c2, c3), shift(c3, c4), shift(c4, c5)};
        case 2: return u32x4{shift(c2, c3), shift(c3, c4), shift(c4, c5), shift(c5, c6)};
        default: return u32x4{shift(c3, c4), shift(c4, c5), shift(c5, c6), shift(c6, c7)};
        }
    } else {
        // rows of different lanes may differ: select per lane
        const unsigned s0 = q == 0 ? c0 : q == 1 ? c1 : q == 2 ? c2 : c3;
        const unsigned s1 = q == 0 ? c1 : q == 1 ? c2 : q == 2 ? c3 : c4;
        const unsigned s2 = q == 0 ? c2 : q == 1 ? c3 : q == 2 ? c4 : c5;
        const unsigned s3 = q == 0 ? c3 : q == 1 ? c4 : q == 2 ? c5 : c6;
        const unsigned s4 = q == 0 ? c4 : q == 1 ? c5 : q == 2 ? c6 : c7;
        return u32x4{shift(s0, s1), shift(s1, s2), shift(s2, s3), shift(s3, s4)};
    }
}

// The exchange has to run with every lane of the wavefront active: a DPP read
// of an inactive lane returns nothing.  The empty asm consumes the result in
// every lane, so the compiler cannot move the exchange into a branch taken
// only by the lanes that use it.
__device__ __forceinline__ u32x4 next_lane_words(u32x4 v) {
    u32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const unsigned w = v[k];
        unsigned r = (unsigned)__builtin_amdgcn_update_dpp(0, (int)w, 0x130 /* wave_shl:1 */, 0xf, 0xf, false);
        asm volatile("" : "+v"(r));
        o[k] = r;
    }
    return o;
}

// Teams of at most 64 lanes lie within one wavefront: lane t of a team
// reads lane t + 1 of the same team, the team's last lane its first lane
// (ds_bpermute; every lane active, as above).
template <int TEAM>
__device__ __forceinline__ u32x4 team_rotate_words(u32x4 v) {
    static_assert(TEAM <= 64 && (TEAM & (TEAM - 1)) == 0, "a power-of-two team within one wavefront");
    const int l = lane_id();
    const int src = ((l & ~(TEAM - 1)) | ((l + 1) & (TEAM - 1))) << 2;
    u32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const unsigned w = v[k];
        unsigned r = (unsigned)__builtin_amdgcn_ds_bpermute(src, (int)w);
        asm volatile("" : "+v"(r));
        o[k] = r;
    }
    return o;
}

}  // namespace mi355norm
