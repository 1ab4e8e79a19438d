// split.hpp -- rows too long for one workgroup's registers.  A row is cut
// into chunks of CV = WG*VPL vectors; a chunk is one workgroup's work item.
//
// Per chunk, LayerNorm computes (mean about K, M2) over its n_c elements by
// two passes over the chunk in registers, K = x[row, 0] being the row shift
// every chunk of the row shares; RMSNorm computes its sum of squares.  A row's
// partials are merged in chunk order with Chan's formula; every workgroup of
// the row runs the identical merge, so all chunks of a row normalise with
// bitwise-identical mean and rstd.  Merging (n, mean, M2) partials is what
// "T3 讲解" part ② recommends once a row has to be read in segments, with the
// associative merge of "CUDA 算子工程" ch. 7 section 7.4.1.
//
// Two schedules:
//   norm_split_stats_kernel  two kernels.  Partials (x read through the
//   + norm_split_apply_kernel  caches), then a second kernel that merges
//                            the row's partials, re-reads x and stores y (the
//                            two may cut rows into chunks of different
//                            sizes).  x crosses from memory to the CUs twice;
//                            measured on MI355X, the second read is served
//                            partly from the Infinity Cache (the normalising
//                            kernel takes 42-44 us after the statistics
//                            kernel on LN bf16 64 x 2^20, 52.5 us when x
//                            comes from HBM), while rocprofv3's FETCH_SIZE
//                            counts both reads either way.
//   norm_split_pass_kernel   single pass, x read once, ordinary launch.  Each
//                            workgroup keeps its chunk in VGPRs, publishes
//                            its partial in the row's slot for it, waits
//                            (one wavefront polling, bounded in time) until
//                            every slot of the row holds a partial, merges
//                            them and normalises from registers.  Teams of S
//                            workgroups walk the rows.  A slot holds its
//                            partial's bits inverted, zero meaning "not yet
//                            published", so waiting on the slots themselves
//                            needs no ordering between separate variables;
//                            the last workgroup of a row to finish returns
//                            the row's slots and departure counter to zero.
//                            If the wait runs out (a workgroup of the team
//                            is not resident, e.g. while another kernel
//                            holds CUs), the workgroup computes every
//                            chunk's partial of the row itself from x,
//                            publishes them and goes on: the same bits,
//                            just slower, so the result never depends on
//                            co-residency and nothing can hang.  With
//                            16-byte vectors, the workgroup's next row's
//                            chunk streams into LDS while it waits on this
//                            one (global_load_lds, no VGPRs held): LN bf16
//                            64 x 2^20 65.0 us vs 68.5-68.9 without.
#pragma once

#include "prims.hpp"

namespace mi355norm {

// workgroup-wide sum (WG/64 wavefronts), bitwise identical in every lane
template <int WG>
__device__ __forceinline__ float wg_sum(float v, float* slots) {
    v = team_sum<64>(v);
    if constexpr (WG > 64) {
        constexpr int W = WG / 64;
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        if (lane_id() == 0) slots[wave] = v;
        lds_barrier();
        float s = slots[0];
#pragma unroll
        for (int w = 1; w < W; ++w) s += slots[w];
        v = s;
    }
    return v;
}

// cache-policy operand of global_load_lds for a nontemporal load (gfx950)
constexpr int kAuxNontemporal = 2;

// RA: x's rows may start off a 16-byte boundary (16-byte vectors only); the
// chunk is read in aligned blocks and realigned in registers.
template <class T, int WG, int VPL, int EPV, bool RA = false>
struct Chunk {
    using V = Vec<T, EPV>;
    using S = typename T::storage;
    static constexpr int CV = WG * VPL;      // vectors per chunk
    static_assert(!RA || EPV * sizeof(S) == 16, "realigned chunks hold 16-byte vectors");
    V xv[VPL];
    bool ok[VPL];
    int v0;                                  // first vector of the chunk

    // xr: the row (wavefront-uniform); lane offsets are 32-bit (N < 2^24).
    // STREAM: nontemporal (x's last read); otherwise cached, so that a second
    // read soon after can be served by the on-die caches.
    template <bool STREAM = true>
    __device__ __forceinline__ void load(const S* xr, int c, int NV) {
        v0 = c * CV;
        // realigned: the row's byte misalignment (one row per workgroup, so
        // wave-uniform) and the aligned address below the row's start
        unsigned mb = 0;
        const S* xa = xr;
        if constexpr (RA) {
            mb = __builtin_amdgcn_readfirstlane((unsigned)(reinterpret_cast<uintptr_t>(xr) & 15u));
            xa = reinterpret_cast<const S*>(reinterpret_cast<uintptr_t>(xr) - mb);
        }
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            const unsigned v = (unsigned)(v0 + j * WG) + threadIdx.x;
            ok[j] = (int)v < NV;
            if (ok[j]) {
                if constexpr (STREAM) xv[j].load_stream(xa + v * EPV);
                else xv[j].load(xa + v * EPV);
            } else {
                xv[j].zero();
            }
        }
        if constexpr (RA) {
            // the block after the lane's own: from the next lane, or loaded
            // by the wavefront's last lane and the row's last vector
            V ex[VPL];
            bool own[VPL];
#pragma unroll
            for (int j = 0; j < VPL; ++j) {
                const unsigned v = (unsigned)(v0 + j * WG) + threadIdx.x;
                own[j] = mb != 0u && ok[j] && (lane_id() == 63 || (int)v == NV - 1);
                if (own[j]) {
                    if constexpr (STREAM) ex[j].load_stream(xa + (v + 1) * EPV);
                    else ex[j].load(xa + (v + 1) * EPV);
                }
            }
#pragma unroll
            for (int j = 0; j < VPL; ++j) {
                const u32x4 nl = next_lane_words(xv[j].w);    // every lane active
                xv[j].w = realign_words<true>(xv[j].w, own[j] ? ex[j].w : nl, mb);
            }
        }
    }

    // Single pass, 16-byte vectors only: the next row's chunk goes straight
    // into LDS (global_load_lds_dwordx4, no VGPRs held), lane t's vectors at
    // pre[j][t], nontemporal (x's only read).  from_lds() waits for this
    // wavefront's loads and reads back the lane's own vectors, so no barrier
    // is needed.
    __device__ __forceinline__ void prefetch(const typename T::storage* xr, int c, int NV, u32x4 (*pre)[WG]) const {
        const int wave = threadIdx.x >> 6;
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            const unsigned v = (unsigned)(c * CV + j * WG) + threadIdx.x;
            if ((int)v < NV)
                __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(xr + v * EPV),
                                                 (__attribute__((address_space(3))) void*)&pre[j][wave * 64], 16, 0,
                                                 kAuxNontemporal);
        }
    }
    __device__ __forceinline__ void from_lds(int c, int NV, const u32x4 (*pre)[WG]) {
        v0 = c * CV;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            const unsigned v = (unsigned)(v0 + j * WG) + threadIdx.x;
            ok[j] = (int)v < NV;
            if (ok[j]) xv[j].w = pre[j][threadIdx.x];
            else xv[j].zero();
        }
    }

    // residual add: the chunk becomes h = x + r (rounded to the storage
    // type), which is also stored to hr (nontemporal if STREAM, else cached
    // so that a second read soon after is served on-die)
    template <bool STREAM>
    __device__ __forceinline__ void add_residual(const typename T::storage* rr, typename T::storage* hr) {
        V rv[VPL];
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            const unsigned v = (unsigned)(v0 + j * WG) + threadIdx.x;
            if (ok[j]) {
                if constexpr (STREAM) rv[j].load_stream(rr + v * EPV);
                else rv[j].load(rr + v * EPV);
            }
        }
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            if (!ok[j]) continue;
            const unsigned v = (unsigned)(v0 + j * WG) + threadIdx.x;
            add_into(xv[j], rv[j]);
            if constexpr (STREAM) xv[j].put_stream(hr + v * EPV);
            else xv[j].put(hr + v * EPV);
        }
    }

    // keep widened copies from living across phases: re-widen instead
    __device__ __forceinline__ void opaque() {
#pragma unroll
        for (int j = 0; j < VPL; ++j) xv[j].opaque();
    }

    // LayerNorm: (mean of x - K, M2 about that mean) over the chunk's valid
    // elements; RMSNorm: (sum of squares, 0).  Uses both LDS slot sets.
    // Masked vectors are dropped by one select per vector.
    // Contraction is off: every inlined copy (the single pass computes the
    // same chunk's partial in two places) performs exactly these IEEE
    // operations, so all copies give the same bits.
    template <bool RMS>
    __device__ __forceinline__ float2 partial(float K, int NV, float (*red)[WG / 64]) {
#pragma clang fp contract(off)
        if constexpr (RMS) {
            float q = 0.0f;
#pragma unroll
            for (int j = 0; j < VPL; ++j) {
                float t = 0.0f;
#pragma unroll
                for (int k = 0; k < EPV; ++k) t = __builtin_fmaf(xv[j].get(k), xv[j].get(k), t);
                q += ok[j] ? t : 0.0f;
            }
            return make_float2(wg_sum<WG>(q, red[0]), 0.0f);
        } else {
            const int nvec = min(CV, NV - v0);
            const float nc = (float)nvec * (float)EPV;
            float s = 0.0f;
#pragma unroll
            for (int j = 0; j < VPL; ++j) {
                float t[EPV];
#pragma unroll
                for (int k = 0; k < EPV; ++k) t[k] = xv[j].get(k) - K;
#pragma unroll
                for (int h = 1; h < EPV; h *= 2)
#pragma unroll
                    for (int k = 0; k + h < EPV; k += 2 * h) t[k] += t[k + h];
                s += ok[j] ? t[0] : 0.0f;
            }
            s = wg_sum<WG>(s, red[0]);
            const float mc = s / nc;
            opaque();
            float q = 0.0f;
#pragma unroll
            for (int j = 0; j < VPL; ++j) {
                float t = 0.0f;
#pragma unroll
                for (int k = 0; k < EPV; ++k) {
                    const float e = (xv[j].get(k) - K) - mc;
                    t = __builtin_fmaf(e, e, t);
                }
                q += ok[j] ? t : 0.0f;
            }
            return make_float2(mc, wg_sum<WG>(q, red[1]));
        }
    }

    // normalise the chunk from registers, apply the affine, store; gamma /
    // beta loads run at most four vectors ahead of their use
    // Q8: yr points at one byte per element and receives the E4M3 codes of
    // the results times qinv
    template <bool RMS, bool Q8 = false>
    __device__ __forceinline__ void apply(void* yr, const typename T::storage* gamma,
                                          const typename T::storage* beta, float K, float mu,
                                          float rs, float qinv = 1.0f) {
        const bool has_g = gamma != nullptr;
        const bool has_b = beta != nullptr;
        if constexpr (Q8) rs *= qinv;      // the 1/scale factor rides on rstd
        opaque();
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            if (j % 4 == 0 && j > 0) __builtin_amdgcn_sched_barrier(0);
            if (!ok[j]) continue;
            const unsigned off = ((unsigned)(v0 + j * WG) + threadIdx.x) * EPV;
            V gv, bv;
            if (has_g) gv.load(gamma + off);
            if (!RMS && has_b) bv.load(beta + off);
            float o[EPV];
#pragma unroll
            for (int k = 0; k < EPV; ++k) {
                const float g = has_g ? gv.get(k) : 1.0f;
                if constexpr (RMS) o[k] = (xv[j].get(k) * rs) * g;
                else o[k] = __builtin_fmaf(((xv[j].get(k) - K) - mu) * rs, g, has_b ? bv.get(k) : 0.0f);
            }
            if constexpr (Q8) {
                store_e4m3<EPV>(static_cast<uint8_t*>(yr) + off, o);
            } else {
                V::store(static_cast<typename T::storage*>(yr) + off, o);
            }
        }
    }

};

// start of row `row` of an output of the I/O dtype, or of FP8 codes
template <class T, bool Q8>
__device__ __forceinline__ void* row_out(void* y, int64_t row, int64_t ldy) {
    if constexpr (Q8) return static_cast<uint8_t*>(y) + row * ldy;
    else return static_cast<typename T::storage*>(y) + row * ldy;
}

// Merge a row's S partials (read(c) gives partial c; S arbitrary) inside one
// wavefront; the result is wave-uniform and identical in every wavefront
// that runs it on the same data.  Lane l folds partials l, l+64, l+128, ...
// in order; the 64 lane states are then merged by a butterfly whose every
// step puts the lower lane's state first, so partners compute bitwise-
// identical results.
template <class Read>
__device__ __forceinline__ Welford merge_partials(Read&& read, int S, int CE, int N) {
    const int l = lane_id();
    Welford a = {0.0f, 0.0f, 0.0f};
    for (int c = l; c < S; c += 64) {
        const float2 v = read(c);
        const int n = min(CE, N - c * CE);
        a = chan_merge(a, Welford{(float)n, v.x, v.y});
    }
#define MI355_CHAN_STEP(CTRL, BIT)                                              \
    {                                                                           \
        Welford b = {dpp<CTRL>(a.n), dpp<CTRL>(a.mean), dpp<CTRL>(a.m2)};      \
        const bool upper = (l & (BIT)) != 0;                                    \
        a = upper ? chan_merge(b, a) : chan_merge(a, b);                        \
    }
    MI355_CHAN_STEP(DPP_QUAD_XOR1, 1)
    MI355_CHAN_STEP(DPP_QUAD_XOR2, 2)
    MI355_CHAN_STEP(DPP_ROW_HALF_MIRROR, 4)
    MI355_CHAN_STEP(DPP_ROW_MIRROR, 8)
#undef MI355_CHAN_STEP
    Welford r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        r[i] = Welford{readlane(a.n, 16 * i), readlane(a.mean, 16 * i), readlane(a.m2, 16 * i)};
    return chan_merge(chan_merge(r[0], r[1]), chan_merge(r[2], r[3]));
}

// Row statistics from its S partials (read(c) gives partial c): (mean about
// K, rstd), wave-uniform.
template <bool RMS, class Read>
__device__ __forceinline__ float2 row_stats(Read&& read, int S, int CE, int N, float eps) {
    const float inv_n = 1.0f / (float)N;
    if constexpr (RMS) {
        float q = 0.0f;
        for (int cc = lane_id(); cc < S; cc += 64) q += read(cc).x;
        q = team_sum<64>(q);
        return make_float2(0.0f, rsqrt_hw(__builtin_fmaf(q, inv_n, eps)));
    } else {
        const Welford w = merge_partials(read, S, CE, N);
        return make_float2(w.mean, rsqrt_hw(__builtin_fmaf(w.m2, inv_n, eps)));
    }
}

// x[row, 0] through the scalar cache: the aligned dword that holds it (split
// rows have more than two elements, so that dword lies within the row, or
// takes the element before it).
template <class T>
__device__ __forceinline__ float shift_scalar(const typename T::storage* xr) {
    typedef __attribute__((address_space(4))) const unsigned cu32;
    const uintptr_t a = (uintptr_t)xr;
    const unsigned w = *(cu32*)(a & ~uintptr_t(3));
    if constexpr (sizeof(typename T::storage) == 4) return __uint_as_float(w);
    else return T::widen((uint16_t)((a & 2) ? (w >> 16) : (w & 0xffffu)));
}

// ---------------------------------------------------------------------------
// single pass
// ---------------------------------------------------------------------------

// A published partial is its 64 bits inverted, so that zero -- what the
// workspace holds when allocated and after each row's reset -- means "not
// yet published".  Only a partial of two NaNs with every payload bit set
// inverts to zero; such a row waits out its bound and takes the recompute
// path, which gives the same (NaN) result.
__device__ __forceinline__ void publish_slot(unsigned long long* slot, float2 v) {
    const unsigned long long bits =
        ((unsigned long long)__float_as_uint(v.y) << 32) | (unsigned long long)__float_as_uint(v.x);
    __hip_atomic_store(slot, ~bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned long long read_slot(const unsigned long long* slot) {
    return __hip_atomic_load(const_cast<unsigned long long*>(slot), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float2 slot_value(unsigned long long s) {
    const unsigned long long bits = ~s;
    return make_float2(__uint_as_float((unsigned)bits), __uint_as_float((unsigned)(bits >> 32)));
}

// One wavefront: whether all S slots hold a partial, polling until they do
// or `ticks` of the 100 MHz real-time clock have passed (ticks == 0: no
// polling at all, the caller recomputes).
__device__ __forceinline__ bool wait_slots(const unsigned long long* slots, int S, unsigned ticks) {
    if (ticks == 0) return false;
    const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
    const int l = lane_id();
    while (true) {
        bool have = true;
        for (int c = l; c < S; c += 64) have = have && read_slot(slots + c) != 0ull;
        if (__builtin_amdgcn_ballot_w64(!have) == 0ull) return true;
        if (__builtin_amdgcn_s_memrealtime() - t0 >= ticks) return false;
        __builtin_amdgcn_s_sleep(2);
    }
}

// One wavefront, after merging the row: count this workgroup's departure;
// the last of the row's S returns the S slots and the counter to zero.
__device__ __forceinline__ void depart_row(unsigned* dep, unsigned long long* slots, int S) {
    unsigned last = 0;
    if (lane_id() == 0)
        last = __hip_atomic_fetch_add(dep, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (unsigned)S - 1;
    last = __builtin_amdgcn_readfirstlane(last);
    if (last) {
        for (int c = lane_id(); c < S; c += 64)
            __hip_atomic_store(slots + c, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (lane_id() == 0) __hip_atomic_store(dep, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Workgroup (team, c) handles chunk c of rows team, team + teams, ...  slots:
// [M, S] published partials; dep: row r's departure counter at dep[64 r].
// Both are zero at launch and again at exit.  The second half of the teams
// starts `stagger` ticks late, so that on a CU holding one workgroup of each
// half their loads, arithmetic and waits interleave.
template <class T, bool RMS, bool Q8, int WG, int VPL, int EPV>
__global__ __launch_bounds__(WG)
void norm_split_pass_kernel(const typename T::storage* __restrict__ x,
                            const typename T::storage* __restrict__ gamma,
                            const typename T::storage* __restrict__ beta,
                            void* y,
                            float* __restrict__ mean_out,
                            float* __restrict__ rstd_out,
                            unsigned long long* __restrict__ slots,
                            unsigned* __restrict__ dep,
                            int64_t M, int N, Strides ld, int S, int teams, float eps, float qinv,
                            unsigned wait_ticks, unsigned stagger)
{
    static_assert(!Q8 || RMS, "FP8 output is fused with RMSNorm only");
    using C = Chunk<T, WG, VPL, EPV>;
    constexpr int CE = C::CV * EPV;           // elements per chunk
    __shared__ float red[2][WG / 64];
    __shared__ float2 stats;                  // (mean about K, rstd) of the current row
    __shared__ int late;
    // next row's chunk, loaded during this row's wait (16-byte vectors)
    constexpr bool PRE = EPV * sizeof(typename T::storage) == 16;
    __shared__ u32x4 pre[PRE ? VPL : 1][PRE ? WG : 1];
    bool have_pre = false;
    const int tid = threadIdx.x;
    const int NV = N / EPV;
    const int team = blockIdx.x / S;          // grid is exactly teams * S
    const int c = blockIdx.x - team * S;

    if (stagger && 2 * team >= teams) {
        const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
        while (__builtin_amdgcn_s_memrealtime() - t0 < stagger) __builtin_amdgcn_s_sleep(8);
    }
    auto read = [](const unsigned long long* sl) { return [sl](int cc) { return slot_value(read_slot(sl + cc)); }; };
    for (int64_t row = team; row < M; row += teams) {
        const typename T::storage* xr = x + row * ld.x;
        unsigned long long* rs = slots + row * S;
        const float K = RMS ? 0.0f : shift_scalar<T>(xr);
        C ch;
        if constexpr (PRE) {
            if (have_pre) ch.from_lds(c, NV, pre);
            else ch.load(xr, c, NV);
        } else {
            ch.load(xr, c, NV);
        }
        const float2 p = ch.template partial<RMS>(K, NV, red);
        if (tid == 0) publish_slot(rs + c, p);
        if constexpr (PRE) {
            // the next row's chunk streams into LDS during the wait, the
            // merge and this row's stores (issued after the publication:
            // earlier, it slowed the partial and the polling wavefront)
            have_pre = row + teams < M;
            if (have_pre) ch.prefetch(x + (row + teams) * ld.x, c, NV, pre);
        }
        if (tid < 64) {
            const bool have = wait_slots(rs, S, wait_ticks);
            if (have) {
                const float2 st = row_stats<RMS>(read(rs), S, CE, N, eps);
                if (tid == 0) stats = st;
                depart_row(dep + row * 64, rs, S);
            }
            if (tid == 0) late = !have;
        }
        lds_barrier();
        if (late) {
            // recompute: every chunk's partial of the row from x, published
            // (the same bits its own workgroup publishes), then the merge
            for (int cc = 0; cc < S; ++cc) {
                ch.load(xr, cc, NV);
                const float2 q = ch.template partial<RMS>(K, NV, red);
                if (tid == 0) publish_slot(rs + cc, q);
                // RMSNorm's partial has one reduction, whose LDS slots the
                // next chunk's would otherwise rewrite while a wavefront
                // still reads them
                if constexpr (RMS) lds_barrier();
            }
            if (tid < 64) {
                const float2 st = row_stats<RMS>(read(rs), S, CE, N, eps);
                if (tid == 0) stats = st;
                depart_row(dep + row * 64, rs, S);
            }
            lds_barrier();
            ch.load(xr, c, NV);
        }
        const float2 st = stats;
        if (c == 0 && tid == 0) {
            if (!RMS && mean_out) mean_out[row] = K + st.x;
            if (rstd_out) rstd_out[row] = st.y;
        }
        ch.template apply<RMS, Q8>(row_out<T, Q8>(y, row, ld.y), gamma, beta, K, st.x, st.y, qinv);
        lds_barrier();           // `stats` and `late` are rewritten for the next row
    }
}

// ---------------------------------------------------------------------------
// two kernels
// ---------------------------------------------------------------------------

// Kernel 1: per-chunk partials, x read through the caches (a second read
// soon after is served on-die).  Chunks of CV = WG*VPL vectors.
// ADD: the chunk is h = x + res (rounded), stored to hout through the caches;
// the normalising kernel then reads hout in place of x.
template <class T, bool RMS, bool ADD, int WG, int VPL, int EPV, bool RA = false>
__global__ __launch_bounds__(WG)
void norm_split_stats_kernel(const typename T::storage* x,
                             const typename T::storage* res,
                             typename T::storage* hout,
                             float2* __restrict__ part,      // [M, S] partials
                             int64_t M, int N, Strides ld, int S)
{
    static_assert(!ADD || RMS, "the residual add is fused with RMSNorm only");
    static_assert(!RA || !ADD, "realigned x: no residual");
    using C = Chunk<T, WG, VPL, EPV, RA>;
    __shared__ float red[2][WG / 64];
    const int NV = N / EPV;
    const int64_t items = M * (int64_t)S;
    for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
        const int64_t row = it / S;
        const int c = (int)(it - row * S);
        const typename T::storage* xr = x + row * ld.x;
        C ch;
        ch.template load<false>(xr, c, NV);
        if constexpr (ADD) ch.template add_residual<false>(res + row * ld.r, hout + row * ld.h);
        const float K = RMS ? 0.0f : T::widen(xr[0]);
        const float2 p = ch.template partial<RMS>(K, NV, red);
        if (threadIdx.x == 0) part[row * S + c] = p;
        __syncthreads();          // LDS slots are rewritten by the next item
    }
}

// Kernel 2: per chunk of its own size (A chunks per row), issue the loads of
// x (its last read), merge the row's S partials of CE elements each while
// they are in flight, normalise and store.  Every wavefront runs the same
// merge in chunk order, so every chunk of a row uses the same bits of mean
// and rstd.  The row's first chunk stores mean and rstd.
template <class T, bool RMS, bool Q8, int WG, int VPL, int EPV, bool RA = false>
__global__ __launch_bounds__(WG)
void norm_split_apply_kernel(const typename T::storage* x,
                             const typename T::storage* __restrict__ gamma,
                             const typename T::storage* __restrict__ beta,
                             void* y,
                             const float2* __restrict__ part,
                             float* __restrict__ mean_out,
                             float* __restrict__ rstd_out,
                             int64_t M, int N, Strides ld, int S, int CE, int A, float eps, float qinv)
{
    static_assert(!Q8 || RMS, "FP8 output is fused with RMSNorm only");
    using C = Chunk<T, WG, VPL, EPV, RA>;
    const int NV = N / EPV;
    const int64_t items = M * (int64_t)A;
    for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
        const int64_t row = it / A;
        const int c = (int)(it - row * A);
        const typename T::storage* xr = x + row * ld.x;
        C ch;
        ch.load(xr, c, NV);
        const float K = RMS ? 0.0f : T::widen(xr[0]);
        const float2* pr = part + row * S;
        const float2 st = row_stats<RMS>([pr](int cc) { return pr[cc]; }, S, CE, N, eps);
        if (c == 0 && threadIdx.x == 0) {
            if (!RMS && mean_out) mean_out[row] = K + st.x;
            if (rstd_out) rstd_out[row] = st.y;
        }
        ch.template apply<RMS, Q8>(row_out<T, Q8>(y, row, ld.y), gamma, beta, K, st.x, st.y, qinv);
    }
}

}  // namespace mi355norm
