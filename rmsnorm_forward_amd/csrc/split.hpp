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
//   norm_split_stats_kernel  the default: two kernels.  Partials (x read
//   + norm_split_apply_kernel  through the caches), then a second kernel that
//                            merges the row's partials, re-reads x and
//                            stores y (the two may cut rows into chunks of
//                            different sizes).  When a batch of rows fits in
//                            the 256 MB Infinity Cache the re-read is served
//                            on-die, so HBM sees x about once.
//   norm_split_coop_kernel   on request: single pass, x read once.  Each
//                            workgroup keeps its chunk in VGPRs, publishes
//                            its partial, waits at a per-row team barrier
//                            (all S workgroups of a team are co-resident:
//                            cooperative launch), merges and normalises from
//                            registers.  Teams walk the rows with a stride of
//                            the team count, each workgroup loading its
//                            next row's chunk while it waits and normalises.
//                            The barrier's counters return to zero by the
//                            end of every launch, so a kept workspace needs
//                            no reset.
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
        __syncthreads();
        float s = slots[0];
#pragma unroll
        for (int w = 1; w < W; ++w) s += slots[w];
        v = s;
    }
    return v;
}

template <class T, int WG, int VPL, int EPV>
struct Chunk {
    using V = Vec<T, EPV>;
    static constexpr int CV = WG * VPL;      // vectors per chunk
    V xv[VPL];
    bool ok[VPL];
    int v0;                                  // first vector of the chunk

    // xr: the row (wavefront-uniform); lane offsets are 32-bit (N < 2^24).
    // STREAM: nontemporal (x's last read); otherwise cached, so that a second
    // read soon after can be served by the on-die caches.
    template <bool STREAM = true>
    __device__ __forceinline__ void load(const typename T::storage* xr, int c, int NV) {
        v0 = c * CV;
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            const unsigned v = (unsigned)(v0 + j * WG) + threadIdx.x;
            ok[j] = (int)v < NV;
            if (ok[j]) {
                if constexpr (STREAM) xv[j].load_stream(xr + v * EPV);
                else xv[j].load(xr + v * EPV);
            } else {
                xv[j].zero();
            }
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
    template <bool RMS>
    __device__ __forceinline__ float2 partial(float K, int NV, float (*red)[WG / 64]) {
        if constexpr (RMS) {
            float q = 0.0f;
#pragma unroll
            for (int j = 0; j < VPL; ++j)
#pragma unroll
                for (int k = 0; k < EPV; ++k) q = __builtin_fmaf(xv[j].get(k), xv[j].get(k), q);
            return make_float2(wg_sum<WG>(q, red[0]), 0.0f);
        } else {
            const int nvec = min(CV, NV - v0);
            const float nc = (float)nvec * (float)EPV;
            float s = 0.0f;
#pragma unroll
            for (int j = 0; j < VPL; ++j)
#pragma unroll
                for (int k = 0; k < EPV; ++k) s += ok[j] ? xv[j].get(k) - K : 0.0f;
            s = wg_sum<WG>(s, red[0]);
            const float mc = s / nc;
            opaque();
            float q = 0.0f;
#pragma unroll
            for (int j = 0; j < VPL; ++j)
#pragma unroll
                for (int k = 0; k < EPV; ++k) {
                    const float e = ok[j] ? (xv[j].get(k) - K) - mc : 0.0f;
                    q = __builtin_fmaf(e, e, q);
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

// Merge a row's S partials (S arbitrary) inside one wavefront; the result is
// wave-uniform and identical in every wavefront that runs it on the same data.
// Lane l folds partials l, l+64, l+128, ... in order; the 64 lane states are
// then merged by a butterfly whose every step puts the lower lane's state
// first, so partners compute bitwise-identical results.
// A partial as one 64-bit atomic access at agent scope: coherent across the
// XCDs' L2 caches without any cache write-back or invalidation.
__device__ __forceinline__ void store_partial_coherent(float2* p, float2 v) {
    const unsigned long long bits =
        ((unsigned long long)__float_as_uint(v.y) << 32) | (unsigned long long)__float_as_uint(v.x);
    __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), bits, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float2 load_partial_coherent(const float2* p) {
    const unsigned long long bits = __hip_atomic_load(
        reinterpret_cast<unsigned long long*>(const_cast<float2*>(p)), __ATOMIC_RELAXED,
        __HIP_MEMORY_SCOPE_AGENT);
    return make_float2(__uint_as_float((unsigned)bits), __uint_as_float((unsigned)(bits >> 32)));
}

// The per-row barrier of the single-pass kernels.  Row r's counters sit in
// one 256-byte line at sync + 64 r (arrivals) and + 32 (departures), so rows
// in flight never share a line; they are zero at launch and again at exit.
// Every member is called by one thread of the workgroup.
struct RowBarrier {
    unsigned* arrived;
    unsigned* departed;
    __device__ RowBarrier(unsigned* sync, int64_t row) : arrived(sync + row * 64), departed(arrived + 32) {}

    // publish this workgroup's partial (a coherent 64-bit store, complete
    // before the count), then count its arrival
    __device__ void arrive(float2* slot, float2 v) const {
        store_partial_coherent(slot, v);
        __builtin_amdgcn_s_waitcnt(0);
        __hip_atomic_fetch_add(arrived, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // wait for `need` arrivals (the row's chunk count; a host test hook can
    // ask for one more, which never comes), polling with relaxed loads at most
    // spin_limit times so that a broken co-residency assumption cannot hang;
    // returns 1 if the bound was reached
    __device__ int wait(unsigned need, unsigned spin_limit) const {
        unsigned spins = 0;
        while (__hip_atomic_load(arrived, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need) {
            if (++spins > spin_limit) return 1;
            __builtin_amdgcn_s_sleep(8);
        }
        return 0;
    }

    // count this workgroup's departure (it has read every partial); the last
    // of the row's S returns both counters to zero for the next call
    __device__ void depart(int S) const {
        if (__hip_atomic_fetch_add(departed, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (unsigned)S - 1) {
            __hip_atomic_store(arrived, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(departed, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
};

// start of row `row` of an output of the I/O dtype, or of FP8 codes
template <class T, bool Q8>
__device__ __forceinline__ void* row_out(void* y, int64_t row, int64_t ldy) {
    if constexpr (Q8) return static_cast<uint8_t*>(y) + row * ldy;
    else return static_cast<typename T::storage*>(y) + row * ldy;
}

template <bool COHERENT>
__device__ __forceinline__ float2 read_partial(const float2* p) {
    if constexpr (COHERENT) return load_partial_coherent(p);
    else return *p;
}

template <bool COHERENT = false>
__device__ __forceinline__ Welford merge_row_partials(const float2* p, int S, int CE, int N) {
    const int l = lane_id();
    Welford a = {0.0f, 0.0f, 0.0f};
    for (int c = l; c < S; c += 64) {
        const float2 v = read_partial<COHERENT>(p + c);
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

// Row statistics from its S partials: (mean about K, rstd).
template <bool RMS, bool COHERENT = false>
__device__ __forceinline__ float2 row_stats(const float2* pr, int S, int CE, int N, float eps) {
    const float inv_n = 1.0f / (float)N;
    if constexpr (RMS) {
        float q = 0.0f;
        for (int cc = lane_id(); cc < S; cc += 64) q += read_partial<COHERENT>(pr + cc).x;
        q = team_sum<64>(q);
        return make_float2(0.0f, rsqrt_hw(__builtin_fmaf(q, inv_n, eps)));
    } else {
        const Welford w = merge_row_partials<COHERENT>(pr, S, CE, N);
        return make_float2(w.mean, rsqrt_hw(__builtin_fmaf(w.m2, inv_n, eps)));
    }
}

// ---------------------------------------------------------------------------
// single pass, cooperative
// ---------------------------------------------------------------------------

// Publication of the partials: each is one coherent 64-bit atomic store,
// complete before the arrival count is incremented, and read back with
// coherent 64-bit loads; no L2 write-back or invalidation is needed (agent-
// scope release / acquire would cost one of each per workgroup and row).


template <class T, bool RMS, bool ADD, bool Q8, int WG, int VPL, int EPV>
__global__ __launch_bounds__(WG)
void norm_split_coop_kernel(const typename T::storage* x,
                            const typename T::storage* res,
                            const typename T::storage* __restrict__ gamma,
                            const typename T::storage* __restrict__ beta,
                            void* y,
                            typename T::storage* hout,
                            float* __restrict__ mean_out,
                            float* __restrict__ rstd_out,
                            float2* __restrict__ part,      // [M, S] partials
                            unsigned* __restrict__ sync,    // row r: [64r], [64r+32]; zero at
                                                            // launch and again at exit
                            int64_t M, int N, Strides ld, int S, int teams, float eps, float qinv,
                            unsigned need, unsigned spin_limit)
{
    static_assert(!ADD || RMS, "the residual add is fused with RMSNorm only");
    static_assert(!Q8 || RMS, "FP8 output is fused with RMSNorm only");
    using C = Chunk<T, WG, VPL, EPV>;
    __shared__ float red[2][WG / 64];
    __shared__ int late;
    const int tid = threadIdx.x;
    const int NV = N / EPV;
    const int team = blockIdx.x / S;          // grid is exactly teams * S
    const int c = blockIdx.x - team * S;

    // One row's chunk: partial, publish, wait, merge, normalise.  during_wait
    // runs between the publication and the wait (the next row's loads go
    // there), before_stores once the statistics are known, before y is
    // stored.
    auto finish = [&](C& ch, float K, int64_t row, auto&& during_wait, auto&& before_stores) {
        const float2 p = ch.template partial<RMS>(K, NV, red);
        const RowBarrier bar(sync, row);
        if (tid == 0) bar.arrive(part + row * S + c, p);
        during_wait();
        if (tid == 0) late = bar.wait(need, spin_limit);
        __syncthreads();
        float2 st = row_stats<RMS, true>(part + row * S, S, C::CV * EPV, N, eps);
        if (late) st = make_float2(__builtin_nanf(""), __builtin_nanf(""));   // visible failure
        if (tid == 0) bar.depart(S);
        if (c == 0 && tid == 0) {
            if (!RMS && mean_out) mean_out[row] = K + st.x;
            if (rstd_out) rstd_out[row] = st.y;
        }
        before_stores();
        ch.template apply<RMS, Q8>(row_out<T, Q8>(y, row, ld.y), gamma, beta, K, st.x, st.y, qinv);
    };

    if constexpr (ADD) {
        for (int64_t row = team; row < M; row += teams) {
            const typename T::storage* xr = x + row * ld.x;
            C ch;
            ch.load(xr, c, NV);
            ch.template add_residual<true>(res + row * ld.r, hout + row * ld.h);
            finish(ch, 0.0f, row, [] {}, [] {});   // RMSNorm only: no shift
        }
    } else {
        // the next row's chunk is loaded while this row waits at its barrier
        // and is normalised: two chunk register sets, the loop unrolled by
        // two so that no copy between them forces an early wait.  Loads and
        // stores share one completion counter, so the next chunk's loads are
        // waited for (ready) before this chunk's stores are issued; the merge
        // of the row's partials, whose loads come after them, waits for them
        // anyway.  (The residual add keeps one set: its chunk is added and
        // stored as soon as it arrives.)
        C ca, cb;
        float Ka = 0.0f, Kb = 0.0f;
        auto fetch = [&](C& ch, float& K, int64_t row) {
            if (row >= M) return;
            const typename T::storage* xr = x + row * ld.x;
            ch.load(xr, c, NV);
            K = RMS ? 0.0f : T::widen(xr[0]);
        };
        auto ready = [&](C& ch, float& K) {
            ch.opaque();
            asm volatile("" : "+v"(K));
        };
        fetch(ca, Ka, team);
        ready(ca, Ka);
        for (int64_t row = team; row < M;) {
            finish(ca, Ka, row, [&] { fetch(cb, Kb, row + teams); }, [&] { ready(cb, Kb); });
            row += teams;
            if (row >= M) break;
            finish(cb, Kb, row, [&] { fetch(ca, Ka, row + teams); }, [&] { ready(ca, Ka); });
            row += teams;
        }
    }
}

// ---------------------------------------------------------------------------
// two kernels
// ---------------------------------------------------------------------------

// Kernel 1: per-chunk partials, x read through the caches (a second read
// soon after is served on-die).  Chunks of CV = WG*VPL vectors.
// ADD: the chunk is h = x + res (rounded), stored to hout through the caches;
// the normalising kernel then reads hout in place of x.
template <class T, bool RMS, bool ADD, int WG, int VPL, int EPV>
__global__ __launch_bounds__(WG)
void norm_split_stats_kernel(const typename T::storage* x,
                             const typename T::storage* res,
                             typename T::storage* hout,
                             float2* __restrict__ part,      // [M, S] partials
                             int64_t M, int N, Strides ld, int S)
{
    static_assert(!ADD || RMS, "the residual add is fused with RMSNorm only");
    using C = Chunk<T, WG, VPL, EPV>;
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
template <class T, bool RMS, bool Q8, int WG, int VPL, int EPV>
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
    using C = Chunk<T, WG, VPL, EPV>;
    const int NV = N / EPV;
    const int64_t items = M * (int64_t)A;
    for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
        const int64_t row = it / A;
        const int c = (int)(it - row * A);
        const typename T::storage* xr = x + row * ld.x;
        C ch;
        ch.load(xr, c, NV);
        const float K = RMS ? 0.0f : T::widen(xr[0]);
        const float2 st = row_stats<RMS>(part + row * S, S, CE, N, eps);
        if (c == 0 && threadIdx.x == 0) {
            if (!RMS && mean_out) mean_out[row] = K + st.x;
            if (rstd_out) rstd_out[row] = st.y;
        }
        ch.template apply<RMS, Q8>(row_out<T, Q8>(y, row, ld.y), gamma, beta, K, st.x, st.y, qinv);
    }
}

}  // namespace mi355norm
