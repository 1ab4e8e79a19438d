// rows.hpp -- register-resident row kernel: one team of TEAM lanes owns one
// row and holds the whole row in VGPRs, so x is read from HBM exactly once.
//
//   TEAM <  64 : 64/TEAM rows per wavefront, reductions stay inside the wave
//                (DPP only, no LDS, no barrier);
//   TEAM == 64 : one row per wavefront;
//   TEAM >  64 : TEAM/64 wavefronts per row, one LDS exchange per reduction.
//
// Lane t of a team holds VPL vectors; vector j covers elements
// [(j*TEAM + t)*EPV, (j*TEAM + t + 1)*EPV), so each load instruction of the
// team reads TEAM*EPV contiguous elements (fully coalesced).  A vector is
// either wholly inside the row or wholly past its end (EPV divides N).
//
// LayerNorm statistics are the stable two-pass of "T3 讲解" part ② taken over
// the register copy of the row, with a shift: K = x[row, 0] is subtracted
// first (exact when the values are within a factor of two of K), the mean of
// d = x - K is mu', and the variance is the mean of (d - mu')^2.  The mean of
// the row is K + mu', and y = (d - mu') * rstd * gamma + beta, so the fp32
// rounding of the mean never enters y (the large-mean rows of "CUDA 算子工程"
// ch. 7 section 7.3 need this: at |x| ~ 1000 an fp32 mean is only known to
// ~3e-5).  RMSNorm needs a single sum of squares.

#pragma once

#include "prims.hpp"

namespace mi355norm {

template <int TEAM>
struct TeamGeom {
    static constexpr int WG = TEAM >= 256 ? TEAM : 256;   // threads per workgroup
    static constexpr int ROWS = WG / TEAM;                 // rows per workgroup
    static constexpr int WPT = TEAM > 64 ? TEAM / 64 : 1;  // wavefronts per team
};

// Sum over the team.  Result is bitwise identical in every lane of the team.
// `slots` is this team's LDS row (WPT floats), used only when TEAM > 64.
template <int TEAM>
__device__ __forceinline__ float team_reduce(float v, float* slots, int wave_in_team) {
    v = team_sum<(TEAM < 64 ? TEAM : 64)>(v);
    if constexpr (TEAM > 64) {
        constexpr int WPT = TEAM / 64;
        if (lane_id() == 0) slots[wave_in_team] = v;
        lds_barrier();
        float s = slots[0];
#pragma unroll
        for (int w = 1; w < WPT; ++w) s += slots[w];
        v = s;
    }
    return v;
}

// Keep the shifted fp32 copy of a lane's elements in VGPRs (instead of
// re-widening the packed copy in each pass) when a lane holds at most this
// many elements.
#ifndef MI355_CACHE_F32_MAX
#define MI355_CACHE_F32_MAX 32
#endif
template <bool B>
struct bool_c {
    static constexpr bool value = B;
};

// sum of the EPV widened elements of a vector minus K, as a pairwise tree
template <class V, int EPV>
__device__ __forceinline__ float vec_sum_shifted(const V& v, float K) {
    float t[EPV];
#pragma unroll
    for (int k = 0; k < EPV; ++k) t[k] = v.get(k) - K;
#pragma unroll
    for (int h = 1; h < EPV; h *= 2)
#pragma unroll
        for (int k = 0; k + h < EPV; k += 2 * h) t[k] += t[k + h];
    return t[0];
}

// ADD (RMSNorm only): the row is first h = x + res rounded to the storage
// type; h is stored to hout (the updated residual) and normalised in place of
// x.  res / hout may be the same buffer, and y may be x: every element is
// read into registers by the lane that later writes it, before it writes.
// Q8 (RMSNorm only): y is FP8 E4M3 codes of (the normalised value * qinv),
// one byte per element, instead of the I/O dtype.
// REALIGN (no residual; 16-byte vectors): rows of x may start off a 16-byte
// boundary while gamma, beta and y do not.  Each lane loads the aligned
// blocks below its vectors and realigns them in registers with the next
// block, taken from the next lane (see realign_words in prims.hpp); the
// tile, the arithmetic and so the results are those of an aligned x.
//
// Two memory schedules, fixed per (operation, team) by measurement on MI355X
// (steady state, 200 launches, us):
//   hoisted (RMSNorm, teams of at most 256 lanes): every load of the row (x,
//     the residual, gamma) is issued before any arithmetic, unconditionally,
//     from an address clamped into the row (a vector past the row's end
//     reads the row's last vector, a row past M reads row M - 1; those values
//     are never used), and only the stores are masked, so no load waits
//     behind a branch or a store.  RMS bf16 65536 x 2048 64x4: 84.8 vs 87.6;
//     fp32 65536 x 2048 256x2: 171.5 vs 175.0; 2 rows per wavefront (bf16
//     32x8) 86.4 vs 100.5.
//   interleaved (LayerNorm; RMSNorm teams of 512+ lanes): x loaded under the
//     per-vector mask, gamma / beta loaded vector by vector in the output
//     loop, each vector's loads waited for (with the previous vector's store)
//     just before it is computed and stored.  LN bf16 16384 x 8192 256x4: 89.0
//     vs 93.0 with gamma / beta hoisted before the statistics (their 32 VGPRs
//     cost a wave per SIMD) and 98.7 hoisted after them; RMS fp32 8192 x 4096
//     512x2: 44.0 vs 44.9.
template <class T, bool RMS, bool ADD, bool Q8, int TEAM, int VPL, int EPV, bool REALIGN = false>
__global__ __launch_bounds__(TeamGeom<TEAM>::WG)
void norm_rows_kernel(const typename T::storage* x,
                      const typename T::storage* res,
                      const typename T::storage* __restrict__ gamma,
                      const typename T::storage* __restrict__ beta,
                      void* yv,
                      typename T::storage* hout,
                      float* __restrict__ mean_out,
                      float* __restrict__ rstd_out,
                      int64_t M, int N, Strides ld, float eps, float qinv)
{
    static_assert(!ADD || RMS, "the residual add is fused with RMSNorm only");
    static_assert(!Q8 || RMS, "FP8 output is fused with RMSNorm only");
    static_assert(!REALIGN || (!ADD && EPV * sizeof(typename T::storage) == 16),
                  "realigned x: 16-byte vectors, no residual");
    using G = TeamGeom<TEAM>;
    using S = typename T::storage;
    using V = Vec<T, EPV>;
    constexpr int E = VPL * EPV;               // elements per lane
    constexpr bool CACHE_F32 = E <= MI355_CACHE_F32_MAX;
    constexpr bool HOIST = RMS && TEAM <= 256;

    // cross-wavefront exchange slots: two sets, one float per wavefront
    __shared__ float red[2][G::ROWS][G::WPT];

    const int tid = threadIdx.x;
    const int team = TEAM >= 64 ? __builtin_amdgcn_readfirstlane(tid / TEAM) : tid / TEAM;
    const int tl = tid % TEAM;
    const int wave_in_team = TEAM > 64 ? __builtin_amdgcn_readfirstlane(tl >> 6) : 0;
    const int NV = N / EPV;                    // EPV divides N on every path
    const float inv_n = 1.0f / (float)N;        // divisor is the true N
    const bool has_g = gamma != nullptr;
    const bool has_b = beta != nullptr;

    // this lane's vectors: in-row flags and (hoisted schedule) element
    // offsets clamped into the row; the same for every row
    bool vin[VPL];
    unsigned off[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
        const int v = j * TEAM + tl;
        vin[j] = v < NV;
        off[j] = (unsigned)(vin[j] || !HOIST ? v : NV - 1) * EPV;
    }

    const int64_t groups = (M + G::ROWS - 1) / G::ROWS;
    int par = 0;    // RMS alternates LDS slot sets between iterations
    for (int64_t grp = blockIdx.x; grp < groups; grp += gridDim.x, par ^= 1) {
        const int64_t row = grp * G::ROWS + team;
        const bool row_ok = row < M;
        // row bases (wavefront-uniform when TEAM >= 64) plus 32-bit lane offsets
        const int64_t rr = row_ok ? row : (HOIST ? M - 1 : 0);
        const S* xr = x + rr * ld.x;
        S* yr = static_cast<S*>(yv) + rr * ld.y;
        uint8_t* yq = static_cast<uint8_t*>(yv) + rr * ld.y;

        V xv[VPL];
        bool ok[VPL];
        V gl[HOIST ? VPL : 1];
        // realigned x: loads from the aligned block below the row's start
        unsigned mb = 0;
        const S* xa = xr;
        if constexpr (REALIGN) {
            mb = (unsigned)(reinterpret_cast<uintptr_t>(xr) & 15u);
            if constexpr (TEAM >= 64) mb = __builtin_amdgcn_readfirstlane(mb);
            xa = reinterpret_cast<const S*>(reinterpret_cast<uintptr_t>(xr) - mb);
        }
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            ok[j] = row_ok && vin[j];
            if (HOIST || ok[j]) xv[j].load_stream(xa + off[j]);   // masked vectors: never used
        }
        if constexpr (REALIGN && TEAM <= 64) {
            // the team lies within this wavefront: the block after lane t's
            // is lane t + 1's, and for the team's last lane the team's first
            // lane's next vector; only the row's last vector loads its own
            V tail;
#pragma unroll
            for (int j = 0; j < VPL; ++j)
                if (mb != 0u && ok[j] && j * TEAM + tl == NV - 1) tail.load_stream(xa + (unsigned)NV * EPV);
            // several rows per wavefront: one scalar branch when they share
            // the misalignment (row strides that keep 16-byte steps), else a
            // select per lane
            unsigned mbu = mb;
            bool uniform = true;
            if constexpr (TEAM < 64) {
                mbu = __builtin_amdgcn_readfirstlane(mb);
                uniform = __builtin_amdgcn_readfirstlane((int)(__builtin_amdgcn_ballot_w64(mb != mbu) == 0)) != 0;
            }
            const bool last = tl == TEAM - 1;
            u32x4 rc = TEAM == 64 ? next_lane_words(xv[0].w) : team_rotate_words<(TEAM < 64 ? TEAM : 64)>(xv[0].w);
#pragma unroll
            for (int j = 0; j < VPL; ++j) {
                // lane t + 1's block of vector j + 1 (team-rotated), read
                // before vector j + 1 is realigned
                u32x4 rn = rc;
                if (j + 1 < VPL) {
                    const u32x4 nx = xv[j + 1 < VPL ? j + 1 : j].w;
                    if constexpr (TEAM == 64) {
                        // the wavefront's first lane, for its last lane
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            const unsigned w = nx[k];
                            rn[k] = __builtin_amdgcn_readlane(w, 0);
                        }
                    } else {
                        rn = team_rotate_words<(TEAM < 64 ? TEAM : 64)>(nx);
                    }
                }
                const u32x4 nb = j * TEAM + tl == NV - 1 ? tail.w : (last ? rn : rc);
                xv[j].w = uniform ? realign_words<true>(xv[j].w, nb, mbu) : realign_words<false>(xv[j].w, nb, mb);
                // the next vector's own-lane neighbours
                if (j + 1 < VPL) {
                    if constexpr (TEAM == 64) rc = next_lane_words(xv[j + 1 < VPL ? j + 1 : j].w);
                    else rc = rn;
                }
            }
        }
        if constexpr (REALIGN && TEAM > 64) {
            // teams of several wavefronts: the wavefronts' last lanes, and
            // the row's last vector, load their next block themselves
            V ex[VPL];
            bool own[VPL];
#pragma unroll
            for (int j = 0; j < VPL; ++j) {
                const int v = j * TEAM + tl;
                own[j] = mb != 0u && ok[j] &&
                         (tl == TEAM - 1 || lane_id() == 63 || v == NV - 1);
                if (own[j]) ex[j].load_stream(xa + (unsigned)(v + 1) * EPV);
            }
#pragma unroll
            for (int j = 0; j < VPL; ++j) {
                const u32x4 nl = next_lane_words(xv[j].w);    // every lane active
                xv[j].w = realign_words<true>(xv[j].w, own[j] ? ex[j].w : nl, mb);
            }
        }
        if constexpr (ADD) {
            V rv[VPL];
#pragma unroll
            for (int j = 0; j < VPL; ++j)
                if (HOIST || ok[j]) rv[j].load_stream(res + rr * ld.r + off[j]);
            if constexpr (HOIST) {
#pragma unroll
                for (int j = 0; j < VPL; ++j)
                    if (has_g) gl[j].load(gamma + off[j]);
            }
#pragma unroll
            for (int j = 0; j < VPL; ++j) {
                if (!HOIST && !ok[j]) continue;
                add_into(xv[j], rv[j]);
                if (ok[j]) xv[j].put_stream(hout + rr * ld.h + off[j]);
            }
        } else if constexpr (HOIST) {
#pragma unroll
            for (int j = 0; j < VPL; ++j)
                if (has_g) gl[j].load(gamma + off[j]);
        }
        float rs, mu = 0.0f, K = 0.0f;
        float d[CACHE_F32 ? VPL : 1][EPV];
        if constexpr (RMS) {
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < VPL; ++j) {
                float t = 0.0f;
#pragma unroll
                for (int k = 0; k < EPV; ++k) t = __builtin_fmaf(xv[j].get(k), xv[j].get(k), t);
                acc += ok[j] ? t : 0.0f;
            }
            // one exchange per iteration: alternating slot sets keep a fast
            // wavefront's next write away from slots a slow one still reads
            acc = team_reduce<TEAM>(acc, red[par][team], wave_in_team);
            rs = rsqrt_hw(__builtin_fmaf(acc, inv_n, eps));
        } else {
            K = row_ok ? T::widen(xr[0]) : 0.0f;
            // pass 1: sum of d = x - K over the valid vectors
            float s = 0.0f;
#pragma unroll
            for (int j = 0; j < VPL; ++j) {
                if constexpr (CACHE_F32) {
#pragma unroll
                    for (int k = 0; k < EPV; ++k) d[j][k] = xv[j].get(k) - K;
                }
                const float t = vec_sum_shifted<V, EPV>(xv[j], K);
                s += ok[j] ? t : 0.0f;
            }
            s = team_reduce<TEAM>(s, red[0][team], wave_in_team);
            mu = s * inv_n;
            if constexpr (!CACHE_F32) {
#pragma unroll
                for (int j = 0; j < VPL; ++j) xv[j].opaque();
            }
            // pass 2: sum of (d - mu')^2 over the valid vectors
            float q = 0.0f;
#pragma unroll
            for (int j = 0; j < VPL; ++j) {
                float t = 0.0f;
#pragma unroll
                for (int k = 0; k < EPV; ++k) {
                    float dv;
                    if constexpr (CACHE_F32) dv = d[j][k];
                    else dv = xv[j].get(k) - K;
                    const float e = dv - mu;
                    if constexpr (CACHE_F32) d[j][k] = e;
                    t = __builtin_fmaf(e, e, t);
                }
                q += ok[j] ? t : 0.0f;
            }
            // two exchanges per iteration (slot sets 0 then 1): the barrier of
            // the second orders every read of set 0 before the next write
            q = team_reduce<TEAM>(q, red[1][team], wave_in_team);
            rs = rsqrt_hw(__builtin_fmaf(q, inv_n, eps));
        }

        if constexpr (!CACHE_F32) {
#pragma unroll
            for (int j = 0; j < VPL; ++j) xv[j].opaque();
        }
        if (tl == 0 && row_ok) {
            if (!RMS && mean_out) mean_out[row] = K + mu;
            if (rstd_out) rstd_out[row] = rs;
        }

        // normalise from the register copy, apply the affine, store; the
        // presence of gamma / beta is resolved by a uniform branch, so the
        // inner loop carries no per-element selects
        // FP8 output: the 1/scale factor rides on rstd (one multiply per row)
        const float rsy = Q8 ? rs * qinv : rs;
        auto emit = [&](auto hg, auto hb) {
            constexpr bool HG = decltype(hg)::value;
            constexpr bool HB = !RMS && decltype(hb)::value;
#pragma unroll
            for (int j = 0; j < VPL; ++j) {
                if (!HOIST && !ok[j]) continue;
                V gv, bl;
                if constexpr (HG && !HOIST) gv.load(gamma + off[j]);
                if constexpr (HB) bl.load(beta + off[j]);
                const V& g = HOIST ? gl[j] : gv;
                float o[EPV];
#pragma unroll
                for (int k = 0; k < EPV; ++k) {
                    float t;
                    if constexpr (RMS) t = xv[j].get(k) * rsy;
                    else if constexpr (CACHE_F32) t = d[j][k] * rs;
                    else t = ((xv[j].get(k) - K) - mu) * rs;
                    if constexpr (HG && HB) o[k] = __builtin_fmaf(t, g.get(k), bl.get(k));
                    else if constexpr (HG) o[k] = t * g.get(k);
                    else if constexpr (HB) o[k] = t + bl.get(k);
                    else o[k] = t;
                }
                if (HOIST && !ok[j]) continue;
                if constexpr (Q8) {
                    store_e4m3<EPV>(yq + off[j], o);
                } else {
                    V::store(yr + off[j], o);
                }
            }
        };
        using TT = bool_c<true>;
        using FF = bool_c<false>;
        if (has_g) {
            if (has_b) emit(TT{}, TT{});
            else emit(TT{}, FF{});
        } else {
            if (has_b) emit(FF{}, TT{});
            else emit(FF{}, FF{});
        }
    }
}

}  // namespace mi355norm
