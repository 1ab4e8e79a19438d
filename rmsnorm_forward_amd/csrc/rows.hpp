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
// team reads TEAM*EPV contiguous elements (fully coalesced).
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
        __syncthreads();
        float s = slots[0];
#pragma unroll
        for (int w = 1; w < WPT; ++w) s += slots[w];
        v = s;
    }
    return v;
}

template <class T, bool RMS, int TEAM, int VPL, int EPV>
__global__ __launch_bounds__(TeamGeom<TEAM>::WG)
void norm_rows_kernel(const typename T::storage* __restrict__ x,
                      const typename T::storage* __restrict__ gamma,
                      const typename T::storage* __restrict__ beta,
                      typename T::storage* __restrict__ y,
                      float* __restrict__ mean_out,
                      float* __restrict__ rstd_out,
                      int64_t M, int N, float eps)
{
    using G = TeamGeom<TEAM>;
    using S = typename T::storage;
    using V = Vec<T, EPV>;
    constexpr int E = VPL * EPV;               // elements per lane
    // keep the shifted fp32 copy of the row when it fits comfortably in VGPRs
    constexpr bool CACHE_F32 = E <= 32;

    __shared__ float red[2][G::ROWS][G::WPT];

    const int tid = threadIdx.x;
    const int team = tid / TEAM;
    const int tl = tid % TEAM;
    const int wave_in_team = TEAM > 64 ? __builtin_amdgcn_readfirstlane(tl >> 6) : 0;
    const int NV = N / EPV;                    // EPV divides N on every path
    const float fN = (float)N;
    const bool has_g = gamma != nullptr;
    const bool has_b = beta != nullptr;

    const int64_t groups = (M + G::ROWS - 1) / G::ROWS;
    int par = 0;    // RMS alternates LDS slot sets between iterations
    for (int64_t grp = blockIdx.x; grp < groups; grp += gridDim.x, par ^= 1) {
        const int64_t row = grp * G::ROWS + team;
        const bool row_ok = row < M;
        const S* xr = x + (row_ok ? row : 0) * (int64_t)N;
        S* yr = y + (row_ok ? row : 0) * (int64_t)N;

        V xv[VPL];
        bool ok[VPL];
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            const int v = j * TEAM + tl;
            ok[j] = row_ok && v < NV;
            if (ok[j]) xv[j].load(xr + (int64_t)v * EPV);
            else xv[j].zero();
        }

        float rs, mu = 0.0f, K = 0.0f;
        float d[CACHE_F32 ? VPL : 1][EPV];
        if constexpr (RMS) {
            float acc[EPV];
#pragma unroll
            for (int k = 0; k < EPV; ++k) acc[k] = 0.0f;
#pragma unroll
            for (int j = 0; j < VPL; ++j)
#pragma unroll
                for (int k = 0; k < EPV; ++k) {
                    const float v = xv[j].get(k);       // masked vectors hold zeros
                    acc[k] = __builtin_fmaf(v, v, acc[k]);
                }
            float q = acc[0];
#pragma unroll
            for (int k = 1; k < EPV; ++k) q += acc[k];
            // one exchange per iteration: alternating slot sets keep a fast
            // wavefront's next write away from slots a slow one still reads
            q = team_reduce<TEAM>(q, red[par][team], wave_in_team);
            rs = 1.0f / __builtin_sqrtf(q / fN + eps);
        } else {
            // two exchanges per iteration (slot sets 0 then 1): the barrier of
            // the second orders every read of set 0 before the next write
            K = row_ok ? T::widen(xr[0]) : 0.0f;
            // pass 1: sum of d = x - K over the valid elements
            float acc[EPV];
#pragma unroll
            for (int k = 0; k < EPV; ++k) acc[k] = 0.0f;
#pragma unroll
            for (int j = 0; j < VPL; ++j)
#pragma unroll
                for (int k = 0; k < EPV; ++k) {
                    const float dv = ok[j] ? xv[j].get(k) - K : 0.0f;
                    if constexpr (CACHE_F32) d[j][k] = dv;
                    acc[k] += dv;
                }
            float s = acc[0];
#pragma unroll
            for (int k = 1; k < EPV; ++k) s += acc[k];
            s = team_reduce<TEAM>(s, red[0][team], wave_in_team);
            mu = s / fN;
            // pass 2: sum of (d - mu')^2 over the valid elements
#pragma unroll
            for (int k = 0; k < EPV; ++k) acc[k] = 0.0f;
#pragma unroll
            for (int j = 0; j < VPL; ++j)
#pragma unroll
                for (int k = 0; k < EPV; ++k) {
                    float dv;
                    if constexpr (CACHE_F32) dv = d[j][k];
                    else dv = xv[j].get(k) - K;
                    const float e = ok[j] ? dv - mu : 0.0f;
                    if constexpr (CACHE_F32) d[j][k] = e;
                    acc[k] = __builtin_fmaf(e, e, acc[k]);
                }
            float q = acc[0];
#pragma unroll
            for (int k = 1; k < EPV; ++k) q += acc[k];
            q = team_reduce<TEAM>(q, red[1][team], wave_in_team);
            rs = 1.0f / __builtin_sqrtf(q / fN + eps);
        }

        if (tl == 0 && row_ok) {
            if (!RMS && mean_out) mean_out[row] = K + mu;
            if (rstd_out) rstd_out[row] = rs;
        }

        // normalise from the register copy, apply the affine, store
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            if (!ok[j]) continue;
            const int64_t off = (int64_t)(j * TEAM + tl) * EPV;
            V gv, bv;
            if (has_g) gv.load(gamma + off);
            if (!RMS && has_b) bv.load(beta + off);
            float o[EPV];
#pragma unroll
            for (int k = 0; k < EPV; ++k) {
                float t;
                if constexpr (RMS) t = xv[j].get(k) * rs;
                else if constexpr (CACHE_F32) t = d[j][k] * rs;
                else t = ((xv[j].get(k) - K) - mu) * rs;
                const float g = has_g ? gv.get(k) : 1.0f;
                if constexpr (RMS) o[k] = t * g;
                else o[k] = __builtin_fmaf(t, g, has_b ? bv.get(k) : 0.0f);
            }
            V::store(yr + off, o);
        }
    }
}

}  // namespace mi355norm
