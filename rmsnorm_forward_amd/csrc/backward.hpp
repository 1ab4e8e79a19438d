// backward.hpp -- LayerNorm / RMSNorm backward ("CUDA 算子工程" ch. 7,
// section 7.7), from the mean and rstd the forward pass stored.
//
// norm_bwd_rows_kernel: a team of TEAM lanes owns a row, as in the forward
// row kernel (lane t holds vectors j*TEAM + t).  Per row it reads dy and x
// once, forms xhat = (x - mean) * rstd and g = dy * gamma, reduces the two
// row sums the section names -- sum(g) and sum(g * xhat) for LayerNorm,
// sum(g * x) for RMSNorm -- in one exchange, and writes
//   LayerNorm  dx = rstd * (g - mean(g) - xhat * mean(g xhat))
//   RMSNorm    dx = rstd * g - x * rstd^3 * mean(g x)
// The column sums dgamma = sum_rows dy * xhat (RMSNorm: dy * x * rstd) and
// dbeta = sum_rows dy are accumulated in fp32 registers by the lane that
// owns each column, over the rows its team visits (a fixed grid, row groups
// grid-strided), summed over the workgroup's teams and written as one
// partial row per workgroup: part_* is [gridDim.x, N].
//
// norm_colsum_kernel: sums the partial rows of each column in a fixed order,
// so dgamma and dbeta are bitwise reproducible for a given grid.
#pragma once

#include "prims.hpp"
#include "rows.hpp"

namespace mi355norm {

template <class T, bool RMS, int TEAM, int VPL, int EPV>
__global__ __launch_bounds__(TeamGeom<TEAM>::WG)
void norm_bwd_rows_kernel(const typename T::storage* dy,      // dx may be written over dy or x
                          const typename T::storage* x,
                          const typename T::storage* __restrict__ gamma,
                          const float* __restrict__ mean,
                          const float* __restrict__ rstd,
                          typename T::storage* dx,
                          float* __restrict__ part_g,      // [P, N] partial dgamma rows (or null)
                          float* __restrict__ part_b,      // [P, N] partial dbeta rows (or null)
                          int64_t M, int N, int64_t ldy, int64_t ldx, int64_t lddx)
{
    using G = TeamGeom<TEAM>;
    using S = typename T::storage;
    using V = Vec<T, EPV>;
    __shared__ float2 red[2][G::ROWS][G::WPT];

    const int tid = threadIdx.x;
    const int team = TEAM >= 64 ? __builtin_amdgcn_readfirstlane(tid / TEAM) : tid / TEAM;
    const int tl = tid % TEAM;
    const int wave_in_team = TEAM > 64 ? __builtin_amdgcn_readfirstlane(tl >> 6) : 0;
    const int NV = N / EPV;
    const float inv_n = 1.0f / (float)N;
    const bool has_g = gamma != nullptr;
    const bool want_g = part_g != nullptr;
    const bool want_b = part_b != nullptr;

    float acc_g[VPL][EPV], acc_b[RMS ? 1 : VPL][EPV];
#pragma unroll
    for (int j = 0; j < VPL; ++j)
#pragma unroll
        for (int k = 0; k < EPV; ++k) {
            acc_g[j][k] = 0.0f;
            if constexpr (!RMS) acc_b[j][k] = 0.0f;
        }
    bool col_ok[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) col_ok[j] = (int)(j * TEAM + tl) < NV;

    const int64_t groups = (M + G::ROWS - 1) / G::ROWS;
    int par = 0;
    for (int64_t grp = blockIdx.x; grp < groups; grp += gridDim.x, par ^= 1) {
        const int64_t row = grp * G::ROWS + team;
        const bool row_ok = row < M;
        const int64_t rr = row_ok ? row : 0;
        const S* dyr = dy + rr * ldy;
        const S* xr = x + rr * ldx;
        V dv[VPL], xv[VPL];
        bool ok[VPL];
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            const unsigned v = (unsigned)(j * TEAM + tl);
            ok[j] = row_ok && col_ok[j];
            if (ok[j]) {
                dv[j].load_stream(dyr + v * EPV);
                xv[j].load_stream(xr + v * EPV);
            }
        }
        const float mu = RMS ? 0.0f : (row_ok ? mean[rr] : 0.0f);
        const float rs = row_ok ? rstd[rr] : 0.0f;

        // the row sums: (sum g, sum g xhat) for LayerNorm, (0, sum g x) for RMSNorm
        float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            if (!ok[j]) continue;
            const unsigned off = (unsigned)(j * TEAM + tl) * EPV;
            V gv;
            if (has_g) gv.load(gamma + off);
#pragma unroll
            for (int k = 0; k < EPV; ++k) {
                const float g = dv[j].get(k) * (has_g ? gv.get(k) : 1.0f);
                const float xh = RMS ? xv[j].get(k) : (xv[j].get(k) - mu) * rs;
                if constexpr (!RMS) s1 += g;
                s2 = __builtin_fmaf(g, xh, s2);
            }
        }
        if constexpr (!RMS) s1 = team_sum<(TEAM < 64 ? TEAM : 64)>(s1);
        s2 = team_sum<(TEAM < 64 ? TEAM : 64)>(s2);
        if constexpr (TEAM > 64) {
            if (lane_id() == 0) red[par][team][wave_in_team] = make_float2(s1, s2);
            __syncthreads();
            float a = 0.0f, b = 0.0f;
#pragma unroll
            for (int w = 0; w < G::WPT; ++w) {
                a += red[par][team][w].x;
                b += red[par][team][w].y;
            }
            s1 = a;
            s2 = b;
        }
        // LayerNorm: dx = rs (g - c1 - xhat c2); RMSNorm: dx = rs g - x c2
        const float c1 = s1 * inv_n;
        const float c2 = RMS ? rs * rs * rs * (s2 * inv_n) : s2 * inv_n;
        S* dxr = dx + rr * lddx;
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            if (!ok[j]) continue;
            const unsigned off = (unsigned)(j * TEAM + tl) * EPV;
            V gv;
            if (has_g) gv.load(gamma + off);
            float o[EPV];
#pragma unroll
            for (int k = 0; k < EPV; ++k) {
                const float d = dv[j].get(k);
                const float g = d * (has_g ? gv.get(k) : 1.0f);
                if constexpr (RMS) {
                    const float xv_k = xv[j].get(k);
                    o[k] = __builtin_fmaf(rs, g, -xv_k * c2);
                    acc_g[j][k] = __builtin_fmaf(d, xv_k * rs, acc_g[j][k]);
                } else {
                    const float xh = (xv[j].get(k) - mu) * rs;
                    o[k] = rs * ((g - c1) - xh * c2);
                    acc_g[j][k] = __builtin_fmaf(d, xh, acc_g[j][k]);
                    acc_b[j][k] += d;
                }
            }
            V::store(dxr + off, o);
        }
    }
    // One partial row per workgroup.  Teams own the same columns lane for
    // lane (lane tl of every team holds vectors j*TEAM + tl), so with several
    // teams per workgroup team 0 adds the others' accumulators, one element
    // at a time through LDS, in team order.
    if constexpr (G::ROWS > 1) {
        __shared__ float xch[G::WG];
        auto fold = [&](float& a) {
            __syncthreads();
            xch[tid] = a;
            __syncthreads();
            if (team == 0) {
                float s = xch[tl];
#pragma unroll
                for (int r = 1; r < G::ROWS; ++r) s += xch[r * TEAM + tl];
                a = s;
            }
        };
#pragma unroll
        for (int j = 0; j < VPL; ++j)
#pragma unroll
            for (int k = 0; k < EPV; ++k) {
                if (want_g) fold(acc_g[j][k]);
                if constexpr (!RMS)
                    if (want_b) fold(acc_b[j][k]);
            }
        if (team != 0) return;
    }
    const int64_t prow = blockIdx.x;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
        if (!col_ok[j]) continue;
        const unsigned off = (unsigned)(j * TEAM + tl) * EPV;
#pragma unroll
        for (int k = 0; k < EPV; ++k) {
            if (want_g) part_g[prow * N + off + k] = acc_g[j][k];
            if constexpr (!RMS)
                if (want_b) part_b[prow * N + off + k] = acc_b[j][k];
        }
    }
}

// out[c] = sum over p = 0 .. P-1 of part[p * N + c], in a fixed order: a
// workgroup of 1024 lanes takes 64 columns; its 16 wavefronts sum
// interleaved sixteenths of the partial rows (wavefront w: rows w, w + 16,
// ...), then wavefront 0 adds the sixteen sums in order.  P = 0 gives zeros.
template <int WAVES>
__global__ __launch_bounds__(64 * WAVES)
void norm_colsum_kernel(const float* __restrict__ part, int64_t P, int N, float* __restrict__ out)
{
    __shared__ float q[WAVES][64];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int64_t c = (int64_t)blockIdx.x * 64 + lane;
    float s = 0.0f;
    if (c < N)
        for (int64_t p = w; p < P; p += WAVES) s += part[p * N + c];
    q[w][lane] = s;
    __syncthreads();
    if (w == 0 && c < N) {
        float t = q[0][lane];
#pragma unroll
        for (int i = 1; i < WAVES; ++i) t += q[i][lane];
        out[c] = t;
    }
}
constexpr int kColsumWaves = 16;

}  // namespace mi355norm
