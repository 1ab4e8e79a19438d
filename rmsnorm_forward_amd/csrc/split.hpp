// split.hpp -- rows too long for one workgroup's registers.  A row is cut
// into chunks of CV = WG*VPL vectors; a chunk is one workgroup's work item.
//
//   norm_split_stats_kernel : per chunk, LayerNorm (n_c, mu_c, M2_c) relative
//                             to the row shift K = x[row, 0] (two passes over
//                             the chunk in registers), or RMSNorm sum of
//                             squares; written to a [M, S] float2 workspace.
//   norm_split_apply_kernel : per chunk, merge the row's S partials in chunk
//                             order with Chan's formula (every workgroup of a
//                             row runs the identical merge, so all chunks of a
//                             row use bitwise-identical mean and rstd), then
//                             normalise the chunk and store it.
//
// Merging (n, mean, M2) partials is what "T3 讲解" part ② recommends once a
// row has to be read in segments, with the associative merge of
// "CUDA 算子工程" ch. 7 section 7.4.1.  This two-kernel form reads x twice;
// rows are independent, so the second read of a chunk is issued soon after
// the first for small M and often hits the on-die caches.
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

template <class T, bool RMS, int WG, int VPL, int EPV>
__global__ __launch_bounds__(WG)
void norm_split_stats_kernel(const typename T::storage* __restrict__ x,
                             float2* __restrict__ ws,
                             int64_t M, int N, int S)
{
    using V = Vec<T, EPV>;
    constexpr int CV = WG * VPL;
    __shared__ float red[2][WG / 64];
    const int tid = threadIdx.x;
    const int NV = N / EPV;
    const int64_t items = M * (int64_t)S;

    for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
        const int64_t row = it / S;
        const int c = (int)(it - row * S);
        const typename T::storage* xr = x + row * (int64_t)N;
        const int v0 = c * CV;
        V xv[VPL];
        bool ok[VPL];
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            const int v = v0 + j * WG + tid;
            ok[j] = v < NV;
            if (ok[j]) xv[j].load_stream(xr + (int64_t)v * EPV);
            else xv[j].zero();
        }
        float2 out;
        if constexpr (RMS) {
            float q = 0.0f;
#pragma unroll
            for (int j = 0; j < VPL; ++j)
#pragma unroll
                for (int k = 0; k < EPV; ++k) {
                    const float v = xv[j].get(k);
                    q = __builtin_fmaf(v, v, q);
                }
            q = wg_sum<WG>(q, red[0]);
            out = make_float2(q, 0.0f);
        } else {
            const float K = T::widen(xr[0]);
            const int nvec = min(CV, NV - v0);
            const float nc = (float)nvec * (float)EPV;
            float s = 0.0f;
#pragma unroll
            for (int j = 0; j < VPL; ++j)
#pragma unroll
                for (int k = 0; k < EPV; ++k) s += ok[j] ? xv[j].get(k) - K : 0.0f;
            s = wg_sum<WG>(s, red[0]);
            const float mc = s / nc;
            float q = 0.0f;
#pragma unroll
            for (int j = 0; j < VPL; ++j)
#pragma unroll
                for (int k = 0; k < EPV; ++k) {
                    const float e = ok[j] ? (xv[j].get(k) - K) - mc : 0.0f;
                    q = __builtin_fmaf(e, e, q);
                }
            q = wg_sum<WG>(q, red[1]);
            out = make_float2(mc, q);
        }
        if (tid == 0) ws[it] = out;
        // the LDS slots are rewritten by the next item
        __syncthreads();
    }
}

// Merge a row's S partials (S arbitrary) inside one wavefront; the result is
// wave-uniform and identical in every wavefront that runs it on the same data.
// Lane l folds partials l, l+64, l+128, ... in order; the 64 lane states are
// then merged by a butterfly whose every step puts the lower lane's state
// first, so partners compute bitwise-identical results.
__device__ __forceinline__ Welford merge_row_partials(const float2* p, int S, int CE, int N) {
    const int l = lane_id();
    Welford a = {0.0f, 0.0f, 0.0f};
    for (int c = l; c < S; c += 64) {
        const float2 v = p[c];
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

template <class T, bool RMS, int WG, int VPL, int EPV>
__global__ __launch_bounds__(WG)
void norm_split_apply_kernel(const typename T::storage* __restrict__ x,
                             const typename T::storage* __restrict__ gamma,
                             const typename T::storage* __restrict__ beta,
                             typename T::storage* __restrict__ y,
                             float* __restrict__ mean_out,
                             float* __restrict__ rstd_out,
                             const float2* __restrict__ ws,
                             int64_t M, int N, int S, float eps)
{
    using V = Vec<T, EPV>;
    constexpr int CV = WG * VPL;
    const int tid = threadIdx.x;
    const int NV = N / EPV;
    const float fN = (float)N;
    const int64_t items = M * (int64_t)S;
    const bool has_g = gamma != nullptr;
    const bool has_b = beta != nullptr;

    for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
        const int64_t row = it / S;
        const int c = (int)(it - row * S);
        const typename T::storage* xr = x + row * (int64_t)N;
        typename T::storage* yr = y + row * (int64_t)N;
        const int v0 = c * CV;
        V xv[VPL];
        bool ok[VPL];
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            const int v = v0 + j * WG + tid;
            ok[j] = v < NV;
            if (ok[j]) xv[j].load_stream(xr + (int64_t)v * EPV);
            else xv[j].zero();
        }
        const float2* pr = ws + row * (int64_t)S;
        float rs, mu = 0.0f, K = 0.0f;
        if constexpr (RMS) {
            float q = 0.0f;
            for (int cc = lane_id(); cc < S; cc += 64) q += pr[cc].x;
            q = team_sum<64>(q);
            rs = rsqrt_hw(q / fN + eps);
        } else {
            K = T::widen(xr[0]);
            const Welford w = merge_row_partials(pr, S, CV * EPV, N);
            mu = w.mean;
            rs = rsqrt_hw(w.m2 / fN + eps);
        }
        if (c == 0 && tid == 0) {
            if (!RMS && mean_out) mean_out[row] = K + mu;
            if (rstd_out) rstd_out[row] = rs;
        }
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            if (!ok[j]) continue;
            const int64_t off = (int64_t)(v0 + j * WG + tid) * EPV;
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
            V::store(yr + off, o);
        }
    }
}

}  // namespace mi355norm
