// inst_impl.hpp -- kernel selection for one I/O dtype.  Included by
// inst_f32.hip / inst_bf16.hip / inst_f16.hip with MI355_T and MI355_NAME set,
// so the three dtypes compile as separate translation units in parallel.
#pragma once

#include "dispatch.hpp"
#include "rows.hpp"
#include "split.hpp"

namespace mi355norm {
namespace detail {

template <class T>
using St = typename T::storage;

template <class T, bool RMS, int TEAM, int VPL, int EPV>
hipError_t go_rows(const NormCall& c, const Plan& p) {
    const St<T>* x = static_cast<const St<T>*>(c.x);
    const St<T>* g = static_cast<const St<T>*>(c.gamma);
    const St<T>* b = static_cast<const St<T>*>(c.beta);
    St<T>* y = static_cast<St<T>*>(c.y);
    float* mean = c.mean;
    float* rstd = c.rstd;
    int64_t M = c.M;
    int N = c.N;
    float eps = c.eps;
    void* args[] = {&x, &g, &b, &y, &mean, &rstd, &M, &N, &eps};
    return hipLaunchKernel(reinterpret_cast<const void*>(&norm_rows_kernel<T, RMS, TEAM, VPL, EPV>),
                           dim3((unsigned)p.grid), dim3(TeamGeom<TEAM>::WG), args, 0, c.stream);
}

template <class T, bool RMS, int TEAM, int EPV>
hipError_t rows_by_vpl(const NormCall& c, const Plan& p) {
    switch (p.vpl) {
    case 1: return go_rows<T, RMS, TEAM, 1, EPV>(c, p);
    case 2: return go_rows<T, RMS, TEAM, 2, EPV>(c, p);
    case 4: return go_rows<T, RMS, TEAM, 4, EPV>(c, p);
    case 8: return go_rows<T, RMS, TEAM, 8, EPV>(c, p);
    case 16: return go_rows<T, RMS, TEAM, 16, EPV>(c, p);
    }
    return hipErrorInvalidValue;
}

template <class T, bool RMS, int EPV>
hipError_t rows_by_team(const NormCall& c, const Plan& p) {
    switch (p.team) {
    case 4: return rows_by_vpl<T, RMS, 4, EPV>(c, p);
    case 8: return rows_by_vpl<T, RMS, 8, EPV>(c, p);
    case 16: return rows_by_vpl<T, RMS, 16, EPV>(c, p);
    case 32: return rows_by_vpl<T, RMS, 32, EPV>(c, p);
    case 64: return rows_by_vpl<T, RMS, 64, EPV>(c, p);
    case 128: return rows_by_vpl<T, RMS, 128, EPV>(c, p);
    case 256: return rows_by_vpl<T, RMS, 256, EPV>(c, p);
    case 512: return rows_by_vpl<T, RMS, 512, EPV>(c, p);
    case 1024: return rows_by_vpl<T, RMS, 1024, EPV>(c, p);
    }
    return hipErrorInvalidValue;
}

template <class T>
hipError_t launch_rows(bool rms, const NormCall& c, const Plan& p) {
    constexpr int VEC = 16 / T::bytes;
    if (p.epv == VEC) return rms ? rows_by_team<T, true, VEC>(c, p) : rows_by_team<T, false, VEC>(c, p);
    if (p.epv == 1) return rms ? rows_by_team<T, true, 1>(c, p) : rows_by_team<T, false, 1>(c, p);
    return hipErrorInvalidValue;
}

template <class T, bool RMS, int EPV>
hipError_t go_split(const NormCall& c, const Plan& p, float2* ws) {
    const St<T>* x = static_cast<const St<T>*>(c.x);
    const St<T>* g = static_cast<const St<T>*>(c.gamma);
    const St<T>* b = static_cast<const St<T>*>(c.beta);
    St<T>* y = static_cast<St<T>*>(c.y);
    float* mean = c.mean;
    float* rstd = c.rstd;
    int64_t M = c.M;
    int N = c.N;
    int S = p.chunks;
    int CE = kStatsWG * kStatsVPL * EPV;
    int A = p.apply_chunks;
    float eps = c.eps;
    {
        void* args[] = {&x, &ws, &M, &N, &S};
        hipError_t e = hipLaunchKernel(
            reinterpret_cast<const void*>(&norm_split_stats_kernel<T, RMS, kStatsWG, kStatsVPL, EPV>),
            dim3((unsigned)p.grid), dim3(kStatsWG), args, 0, c.stream);
        if (e != hipSuccess) return e;
    }
    const float2* pp = ws;
    void* args[] = {&x, &g, &b, &y, &pp, &mean, &rstd, &M, &N, &S, &CE, &A, &eps};
    return hipLaunchKernel(
        reinterpret_cast<const void*>(&norm_split_apply_kernel<T, RMS, kApplyWG, kApplyVPL, EPV>),
        dim3((unsigned)p.apply_grid), dim3(kApplyWG), args, 0, c.stream);
}

template <class T, bool RMS, int EPV>
const void* coop_kernel() {
    return reinterpret_cast<const void*>(&norm_split_coop_kernel<T, RMS, kCoopWG, kCoopVPL, EPV>);
}

template <class T>
int coop_blocks_per_cu(bool rms, int epv) {
    constexpr int VEC = 16 / T::bytes;
    const void* f = nullptr;
    if (epv == VEC) f = rms ? coop_kernel<T, true, VEC>() : coop_kernel<T, false, VEC>();
    else if (epv == 1) f = rms ? coop_kernel<T, true, 1>() : coop_kernel<T, false, 1>();
    if (!f) return 0;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, kCoopWG, 0) != hipSuccess) return 0;
    return n;
}

template <class T, bool RMS, int EPV>
hipError_t go_split_coop(const NormCall& c, const Plan& p, float2* ws, unsigned* sync,
                         unsigned need, unsigned spin_limit) {
    const St<T>* x = static_cast<const St<T>*>(c.x);
    const St<T>* g = static_cast<const St<T>*>(c.gamma);
    const St<T>* b = static_cast<const St<T>*>(c.beta);
    St<T>* y = static_cast<St<T>*>(c.y);
    float* mean = c.mean;
    float* rstd = c.rstd;
    int64_t M = c.M;
    int N = c.N;
    int S = p.chunks;
    int teams = p.teams;
    float eps = c.eps;
    void* args[] = {&x, &g, &b, &y, &mean, &rstd, &ws, &sync, &M, &N, &S, &teams, &eps, &need, &spin_limit};
    return hipLaunchCooperativeKernel(coop_kernel<T, RMS, EPV>(), dim3((unsigned)(teams * S)),
                                      dim3(kCoopWG), args, 0, c.stream);
}

template <class T>
hipError_t launch_split_coop(bool rms, const NormCall& c, const Plan& p, float2* ws, unsigned* sync,
                             unsigned need, unsigned spin_limit) {
    constexpr int VEC = 16 / T::bytes;
    if (p.epv == VEC)
        return rms ? go_split_coop<T, true, VEC>(c, p, ws, sync, need, spin_limit)
                   : go_split_coop<T, false, VEC>(c, p, ws, sync, need, spin_limit);
    if (p.epv == 1)
        return rms ? go_split_coop<T, true, 1>(c, p, ws, sync, need, spin_limit)
                   : go_split_coop<T, false, 1>(c, p, ws, sync, need, spin_limit);
    return hipErrorInvalidValue;
}

template <class T>
hipError_t launch_split(bool rms, const NormCall& c, const Plan& p, float2* ws) {
    constexpr int VEC = 16 / T::bytes;
    if (p.epv == VEC) return rms ? go_split<T, true, VEC>(c, p, ws) : go_split<T, false, VEC>(c, p, ws);
    if (p.epv == 1) return rms ? go_split<T, true, 1>(c, p, ws) : go_split<T, false, 1>(c, p, ws);
    return hipErrorInvalidValue;
}

}  // namespace detail
}  // namespace mi355norm
