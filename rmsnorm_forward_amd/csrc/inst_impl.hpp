// inst_impl.hpp -- kernel selection for one I/O dtype.  Included by
// inst_f32.hip / inst_bf16.hip / inst_f16.hip, so the three dtypes compile as
// separate translation units in parallel.
#pragma once

#include "dispatch.hpp"
#include "rows.hpp"
#include "split.hpp"

namespace mi355norm {
namespace detail {

template <class T>
using St = typename T::storage;

template <bool B>
using bc = std::integral_constant<bool, B>;

// Calls f(bc<RMS>, bc<ADD>, bc<Q8>) for the operation.
template <class F>
hipError_t with_op(int op, F&& f) {
    switch (op) {
    case OP_LN: return f(bc<false>{}, bc<false>{}, bc<false>{});
    case OP_RMS: return f(bc<true>{}, bc<false>{}, bc<false>{});
    case OP_ADD_RMS: return f(bc<true>{}, bc<true>{}, bc<false>{});
    case OP_RMS_Q8: return f(bc<true>{}, bc<false>{}, bc<true>{});
    case OP_ADD_RMS_Q8: return f(bc<true>{}, bc<true>{}, bc<true>{});
    }
    return hipErrorInvalidValue;
}

// Calls f(integral_constant<int, EPV>) for the plan's vector width.
template <class T, class F>
hipError_t with_epv(int epv, F&& f) {
    constexpr int VEC = 16 / T::bytes;
    if (epv == VEC) return f(std::integral_constant<int, VEC>{});
    if (epv == 1) return f(std::integral_constant<int, 1>{});
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// row kernel
// ---------------------------------------------------------------------------

template <class T, bool RMS, bool ADD, bool Q8, int TEAM, int VPL, int EPV, bool RA>
hipError_t go_rows(const NormCall& c, const Plan& p) {
    const St<T>* x = static_cast<const St<T>*>(c.x);
    const St<T>* r = static_cast<const St<T>*>(c.res);
    const St<T>* g = static_cast<const St<T>*>(c.gamma);
    const St<T>* b = static_cast<const St<T>*>(c.beta);
    void* y = c.y;
    St<T>* h = static_cast<St<T>*>(c.hout);
    float* mean = c.mean;
    float* rstd = c.rstd;
    int64_t M = c.M;
    int N = c.N;
    float eps = c.eps;
    float qinv = c.qinv;
    Strides ld = c.ld;
    void* args[] = {&x, &r, &g, &b, &y, &h, &mean, &rstd, &M, &N, &ld, &eps, &qinv};
    return hipLaunchKernel(reinterpret_cast<const void*>(&norm_rows_kernel<T, RMS, ADD, Q8, TEAM, VPL, EPV, RA>),
                           dim3((unsigned)p.grid), dim3(TeamGeom<TEAM>::WG), args, 0, c.stream);
}

template <class T, bool RMS, bool ADD, bool Q8, int TEAM, int EPV, bool RA>
hipError_t rows_by_vpl(const NormCall& c, const Plan& p) {
    switch (p.vpl) {
    case 1: return go_rows<T, RMS, ADD, Q8, TEAM, 1, EPV, RA>(c, p);
    case 2: return go_rows<T, RMS, ADD, Q8, TEAM, 2, EPV, RA>(c, p);
    case 4: return go_rows<T, RMS, ADD, Q8, TEAM, 4, EPV, RA>(c, p);
    case 8: return go_rows<T, RMS, ADD, Q8, TEAM, 8, EPV, RA>(c, p);
    case 16: return go_rows<T, RMS, ADD, Q8, TEAM, 16, EPV, RA>(c, p);
    case 5:
        if constexpr (TEAM == 64) return go_rows<T, RMS, ADD, Q8, TEAM, 5, EPV, RA>(c, p);
        break;
    case 10:
        if constexpr (TEAM == 64) return go_rows<T, RMS, ADD, Q8, TEAM, 10, EPV, RA>(c, p);
        break;
    }
    return hipErrorInvalidValue;
}

template <class T, bool RMS, bool ADD, bool Q8, int EPV, bool RA = false>
hipError_t rows_by_team(const NormCall& c, const Plan& p) {
    switch (p.team) {
    case 4: return rows_by_vpl<T, RMS, ADD, Q8, 4, EPV, RA>(c, p);
    case 8: return rows_by_vpl<T, RMS, ADD, Q8, 8, EPV, RA>(c, p);
    case 16: return rows_by_vpl<T, RMS, ADD, Q8, 16, EPV, RA>(c, p);
    case 32: return rows_by_vpl<T, RMS, ADD, Q8, 32, EPV, RA>(c, p);
    case 64: return rows_by_vpl<T, RMS, ADD, Q8, 64, EPV, RA>(c, p);
    case 128: return rows_by_vpl<T, RMS, ADD, Q8, 128, EPV, RA>(c, p);
    case 256: return rows_by_vpl<T, RMS, ADD, Q8, 256, EPV, RA>(c, p);
    case 512: return rows_by_vpl<T, RMS, ADD, Q8, 512, EPV, RA>(c, p);
    case 1024: return rows_by_vpl<T, RMS, ADD, Q8, 1024, EPV, RA>(c, p);
    }
    return hipErrorInvalidValue;
}

template <class T>
hipError_t launch_rows(int op, const NormCall& c, const Plan& p) {
    return with_op(op, [&](auto rms, auto add, auto q8) {
        return with_epv<T>(p.epv, [&](auto epv) {
            return rows_by_team<T, decltype(rms)::value, decltype(add)::value, decltype(q8)::value,
                                decltype(epv)::value>(c, p);
        });
    });
}

// Row kernel with realigned loads of x (x not 16-byte aligned, the other
// operands aligned): LayerNorm, RMSNorm and RMSNorm with FP8 output on
// 16-byte vectors.  Instantiated, with the split rows' two kernels below, in
// translation units of their own.
template <class T>
hipError_t launch_rows_realigned(int op, const NormCall& c, const Plan& p) {
    constexpr int VEC = 16 / T::bytes;
    if (p.epv != VEC) return hipErrorInvalidValue;
    switch (op) {
    case OP_LN: return rows_by_team<T, false, false, false, VEC, true>(c, p);
    case OP_RMS: return rows_by_team<T, true, false, false, VEC, true>(c, p);
    case OP_RMS_Q8: return rows_by_team<T, true, false, true, VEC, true>(c, p);
    }
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// split rows, two kernels
// ---------------------------------------------------------------------------

template <class T, bool RMS, bool ADD, bool Q8, int EPV, bool RA = false>
hipError_t go_split(const NormCall& c, const Plan& p, float2* ws) {
    const St<T>* x = static_cast<const St<T>*>(c.x);
    const St<T>* r = static_cast<const St<T>*>(c.res);
    const St<T>* g = static_cast<const St<T>*>(c.gamma);
    const St<T>* b = static_cast<const St<T>*>(c.beta);
    void* y = c.y;
    St<T>* h = static_cast<St<T>*>(c.hout);
    float* mean = c.mean;
    float* rstd = c.rstd;
    int64_t M = c.M;
    int N = c.N;
    int S = p.chunks;
    int CE = kStatsWG * kStatsVPL * EPV;
    int A = p.apply_chunks;
    float eps = c.eps;
    float qinv = c.qinv;
    Strides ld = c.ld;
    {
        void* args[] = {&x, &r, &h, &ws, &M, &N, &ld, &S};
        hipError_t e = hipLaunchKernel(
            reinterpret_cast<const void*>(&norm_split_stats_kernel<T, RMS, ADD, kStatsWG, kStatsVPL, EPV, RA>),
            dim3((unsigned)p.grid), dim3(kStatsWG), args, 0, c.stream);
        if (e != hipSuccess) return e;
    }
    // with the residual add the normalising kernel reads the stored sum
    const St<T>* src = ADD ? h : x;
    Strides lda = ld;
    if (ADD) lda.x = ld.h;
    const float2* pp = ws;
    void* args[] = {&src, &g, &b, &y, &pp, &mean, &rstd, &M, &N, &lda, &S, &CE, &A, &eps, &qinv};
    return hipLaunchKernel(
        reinterpret_cast<const void*>(&norm_split_apply_kernel<T, RMS, Q8, kApplyWG, kApplyVPL, EPV, RA>),
        dim3((unsigned)p.apply_grid), dim3(kApplyWG), args, 0, c.stream);
}

template <class T>
hipError_t launch_split(int op, const NormCall& c, const Plan& p, float2* ws) {
    return with_op(op, [&](auto rms, auto add, auto q8) {
        return with_epv<T>(p.epv, [&](auto epv) {
            return go_split<T, decltype(rms)::value, decltype(add)::value, decltype(q8)::value,
                            decltype(epv)::value>(c, p, ws);
        });
    });
}

// The two kernels with realigned loads of x (as the row kernel's).
template <class T>
hipError_t launch_split_realigned(int op, const NormCall& c, const Plan& p, float2* ws) {
    constexpr int VEC = 16 / T::bytes;
    if (p.epv != VEC) return hipErrorInvalidValue;
    switch (op) {
    case OP_LN: return go_split<T, false, false, false, VEC, true>(c, p, ws);
    case OP_RMS: return go_split<T, true, false, false, VEC, true>(c, p, ws);
    case OP_RMS_Q8: return go_split<T, true, false, true, VEC, true>(c, p, ws);
    }
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// split rows, single pass (LayerNorm, RMSNorm, RMSNorm with FP8 output)
// ---------------------------------------------------------------------------

template <class T, bool RMS, bool Q8, int EPV, int WG>
const void* pass_kernel() {
    return reinterpret_cast<const void*>(&norm_split_pass_kernel<T, RMS, Q8, WG, kPassVPL, EPV>);
}

// Calls f(bc<RMS>, bc<Q8>) for the operations the single pass runs.
template <class F>
hipError_t with_pass_op(int op, F&& f) {
    switch (op) {
    case OP_LN: return f(bc<false>{}, bc<false>{});
    case OP_RMS: return f(bc<true>{}, bc<false>{});
    case OP_RMS_Q8: return f(bc<true>{}, bc<true>{});
    }
    return hipErrorInvalidValue;
}

// Whether the wide chunks (kPassWideWG lanes) are built for this operation,
// dtype and vector width: 16-byte vectors, RMSNorm of every dtype and fp32
// LayerNorm (LayerNorm with 16-bit I/O runs 128 VGPRs and spills at that
// width).
template <class T, bool RMS, int EPV>
constexpr bool pass_wide_built() {
    return EPV * sizeof(St<T>) == 16 && (RMS || std::is_same<T, F32>::value);
}

// Calls f(integral_constant<int, WG>) for the plan's chunk width.
template <class T, bool RMS, int EPV, class F>
hipError_t with_pass_wg(int wg, F&& f) {
    if (wg == kPassWG) return f(std::integral_constant<int, kPassWG>{});
    if constexpr (pass_wide_built<T, RMS, EPV>())
        if (wg == kPassWideWG) return f(std::integral_constant<int, kPassWideWG>{});
    return hipErrorInvalidValue;
}

// Workgroups of the single pass resident per CU for this chunk width (0 if
// that width is not built for the operation).
template <class T>
int pass_blocks_per_cu(int op, int epv, int wg) {
    const void* f = nullptr;
    (void)with_pass_op(op, [&](auto rms, auto q8) {
        return with_epv<T>(epv, [&](auto e) {
            return with_pass_wg<T, decltype(rms)::value, decltype(e)::value>(wg, [&](auto w) {
                f = pass_kernel<T, decltype(rms)::value, decltype(q8)::value, decltype(e)::value,
                                decltype(w)::value>();
                return hipSuccess;
            });
        });
    });
    if (!f) return 0;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, wg, 0) != hipSuccess) return 0;
    return n;
}

template <class T, bool RMS, bool Q8, int EPV, int WG>
hipError_t go_split_pass(const NormCall& c, const Plan& p, unsigned long long* slots, unsigned* dep,
                         unsigned wait_ticks, unsigned stagger) {
    const St<T>* x = static_cast<const St<T>*>(c.x);
    const St<T>* g = static_cast<const St<T>*>(c.gamma);
    const St<T>* b = static_cast<const St<T>*>(c.beta);
    void* y = c.y;
    float* mean = c.mean;
    float* rstd = c.rstd;
    int64_t M = c.M;
    int N = c.N;
    int S = p.chunks;
    int teams = p.teams;
    float eps = c.eps;
    float qinv = c.qinv;
    Strides ld = c.ld;
    void* args[] = {&x, &g, &b, &y, &mean, &rstd, &slots, &dep, &M, &N, &ld, &S, &teams, &eps, &qinv,
                    &wait_ticks, &stagger};
    return hipLaunchKernel(pass_kernel<T, RMS, Q8, EPV, WG>(), dim3((unsigned)(teams * S)), dim3(WG), args, 0,
                           c.stream);
}

template <class T>
hipError_t launch_split_pass(int op, const NormCall& c, const Plan& p, unsigned long long* slots, unsigned* dep,
                             unsigned wait_ticks, unsigned stagger) {
    return with_pass_op(op, [&](auto rms, auto q8) {
        return with_epv<T>(p.epv, [&](auto epv) {
            return with_pass_wg<T, decltype(rms)::value, decltype(epv)::value>(p.wg, [&](auto w) {
                return go_split_pass<T, decltype(rms)::value, decltype(q8)::value, decltype(epv)::value,
                                     decltype(w)::value>(c, p, slots, dep, wait_ticks, stagger);
            });
        });
    });
}

}  // namespace detail
}  // namespace mi355norm
