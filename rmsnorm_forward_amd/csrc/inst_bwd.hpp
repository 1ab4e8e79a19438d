// inst_bwd.hpp -- backward kernel selection for one I/O dtype (row kernel
// and split rows).  Included by inst_f32.hip / inst_bf16.hip / inst_f16.hip
// after the forward's selection, whose helpers it uses.
#pragma once

#include <algorithm>

#include "backward.hpp"
#include "backward_split.hpp"
#include "inst_impl.hpp"

namespace mi355norm {
namespace detail {

// ---------------------------------------------------------------------------
// backward
// ---------------------------------------------------------------------------

template <class T, bool RMS, int TEAM, int VPL, int EPV>
hipError_t go_bwd(const BwdCall& c, const Plan& p) {
    const St<T>* dy = static_cast<const St<T>*>(c.dy);
    const St<T>* x = static_cast<const St<T>*>(c.x);
    const St<T>* g = static_cast<const St<T>*>(c.gamma);
    const float* mean = c.mean;
    const float* rstd = c.rstd;
    St<T>* dx = static_cast<St<T>*>(c.dx);
    float* pg = c.part_g;
    float* pb = c.part_b;
    int64_t M = c.M;
    int N = c.N;
    int64_t ldy = c.ldy, ldx = c.ldx, lddx = c.lddx;
    void* args[] = {&dy, &x, &g, &mean, &rstd, &dx, &pg, &pb, &M, &N, &ldy, &ldx, &lddx};
    return hipLaunchKernel(reinterpret_cast<const void*>(&norm_bwd_rows_kernel<T, RMS, TEAM, VPL, EPV>),
                           dim3((unsigned)p.grid), dim3(kBwdWG), args, 0, c.stream);
}

template <class T, bool RMS, int TEAM, int EPV>
hipError_t bwd_by_vpl(const BwdCall& c, const Plan& p) {
    switch (p.vpl) {
    case 1: return go_bwd<T, RMS, TEAM, 1, EPV>(c, p);
    case 2: return go_bwd<T, RMS, TEAM, 2, EPV>(c, p);
    case 4: return go_bwd<T, RMS, TEAM, 4, EPV>(c, p);
    case 8:
        if constexpr (8 * EPV <= kBwdMaxElems) return go_bwd<T, RMS, TEAM, 8, EPV>(c, p);
        break;
    case 16:
        if constexpr (16 * EPV <= kBwdMaxElems) return go_bwd<T, RMS, TEAM, 16, EPV>(c, p);
        break;
    }
    return hipErrorInvalidValue;
}

template <class T, bool RMS, int EPV>
hipError_t bwd_by_team(const BwdCall& c, const Plan& p) {
    switch (p.team) {
    case 8: return bwd_by_vpl<T, RMS, 8, EPV>(c, p);
    case 16: return bwd_by_vpl<T, RMS, 16, EPV>(c, p);
    case 32: return bwd_by_vpl<T, RMS, 32, EPV>(c, p);
    case 64: return bwd_by_vpl<T, RMS, 64, EPV>(c, p);
    case 128: return bwd_by_vpl<T, RMS, 128, EPV>(c, p);
    case 256: return bwd_by_vpl<T, RMS, 256, EPV>(c, p);
    case 512: return bwd_by_vpl<T, RMS, 512, EPV>(c, p);
    case 1024: return bwd_by_vpl<T, RMS, 1024, EPV>(c, p);
    }
    return hipErrorInvalidValue;
}

template <class T>
hipError_t launch_bwd(int op, const BwdCall& c, const Plan& p) {
    if (op != OP_LN && op != OP_RMS) return hipErrorInvalidValue;
    return with_epv<T>(p.epv, [&](auto epv) {
        constexpr int E = decltype(epv)::value;
        return op == OP_RMS ? bwd_by_team<T, true, E>(c, p) : bwd_by_team<T, false, E>(c, p);
    });
}

template <class T, bool RMS, int EPV>
hipError_t go_bwd_split(const BwdCall& c, const Plan& p, float2* part, float2* rows, int accumulate) {
    const St<T>* dy = static_cast<const St<T>*>(c.dy);
    const St<T>* x = static_cast<const St<T>*>(c.x);
    const St<T>* g = static_cast<const St<T>*>(c.gamma);
    const float* mean = c.mean;
    const float* rstd = c.rstd;
    St<T>* dx = static_cast<St<T>*>(c.dx);
    float* pg = c.part_g;
    float* pb = c.part_b;
    int64_t M = c.M;
    int N = c.N;
    int64_t ldy = c.ldy, ldx = c.ldx, lddx = c.lddx;
    int S = p.chunks, A = p.apply_chunks;
    const float2* pc = part;
    const float2* rc = rows;
    {
        void* args[] = {&dy, &x, &g, &mean, &rstd, &part, &M, &N, &ldy, &ldx, &S};
        const int64_t grid = std::min<int64_t>(p.grid, M * S);
        hipError_t e = hipLaunchKernel(
            reinterpret_cast<const void*>(&norm_bwd_split_sums_kernel<T, RMS, kBwdSplitWG, bwd_sums_vpl(EPV), EPV>),
            dim3((unsigned)grid), dim3(kBwdSplitWG), args, 0, c.stream);
        if (e != hipSuccess) return e;
    }
    {
        void* args[] = {&pc, &rows, &M, &S};
        const int64_t grid = std::min<int64_t>((M + 3) / 4, int64_t(1) << 20);   // rows grid-strided
        hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&norm_bwd_split_rowsum_kernel<4>),
                                       dim3((unsigned)grid), dim3(256), args, 0, c.stream);
        if (e != hipSuccess) return e;
    }
    void* args[] = {&dy, &x, &g, &mean, &rstd, &rc, &dx, &pg, &pb, &accumulate, &M, &N, &ldy, &ldx, &lddx, &A};
    return hipLaunchKernel(
        reinterpret_cast<const void*>(&norm_bwd_split_apply_kernel<T, RMS, kBwdSplitWG, kBwdSplitApplyVPL, EPV>),
        dim3((unsigned)(int64_t(A) * p.teams)), dim3(kBwdSplitWG), args, 0, c.stream);
}

template <class T>
hipError_t launch_bwd_split(int op, const BwdCall& c, const Plan& p, float2* part, float2* rows, int accumulate) {
    if (op != OP_LN && op != OP_RMS) return hipErrorInvalidValue;
    return with_epv<T>(p.epv, [&](auto epv) {
        constexpr int E = decltype(epv)::value;
        return op == OP_RMS ? go_bwd_split<T, true, E>(c, p, part, rows, accumulate)
                            : go_bwd_split<T, false, E>(c, p, part, rows, accumulate);
    });
}

// ---------------------------------------------------------------------------
// split backward, single pass
// ---------------------------------------------------------------------------

template <class T, bool RMS, int EPV>
const void* bwd_pass_kernel() {
    return reinterpret_cast<const void*>(&norm_bwd_pass_kernel<T, RMS, kBwdPassWG, kBwdPassVPL, EPV>);
}

template <class T>
int bwd_pass_blocks_per_cu(int op, int epv) {
    if (op != OP_LN && op != OP_RMS) return 0;
    const void* f = nullptr;
    (void)with_epv<T>(epv, [&](auto e) {
        constexpr int E = decltype(e)::value;
        f = op == OP_RMS ? bwd_pass_kernel<T, true, E>() : bwd_pass_kernel<T, false, E>();
        return hipSuccess;
    });
    if (!f) return 0;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, kBwdPassWG, 0) != hipSuccess) return 0;
    return n;
}

template <class T, bool RMS, int EPV>
hipError_t go_bwd_pass(const BwdCall& c, const Plan& p, unsigned long long* slots, unsigned* dep,
                       unsigned wait_ticks) {
    const St<T>* dy = static_cast<const St<T>*>(c.dy);
    const St<T>* x = static_cast<const St<T>*>(c.x);
    const St<T>* g = static_cast<const St<T>*>(c.gamma);
    const float* mean = c.mean;
    const float* rstd = c.rstd;
    St<T>* dx = static_cast<St<T>*>(c.dx);
    float* pg = c.part_g;
    float* pb = c.part_b;
    int64_t M = c.M;
    int N = c.N;
    int64_t ldy = c.ldy, ldx = c.ldx, lddx = c.lddx;
    int S = p.chunks, teams = p.teams;
    void* args[] = {&dy, &x, &g, &mean, &rstd, &dx, &pg, &pb, &slots, &dep, &M, &N, &ldy, &ldx, &lddx, &S,
                    &teams, &wait_ticks};
    return hipLaunchKernel(bwd_pass_kernel<T, RMS, EPV>(), dim3((unsigned)(teams * S)), dim3(kBwdPassWG), args, 0,
                           c.stream);
}

template <class T>
hipError_t launch_bwd_pass(int op, const BwdCall& c, const Plan& p, unsigned long long* slots, unsigned* dep,
                           unsigned wait_ticks) {
    if (op != OP_LN && op != OP_RMS) return hipErrorInvalidValue;
    return with_epv<T>(p.epv, [&](auto epv) {
        constexpr int E = decltype(epv)::value;
        return op == OP_RMS ? go_bwd_pass<T, true, E>(c, p, slots, dep, wait_ticks)
                            : go_bwd_pass<T, false, E>(c, p, slots, dep, wait_ticks);
    });
}

}  // namespace detail
}  // namespace mi355norm
