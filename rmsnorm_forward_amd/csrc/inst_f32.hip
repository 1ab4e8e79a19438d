// inst_f32.hip -- f32 instantiations of the row, split-row and backward
// kernels, and the launch of the (type-free) column-sum kernel.
#include "inst_bwd.hpp"
#include "inst_impl.hpp"

namespace mi355norm {
hipError_t launch_rows_f32(int op, const NormCall& c, const Plan& p) {
    return detail::launch_rows<F32>(op, c, p);
}
hipError_t launch_split_f32(int op, const NormCall& c, const Plan& p, float2* ws) {
    return detail::launch_split<F32>(op, c, p, ws);
}
hipError_t launch_split_pass_f32(int op, const NormCall& c, const Plan& p, unsigned long long* slots,
                                  unsigned* dep, unsigned wait_ticks, unsigned stagger) {
    return detail::launch_split_pass<F32>(op, c, p, slots, dep, wait_ticks, stagger);
}
int pass_blocks_per_cu_f32(int op, int epv, int wg) {
    return detail::pass_blocks_per_cu<F32>(op, epv, wg);
}
hipError_t launch_bwd_f32(int op, const BwdCall& c, const Plan& p) {
    return detail::launch_bwd<F32>(op, c, p);
}
hipError_t launch_bwd_split_f32(int op, const BwdCall& c, const Plan& p, float2* part, float2* rows, int accumulate) {
    return detail::launch_bwd_split<F32>(op, c, p, part, rows, accumulate);
}
hipError_t launch_bwd_pass_f32(int op, const BwdCall& c, const Plan& p, unsigned long long* slots, unsigned* dep,
                               unsigned wait_ticks) {
    return detail::launch_bwd_pass<F32>(op, c, p, slots, dep, wait_ticks);
}
int bwd_pass_blocks_per_cu_f32(int op, int epv) {
    return detail::bwd_pass_blocks_per_cu<F32>(op, epv);
}
hipError_t launch_colsum(const float* part_g, float* out_g, const float* part_b, float* out_b, int64_t P, int N,
                         hipStream_t stream) {
    // wavefronts per 64 columns: as many as the partial rows keep busy; few
    // partial rows: one lane per four columns
    const unsigned pairs = out_b ? 2u : 1u;
    const dim3 grid((unsigned)((N + 63) / 64), pairs);
    if (P >= 4 * kColsumWaves) {
        hipLaunchKernelGGL(norm_colsum_kernel<kColsumWaves>, grid, dim3(64 * kColsumWaves), 0, stream, part_g,
                           out_g, part_b, out_b, P, N);
    } else if (P >= 16) {
        hipLaunchKernelGGL(norm_colsum_kernel<4>, grid, dim3(64 * 4), 0, stream, part_g, out_g, part_b, out_b, P, N);
    } else if (N % 4 == 0) {
        const dim3 g4((unsigned)((N / 4 + 255) / 256), pairs);
        hipLaunchKernelGGL(norm_colsum_narrow_kernel<true>, g4, dim3(256), 0, stream, part_g, out_g, part_b, out_b,
                           P, N);
    } else {
        const dim3 g1((unsigned)((N + 255) / 256), pairs);
        hipLaunchKernelGGL(norm_colsum_narrow_kernel<false>, g1, dim3(256), 0, stream, part_g, out_g, part_b, out_b,
                           P, N);
    }
    return hipGetLastError();
}
}  // namespace mi355norm
