// inst_f16.hip -- f16 instantiations of the row, split-row and backward kernels.
#include "inst_bwd.hpp"
#include "inst_impl.hpp"

namespace mi355norm {
hipError_t launch_rows_f16(int op, const NormCall& c, const Plan& p) {
    return detail::launch_rows<F16>(op, c, p);
}
hipError_t launch_split_f16(int op, const NormCall& c, const Plan& p, float2* ws) {
    return detail::launch_split<F16>(op, c, p, ws);
}
hipError_t launch_split_pass_f16(int op, const NormCall& c, const Plan& p, unsigned long long* slots,
                                  unsigned* dep, unsigned wait_ticks, unsigned stagger) {
    return detail::launch_split_pass<F16>(op, c, p, slots, dep, wait_ticks, stagger);
}
int pass_blocks_per_cu_f16(int op, int epv, int wg) {
    return detail::pass_blocks_per_cu<F16>(op, epv, wg);
}
hipError_t launch_bwd_f16(int op, const BwdCall& c, const Plan& p) {
    return detail::launch_bwd<F16>(op, c, p);
}
hipError_t launch_bwd_split_f16(int op, const BwdCall& c, const Plan& p, float2* part, float2* rows, int accumulate) {
    return detail::launch_bwd_split<F16>(op, c, p, part, rows, accumulate);
}
hipError_t launch_bwd_pass_f16(int op, const BwdCall& c, const Plan& p, unsigned long long* slots, unsigned* dep,
                               unsigned wait_ticks) {
    return detail::launch_bwd_pass<F16>(op, c, p, slots, dep, wait_ticks);
}
int bwd_pass_blocks_per_cu_f16(int op, int epv) {
    return detail::bwd_pass_blocks_per_cu<F16>(op, epv);
}
}  // namespace mi355norm
