// inst_realign_f16.hip -- f16 instantiations of the row kernel and the split
// rows' two kernels with realigned loads of x (x not 16-byte aligned; the
// other operands aligned).
#include "inst_impl.hpp"

namespace mi355norm {
hipError_t launch_rows_realigned_f16(int op, const NormCall& c, const Plan& p) {
    return detail::launch_rows_realigned<F16>(op, c, p);
}
hipError_t launch_split_realigned_f16(int op, const NormCall& c, const Plan& p, float2* ws) {
    return detail::launch_split_realigned<F16>(op, c, p, ws);
}
}  // namespace mi355norm
