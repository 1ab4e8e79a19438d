// inst_realign_bf16.hip -- bf16 instantiations of the row kernel with realigned
// loads of x (x not 16-byte aligned; the other operands aligned).
#include "inst_impl.hpp"

namespace mi355norm {
hipError_t launch_rows_realigned_bf16(int op, const NormCall& c, const Plan& p) {
    return detail::launch_rows_realigned<BF16>(op, c, p);
}
}  // namespace mi355norm
