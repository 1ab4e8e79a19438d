// inst_realign_f32.hip -- f32 instantiations of the row kernel with realigned
// loads of x (x not 16-byte aligned; the other operands aligned).
#include "inst_impl.hpp"

namespace mi355norm {
hipError_t launch_rows_realigned_f32(int op, const NormCall& c, const Plan& p) {
    return detail::launch_rows_realigned<F32>(op, c, p);
}
}  // namespace mi355norm
