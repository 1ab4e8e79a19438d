// inst_bf16.hip -- bf16 instantiations of the row and split-row kernels.
#include "inst_impl.hpp"

namespace mi355norm {
hipError_t launch_rows_bf16(bool rms, const NormCall& c, const Plan& p) {
    return detail::launch_rows<BF16>(rms, c, p);
}
hipError_t launch_split_bf16(bool rms, const NormCall& c, const Plan& p, float2* ws) {
    return detail::launch_split<BF16>(rms, c, p, ws);
}
}  // namespace mi355norm
