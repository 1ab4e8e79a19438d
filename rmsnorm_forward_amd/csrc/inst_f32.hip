// inst_f32.hip -- f32 instantiations of the row and split-row kernels.
#include "inst_impl.hpp"

namespace mi355norm {
hipError_t launch_rows_f32(bool rms, const NormCall& c, const Plan& p) {
    return detail::launch_rows<F32>(rms, c, p);
}
hipError_t launch_split_f32(bool rms, const NormCall& c, const Plan& p, float2* ws) {
    return detail::launch_split<F32>(rms, c, p, ws);
}
}  // namespace mi355norm
