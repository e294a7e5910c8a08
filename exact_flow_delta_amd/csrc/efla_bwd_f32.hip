// efla_bwd_f32.hip -- fp32-input instantiations of the backward pass.
#include "efla_bwd.hpp"

namespace efla {
hipError_t launch_bwd_f32(const BwdArgs& a, hipStream_t s) { return launch_bwd_e<float>(a, s); }
}  // namespace efla
