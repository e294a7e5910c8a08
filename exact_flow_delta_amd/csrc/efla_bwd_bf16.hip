// efla_bwd_bf16.hip -- bf16-input instantiations of the backward pass.
#include "efla_bwd.hpp"

namespace efla {
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t s) { return launch_bwd_e<bf16>(a, s); }
}  // namespace efla
