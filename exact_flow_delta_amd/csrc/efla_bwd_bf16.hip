// efla_bwd_bf16.hip -- bf16-input instantiations of the backward pass (the state-gradient pass and the per-chunk
// gradients on bf16 matrix cores where efla_bwd_chain_mx.hpp and efla_bwd_mx.hpp apply).
#include "efla_bwd.hpp"
#include "efla_bwd_chain_mx.hpp"
#include "efla_bwd_mx.hpp"

namespace efla {
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t s) { return launch_bwd_e<bf16>(a, s); }
}  // namespace efla
