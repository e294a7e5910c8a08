// efla_chunk_bf16.hip -- bf16-input instantiations of the one-launch chunked forward: for d_k >= 32 and
// 64-token chunks the state pass with an in-workgroup UT transform, else the fused chunk kernel.
#include "efla_chain_bf16.hpp"
#include "efla_chunk_fwd.hpp"

namespace efla {
hipError_t launch_chunk_fwd_bf16(const ChunkArgs& a, hipStream_t stream) {
    if (a.d_k >= 32 && a.chunk == 64) return launch_chain_ut_bf16(a, stream);
    return launch_chunk_e<bf16>(a, stream);
}
}  // namespace efla
