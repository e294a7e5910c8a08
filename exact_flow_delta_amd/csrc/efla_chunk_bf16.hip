// efla_chunk_bf16.hip -- bf16-input instantiations of the fused chunked forward.
#include "efla_chunk_fwd.hpp"

namespace efla {
hipError_t launch_chunk_fwd_bf16(const ChunkArgs& a, hipStream_t stream) { return launch_chunk_e<bf16>(a, stream); }
}  // namespace efla
