// efla_chunk_f32.hip -- fp32-input instantiations of the fused chunked forward.
#include "efla_chunk_fwd.hpp"

namespace efla {
hipError_t launch_chunk_fwd_f32(const ChunkArgs& a, hipStream_t stream) { return launch_chunk_e<float>(a, stream); }
}  // namespace efla
