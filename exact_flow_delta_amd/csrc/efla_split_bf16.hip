// efla_split_bf16.hip -- bf16-input instantiations of the two-launch chunked forward.
#include "efla_chain_bf16.hpp"
#include "efla_chunk_split.hpp"

namespace efla {
hipError_t launch_split_fwd_bf16(const SplitArgs& a, bool with_ut, hipStream_t stream) {
    return launch_split_e<bf16>(a, with_ut, stream);
}
hipError_t launch_ut_bf16(const void* k, const float* beta, void* tw, int BH, int L, int d_k, int chunk, int gate,
                          hipStream_t stream, void* tt, const TokLayout* layout) {
    return launch_ut_e<bf16>(k, beta, tw, BH, L, d_k, chunk, gate, stream, tt, layout);
}
}  // namespace efla
