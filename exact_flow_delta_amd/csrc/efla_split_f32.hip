// efla_split_f32.hip -- fp32-input instantiations of the two-launch chunked forward.
#include "efla_chunk_split.hpp"

namespace efla {
hipError_t launch_split_fwd_f32(const SplitArgs& a, bool with_ut, hipStream_t stream) {
    return launch_split_e<float>(a, with_ut, stream);
}
hipError_t launch_ut_f32(const void* k, const float* beta, void* tw, int BH, int L, int d_k, int chunk, int gate,
                         hipStream_t stream, const TokLayout* layout) {
    return launch_ut_e<float>(k, beta, tw, BH, L, d_k, chunk, gate, stream, nullptr, layout);
}
}  // namespace efla
