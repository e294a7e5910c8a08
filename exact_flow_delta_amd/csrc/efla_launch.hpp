// efla_launch.hpp -- internal launchers behind the C ABI (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "efla.h"

namespace efla {

// Exact gate for n tokens of d_k keys.
hipError_t launch_alpha(const void* k, efla_dtype dt, const float* beta, float* alpha, int64_t n, int d_k,
                        hipStream_t stream);

// One decode token for NH independent states (in place).
hipError_t launch_recurrent_step(const void* q, const void* k, const void* v, const float* beta, efla_dtype dt,
                                 float* state, void* o, int64_t NH, int d_k, int d_v, hipStream_t stream);

// Chunked forward.  One workgroup per (batch*head, d_v slab of `dvs` columns); every workgroup
// walks the chunks of its sequence in order, carrying its slab of the state.
struct ChunkArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* beta;
    void* o;
    const float* s0;   // may be null
    float* sf;         // may be null
    int BH, L, d_k, d_v, chunk, dvs;
};

// LDS bytes of the chunk kernel for these sizes, or -1 when no kernel is built for them.
int chunk_lds_bytes(efla_dtype dt, int d_k, int chunk, int dvs);
// Workgroups of the chunk kernel (including the XCD padding of the grid).
int64_t chunk_grid(int BH, int d_v, int dvs);

hipError_t launch_chunk_fwd_f32(const ChunkArgs& a, hipStream_t stream);
hipError_t launch_chunk_fwd_bf16(const ChunkArgs& a, hipStream_t stream);

}  // namespace efla
