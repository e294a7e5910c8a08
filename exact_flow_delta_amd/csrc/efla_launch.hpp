// efla_launch.hpp -- internal launchers behind the C ABI (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "efla.h"

namespace efla {

// Exact gate for n tokens of d_k keys.
// gate: 0 for the exact coefficient, p in 1 .. 16 for the p-th order Runge-Kutta one (gate_alpha)
hipError_t launch_alpha(const void* k, efla_dtype dt, const float* beta, float* alpha, int64_t n, int d_k, int gate,
                        hipStream_t stream);

// One decode token for NH independent states (in place).
hipError_t launch_recurrent_step(const void* q, const void* k, const void* v, const float* beta, efla_dtype dt,
                                 float* state, void* o, int64_t NH, int d_k, int d_v, int gate, hipStream_t stream);

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
    int gate;          // 0: exact coefficient; p: p-th order Runge-Kutta (gate_alpha)
};

// LDS bytes of the chunk kernel for these sizes, or -1 when no kernel is built for them.
int chunk_lds_bytes(efla_dtype dt, int d_k, int chunk, int dvs);
// Workgroups of the chunk kernel (including the XCD padding of the grid).
int64_t chunk_grid(int BH, int d_v, int dvs);

hipError_t launch_chunk_fwd_f32(const ChunkArgs& a, hipStream_t stream);
hipError_t launch_chunk_fwd_bf16(const ChunkArgs& a, hipStream_t stream);

// Two-launch chunked forward: the UT transform of every (batch*head, chunk) into the workspace `tw`,
// then the state pass (one workgroup per (batch*head, d_v slab)) reading it.
struct SplitArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* beta;
    void* o;
    const float* s0;   // may be null
    float* sf;         // may be null
    void* tw;          // T diag(alpha) blocks, BH * ceil(L / chunk) * ut_block_elems(chunk) elements
    int BH, L, d_k, d_v, chunk, dvs;
    int gate;          // 0: exact coefficient; p: p-th order Runge-Kutta (gate_alpha)
};

// elements of the UT output per chunk: (chunk/16)(chunk/16 + 1)/2 blocks of 256
inline int64_t ut_block_elems(int chunk) { return (int64_t)(chunk / 16) * (chunk / 16 + 1) / 2 * 256; }
// LDS bytes of the state-pass kernel, or -1 when none is built for these sizes
int chain_lds_bytes(efla_dtype dt, int d_k, int chunk, int dvs);
// LDS bytes of the UT kernel
int ut_lds_bytes(efla_dtype dt, int d_k, int chunk);

// with_ut = false: a.tw already holds the UT output; only the state pass is launched
hipError_t launch_split_fwd_f32(const SplitArgs& a, bool with_ut, hipStream_t stream);
hipError_t launch_split_fwd_bf16(const SplitArgs& a, bool with_ut, hipStream_t stream);
hipError_t launch_ut_f32(const void* k, const float* beta, void* tw, int BH, int L, int d_k, int chunk, int gate,
                         hipStream_t stream);
hipError_t launch_ut_bf16(const void* k, const float* beta, void* tw, int BH, int L, int d_k, int chunk, int gate,
                          hipStream_t stream);

}  // namespace efla
