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
    // segment-parallel scan (all zero: the whole sequence in one pass)
    int nseg;          // segments (grid y); 0 or 1: one
    int seg_chunks;    // chunks per segment; 0: all
    int aug;           // 1: d_k transition columns after the d_v value columns (zero values, identity start)
    int sf_all;        // 1: final state of every segment into sf [BH][nseg][d_k][d_v (+ d_k)]; 0: the last's, [BH][d_k][d_v]
};

// The segment parameters a state-pass kernel receives.  s0, when given, holds one initial state per
// (head, segment): s0[((bh * nseg + seg) * d_k + row) * d_v + col].
struct ChainSeg {
    int seg_chunks;   // chunks per segment (>= 1)
    int nslab_v;      // slabs of value columns; slabs from here on are transition slabs
    int ld_sf;        // row stride of sf when sf_all
    int sf_all;
};
inline ChainSeg chain_seg(const SplitArgs& a, int dk, int c, int dvs) {
    const int nc = (a.L + c - 1) / c;
    ChainSeg sg;
    sg.seg_chunks = a.seg_chunks > 0 ? a.seg_chunks : (nc > 0 ? nc : 1);
    sg.nslab_v = a.d_v / dvs;
    sg.ld_sf = a.d_v + (a.aug ? dk : 0);
    sg.sf_all = a.sf_all;
    return sg;
}

// elements of the UT output per chunk: (chunk/16)(chunk/16 + 1)/2 blocks of 256
inline int64_t ut_block_elems(int chunk) { return (int64_t)(chunk / 16) * (chunk / 16 + 1) / 2 * 256; }
// LDS bytes of the state-pass kernel, or -1 when none is built for these sizes
int chain_lds_bytes(efla_dtype dt, int d_k, int chunk, int dvs);
// LDS bytes of the UT kernel
int ut_lds_bytes(efla_dtype dt, int d_k, int chunk);

// with_ut = false: a.tw already holds the UT output; only the state pass is launched
hipError_t launch_split_fwd_f32(const SplitArgs& a, bool with_ut, hipStream_t stream);
hipError_t launch_split_fwd_bf16(const SplitArgs& a, bool with_ut, hipStream_t stream);
// Initial states of the segments of the segment-parallel forward (efla_seg_scan.hip): S_in[0] = s0 (or 0),
// S_in[g+1] = M_g S_in[g] + S_g(0) from seg_states [BH][nseg][d_k][d_v + d_k] = [S_g(0) | M_g]; s_in
// [BH][nseg][d_k][d_v].
hipError_t launch_seg_scan(const float* seg_states, const float* s0, float* s_in, int BH, int nseg, int d_k, int d_v,
                           hipStream_t stream);

hipError_t launch_ut_f32(const void* k, const float* beta, void* tw, int BH, int L, int d_k, int chunk, int gate,
                         hipStream_t stream);
hipError_t launch_ut_bf16(const void* k, const float* beta, void* tw, int BH, int L, int d_k, int chunk, int gate,
                          hipStream_t stream);

}  // namespace efla
