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

struct TokLayout;

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
    const TokLayout* layout = nullptr;   // null: contiguous [B,H,L,d] (the one-launch kernel takes any other)
};

// LDS bytes of the chunk kernel for these sizes, or -1 when no kernel is built for them.
int chunk_lds_bytes(efla_dtype dt, int d_k, int chunk, int dvs);
// Workgroups of the chunk kernel (including the XCD padding of the grid).
int64_t chunk_grid(int BH, int d_v, int dvs);

hipError_t launch_chunk_fwd_f32(const ChunkArgs& a, hipStream_t stream);
hipError_t launch_chunk_fwd_bf16(const ChunkArgs& a, hipStream_t stream);

// Where the tokens of each (batch, head) live.  Element strides (batch, head, token) per tensor, the feature
// dimension contiguous; with cu_seqlens the batch entries are packed sequences: sequence b holds tokens
// cu_seqlens[b] .. cu_seqlens[b+1]-1 of the token dimension, batch strides unused, and head h of it has its
// chunks from chunk h * TC + cu_chunks[b] of the UT workspace, TC = cu_chunks[nseq] (head-major order).  The
// arrays are made on the device by launch_varlen_prep from the caller's offsets: cu_seqlens here is their
// sanitised copy (clamped to [0, L] and non-decreasing, so the sequences are disjoint and hold at most L
// tokens together), cu_chunks the prefix of the sequences' chunk counts (TC <= ceil(L / C) + nseq), and
// chunk_seq[j] the sequence of chunk j < TC of a head.  Without cu_seqlens every sequence has L tokens and
// (batch b, head h) = bh starts at chunk bh * ceil(L / C).
struct TokLayout {
    int64_t q_b, q_h, q_t, k_b, k_h, k_t, v_b, v_h, v_t, o_b, o_h, o_t, be_b, be_h, be_t;
    const int* cu_seqlens;   // device, nseq + 1 sanitised offsets, or null
    const int* cu_chunks;    // device, nseq + 1 entries, or null
    const int* chunk_seq;    // device, cu_chunks[nseq] entries, or null
    int H;
    int nseq;
};

// contiguous [B,H,L,d] q, k, v, o and [B,H,L] beta
inline TokLayout contiguous_layout(int H, int L, int d_k, int d_v) {
    TokLayout t{};
    t.q_t = t.k_t = d_k;
    t.q_h = t.k_h = (int64_t)L * d_k;
    t.q_b = t.k_b = (int64_t)H * L * d_k;
    t.v_t = t.o_t = d_v;
    t.v_h = t.o_h = (int64_t)L * d_v;
    t.v_b = t.o_b = (int64_t)H * L * d_v;
    t.be_t = 1;
    t.be_h = L;
    t.be_b = (int64_t)H * L;
    t.H = H;
    return t;
}

// One (batch, head)'s tokens: element offsets of its token 0 in q, k, v, o, beta, its length and its first chunk
// in the UT workspace.
struct SeqView {
    int64_t q0, k0, v0, o0, be0;
    int len;
    int chunk0;
};
// VL: packed sequences (ly.cu_seqlens set); the kernels that call these helpers inside their loops take it as a
// template argument so that the fixed-length form stays free of branches.
template <bool VL>
__device__ inline SeqView seq_view_t(const TokLayout& ly, int bh, int L, int C) {
    const int b = bh / ly.H, h = bh - b * ly.H;
    SeqView s;
    if constexpr (VL) {
        const int t0 = ly.cu_seqlens[b], t1 = ly.cu_seqlens[b + 1];
        s.len = t1 - t0;
        s.q0 = h * ly.q_h + (int64_t)t0 * ly.q_t;
        s.k0 = h * ly.k_h + (int64_t)t0 * ly.k_t;
        s.v0 = h * ly.v_h + (int64_t)t0 * ly.v_t;
        s.o0 = h * ly.o_h + (int64_t)t0 * ly.o_t;
        s.be0 = h * ly.be_h + (int64_t)t0 * ly.be_t;
        s.chunk0 = h * ly.cu_chunks[ly.nseq] + ly.cu_chunks[b];
    } else {
        s.len = L;
        s.q0 = b * ly.q_b + h * ly.q_h;
        s.k0 = b * ly.k_b + h * ly.k_h;
        s.v0 = b * ly.v_b + h * ly.v_h;
        s.o0 = b * ly.o_b + h * ly.o_h;
        s.be0 = b * ly.be_b + h * ly.be_h;
        s.chunk0 = bh * ((L + C - 1) / C);
    }
    return s;
}
__device__ inline SeqView seq_view(const TokLayout& ly, int bh, int L, int C) {
    return ly.cu_seqlens ? seq_view_t<true>(ly, bh, L, C) : seq_view_t<false>(ly, bh, L, C);
}

// Chunk u of the UT workspace -> (batch*head, chunk within that sequence); u < ut_chunks(ly, ...).
template <bool VL>
__device__ inline void chunk_of(const TokLayout& ly, int u, int NC, int& bh, int& c) {
    if constexpr (VL) {
        const int tc = ly.cu_chunks[ly.nseq];   // chunks of one head (> 0 whenever u is a chunk)
        const int h = u / tc, j = u - h * tc;
        const int b = ly.chunk_seq[j];
        bh = b * ly.H + h;
        c = j - ly.cu_chunks[b];
    } else {
        bh = u / NC;
        c = u - bh * NC;
    }
}

// Chunks of the UT workspace: BH * ceil(L / C), or with packed sequences H times their total (device read).
template <bool VL>
__device__ inline int ut_chunks(const TokLayout& ly, int BH, int NC) {
    if constexpr (VL) return ly.H * ly.cu_chunks[ly.nseq]; else return BH * NC;
}

// From the caller's offsets cu_seqlens[0..nseq]: cu_tok[b] = max over b' <= b of clamp(cu_seqlens[b'], 0, L),
// cu_chunks[b] = sum over b' < b of ceil((cu_tok[b'+1] - cu_tok[b']) / C), and chunk_seq[j] = the b with
// cu_chunks[b] <= j < cu_chunks[b+1] for j < cu_chunks[nseq] (which is at most max_chunks).  Two launches.
hipError_t launch_varlen_prep(const int* cu_seqlens, int* cu_tok, int* cu_chunks, int* chunk_seq, int nseq, int L,
                              int C, int max_chunks, hipStream_t stream);

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
    const TokLayout* layout;   // null: contiguous [B,H,L,d]
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

// layout: null for contiguous [B,H,L,d_k] keys and [B,H,L] betas, else the tensors' strides (and packed sequences)
hipError_t launch_ut_f32(const void* k, const float* beta, void* tw, int BH, int L, int d_k, int chunk, int gate,
                         hipStream_t stream, const TokLayout* layout = nullptr);
// tt (optional; d_k >= 32): also T^T of every chunk as a row-major chunk x chunk bf16 matrix, for the backward pass
hipError_t launch_ut_bf16(const void* k, const float* beta, void* tw, int BH, int L, int d_k, int chunk, int gate,
                          hipStream_t stream, void* tt = nullptr, const TokLayout* layout = nullptr);

}  // namespace efla
