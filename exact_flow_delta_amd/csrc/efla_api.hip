// efla_api.hip -- the exported C ABI of libefla.so: argument checks, launch planning, error mapping.
// Every check runs before anything is enqueued; on error no output is touched.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "efla.h"
#include "efla_bwd.hpp"
#include "efla_chain_bf16.hpp"
#include "efla_chunk_fwd.hpp"
#include "efla_chunk_split.hpp"
#include "efla_launch.hpp"

namespace {

thread_local char g_last_error[512] = "";

efla_status fail_hip(hipError_t e, const char* where) {
    snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%s)", where, hipGetErrorName(e), hipGetErrorString(e));
    return EFLA_ERR_HIP;
}

bool valid_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool valid_chunk(int c) { return c == 16 || c == 32 || c == 64; }
bool valid_dtype(efla_dtype dt) { return dt == EFLA_F32 || dt == EFLA_BF16; }
bool valid_gate(int gate) { return gate >= EFLA_GATE_EXACT && gate <= EFLA_GATE_MAX_ORDER; }
size_t esize(efla_dtype dt) { return dt == EFLA_BF16 ? 2 : 4; }
bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// do [a, a+na) and [b, b+nb) share a byte?  (null or empty ranges never overlap)
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
    return pa < pb + nb && pb < pa + na;
}

efla_status device_present() {
    int n = 0;
    const hipError_t e = hipGetDeviceCount(&n);
    if (e != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        snprintf(g_last_error, sizeof(g_last_error), "no HIP device visible (%s)",
                 e != hipSuccess ? hipGetErrorName(e) : "0 devices");
        return EFLA_ERR_NO_DEVICE;
    }
    return EFLA_OK;
}

int split_lds_bytes(efla_dtype dt, int d_k, int chunk, int dvs) {
    const int b = dt == EFLA_BF16 ? efla::chain_layout_bytes<2>(d_k, chunk, dvs)
                                  : efla::chain_layout_bytes<4>(d_k, chunk, dvs);
    const int u = dt == EFLA_BF16 ? efla::ut_layout_bytes<2>(d_k, chunk) : efla::ut_layout_bytes<4>(d_k, chunk);
    return (b <= efla::kMaxLdsBytes && u <= efla::kMaxLdsBytes) ? b : -1;
}

// LDS of the one-launch forward: bf16 with d_k >= 32 and 64-token chunks runs the state pass with its own UT
// wave, everything else the fused chunk kernel
int lds_bytes(efla_dtype dt, int d_k, int chunk, int dvs) {
    const int b = dt == EFLA_BF16 && d_k >= 32 && chunk == 64 ? efla::chain_ut_bf16_bytes(d_k, dvs)
                  : dt == EFLA_BF16                           ? efla::chunk_layout_bytes<2>(d_k, chunk, dvs)
                                                              : efla::chunk_layout_bytes<4>(d_k, chunk, dvs);
    return b <= efla::kMaxLdsBytes ? b : -1;
}

// Slab width: the widest (fewest waves re-reading the chunk data) that still gives the GPU enough
// workgroups; narrower when B*H is small so that more compute units carry a slab.
int kernel_lds(bool split, efla_dtype dt, int d_k, int chunk, int dvs) {
    return split ? split_lds_bytes(dt, d_k, chunk, dvs) : lds_bytes(dt, d_k, chunk, dvs);
}

int auto_slab(bool split, int64_t BH, int d_k, int d_v, int chunk, efla_dtype dt) {
    int dvs = d_v < 64 ? d_v : 64;
    while (dvs > 16 && BH * (d_v / dvs) < 256) dvs /= 2;
    while (dvs > 16 && kernel_lds(split, dt, d_k, chunk, dvs) < 0) dvs /= 2;
    return dvs;
}

efla_status check_chunk_sizes(bool split, int B, int H, int L, int d_k, int d_v, int chunk, efla_dtype dt,
                              int dv_slab, int* dvs_out) {
    if (!valid_dtype(dt)) return EFLA_ERR_INVALID_ARG;
    if (B < 0 || H < 0 || L < 0) return EFLA_ERR_INVALID_ARG;
    if ((int64_t)B * H > INT32_MAX) return EFLA_ERR_INVALID_ARG;
    if (!valid_dim(d_k) || !valid_dim(d_v) || !valid_chunk(chunk)) return EFLA_ERR_UNSUPPORTED;
    if (dv_slab != 0 && dv_slab != 16 && dv_slab != 32 && dv_slab != 64) return EFLA_ERR_UNSUPPORTED;
    if (dv_slab != 0 && (dv_slab > d_v || d_v % dv_slab != 0)) return EFLA_ERR_UNSUPPORTED;
    const int dvs = dv_slab ? dv_slab : auto_slab(split, (int64_t)B * H, d_k, d_v, chunk, dt);
    if (kernel_lds(split, dt, d_k, chunk, dvs) < 0) return EFLA_ERR_UNSUPPORTED;
    if (efla::chunk_grid((int)((int64_t)B * H), d_v, dvs) > INT32_MAX) return EFLA_ERR_INVALID_ARG;
    // the UT launch has one workgroup per (batch*head, chunk)
    if (split && (int64_t)B * H * ((L + chunk - 1) / chunk) > INT32_MAX) return EFLA_ERR_INVALID_ARG;
    *dvs_out = dvs;
    return EFLA_OK;
}

// pointer checks shared by the chunked-forward entry points (sizes already validated); beta is
// required unless need_beta is false (the state pass alone does not read it)
efla_status check_fwd_buffers(const void* q, const void* k, const void* v, const float* beta, efla_dtype dtype,
                              const void* o, const float* initial_state, const float* final_state, int64_t BH, int L,
                              int d_k, int d_v, bool need_beta = true) {
    const size_t es = esize(dtype);
    const size_t nq = (size_t)BH * L * d_k * es, nv = (size_t)BH * L * d_v * es, nb = (size_t)BH * L * 4;
    const size_t ns = (size_t)BH * d_k * d_v * 4;
    if (L > 0 && BH > 0) {
        if (!q || !k || !v || (need_beta && !beta) || !o) return EFLA_ERR_INVALID_ARG;
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(beta, 4))
            return EFLA_ERR_INVALID_ARG;
    }
    if ((initial_state && !aligned(initial_state, 16)) || (final_state && !aligned(final_state, 16)))
        return EFLA_ERR_INVALID_ARG;
    // o overlaps nothing; the final state overlaps no input; initial and final state are identical or disjoint
    if (overlap(o, nv, q, nq) || overlap(o, nv, k, nq) || overlap(o, nv, v, nv) || overlap(o, nv, beta, nb) ||
        overlap(o, nv, initial_state, ns) || overlap(o, nv, final_state, ns))
        return EFLA_ERR_INVALID_ARG;
    if (overlap(final_state, ns, q, nq) || overlap(final_state, ns, k, nq) || overlap(final_state, ns, v, nv) ||
        overlap(final_state, ns, beta, nb))
        return EFLA_ERR_INVALID_ARG;
    if ((const void*)initial_state != (const void*)final_state && overlap(initial_state, ns, final_state, ns))
        return EFLA_ERR_INVALID_ARG;
    return EFLA_OK;
}

size_t ut_bytes(int64_t BH, int L, int chunk, efla_dtype dt) {
    return (size_t)BH * (size_t)((L + chunk - 1) / chunk) * (size_t)efla::ut_block_elems(chunk) * esize(dt);
}

size_t round_up_256(size_t n) { return (n + 255) / 256 * 256; }

// The segment-parallel forward's launch shape and workspace: a slab width dividing d_v and d_k, the number of
// segments (0 asked = automatic: as many as keep the second pass within one workgroup per compute unit, with at
// least 16 chunks per segment) and the chunks per segment; workspace = UT output, then the per-segment states
// [S_g(0) | M_g] (fp32, d_k x (d_v + d_k)), then the segments' initial states (fp32, d_k x d_v).
struct ScanPlan {
    int dvs, nseg, seg_chunks;
    int dvs1;   // slab width of the first pass (transition columns included)
    size_t off_states, off_sin, total;
};

efla_status scan_plan(int B, int H, int L, int d_k, int d_v, int chunk, efla_dtype dt, int segments, ScanPlan* p) {
    if (!valid_dtype(dt) || B < 0 || H < 0 || L < 0 || segments < 0) return EFLA_ERR_INVALID_ARG;
    if (!valid_dim(d_k) || !valid_dim(d_v) || !valid_chunk(chunk)) return EFLA_ERR_UNSUPPORTED;
    const int64_t BH = (int64_t)B * H;
    const int64_t NC = (L + chunk - 1) / chunk;
    if (BH > INT32_MAX || BH * NC > INT32_MAX) return EFLA_ERR_INVALID_ARG;
    int dvs = 64;
    while (dvs > 16 && (dvs > d_v || dvs > d_k || split_lds_bytes(dt, d_k, chunk, dvs) < 0)) dvs /= 2;
    if (split_lds_bytes(dt, d_k, chunk, dvs) < 0) return EFLA_ERR_UNSUPPORTED;
    if (efla::chunk_grid((int)BH, d_v + d_k, dvs) > INT32_MAX) return EFLA_ERR_INVALID_ARG;
    int64_t G = segments;
    if (G == 0) {
        // Segments pay for a second state pass; they win only when one segment's grid leaves most of the
        // 256 compute units idle.  Measured (d 128, bf16): 16 heads x 65,536 tokens best at 8 segments, 32 x 16,384
        // and 32 x 32,768 at 4; 64 heads x 8,192 tokens is faster unsegmented (2 segments: 20 % slower).
        const int64_t per_seg = BH * (d_v / dvs);   // second-pass workgroups of one segment
        G = 1;
        if (per_seg <= 64)
            while (per_seg * 2 * G <= 256 && NC >= 32 * G) G *= 2;
    }
    if (G > NC) G = NC > 0 ? NC : 1;
    if (G > 65535) return EFLA_ERR_INVALID_ARG;
    const int64_t sc = NC > 0 ? (NC + G - 1) / G : 1;
    G = NC > 0 ? (NC + sc - 1) / sc : 1;   // no empty segment
    p->dvs = dvs;
    // the first pass carries d_v + d_k columns without outputs: at d_k = d_v = 128 (bf16, 64-token chunks) one slab
    // of 128 columns per workgroup (eight compute waves sharing each chunk's K and Ta tiles) while that still gives
    // every compute unit a workgroup
    p->dvs1 = dvs;
    if (dt == EFLA_BF16 && d_k == 128 && d_v == 128 && chunk == 64 && BH * G * 2 >= 256) p->dvs1 = 128;
    p->nseg = (int)G;
    p->seg_chunks = (int)sc;
    const size_t ut = round_up_256(ut_bytes(BH, L, chunk, dt));
    const size_t states = G > 1 ? round_up_256((size_t)BH * G * d_k * (d_v + d_k) * 4) : 0;
    const size_t sin = G > 1 ? round_up_256((size_t)BH * G * d_k * d_v * 4) : 0;
    p->off_states = ut;
    p->off_sin = ut + states;
    p->total = ut + states + sin;
    return EFLA_OK;
}

// The split forward (one segment: UT transform, then the state pass) or the segment-parallel one: UT transform
// of every chunk; pass 1 over every segment from a zero state with the transition columns; the scan of the
// segments' initial states; pass 2 over every segment from its initial state, writing the outputs and the last
// segment's final state.  a.tw is the workspace base (the UT output).
hipError_t run_fwd(bool bf, const efla::SplitArgs& a, const ScanPlan& p, char* ws, hipStream_t s) {
    auto chain = [&](const efla::SplitArgs& x, bool with_ut) {
        return bf ? efla::launch_split_fwd_bf16(x, with_ut, s) : efla::launch_split_fwd_f32(x, with_ut, s);
    };
    if (p.nseg == 1) return chain(a, true);
    float* states = reinterpret_cast<float*>(ws + p.off_states);
    float* s_in = reinterpret_cast<float*>(ws + p.off_sin);
    efla::SplitArgs a1 = a;
    a1.o = nullptr;
    a1.s0 = nullptr;
    a1.sf = states;
    a1.nseg = p.nseg;
    a1.seg_chunks = p.seg_chunks;
    a1.aug = 1;
    a1.sf_all = 1;
    a1.dvs = p.dvs1;
    hipError_t e = chain(a1, true);
    if (e == hipSuccess) e = efla::launch_seg_scan(states, a.s0, s_in, a.BH, p.nseg, a.d_k, a.d_v, s);
    efla::SplitArgs a2 = a;
    a2.s0 = s_in;
    a2.nseg = p.nseg;
    a2.seg_chunks = p.seg_chunks;
    if (e == hipSuccess) e = chain(a2, false);
    return e;
}

}  // namespace

namespace efla {
int chain_lds_bytes(efla_dtype dt, int d_k, int chunk, int dvs) { return split_lds_bytes(dt, d_k, chunk, dvs); }
int ut_lds_bytes(efla_dtype dt, int d_k, int chunk) {
    return dt == EFLA_BF16 ? ut_layout_bytes<2>(d_k, chunk) : ut_layout_bytes<4>(d_k, chunk);
}
}  // namespace efla

namespace efla {
int chunk_lds_bytes(efla_dtype dt, int d_k, int chunk, int dvs) { return lds_bytes(dt, d_k, chunk, dvs); }
int64_t chunk_grid(int BH, int d_v, int dvs) { return (int64_t)((BH + 7) / 8) * 8 * (d_v / dvs); }
}  // namespace efla

extern "C" {

int efla_version(void) { return 20000; }

const char* efla_status_string(efla_status s) {
    switch (s) {
        case EFLA_OK: return "EFLA_OK";
        case EFLA_ERR_INVALID_ARG: return "EFLA_ERR_INVALID_ARG: invalid argument";
        case EFLA_ERR_UNSUPPORTED: return "EFLA_ERR_UNSUPPORTED: size or type combination not built";
        case EFLA_ERR_WORKSPACE: return "EFLA_ERR_WORKSPACE: workspace missing, misaligned or too small";
        case EFLA_ERR_NO_DEVICE: return "EFLA_ERR_NO_DEVICE: no HIP device";
        case EFLA_ERR_HIP: return "EFLA_ERR_HIP: HIP runtime error";
        default: break;
    }
    return "EFLA: unknown status";
}

const char* efla_last_error(void) { return g_last_error; }

efla_status efla_alpha_gate(const void* k, efla_dtype k_dtype, const float* beta, float* alpha, int64_t n_tokens,
                            int d_k, int gate, void* stream) {
    if (!valid_dtype(k_dtype) || n_tokens < 0 || !valid_gate(gate)) return EFLA_ERR_INVALID_ARG;
    if (!valid_dim(d_k)) return EFLA_ERR_UNSUPPORTED;
    if (n_tokens == 0) return EFLA_OK;
    if (!k || !beta || !alpha) return EFLA_ERR_INVALID_ARG;
    if (!aligned(k, 16) || !aligned(beta, 4) || !aligned(alpha, 4)) return EFLA_ERR_INVALID_ARG;
    const size_t nk = (size_t)n_tokens * d_k * esize(k_dtype), nb = (size_t)n_tokens * 4;
    if (overlap(alpha, nb, k, nk) || overlap(alpha, nb, beta, nb)) return EFLA_ERR_INVALID_ARG;
    // keys per workgroup is at least 8 (fp32, d_k = 128)
    if (n_tokens / 8 + 1 > INT32_MAX) return EFLA_ERR_INVALID_ARG;
    efla_status st = device_present();
    if (st != EFLA_OK) return st;
    const hipError_t e = efla::launch_alpha(k, k_dtype, beta, alpha, n_tokens, d_k, gate, (hipStream_t)stream);
    return e == hipSuccess ? EFLA_OK : fail_hip(e, "efla_alpha launch");
}

efla_status efla_alpha(const void* k, efla_dtype k_dtype, const float* beta, float* alpha, int64_t n_tokens, int d_k,
                       void* stream) {
    return efla_alpha_gate(k, k_dtype, beta, alpha, n_tokens, d_k, EFLA_GATE_EXACT, stream);
}

efla_status efla_chunk_fwd_plan(int B, int H, int L, int d_k, int d_v, int chunk, efla_dtype dtype, int dv_slab,
                                int* workgroups, int* slab_width, int* lds) {
    int dvs = 0;
    const efla_status st = check_chunk_sizes(false, B, H, L, d_k, d_v, chunk, dtype, dv_slab, &dvs);
    if (st != EFLA_OK) return st;
    if (workgroups) *workgroups = (int)efla::chunk_grid(B * H, d_v, dvs);
    if (slab_width) *slab_width = dvs;
    if (lds) *lds = lds_bytes(dtype, d_k, chunk, dvs);
    return EFLA_OK;
}

efla_status efla_chunk_fwd_slab_gate(const void* q, const void* k, const void* v, const float* beta, efla_dtype dtype,
                                     void* o, const float* initial_state, float* final_state, int B, int H, int L,
                                     int d_k, int d_v, int chunk, int dv_slab, int gate, void* stream) {
    if (!valid_gate(gate)) return EFLA_ERR_INVALID_ARG;
    int dvs = 0;
    efla_status st = check_chunk_sizes(false, B, H, L, d_k, d_v, chunk, dtype, dv_slab, &dvs);
    if (st != EFLA_OK) return st;
    const int64_t BH = (int64_t)B * H;
    st = check_fwd_buffers(q, k, v, beta, dtype, o, initial_state, final_state, BH, L, d_k, d_v);
    if (st != EFLA_OK) return st;
    if (BH == 0) return EFLA_OK;
    if (L == 0 && !final_state) return EFLA_OK;
    st = device_present();
    if (st != EFLA_OK) return st;
    efla::ChunkArgs a{q, k, v, beta, o, initial_state, final_state, (int)BH, L, d_k, d_v, chunk, dvs, gate};
    const hipError_t e = dtype == EFLA_BF16 ? efla::launch_chunk_fwd_bf16(a, (hipStream_t)stream)
                                            : efla::launch_chunk_fwd_f32(a, (hipStream_t)stream);
    return e == hipSuccess ? EFLA_OK : fail_hip(e, "efla_chunk_fwd launch");
}

efla_status efla_chunk_fwd_slab(const void* q, const void* k, const void* v, const float* beta, efla_dtype dtype,
                                void* o, const float* initial_state, float* final_state, int B, int H, int L, int d_k,
                                int d_v, int chunk, int dv_slab, void* stream) {
    return efla_chunk_fwd_slab_gate(q, k, v, beta, dtype, o, initial_state, final_state, B, H, L, d_k, d_v, chunk,
                                    dv_slab, EFLA_GATE_EXACT, stream);
}


efla_status efla_chunk_split_workspace_size(int B, int H, int L, int chunk, efla_dtype dtype, size_t* bytes) {
    if (!valid_dtype(dtype) || B < 0 || H < 0 || L < 0 || !bytes) return EFLA_ERR_INVALID_ARG;
    if (!valid_chunk(chunk)) return EFLA_ERR_UNSUPPORTED;
    *bytes = ut_bytes((int64_t)B * H, L, chunk, dtype);
    return EFLA_OK;
}

efla_status efla_ut_transform_gate(const void* k, const float* beta, efla_dtype dtype, void* t_out,
                                   size_t t_out_bytes, int B, int H, int L, int d_k, int chunk, int gate, void* stream) {
    if (!valid_dtype(dtype) || B < 0 || H < 0 || L < 0 || !valid_gate(gate)) return EFLA_ERR_INVALID_ARG;
    if (!valid_dim(d_k) || !valid_chunk(chunk)) return EFLA_ERR_UNSUPPORTED;
    const int64_t BH = (int64_t)B * H;
    if (BH > INT32_MAX || BH * ((L + chunk - 1) / chunk) > INT32_MAX) return EFLA_ERR_INVALID_ARG;
    if (BH == 0 || L == 0) return EFLA_OK;
    if (!k || !beta || !aligned(k, 16) || !aligned(beta, 4)) return EFLA_ERR_INVALID_ARG;
    const size_t need = ut_bytes(BH, L, chunk, dtype);
    if (!t_out || !aligned(t_out, 16) || t_out_bytes < need) return EFLA_ERR_WORKSPACE;
    const size_t nk = (size_t)BH * L * d_k * esize(dtype), nb = (size_t)BH * L * 4;
    if (overlap(t_out, need, k, nk) || overlap(t_out, need, beta, nb)) return EFLA_ERR_INVALID_ARG;
    const efla_status st = device_present();
    if (st != EFLA_OK) return st;
    const hipError_t e = dtype == EFLA_BF16
                             ? efla::launch_ut_bf16(k, beta, t_out, (int)BH, L, d_k, chunk, gate, (hipStream_t)stream)
                             : efla::launch_ut_f32(k, beta, t_out, (int)BH, L, d_k, chunk, gate, (hipStream_t)stream);
    return e == hipSuccess ? EFLA_OK : fail_hip(e, "efla_ut_transform launch");
}

efla_status efla_ut_transform(const void* k, const float* beta, efla_dtype dtype, void* t_out, size_t t_out_bytes,
                              int B, int H, int L, int d_k, int chunk, void* stream) {
    return efla_ut_transform_gate(k, beta, dtype, t_out, t_out_bytes, B, H, L, d_k, chunk, EFLA_GATE_EXACT, stream);
}

efla_status efla_chunk_fwd_split_plan(int B, int H, int L, int d_k, int d_v, int chunk, efla_dtype dtype, int dv_slab,
                                      int* workgroups, int* slab_width, int* lds) {
    int dvs = 0;
    const efla_status st = check_chunk_sizes(true, B, H, L, d_k, d_v, chunk, dtype, dv_slab, &dvs);
    if (st != EFLA_OK) return st;
    if (workgroups) *workgroups = (int)efla::chunk_grid(B * H, d_v, dvs);
    if (slab_width) *slab_width = dvs;
    if (lds) *lds = split_lds_bytes(dtype, d_k, chunk, dvs);
    return EFLA_OK;
}

namespace {
efla_status split_entry(bool with_ut, const void* q, const void* k, const void* v, const float* beta,
                        efla_dtype dtype, void* o, const float* initial_state, float* final_state, int B, int H, int L,
                        int d_k, int d_v, int chunk, int dv_slab, int gate, void* tw, size_t tw_bytes, void* stream) {
    if (!valid_gate(gate)) return EFLA_ERR_INVALID_ARG;
    int dvs = 0;
    efla_status st = check_chunk_sizes(true, B, H, L, d_k, d_v, chunk, dtype, dv_slab, &dvs);
    if (st != EFLA_OK) return st;
    const int64_t BH = (int64_t)B * H;
    st = check_fwd_buffers(q, k, v, beta, dtype, o, initial_state, final_state, BH, L, d_k, d_v, with_ut);
    if (st != EFLA_OK) return st;
    const size_t need = ut_bytes(BH, L, chunk, dtype);
    if (need > 0) {
        if (!tw || !aligned(tw, 16) || tw_bytes < need) return EFLA_ERR_WORKSPACE;
        const size_t es = esize(dtype);
        const size_t nq = (size_t)BH * L * d_k * es, nv = (size_t)BH * L * d_v * es, nb = (size_t)BH * L * 4;
        const size_t ns = (size_t)BH * d_k * d_v * 4;
        if (overlap(tw, need, q, nq) || overlap(tw, need, k, nq) || overlap(tw, need, v, nv) ||
            overlap(tw, need, beta, nb) || overlap(tw, need, o, nv) || overlap(tw, need, initial_state, ns) ||
            overlap(tw, need, final_state, ns))
            return EFLA_ERR_INVALID_ARG;
    }
    if (BH == 0) return EFLA_OK;
    if (L == 0 && !final_state) return EFLA_OK;
    st = device_present();
    if (st != EFLA_OK) return st;
    efla::SplitArgs a{q, k, v, beta, o, initial_state, final_state, tw, (int)BH, L, d_k, d_v, chunk, dvs, gate};
    const hipError_t e = dtype == EFLA_BF16 ? efla::launch_split_fwd_bf16(a, with_ut, (hipStream_t)stream)
                                            : efla::launch_split_fwd_f32(a, with_ut, (hipStream_t)stream);
    return e == hipSuccess ? EFLA_OK : fail_hip(e, with_ut ? "efla_chunk_fwd_split launch" : "efla_chunk_state_pass launch");
}
}  // namespace

efla_status efla_chunk_fwd_split_gate(const void* q, const void* k, const void* v, const float* beta,
                                      efla_dtype dtype, void* o, const float* initial_state, float* final_state, int B,
                                      int H, int L, int d_k, int d_v, int chunk, int dv_slab, int gate,
                                      void* workspace, size_t workspace_bytes, void* stream) {
    return split_entry(true, q, k, v, beta, dtype, o, initial_state, final_state, B, H, L, d_k, d_v, chunk, dv_slab,
                       gate, workspace, workspace_bytes, stream);
}

efla_status efla_chunk_fwd_split(const void* q, const void* k, const void* v, const float* beta, efla_dtype dtype,
                                 void* o, const float* initial_state, float* final_state, int B, int H, int L, int d_k,
                                 int d_v, int chunk, int dv_slab, void* workspace, size_t workspace_bytes,
                                 void* stream) {
    return split_entry(true, q, k, v, beta, dtype, o, initial_state, final_state, B, H, L, d_k, d_v, chunk, dv_slab,
                       EFLA_GATE_EXACT, workspace, workspace_bytes, stream);
}

efla_status efla_chunk_state_pass(const void* q, const void* k, const void* v, const void* t_in, size_t t_in_bytes,
                                  efla_dtype dtype, void* o, const float* initial_state, float* final_state, int B,
                                  int H, int L, int d_k, int d_v, int chunk, int dv_slab, void* stream) {
    return split_entry(false, q, k, v, nullptr, dtype, o, initial_state, final_state, B, H, L, d_k, d_v, chunk, dv_slab,
                       EFLA_GATE_EXACT, const_cast<void*>(t_in), t_in_bytes, stream);
}

efla_status efla_chunk_scan_plan(int B, int H, int L, int d_k, int d_v, int chunk, efla_dtype dtype, int segments,
                                 int* nseg, int* seg_chunks, int* slab_width, size_t* workspace_bytes) {
    ScanPlan p;
    const efla_status st = scan_plan(B, H, L, d_k, d_v, chunk, dtype, segments, &p);
    if (st != EFLA_OK) return st;
    if (nseg) *nseg = p.nseg;
    if (seg_chunks) *seg_chunks = p.seg_chunks;
    if (slab_width) *slab_width = p.dvs;
    if (workspace_bytes) *workspace_bytes = p.total;
    return EFLA_OK;
}

efla_status efla_chunk_fwd_scan(const void* q, const void* k, const void* v, const float* beta, efla_dtype dtype,
                                void* o, const float* initial_state, float* final_state, int B, int H, int L, int d_k,
                                int d_v, int chunk, int segments, int gate, void* workspace, size_t workspace_bytes,
                                void* stream) {
    if (!valid_gate(gate)) return EFLA_ERR_INVALID_ARG;
    ScanPlan p;
    efla_status st = scan_plan(B, H, L, d_k, d_v, chunk, dtype, segments, &p);
    if (st != EFLA_OK) return st;
    const int64_t BH = (int64_t)B * H;
    st = check_fwd_buffers(q, k, v, beta, dtype, o, initial_state, final_state, BH, L, d_k, d_v);
    if (st != EFLA_OK) return st;
    if (p.total > 0 && BH > 0 && L > 0) {
        if (!workspace || !aligned(workspace, 256) || workspace_bytes < p.total) return EFLA_ERR_WORKSPACE;
        const size_t es = esize(dtype);
        const size_t nq = (size_t)BH * L * d_k * es, nv = (size_t)BH * L * d_v * es, nb = (size_t)BH * L * 4;
        const size_t ns = (size_t)BH * d_k * d_v * 4;
        const size_t need = p.total;
        if (overlap(workspace, need, q, nq) || overlap(workspace, need, k, nq) || overlap(workspace, need, v, nv) ||
            overlap(workspace, need, beta, nb) || overlap(workspace, need, o, nv) ||
            overlap(workspace, need, initial_state, ns) || overlap(workspace, need, final_state, ns))
            return EFLA_ERR_INVALID_ARG;
    }
    if (BH == 0) return EFLA_OK;
    if (L == 0 && !final_state) return EFLA_OK;
    st = device_present();
    if (st != EFLA_OK) return st;
    efla::SplitArgs a{q, k, v, beta, o, initial_state, final_state, workspace, (int)BH, L, d_k, d_v, chunk, p.dvs, gate};
    const hipError_t e = run_fwd(dtype == EFLA_BF16, a, p, static_cast<char*>(workspace), (hipStream_t)stream);
    return e == hipSuccess ? EFLA_OK : fail_hip(e, "efla_chunk_fwd_scan launch");
}

namespace {

// Launch shape and workspace of efla_chunk_fwd_layout: the scan plan of the sizes (fixed-length sequences), or
// one segment over packed sequences, whose workspace is the sanitised token offsets and the chunk offsets
// (B + 1 int32 each) and the chunk -> sequence table (ceil(L / C) + B int32), then H * (ceil(L / C) + B) UT
// chunks (the sanitised sequences are disjoint, so their sum_b ceil(len_b / C) is at most ceil(L / C) + B).
// One segment takes the split forward's slab.
struct LayoutPlan {
    ScanPlan sp;
    size_t off_ut;
};

efla_status layout_plan(int B, int H, int L, int d_k, int d_v, int chunk, efla_dtype dt, bool varlen, int segments,
                        LayoutPlan* lp) {
    if (segments < 0) return EFLA_ERR_INVALID_ARG;
    if (varlen && segments > 1) return EFLA_ERR_UNSUPPORTED;
    if (varlen) {
        int dvs = 0;
        const efla_status st = check_chunk_sizes(true, B, H, 0, d_k, d_v, chunk, dt, 0, &dvs);
        if (st != EFLA_OK) return st;
        if (L < 0) return EFLA_ERR_INVALID_ARG;
        const int64_t n_ut = (int64_t)H * ((L + chunk - 1) / chunk + B);
        if (n_ut > INT32_MAX || (int64_t)B + 1 > INT32_MAX / 8) return EFLA_ERR_INVALID_ARG;
        lp->sp.dvs = lp->sp.dvs1 = dvs;
        lp->sp.nseg = 1;
        lp->sp.seg_chunks = 0;
        lp->off_ut = round_up_256((size_t)(B + 1) * 8 + (size_t)((L + chunk - 1) / chunk + B) * 4);
        lp->sp.off_states = lp->sp.off_sin = 0;
        lp->sp.total = lp->off_ut + round_up_256((size_t)n_ut * efla::ut_block_elems(chunk) * esize(dt));
        return EFLA_OK;
    }
    efla_status st = scan_plan(B, H, L, d_k, d_v, chunk, dt, segments, &lp->sp);
    if (st != EFLA_OK) return st;
    if (lp->sp.nseg == 1) {
        int dvs = 0;
        st = check_chunk_sizes(true, B, H, L, d_k, d_v, chunk, dt, 0, &dvs);
        if (st != EFLA_OK) return st;
        lp->sp.dvs = dvs;
    }
    lp->off_ut = 0;
    return EFLA_OK;
}

// Elements spanned by a strided tensor of n0 x n1 x n2 rows of `inner` contiguous elements (0 when empty).
int64_t span(const int64_t st[3], int64_t n0, int64_t n1, int64_t n2, int64_t inner) {
    if (n0 <= 0 || n1 <= 0 || n2 <= 0) return 0;
    return (n0 - 1) * st[0] + (n1 - 1) * st[1] + (n2 - 1) * st[2] + inner;
}

// No two rows share an element: the dimensions of more than one row, sorted by stride, each step over at
// least the extent of the ones inside it.  An empty tensor has no rows.
bool rows_disjoint(const int64_t st[3], const int64_t n[3], int64_t inner) {
    if (n[0] <= 0 || n[1] <= 0 || n[2] <= 0) return true;
    int idx[3] = {0, 1, 2};
    for (int i = 0; i < 3; ++i)
        for (int j = i + 1; j < 3; ++j)
            if (st[idx[j]] < st[idx[i]]) { const int t = idx[i]; idx[i] = idx[j]; idx[j] = t; }
    int64_t ext = inner;
    for (int i = 0; i < 3; ++i) {
        const int d = idx[i];
        if (n[d] <= 1) continue;
        if (st[d] < ext) return false;
        ext += (n[d] - 1) * st[d];
    }
    return true;
}

// The kernels' token layout for the caller's (NULL: contiguous [B,H,L,d]), with the stride checks every entry point
// over layouts makes (see efla_chunk_fwd_layout).
efla_status make_layout(const efla_layout* layout, efla_dtype dt, int B, int H, int L, int d_k, int d_v,
                        efla::TokLayout* out) {
    const bool varlen = layout && layout->cu_seqlens;
    const int64_t es = (int64_t)esize(dt);
    efla::TokLayout ly = efla::contiguous_layout(H, L, d_k, d_v);
    if (layout) {
        const int64_t* src[5] = {layout->q, layout->k, layout->v, layout->o, layout->beta};
        int64_t* dst[5] = {&ly.q_b, &ly.k_b, &ly.v_b, &ly.o_b, &ly.be_b};
        for (int i = 0; i < 5; ++i) {
            for (int j = 0; j < 3; ++j) {
                const int64_t x = (varlen && j == 0) ? 0 : src[i][j];   // packed: no batch stride
                if (x < 0) return EFLA_ERR_INVALID_ARG;
                if (i < 4 && x % (16 / es) != 0) return EFLA_ERR_INVALID_ARG;   // 16-byte rows
                dst[i][j] = x;
            }
        }
        // rows of a chunk past the end of a sequence read as zeros only when no token's row overlaps the next
        if (ly.q_t < d_k || ly.k_t < d_k || ly.v_t < d_v || ly.be_t < 1) return EFLA_ERR_INVALID_ARG;
        // in-chunk offsets are 32-bit byte offsets
        const int64_t lim = (int64_t)INT32_MAX / 64;
        if (ly.q_t * es >= lim || ly.k_t * es >= lim || ly.v_t * es >= lim || ly.o_t * es >= lim || ly.be_t * 4 >= lim)
            return EFLA_ERR_INVALID_ARG;
        ly.cu_seqlens = layout->cu_seqlens;
    }
    ly.H = H;
    ly.nseq = B;
    *out = ly;
    return EFLA_OK;
}

// Two strided tensors of the same element size es, strides st and sizes n (rows of `inner` contiguous elements) at
// bases a and b share no element although their address extents overlap -- slices of one fused buffer.  Sufficient
// test: with the dimensions of more than one index sorted by stride, those adjacent to the block so far (stride
// equal to it) merged into it, every remaining stride is a multiple of the smallest remaining one, s, so every block
// of either tensor starts at the same residue modulo s as its base; blocks of `block` elements starting at residues
// 0 and r = |b - a| mod s then miss one another when block <= r <= s - block.
bool rows_interleave(const void* a, const void* b, int64_t es, const int64_t st[3], const int64_t n[3],
                     int64_t inner) {
    const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
    const uint64_t dbytes = pa > pb ? pa - pb : pb - pa;
    if (es <= 0 || dbytes % (uint64_t)es != 0) return false;
    const int64_t delta = (int64_t)(dbytes / (uint64_t)es);
    int idx[3], m = 0;
    for (int d = 0; d < 3; ++d)
        if (n[d] > 1) idx[m++] = d;
    for (int i = 0; i < m; ++i)
        for (int j = i + 1; j < m; ++j)
            if (st[idx[j]] < st[idx[i]]) { const int t = idx[i]; idx[i] = idx[j]; idx[j] = t; }
    int64_t block = inner;
    int i = 0;
    while (i < m && st[idx[i]] == block) block *= n[idx[i++]];
    if (i == m) return false;   // one contiguous block: the extents decide
    const int64_t sm = st[idx[i]];
    if (sm < 2 * block) return false;
    for (int j = i + 1; j < m; ++j)
        if (st[idx[j]] % sm != 0) return false;
    const int64_t r = delta % sm;
    return r >= block && r <= sm - block;
}

// A tensor argument for the overlap checks: its address extent and, when strided (st set), its element size,
// strides, sizes and row length.
struct Ext {
    const void* p;
    size_t bytes;
    int64_t es;
    const int64_t* st;
    const int64_t* n;
    int64_t inner;
};

// No element shared: disjoint extents, or rows that interleave (same element size, strides, sizes and rows)
bool disjoint(const Ext& a, const Ext& b) {
    if (!overlap(a.p, a.bytes, b.p, b.bytes)) return true;
    if (!a.st || !b.st || a.es != b.es || a.inner != b.inner) return false;
    for (int d = 0; d < 3; ++d)
        if (a.st[d] != b.st[d] || a.n[d] != b.n[d]) return false;
    return rows_interleave(a.p, b.p, a.es, a.st, a.n, a.inner);
}

}  // namespace

efla_status efla_chunk_layout_plan(int B, int H, int L, int d_k, int d_v, int chunk, efla_dtype dtype, int varlen,
                                   int segments, int* nseg, size_t* workspace_bytes) {
    LayoutPlan lp;
    const efla_status st = layout_plan(B, H, L, d_k, d_v, chunk, dtype, varlen != 0, segments, &lp);
    if (st != EFLA_OK) return st;
    if (nseg) *nseg = lp.sp.nseg;
    if (workspace_bytes) *workspace_bytes = lp.sp.total;
    return EFLA_OK;
}

efla_status efla_chunk_fwd_layout(const void* q, const void* k, const void* v, const float* beta, efla_dtype dtype,
                                  void* o, const float* initial_state, float* final_state, int B, int H, int L,
                                  int d_k, int d_v, int chunk, int segments, int gate, const efla_layout* layout,
                                  void* workspace, size_t workspace_bytes, void* stream) {
    if (!valid_gate(gate)) return EFLA_ERR_INVALID_ARG;
    const bool varlen = layout && layout->cu_seqlens;
    LayoutPlan lp;
    efla_status st = layout_plan(B, H, L, d_k, d_v, chunk, dtype, varlen, segments, &lp);
    if (st != EFLA_OK) return st;
    const int64_t BH = (int64_t)B * H;
    const int64_t es = (int64_t)esize(dtype);
    efla::TokLayout ly;
    st = make_layout(layout, dtype, B, H, L, d_k, d_v, &ly);
    if (st != EFLA_OK) return st;
    const int64_t nb = varlen ? 1 : B;   // batch extent of the token tensors
    const int64_t so[3] = {ly.o_b, ly.o_h, ly.o_t}, no[3] = {nb, H, L};
    if (!rows_disjoint(so, no, d_v)) return EFLA_ERR_INVALID_ARG;
    const int64_t sq[3] = {ly.q_b, ly.q_h, ly.q_t}, sk[3] = {ly.k_b, ly.k_h, ly.k_t}, sv[3] = {ly.v_b, ly.v_h, ly.v_t};
    const int64_t sb[3] = {ly.be_b, ly.be_h, ly.be_t};
    const size_t nq = (size_t)(span(sq, nb, H, L, d_k) * es), nk = (size_t)(span(sk, nb, H, L, d_k) * es);
    const size_t nv = (size_t)(span(sv, nb, H, L, d_v) * es), nob = (size_t)(span(so, nb, H, L, d_v) * es);
    const size_t nbe = (size_t)(span(sb, nb, H, L, 1) * 4);
    const size_t ns = (size_t)BH * d_k * d_v * 4;
    const size_t ncu = varlen ? (size_t)(B + 1) * 4 : 0;
    if (L > 0 && BH > 0) {
        if (!q || !k || !v || !beta || !o) return EFLA_ERR_INVALID_ARG;
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(beta, 4))
            return EFLA_ERR_INVALID_ARG;
    }
    if (varlen && BH > 0 && !aligned(layout->cu_seqlens, 4)) return EFLA_ERR_INVALID_ARG;
    if ((initial_state && !aligned(initial_state, 16)) || (final_state && !aligned(final_state, 16)))
        return EFLA_ERR_INVALID_ARG;
    const void* cu = varlen ? (const void*)layout->cu_seqlens : nullptr;
    // o overlaps nothing; the final state overlaps no input; initial and final state are identical or disjoint
    if (overlap(o, nob, q, nq) || overlap(o, nob, k, nk) || overlap(o, nob, v, nv) || overlap(o, nob, beta, nbe) ||
        overlap(o, nob, initial_state, ns) || overlap(o, nob, final_state, ns) || overlap(o, nob, cu, ncu))
        return EFLA_ERR_INVALID_ARG;
    if (overlap(final_state, ns, q, nq) || overlap(final_state, ns, k, nk) || overlap(final_state, ns, v, nv) ||
        overlap(final_state, ns, beta, nbe) || overlap(final_state, ns, cu, ncu))
        return EFLA_ERR_INVALID_ARG;
    if ((const void*)initial_state != (const void*)final_state && overlap(initial_state, ns, final_state, ns))
        return EFLA_ERR_INVALID_ARG;
    const bool runs = BH > 0 && (L > 0 || final_state);
    if (runs && lp.sp.total > 0) {
        const size_t need = lp.sp.total;
        if (!workspace || !aligned(workspace, 256) || workspace_bytes < need) return EFLA_ERR_WORKSPACE;
        if (overlap(workspace, need, q, nq) || overlap(workspace, need, k, nk) || overlap(workspace, need, v, nv) ||
            overlap(workspace, need, beta, nbe) || overlap(workspace, need, o, nob) ||
            overlap(workspace, need, initial_state, ns) || overlap(workspace, need, final_state, ns) ||
            overlap(workspace, need, cu, ncu))
            return EFLA_ERR_INVALID_ARG;
    }
    if (!runs) return EFLA_OK;
    st = device_present();
    if (st != EFLA_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    char* ws = static_cast<char*>(workspace);
    hipError_t e = hipSuccess;
    if (varlen) {
        int* cu_tok = reinterpret_cast<int*>(ws);
        int* cu_chunks = cu_tok + (B + 1);
        int* chunk_seq = cu_chunks + (B + 1);
        ly.cu_seqlens = cu_tok;
        ly.cu_chunks = cu_chunks;
        ly.chunk_seq = chunk_seq;
        e = efla::launch_varlen_prep(layout->cu_seqlens, cu_tok, cu_chunks, chunk_seq, B, L, chunk,
                                     (L + chunk - 1) / chunk + B, s);
    }
    if (dtype == EFLA_BF16 && d_k >= 32 && chunk == 64 && lp.sp.nseg == 1) {
        // the one-launch kernel (efla_chunk_fwd's form for these sizes) reads the views and packed sequences itself;
        // of the workspace it uses only the sanitised offsets
        int dvs = 0;
        st = check_chunk_sizes(false, B, H, L, d_k, d_v, chunk, dtype, 0, &dvs);
        if (st != EFLA_OK) return st;
        efla::ChunkArgs a1{q, k, v, beta, o, initial_state, final_state, (int)BH, L, d_k, d_v, chunk, dvs, gate, &ly};
        if (e == hipSuccess) e = efla::launch_chunk_fwd_bf16(a1, s);
        return e == hipSuccess ? EFLA_OK : fail_hip(e, "efla_chunk_fwd_layout launch");
    }
    efla::SplitArgs a{q, k, v, beta, o, initial_state, final_state, ws + lp.off_ut, (int)BH, L, d_k, d_v, chunk,
                      lp.sp.dvs, gate};
    a.layout = &ly;
    if (e == hipSuccess) e = run_fwd(dtype == EFLA_BF16, a, lp.sp, ws, s);
    return e == hipSuccess ? EFLA_OK : fail_hip(e, "efla_chunk_fwd_layout launch");
}

namespace {

// Workspace of efla_chunk_bwd_layout: with packed sequences first the sanitised token offsets, the chunk offsets
// (B + 1 int32 each) and the chunk -> sequence table (ceil(L / C) + B int32); then the UT output (Ta), the state
// entering and the gradient of the state leaving every chunk (d_k x d_v each), then -- where the per-chunk
// gradients run on bf16 matrix cores (bf16, d_k >= 32, chunk 32 or 64, d_v a multiple of 32) -- T^T of every chunk
// (bf16, chunk x chunk); each part 256-byte aligned.  The per-chunk states are bf16 where all three passes run on
// the matrix cores (those sizes with 64-token chunks: the per-chunk kernel takes them as bf16 operands), else
// fp32.  Chunks: B H ceil(L / C), or with packed sequences H (ceil(L / C) + B), which bounds H sum_b
// ceil(len_b / C) for disjoint sequences.
struct BwdPlan {
    size_t off_ut, off_s, off_ds, off_tt, total;
    bool tt, sbf;
};

efla_status bwd_plan(int B, int H, int L, int d_k, int d_v, int chunk, efla_dtype dt, bool varlen, BwdPlan* p) {
    if (!valid_dtype(dt) || B < 0 || H < 0 || L < 0) return EFLA_ERR_INVALID_ARG;
    if (!valid_dim(d_k) || !valid_dim(d_v) || !valid_chunk(chunk)) return EFLA_ERR_UNSUPPORTED;
    const int64_t BH = (int64_t)B * H;
    const int64_t NC = (L + chunk - 1) / chunk;
    const int64_t NU = varlen ? (int64_t)H * (NC + B) : BH * NC;
    if (BH > INT32_MAX || NU > INT32_MAX || BH * (d_v / 16) > INT32_MAX) return EFLA_ERR_INVALID_ARG;
    if (varlen && (int64_t)B + 1 > INT32_MAX / 8) return EFLA_ERR_INVALID_ARG;
    p->tt = dt == EFLA_BF16 && d_k >= 32 && chunk >= 32 && d_v % 32 == 0;
    p->sbf = p->tt && chunk == 64;
    const size_t states = round_up_256((size_t)NU * d_k * d_v * (p->sbf ? 2 : 4));
    p->off_ut = varlen ? round_up_256((size_t)(B + 1) * 8 + (size_t)(NC + B) * 4) : 0;
    p->off_s = p->off_ut + round_up_256((size_t)NU * (size_t)efla::ut_block_elems(chunk) * esize(dt));
    p->off_ds = p->off_s + states;
    p->off_tt = p->off_ds + states;
    p->total = p->off_tt + (p->tt ? round_up_256((size_t)NU * chunk * chunk * 2) : 0);
    return EFLA_OK;
}

}  // namespace

efla_status efla_chunk_bwd_layout_workspace_size(int B, int H, int L, int d_k, int d_v, int chunk, efla_dtype dtype,
                                                 int varlen, size_t* bytes) {
    BwdPlan p;
    const efla_status st = bwd_plan(B, H, L, d_k, d_v, chunk, dtype, varlen != 0, &p);
    if (st != EFLA_OK) return st;
    if (!bytes) return EFLA_ERR_INVALID_ARG;
    *bytes = p.total;
    return EFLA_OK;
}

efla_status efla_chunk_bwd_workspace_size(int B, int H, int L, int d_k, int d_v, int chunk, efla_dtype dtype,
                                          size_t* bytes) {
    return efla_chunk_bwd_layout_workspace_size(B, H, L, d_k, d_v, chunk, dtype, 0, bytes);
}

efla_status efla_chunk_bwd_layout(const void* q, const void* k, const void* v, const float* beta, efla_dtype dtype,
                                  const float* initial_state, const void* d_o, const float* d_final, void* dq,
                                  void* dk, void* dv, float* dbeta, float* d_initial, int B, int H, int L, int d_k,
                                  int d_v, int chunk, int gate, const efla_layout* layout, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    if (!valid_gate(gate)) return EFLA_ERR_INVALID_ARG;
    const bool varlen = layout && layout->cu_seqlens;
    BwdPlan p;
    efla_status st = bwd_plan(B, H, L, d_k, d_v, chunk, dtype, varlen, &p);
    if (st != EFLA_OK) return st;
    efla::TokLayout ly;
    st = make_layout(layout, dtype, B, H, L, d_k, d_v, &ly);
    if (st != EFLA_OK) return st;
    const int64_t BH = (int64_t)B * H;
    const int64_t es = (int64_t)esize(dtype);
    const int64_t nb = varlen ? 1 : B;   // batch extent of the token tensors
    const int64_t sq[3] = {ly.q_b, ly.q_h, ly.q_t}, sk[3] = {ly.k_b, ly.k_h, ly.k_t}, sv[3] = {ly.v_b, ly.v_h, ly.v_t};
    const int64_t so[3] = {ly.o_b, ly.o_h, ly.o_t}, sb[3] = {ly.be_b, ly.be_h, ly.be_t}, n3[3] = {nb, H, L};
    // the gradients take their inputs' strides: no two of their rows (elements for dbeta) may share memory
    if (!rows_disjoint(sq, n3, d_k) || !rows_disjoint(sk, n3, d_k) || !rows_disjoint(sv, n3, d_v) ||
        !rows_disjoint(sb, n3, 1))
        return EFLA_ERR_INVALID_ARG;
    const size_t nq = (size_t)(span(sq, nb, H, L, d_k) * es), nk = (size_t)(span(sk, nb, H, L, d_k) * es);
    const size_t nv = (size_t)(span(sv, nb, H, L, d_v) * es), no = (size_t)(span(so, nb, H, L, d_v) * es);
    const size_t nbe = (size_t)(span(sb, nb, H, L, 1) * 4);
    const size_t ns = (size_t)BH * d_k * d_v * 4;
    const size_t ncu = varlen ? (size_t)(B + 1) * 4 : 0;
    if (L > 0 && BH > 0) {
        if (!q || !k || !v || !beta || !d_o || !dq || !dk || !dv || !dbeta) return EFLA_ERR_INVALID_ARG;
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(d_o, 16) || !aligned(dq, 16) ||
            !aligned(dk, 16) || !aligned(dv, 16) || !aligned(beta, 4) || !aligned(dbeta, 4))
            return EFLA_ERR_INVALID_ARG;
    }
    if (varlen && BH > 0 && !aligned(layout->cu_seqlens, 4)) return EFLA_ERR_INVALID_ARG;
    if ((initial_state && !aligned(initial_state, 16)) || (d_final && !aligned(d_final, 16)) ||
        (d_initial && !aligned(d_initial, 16)))
        return EFLA_ERR_INVALID_ARG;
    // outputs overlap nothing (inputs, one another, the workspace): disjoint address extents, or rows of equal
    // strides that interleave (slices of one fused buffer)
    const void* cu = varlen ? (const void*)layout->cu_seqlens : nullptr;
    const int64_t ek = (int64_t)es;
    const Ext in[8] = {{q, nq, ek, sq, n3, d_k},   {k, nk, ek, sk, n3, d_k},       {v, nv, ek, sv, n3, d_v},
                       {beta, nbe, 4, sb, n3, 1},   {initial_state, ns, 4, nullptr, nullptr, 0},
                       {d_o, no, ek, so, n3, d_v}, {d_final, ns, 4, nullptr, nullptr, 0},
                       {cu, ncu, 4, nullptr, nullptr, 0}};
    const Ext out[5] = {{dq, nq, ek, sq, n3, d_k}, {dk, nk, ek, sk, n3, d_k}, {dv, nv, ek, sv, n3, d_v},
                        {dbeta, nbe, 4, sb, n3, 1}, {d_initial, ns, 4, nullptr, nullptr, 0}};
    for (int i = 0; i < 5; ++i) {
        for (int j = 0; j < 8; ++j)
            if (!disjoint(out[i], in[j])) return EFLA_ERR_INVALID_ARG;
        for (int j = i + 1; j < 5; ++j)
            if (!disjoint(out[i], out[j])) return EFLA_ERR_INVALID_ARG;
    }
    if (BH == 0) return EFLA_OK;
    if (L == 0 && !d_initial) return EFLA_OK;
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < p.total) return EFLA_ERR_WORKSPACE;
    for (int j = 0; j < 8; ++j)
        if (overlap(workspace, p.total, in[j].p, in[j].bytes)) return EFLA_ERR_INVALID_ARG;
    for (int j = 0; j < 5; ++j)
        if (overlap(workspace, p.total, out[j].p, out[j].bytes)) return EFLA_ERR_INVALID_ARG;
    st = device_present();
    if (st != EFLA_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    char* ws = static_cast<char*>(workspace);
    const bool bf = dtype == EFLA_BF16;
    hipError_t e = hipSuccess;
    if (varlen) {
        int* cu_tok = reinterpret_cast<int*>(ws);
        int* cu_chunks = cu_tok + (B + 1);
        int* chunk_seq = cu_chunks + (B + 1);
        ly.cu_seqlens = cu_tok;
        ly.cu_chunks = cu_chunks;
        ly.chunk_seq = chunk_seq;
        e = efla::launch_varlen_prep(layout->cu_seqlens, cu_tok, cu_chunks, chunk_seq, B, L, chunk,
                                     (L + chunk - 1) / chunk + B, s);
    }
    void* tw = ws + p.off_ut;
    void* tt = p.tt ? (void*)(ws + p.off_tt) : nullptr;
    // contiguous tensors: every (batch, head) is one sequence of L tokens
    const efla::TokLayout* lyp = layout ? &ly : nullptr;
    if (L > 0 && e == hipSuccess)
        e = bf ? efla::launch_ut_bf16(k, beta, tw, (int)BH, L, d_k, chunk, gate, s, tt, lyp)
               : efla::launch_ut_f32(k, beta, tw, (int)BH, L, d_k, chunk, gate, s, lyp);
    efla::BwdArgs a{q, k, v, beta, initial_state, d_o, d_final, dq, dk, dv, dbeta, d_initial, (int)BH, L, d_k, d_v,
                    chunk, gate, tw, ws + p.off_s, ws + p.off_ds, tt, lyp, p.sbf};
    if (e == hipSuccess) e = bf ? efla::launch_bwd_bf16(a, s) : efla::launch_bwd_f32(a, s);
    return e == hipSuccess ? EFLA_OK : fail_hip(e, "efla_chunk_bwd launch");
}

efla_status efla_chunk_bwd(const void* q, const void* k, const void* v, const float* beta, efla_dtype dtype,
                           const float* initial_state, const void* d_o, const float* d_final, void* dq, void* dk,
                           void* dv, float* dbeta, float* d_initial, int B, int H, int L, int d_k, int d_v,
                           int chunk, int gate, void* workspace, size_t workspace_bytes, void* stream) {
    return efla_chunk_bwd_layout(q, k, v, beta, dtype, initial_state, d_o, d_final, dq, dk, dv, dbeta, d_initial, B,
                                 H, L, d_k, d_v, chunk, gate, nullptr, workspace, workspace_bytes, stream);
}

namespace {

// The form efla_chunk_fwd takes for these sizes: the segment-parallel one when the automatic segment count is
// above one (few heads, long sequences), else the one-launch kernel for bf16 with d_k >= 32 and 64-token chunks,
// else the split form; and the workspace that form needs.
struct FwdForm {
    int form;
    ScanPlan scan;
    size_t workspace;
};

efla_status fwd_form(int B, int H, int L, int d_k, int d_v, int chunk, efla_dtype dt, FwdForm* f) {
    efla_status st = scan_plan(B, H, L, d_k, d_v, chunk, dt, 0, &f->scan);
    if (st != EFLA_OK) return st;
    int dvs = 0;
    if (f->scan.nseg > 1) {
        f->form = EFLA_FWD_SCAN;
        f->workspace = f->scan.total;
    } else if (dt == EFLA_BF16 && d_k >= 32 && chunk == 64) {
        st = check_chunk_sizes(false, B, H, L, d_k, d_v, chunk, dt, 0, &dvs);
        if (st != EFLA_OK) return st;
        f->form = EFLA_FWD_ONE_LAUNCH;
        f->workspace = 0;
    } else {
        st = check_chunk_sizes(true, B, H, L, d_k, d_v, chunk, dt, 0, &dvs);
        if (st != EFLA_OK) return st;
        f->form = EFLA_FWD_SPLIT;
        f->workspace = ut_bytes((int64_t)B * H, L, chunk, dt);
    }
    return EFLA_OK;
}

}  // namespace

size_t efla_chunk_fwd_workspace_size(int B, int H, int L, int d_k, int d_v, int chunk, efla_dtype dtype) {
    FwdForm f;
    return fwd_form(B, H, L, d_k, d_v, chunk, dtype, &f) == EFLA_OK ? f.workspace : 0;
}

efla_status efla_chunk_fwd_form(int B, int H, int L, int d_k, int d_v, int chunk, efla_dtype dtype, int* form,
                                int* segments, size_t* workspace_bytes) {
    FwdForm f;
    const efla_status st = fwd_form(B, H, L, d_k, d_v, chunk, dtype, &f);
    if (st != EFLA_OK) return st;
    if (form) *form = f.form;
    if (segments) *segments = f.form == EFLA_FWD_SCAN ? f.scan.nseg : 1;
    if (workspace_bytes) *workspace_bytes = f.workspace;
    return EFLA_OK;
}

efla_status efla_chunk_fwd_gate(const void* q, const void* k, const void* v, const float* beta, efla_dtype dtype,
                                void* o, const float* initial_state, float* final_state, int B, int H, int L, int d_k,
                                int d_v, int chunk, int gate, void* workspace, size_t workspace_bytes, void* stream) {
    if (!valid_gate(gate)) return EFLA_ERR_INVALID_ARG;
    FwdForm f;
    const efla_status st = fwd_form(B, H, L, d_k, d_v, chunk, dtype, &f);
    if (st != EFLA_OK) return st;
    if (f.form == EFLA_FWD_ONE_LAUNCH)
        return efla_chunk_fwd_slab_gate(q, k, v, beta, dtype, o, initial_state, final_state, B, H, L, d_k, d_v,
                                        chunk, 0, gate, stream);
    // the workspace is checked against the stricter 256-byte alignment of the scan form for every form
    if (f.workspace > 0 && (int64_t)B * H > 0 && (L > 0 || final_state) && workspace && !aligned(workspace, 256))
        return EFLA_ERR_WORKSPACE;
    if (f.form == EFLA_FWD_SCAN)
        return efla_chunk_fwd_scan(q, k, v, beta, dtype, o, initial_state, final_state, B, H, L, d_k, d_v, chunk, 0,
                                   gate, workspace, workspace_bytes, stream);
    return split_entry(true, q, k, v, beta, dtype, o, initial_state, final_state, B, H, L, d_k, d_v, chunk, 0, gate,
                       workspace, workspace_bytes, stream);
}

efla_status efla_chunk_fwd(const void* q, const void* k, const void* v, const float* beta, efla_dtype dtype, void* o,
                           const float* initial_state, float* final_state, int B, int H, int L, int d_k, int d_v,
                           int chunk, void* workspace, size_t workspace_bytes, void* stream) {
    return efla_chunk_fwd_gate(q, k, v, beta, dtype, o, initial_state, final_state, B, H, L, d_k, d_v, chunk,
                               EFLA_GATE_EXACT, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---- the allocation-free forward's scratch ------------------------------------------------------------------
// A file-scope device array that every GPU running the library holds (from the module's load to the process's
// end).  In host code its name is only a stand-in for the symbol: the device address of each GPU's copy comes
// from hipGetSymbolAddress, once per device, and only that address is ever handed to a kernel or a copy.
static __device__ __align__(256) unsigned char scratch[EFLA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's address of `scratch` (looked up on the first call for that device), or an error.
efla_status scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        snprintf(g_last_error, sizeof(g_last_error), "no HIP device visible (%s)", hipGetErrorName(e));
        return EFLA_ERR_NO_DEVICE;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        snprintf(g_last_error, sizeof(g_last_error), "device %d beyond the %d this library tracks", dev, kMaxDevices);
        return EFLA_ERR_UNSUPPORTED;
    }
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p) return fail_hip(e != hipSuccess ? e : hipErrorInvalidSymbol,
                                                       "efla_chunk_fwd_noalloc: hipGetSymbolAddress(scratch)");
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return EFLA_OK;
}

}  // namespace

extern "C" {

efla_status efla_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* beta, efla_dtype dtype,
                                   void* o, const float* initial_state, float* final_state, int B, int H, int L,
                                   int d_k, int d_v, int chunk, int gate, void* stream) {
    if (!valid_gate(gate)) return EFLA_ERR_INVALID_ARG;
    FwdForm f;
    efla_status st = fwd_form(B, H, L, d_k, d_v, chunk, dtype, &f);
    if (st != EFLA_OK) return st;
    if (f.workspace > EFLA_NOALLOC_SCRATCH_BYTES) {
        snprintf(g_last_error, sizeof(g_last_error),
                 "efla_chunk_fwd_noalloc: these sizes need %zu bytes of scratch, above the library's %zu", f.workspace,
                 (size_t)EFLA_NOALLOC_SCRATCH_BYTES);
        return EFLA_ERR_WORKSPACE;
    }
    void* ws = nullptr;
    if (f.workspace > 0) {
        // argument checks that need no device first, so that bad arguments report as such on any machine
        const int64_t BH = (int64_t)B * H;
        st = check_fwd_buffers(q, k, v, beta, dtype, o, initial_state, final_state, BH, L, d_k, d_v);
        if (st != EFLA_OK) return st;
        if (BH == 0 || (L == 0 && !final_state)) return EFLA_OK;
        st = scratch_address(&ws);
        if (st != EFLA_OK) return st;
    }
    return efla_chunk_fwd_gate(q, k, v, beta, dtype, o, initial_state, final_state, B, H, L, d_k, d_v, chunk, gate, ws,
                               ws ? (size_t)EFLA_NOALLOC_SCRATCH_BYTES : 0, stream);
}

efla_status efla_recurrent_step_gate(const void* q, const void* k, const void* v, const float* beta, efla_dtype dtype,
                                     float* state, void* o, int64_t NH, int d_k, int d_v, int gate, void* stream) {
    if (!valid_dtype(dtype) || NH < 0 || !valid_gate(gate)) return EFLA_ERR_INVALID_ARG;
    if (!valid_dim(d_k) || !valid_dim(d_v)) return EFLA_ERR_UNSUPPORTED;
    if (NH == 0) return EFLA_OK;
    if (NH > INT32_MAX) return EFLA_ERR_INVALID_ARG;
    if (!q || !k || !v || !beta || !state || !o) return EFLA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(state, 16) ||
        !aligned(beta, 4))
        return EFLA_ERR_INVALID_ARG;
    const size_t es = esize(dtype);
    const size_t nq = (size_t)NH * d_k * es, nv = (size_t)NH * d_v * es, nb = (size_t)NH * 4;
    const size_t ns = (size_t)NH * d_k * d_v * 4;
    if (overlap(o, nv, q, nq) || overlap(o, nv, k, nq) || overlap(o, nv, v, nv) || overlap(o, nv, beta, nb) ||
        overlap(o, nv, state, ns))
        return EFLA_ERR_INVALID_ARG;
    if (overlap(state, ns, q, nq) || overlap(state, ns, k, nq) || overlap(state, ns, v, nv) ||
        overlap(state, ns, beta, nb))
        return EFLA_ERR_INVALID_ARG;
    const efla_status st = device_present();
    if (st != EFLA_OK) return st;
    const hipError_t e =
        efla::launch_recurrent_step(q, k, v, beta, dtype, state, o, NH, d_k, d_v, gate, (hipStream_t)stream);
    return e == hipSuccess ? EFLA_OK : fail_hip(e, "efla_recurrent_step launch");
}

efla_status efla_recurrent_step(const void* q, const void* k, const void* v, const float* beta, efla_dtype dtype,
                                float* state, void* o, int64_t NH, int d_k, int d_v, void* stream) {
    return efla_recurrent_step_gate(q, k, v, beta, dtype, state, o, NH, d_k, d_v, EFLA_GATE_EXACT, stream);
}

}  // extern "C"
