// efla_bwd.hpp -- backward pass of the chunked forward: gradients of q, k, v, beta and the initial state.
//
// The pages train every model they report but print no backward pass ("Exact Flow Linear Attention"
// (gist.science), Risultati Sperimentali item 4: training throughput as DeltaNet's), so the gradients are the
// adjoint of the chunked form ("Error-Free Linear Attention is a Free Lunch" (howistudyai.com), Step 4), which
// per chunk of C tokens with entering state S, gates D = diag(alpha), L = strict_lower(K K^T),
// T = (I + D L)^{-1}, Ta = T D, P = lower_incl(Q K^T) computes
//   R = V - K S,   Delta = Ta R,   O = Q S + P Delta,   S' = S + K^T Delta.
// Given dO and dS' (the gradient of the state leaving the chunk):
//   dDelta = P^T dO + K dS'              G = T^T dDelta           dR = D G = Ta^T dDelta,   dV = dR
//   dS     = dS' + Q^T dO - K^T dR       (the gradient of the state entering the chunk)
//   dQ     = dO S^T + (M o (dO Delta^T)) K                                (M: the lower_incl mask)
//   dK     = (M o (dO Delta^T))^T Q + Delta dS'^T - dR S^T + (dL + dL^T) K + 2 dlambda o K
//            with dL = -strict_lower(D (G Delta^T)) (the solve (I + D L) Delta = D R differentiated)
//   dalpha = rowsum(G o R) - rowsum(L o (G Delta^T)),   dbeta = dalpha dalpha/dbeta,
//   dlambda = dalpha dalpha/dlambda                      (gate derivatives: gate_alpha_grad)
// Three launches after the UT transform (Ta into the workspace):
//   bwd_states_kernel  the forward state pass again, writing the state entering every chunk (fp32);
//   bwd_chain_kernel   the state gradient backwards over the chunks, writing the gradient of the state
//                      leaving every chunk (fp32), dV and the initial state's gradient;
//   bwd_chunk_kernel   one workgroup per (head, chunk): T by forward substitution in fp32, then dQ, dK, dbeta.
// The first two are sequential over chunks and independent over (head, slab of state columns); the third is
// parallel over all chunks.  These generic kernels take every product as an fp32 matrix-core instruction
// (16x16x4) on fp32 LDS tiles, each wave owning whole 16x16 output tiles, inputs of either storage type widened on
// load; they serve fp32 inputs and the bf16 sizes the matrix-core kernels below do not take.  bf16 inputs with
// d_k >= 32 run the three on bf16 matrix cores where the sizes allow (launch_bwd_t tries them first):
// efla_bwd_chain_mx.hpp (state recompute and state gradient, 64-token chunks) and efla_bwd_mx.hpp (per-chunk
// gradients, chunks of 32 or 64, d_v a multiple of 32, T^T from the UT launch).
#pragma once

#include "efla_common.hpp"
#include "efla_launch.hpp"

namespace efla {

namespace bwd {

constexpr int NT = 256;   // threads per workgroup: four waves

// An M x N fp32 product distributed over the NWV waves of the workgroup by 16x16 tiles: tile tt = w + NWV s
// (s < TPW) of the row-major tile grid belongs to wave w, whose lane (r, g) (r = lane & 15, g = lane >> 4) holds
// its elements (16 ti + 4 g + i, 16 tj + r), i = 0..3 -- the matrix cores' accumulator layout.
template <int M, int N, int NWV = 4>
struct Acc {
    static constexpr int TN = N / 16, NTT = (M / 16) * (N / 16), TPW = (NTT + NWV - 1) / NWV;
    static constexpr bool ALL = NTT % NWV == 0;   // every wave owns TPW tiles
    f32x4 t[TPW];
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int s = 0; s < TPW; ++s) t[s] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // f(row, col, element) for every element this lane holds
    template <class F>
    __device__ __forceinline__ void each(int w, int lane, F f) {
#pragma unroll
        for (int s = 0; s < TPW; ++s) {
            const int tt = w + NWV * s;
            if (ALL || tt < NTT) {
                const int ti = tt / TN, tj = tt - ti * TN;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float x = t[s][i];
                    f(16 * ti + 4 * (lane >> 4) + i, 16 * tj + (lane & 15), x);
                    t[s][i] = x;
                }
            }
        }
    }
};

// acc += A B over k < K (a multiple of 4), A(i, k) = A[i * ars + k * acs], B(k, j) = B[k * brs + j * bcs] in LDS:
// per 16x16x4 step lane (r, g) supplies A(16 ti + r, k + g) and B(k + g, 16 tj + r).  The reduction steps run in
// the outer loop and the wave's tiles in the inner one, so that consecutive matrix instructions are independent;
// a wave with a single tile splits its reduction into two chains (even and odd steps), summed at the end.
template <int M, int N, int NWV>
__device__ __forceinline__ void mm(Acc<M, N, NWV>& acc, const float* A, int ars, int acs, const float* B, int brs,
                                   int bcs, int K, int w, int lane) {
    typedef Acc<M, N, NWV> AC;
    constexpr int TPW = AC::TPW;
    const int r = lane & 15, g = lane >> 4;
    const float* pa[TPW];
    const float* pb[TPW];
#pragma unroll
    for (int s = 0; s < TPW; ++s) {
        const int tt = w + NWV * s;
        const int ti = tt / AC::TN, tj = tt - ti * AC::TN;
        pa[s] = A + (16 * ti + r) * ars + g * acs;
        pb[s] = B + g * brs + (16 * tj + r) * bcs;
    }
    if constexpr (TPW == 1) {
        if (AC::ALL || w < AC::NTT) {
            f32x4 c0 = acc.t[0], c1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
            for (int k = 0; k < K; k += 8) {
                c0 = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[0][k * acs], pb[0][k * brs], c0, 0, 0, 0);
                if (k + 4 < K) c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[0][(k + 4) * acs], pb[0][(k + 4) * brs], c1, 0, 0, 0);
            }
            acc.t[0] = c0 + c1;
        }
    } else {
        const bool last = AC::ALL || w + NWV * (TPW - 1) < AC::NTT;   // this wave owns a tile in slot TPW - 1
#pragma unroll 2
        for (int k = 0; k < K; k += 4) {
#pragma unroll
            for (int s = 0; s < TPW; ++s) {
                if (s < TPW - 1 || last)
                    acc.t[s] = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[s][k * acs], pb[s][k * brs], acc.t[s], 0, 0, 0);
            }
        }
    }
}

// ROWS x COLS of a row-major global matrix (row stride ld elements, 16-byte aligned rows) held in registers
// between a load (16 bytes per thread and request, all requests issued before any is used; rows >= n read as
// zeros) and a store into LDS (row stride sld) widened to fp32.  Loading the next tile before computing on
// the current one keeps its latency off the critical path.
template <typename E, int ROWS, int COLS, int NTH = NT>
struct Tile {
    typedef typename Vec16<E>::type V;
    static constexpr int VEC = Vec16<E>::N;
    static constexpr int VPR = COLS / VEC;
    static constexpr int TOT = ROWS * VPR;
    static constexpr int N = (TOT + NTH - 1) / NTH;
    static_assert(COLS % VEC == 0, "whole 16-byte vectors per row");
    V x[N];
    __device__ __forceinline__ void load(const E* g, int64_t ld, int n, int tid) {
#pragma unroll
        for (int it = 0; it < N; ++it) {
            const int idx = it * NTH + tid, r = idx / VPR, c = (idx - r * VPR) * VEC;
            x[it] = (idx < TOT && r < n) ? *reinterpret_cast<const V*>(g + (int64_t)r * ld + c)
                                         : __builtin_bit_cast(V, u32x4{0u, 0u, 0u, 0u});
        }
    }
    __device__ __forceinline__ void store(float* s, int sld, int tid) const {
#pragma unroll
        for (int it = 0; it < N; ++it) {
            const int idx = it * NTH + tid, r = idx / VPR, c = (idx - r * VPR) * VEC;
            if (TOT % NTH == 0 || idx < TOT) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) s[r * sld + c + e] = to_f32<E>(x[it][e]);
            }
        }
    }
};

// The lower 16x16 blocks of one chunk's Ta from the UT workspace's operand order: block qi = rb (rb + 1) / 2 + kb
// (kb <= rb) holds at [lane = 16 g + r][j] the entry (16 rb + r, 16 kb + 4 g + j).  The blocks above the
// diagonal are never written here: zero_upper clears them once.
template <typename E, int C, int NTH = NT>
struct TaTile {
    static constexpr int NQ = (C / 16) * (C / 16 + 1) / 2;
    static constexpr int TOT = NQ * 64;   // 4-element groups
    static constexpr int N = (TOT + NTH - 1) / NTH;
    typedef E V4 __attribute__((ext_vector_type(4)));
    V4 x[N];
    __device__ __forceinline__ void load(const E* blk, int tid) {
#pragma unroll
        for (int it = 0; it < N; ++it) {
            const int idx = it * NTH + tid;
            if (TOT % NTH == 0 || idx < TOT) x[it] = *reinterpret_cast<const V4*>(blk + 4 * idx);
        }
    }
    __device__ __forceinline__ void store(float* s, int sld, int tid) const {
#pragma unroll
        for (int it = 0; it < N; ++it) {
            const int idx = it * NTH + tid;
            if (TOT % NTH == 0 || idx < TOT) {
                const int qi = idx >> 6, lane = idx & 63;
                int rb = 0;
                while ((rb + 1) * (rb + 2) / 2 <= qi) ++rb;
                const int kb = qi - rb * (rb + 1) / 2;
                const int row = 16 * rb + (lane & 15), col = 16 * kb + 4 * (lane >> 4);
#pragma unroll
                for (int j = 0; j < 4; ++j) s[row * sld + col + j] = to_f32<E>(x[it][j]);
            }
        }
    }
    static __device__ __forceinline__ void zero_upper(float* s, int sld, int tid) {
        for (int idx = tid; idx < C * C; idx += NTH) {
            const int row = idx / C, col = idx - row * C;
            if ((col >> 4) > (row >> 4)) s[row * sld + col] = 0.0f;
        }
    }
};

}  // namespace bwd

// The (batch*head, chunk) of workgroup u of a launch over every chunk of the UT workspace, and that sequence's
// tokens; false for a workgroup past the last chunk (with packed sequences the grid is an upper bound).
__device__ inline bool chunk_at(const TokLayout& ly, int u, int L, int C, int& bh, int& c, SeqView& sv) {
    const int NC = (L + C - 1) / C;
    if (ly.cu_seqlens) {
        if (u >= ly.H * ly.cu_chunks[ly.nseq]) return false;
        chunk_of<true>(ly, u, NC, bh, c);
        sv = seq_view_t<true>(ly, bh, L, C);
    } else {
        chunk_of<false>(ly, u, NC, bh, c);
        sv = seq_view_t<false>(ly, bh, L, C);
    }
    return true;
}

// ------------------------------------------------------------------------------------------------
// The state entering every chunk: s_all[bh][c][i][j] (fp32, d_k x d_v), from S_0 = s0 (or 0) and
// S <- S + K^T Ta (V - K S).  One workgroup per (head, slab of DVS state columns).
// ------------------------------------------------------------------------------------------------
template <typename E, int DK, int C, int DVS>
__global__ __launch_bounds__(bwd::NT) void bwd_states_kernel(const E* __restrict__ k, const E* __restrict__ v,
                                                             const E* __restrict__ tw, const float* __restrict__ s0,
                                                             float* __restrict__ s_all, int L, int DV, int nslab,
                                                             TokLayout ly) {
    using namespace bwd;
    constexpr int LDK = DK + 2, LDV = DVS + 2, LDC = C + 2;
    constexpr int NQE = (C / 16) * (C / 16 + 1) / 2 * 256;
    // V, then R = V - K S in place, then Delta (76 KB for d_k = 128, 64-token chunks and 32 columns: two
    // workgroups per compute unit)
    __shared__ float sK[C * LDK], sV[C * LDV], sT[C * LDC], sS[DK * LDV];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int bh = blockIdx.x / nslab, slab = blockIdx.x - bh * nslab;
    const int col0 = slab * DVS;
    const SeqView sv = seq_view(ly, bh, L, C);   // this sequence's tokens and first chunk
    const int NC = (sv.len + C - 1) / C;
    Acc<DK, DVS> S;
    S.zero();
    if (s0) S.each(w, lane, [&](int i, int j, float& x) { x = s0[((int64_t)bh * DK + i) * DV + col0 + j]; });
    Tile<E, C, DK> tk;
    Tile<E, C, DVS> tv;
    TaTile<E, C> tt;
    auto load = [&](int c) {
        const int t0 = c * C, n = sv.len - t0 < C ? sv.len - t0 : C;
        tk.load(k + sv.k0 + t0 * ly.k_t, ly.k_t, n, tid);
        tv.load(v + sv.v0 + t0 * ly.v_t + col0, ly.v_t, n, tid);
        tt.load(tw + ((int64_t)sv.chunk0 + c) * NQE, tid);
    };
    TaTile<E, C>::zero_upper(sT, LDC, tid);
    if (NC > 0) load(0);
    for (int c = 0; c < NC; ++c) {
        float* out = s_all + ((int64_t)sv.chunk0 + c) * DK * DV;
        S.each(w, lane, [&](int i, int j, float& x) {
            out[i * DV + col0 + j] = x;
            sS[i * LDV + j] = x;
        });
        tk.store(sK, LDK, tid);
        tv.store(sV, LDV, tid);
        tt.store(sT, LDC, tid);
        __syncthreads();
        if (c + 1 < NC) load(c + 1);
        {   // R = V - K S (each element read and written by the lane that holds it)
            Acc<C, DVS> a;
            a.zero();
            mm(a, sK, LDK, 1, sS, LDV, 1, DK, w, lane);
            a.each(w, lane, [&](int i, int j, float& x) { sV[i * LDV + j] -= x; });
        }
        __syncthreads();
        {   // Delta = Ta R, over R once every wave has read it
            Acc<C, DVS> a;
            a.zero();
            mm(a, sT, LDC, 1, sV, LDV, 1, C, w, lane);
            __syncthreads();
            a.each(w, lane, [&](int i, int j, float& x) { sV[i * LDV + j] = x; });
        }
        __syncthreads();
        mm(S, sK, 1, LDK, sV, LDV, 1, C, w, lane);   // S += K^T Delta
        __syncthreads();
    }
}

constexpr int kChainThreads = 512;   // threads of the state-gradient kernel (eight waves)

// ------------------------------------------------------------------------------------------------
// The state gradient, backwards over the chunks, for one (head, slab of DVS columns): ds_all[bh][c] =
// the gradient of the state leaving chunk c; dV of the slab; d_initial = the gradient of S_0.
// ------------------------------------------------------------------------------------------------
template <typename E, int DK, int C, int DVS>
__global__ __launch_bounds__(kChainThreads) void bwd_chain_kernel(const E* __restrict__ q, const E* __restrict__ k,
                                                            const E* __restrict__ tw, const E* __restrict__ d_o,
                                                            const float* __restrict__ d_final,
                                                            float* __restrict__ ds_all, E* __restrict__ dv,
                                                            float* __restrict__ d_initial, int L, int DV, int nslab,
                                                            TokLayout ly) {
    using namespace bwd;
    constexpr int NWV = kChainThreads / 64;   // two waves per SIMD
    constexpr int NTH = kChainThreads;
    constexpr int LDK = DK + 2, LDV = DVS + 2, LDC = C + 2;
    constexpr int NQE = (C / 16) * (C / 16 + 1) / 2 * 256;
    __shared__ float sQ[C * LDK], sK[C * LDK], sO[C * LDV], sD[C * LDV], sR[C * LDV], sT[C * LDC], sP[C * LDC],
        sS[DK * LDV];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int bh = blockIdx.x / nslab, slab = blockIdx.x - bh * nslab;
    const int col0 = slab * DVS;
    const SeqView sv = seq_view(ly, bh, L, C);
    const int NC = (sv.len + C - 1) / C;
    Acc<DK, DVS, NWV> dS;
    dS.zero();
    if (d_final)
        dS.each(w, lane, [&](int i, int j, float& x) { x = d_final[((int64_t)bh * DK + i) * DV + col0 + j]; });
    Tile<E, C, DK, NTH> tq, tk;
    Tile<E, C, DVS, NTH> to;
    TaTile<E, C, NTH> tt;
    auto load = [&](int c) {
        const int t0 = c * C, n = sv.len - t0 < C ? sv.len - t0 : C;
        tq.load(q + sv.q0 + t0 * ly.q_t, ly.q_t, n, tid);
        tk.load(k + sv.k0 + t0 * ly.k_t, ly.k_t, n, tid);
        to.load(d_o + sv.o0 + t0 * ly.o_t + col0, ly.o_t, n, tid);
        tt.load(tw + ((int64_t)sv.chunk0 + c) * NQE, tid);
    };
    TaTile<E, C, NTH>::zero_upper(sT, LDC, tid);
    if (NC > 0) load(NC - 1);
    for (int c = NC - 1; c >= 0; --c) {
        const int t0 = c * C, n = sv.len - t0 < C ? sv.len - t0 : C;
        float* out = ds_all + ((int64_t)sv.chunk0 + c) * DK * DV;
        dS.each(w, lane, [&](int i, int j, float& x) {
            out[i * DV + col0 + j] = x;
            sS[i * LDV + j] = x;
        });
        tq.store(sQ, LDK, tid);
        tk.store(sK, LDK, tid);
        to.store(sO, LDV, tid);
        tt.store(sT, LDC, tid);
        __syncthreads();
        if (c > 0) load(c - 1);
        {   // P = lower_incl(Q K^T)
            Acc<C, C, NWV> a;
            a.zero();
            mm(a, sQ, LDK, 1, sK, 1, LDK, DK, w, lane);
            a.each(w, lane, [&](int i, int j, float& x) { sP[i * LDC + j] = j <= i ? x : 0.0f; });
        }
        __syncthreads();
        {   // dDelta = P^T dO + K dS'
            Acc<C, DVS, NWV> a;
            a.zero();
            mm(a, sP, 1, LDC, sO, LDV, 1, C, w, lane);
            mm(a, sK, LDK, 1, sS, LDV, 1, DK, w, lane);
            a.each(w, lane, [&](int i, int j, float& x) { sD[i * LDV + j] = x; });
        }
        __syncthreads();
        {   // dR = Ta^T dDelta = dV; -dR kept for the state gradient
            Acc<C, DVS, NWV> a;
            a.zero();
            mm(a, sT, 1, LDC, sD, LDV, 1, C, w, lane);
            a.each(w, lane, [&](int i, int j, float& x) {
                sR[i * LDV + j] = -x;
                if (i < n) dv[sv.v0 + (int64_t)(t0 + i) * ly.v_t + col0 + j] = from_f32<E>(x);
            });
        }
        __syncthreads();
        mm(dS, sQ, 1, LDK, sO, LDV, 1, C, w, lane);   // dS += Q^T dO
        mm(dS, sK, 1, LDK, sR, LDV, 1, C, w, lane);   //    - K^T dR
        __syncthreads();
    }
    if (d_initial)
        dS.each(w, lane, [&](int i, int j, float& x) { d_initial[((int64_t)bh * DK + i) * DV + col0 + j] = x; });
}

// ------------------------------------------------------------------------------------------------
// dQ, dK and dbeta of one chunk (one workgroup per (head, chunk)), from the chunk's entering state
// (s_all) and the gradient of its leaving state (ds_all); the d_v columns are taken 16 at a time.
// ------------------------------------------------------------------------------------------------
constexpr int kChunkThreads = 512;   // threads of the per-chunk gradient kernel (eight waves)

template <typename E, int DK, int C>
struct BwdChunkLds {
    static constexpr int LDK = DK + 2, LDC = C + 2, LDV = 17;
    static constexpr int BYTES = 4 * (2 * C * LDK + 3 * C * LDC + 2 * DK * LDV + 5 * C * LDV + 4 * C);
};

template <typename E, int DK, int C>
__global__ __launch_bounds__(kChunkThreads) void bwd_chunk_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v, const float* __restrict__ beta,
    const E* __restrict__ d_o, const float* __restrict__ s_all, const float* __restrict__ ds_all, E* __restrict__ dq,
    E* __restrict__ dk, float* __restrict__ dbeta, int L, int DV, int gate, TokLayout ly) {
    using namespace bwd;
    constexpr int NWV = kChunkThreads / 64;   // two waves per SIMD: one's LDS reads and barriers overlap the other's products
    constexpr int NTH = kChunkThreads;
    typedef BwdChunkLds<E, DK, C> LY;
    constexpr int LDK = LY::LDK, LDC = LY::LDC, LDV = LY::LDV;
    extern __shared__ float smem[];
    float* sQ = smem;
    float* sK = sQ + C * LDK;
    float* sL = sK + C * LDK;    // K K^T (full)
    float* sP = sL + C * LDC;    // lower_incl(Q K^T); later M o (dO Delta^T)
    float* sT = sP + C * LDC;    // T; later G Delta^T, then dL
    float* sS = sT + C * LDC;    // S[:, slab]
    float* sG2 = sS + DK * LDV;  // dS'[:, slab]
    float* sV = sG2 + DK * LDV;  // V slab; then D R; then -dR
    float* sO = sV + C * LDV;    // dO slab
    float* sDl = sO + C * LDV;   // Delta slab
    float* sDd = sDl + C * LDV;  // dDelta slab
    float* sGs = sDd + C * LDV;  // G slab
    float* sAl = sGs + C * LDV;  // alpha
    float* sDb = sAl + C;        // dalpha/dbeta
    float* sDlam = sDb + C;      // dalpha/dlambda
    float* sDa = sDlam + C;      // dalpha, then dlambda

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int bh, c;
    SeqView sv;
    if (!chunk_at(ly, blockIdx.x, L, C, bh, c, sv)) return;
    const int t0 = c * C, n = sv.len - t0 < C ? sv.len - t0 : C;
    const int64_t q0 = sv.q0 + (int64_t)t0 * ly.q_t, k0 = sv.k0 + (int64_t)t0 * ly.k_t;   // the chunk's first rows
    const int64_t v0 = sv.v0 + (int64_t)t0 * ly.v_t, o0 = sv.o0 + (int64_t)t0 * ly.o_t;
    const int64_t be0 = sv.be0 + (int64_t)t0 * ly.be_t;
    const float* Sg = s_all + (int64_t)blockIdx.x * DK * DV;   // workgroup u works on chunk u of the workspace
    const float* dSg = ds_all + (int64_t)blockIdx.x * DK * DV;
    (void)bh;

    {
        Tile<E, C, DK, NTH> tq, tk;
        tq.load(q + q0, ly.q_t, n, tid);
        tk.load(k + k0, ly.k_t, n, tid);
        tq.store(sQ, LDK, tid);
        tk.store(sK, LDK, tid);
    }
    // the d_v slabs' tiles, loaded one slab ahead
    Tile<float, DK, 16, NTH> ts, tds;
    Tile<E, C, 16, NTH> tv, to;
    auto load_slab = [&](int col0) {
        ts.load(Sg + col0, DV, DK, tid);
        tds.load(dSg + col0, DV, DK, tid);
        tv.load(v + v0 + col0, ly.v_t, n, tid);
        to.load(d_o + o0 + col0, ly.o_t, n, tid);
    };
    load_slab(0);
    if (tid < C) sDa[tid] = 0.0f;
    __syncthreads();
    if (tid < C) {   // gates of the chunk's tokens (rows past the end: zero keys, zero step)
        float lam = 0.0f;
        for (int e = 0; e < DK; ++e) lam = fmaf(sK[tid * LDK + e], sK[tid * LDK + e], lam);
        const float b = tid < n ? beta[be0 + (int64_t)tid * ly.be_t] : 0.0f;
        sAl[tid] = gate_alpha(b, lam, gate);
        float db, dl;
        gate_alpha_grad(b, lam, gate, &db, &dl);
        sDb[tid] = db;
        sDlam[tid] = dl;
    }
    {   // L = K K^T, P = lower_incl(Q K^T)
        Acc<C, C, NWV> a, b;
        a.zero();
        b.zero();
        mm(a, sK, LDK, 1, sK, 1, LDK, DK, w, lane);
        mm(b, sQ, LDK, 1, sK, 1, LDK, DK, w, lane);
        a.each(w, lane, [&](int i, int j, float& x) { sL[i * LDC + j] = x; });
        b.each(w, lane, [&](int i, int j, float& x) { sP[i * LDC + j] = j <= i ? x : 0.0f; });
    }
    __syncthreads();
    // T = (I + D strict_lower(L))^{-1} by forward substitution, one column per lane of wave 0 in registers:
    // T[i][j] = [i == j] - alpha_i sum_{j <= m < i} L[i][m] T[m][j]
    if (tid < 64) {
        const int j = tid;
        float t[C];
#pragma unroll
        for (int i = 0; i < C; ++i) {
            float s4[4] = {0.0f, 0.0f, 0.0f, 0.0f};   // four partial sums: a quarter of the dependent chain
#pragma unroll
            for (int m = 0; m < i; ++m) s4[m & 3] = fmaf(sL[i * LDC + m], t[m], s4[m & 3]);
            t[i] = (i == j ? 1.0f : 0.0f) - sAl[i] * ((s4[0] + s4[1]) + (s4[2] + s4[3]));
            if (i < j) t[i] = 0.0f;
        }
        if (j < C) {
#pragma unroll
            for (int i = 0; i < C; ++i) sT[i * LDC + j] = t[i];
        }
    }
    __syncthreads();

    Acc<C, DK, NWV> aQ, aK;
    Acc<C, C, NWV> W1, W2;
    aQ.zero();
    aK.zero();
    W1.zero();
    W2.zero();
    for (int col0 = 0; col0 < DV; col0 += 16) {
        ts.store(sS, LDV, tid);
        tds.store(sG2, LDV, tid);
        tv.store(sV, LDV, tid);
        to.store(sO, LDV, tid);
        __syncthreads();
        if (col0 + 16 < DV) load_slab(col0 + 16);
        Acc<C, 16, NWV> R;   // R = V - K S, kept for dalpha; D R over V
        R.zero();
        mm(R, sK, LDK, 1, sS, LDV, 1, DK, w, lane);
        R.each(w, lane, [&](int i, int j, float& x) { x = sV[i * LDV + j] - x; });
        __syncthreads();
        R.each(w, lane, [&](int i, int j, float& x) { sV[i * LDV + j] = sAl[i] * x; });
        __syncthreads();
        {   // Delta = T (D R); dDelta = P^T dO + K dS'
            Acc<C, 16, NWV> a, b;
            a.zero();
            b.zero();
            mm(a, sT, LDC, 1, sV, LDV, 1, C, w, lane);
            mm(b, sP, 1, LDC, sO, LDV, 1, C, w, lane);
            mm(b, sK, LDK, 1, sG2, LDV, 1, DK, w, lane);
            a.each(w, lane, [&](int i, int j, float& x) { sDl[i * LDV + j] = x; });
            b.each(w, lane, [&](int i, int j, float& x) { sDd[i * LDV + j] = x; });
        }
        __syncthreads();
        {   // G = T^T dDelta; -dR = -D G over V; dalpha += rowsum(G o R)
            Acc<C, 16, NWV> a;
            a.zero();
            mm(a, sT, 1, LDC, sDd, LDV, 1, C, w, lane);
            a.each(w, lane, [&](int i, int j, float& x) {
                sGs[i * LDV + j] = x;
                sV[i * LDV + j] = -sAl[i] * x;
            });
            // rows of this lane's elements: the same (tile, i) for a and R, summed over the 16 columns (lanes r)
#pragma unroll
            for (int s = 0; s < Acc<C, 16, NWV>::TPW; ++s) {
                const int tt = w + NWV * s;
                if (Acc<C, 16, NWV>::ALL || tt < Acc<C, 16, NWV>::NTT) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float p = a.t[s][i] * R.t[s][i];
                        p = group_sum<16>(p);   // the tile row's 16 columns, by DPP moves
                        if ((lane & 15) == 0) sDa[16 * tt + 4 * (lane >> 4) + i] += p;
                    }
                }
            }
        }
        __syncthreads();
        // dQ += dO S^T; dK += Delta dS'^T - dR S^T; W1 += dO Delta^T; W2 += G Delta^T
        mm(aQ, sO, LDV, 1, sS, 1, LDV, 16, w, lane);
        mm(aK, sDl, LDV, 1, sG2, 1, LDV, 16, w, lane);
        mm(aK, sV, LDV, 1, sS, 1, LDV, 16, w, lane);
        mm(W1, sO, LDV, 1, sDl, 1, LDV, 16, w, lane);
        mm(W2, sGs, LDV, 1, sDl, 1, LDV, 16, w, lane);
        __syncthreads();
    }

    // M o W1 into sP, W2 into sT
    W1.each(w, lane, [&](int i, int j, float& x) { sP[i * LDC + j] = j <= i ? x : 0.0f; });
    W2.each(w, lane, [&](int i, int j, float& x) { sT[i * LDC + j] = x; });
    __syncthreads();
    // dalpha = rowsum(G o R) - rowsum(strict_lower(L) o W2); dbeta; dlambda
    if (tid < C) {
        const int i = tid;
        float s = sDa[i];
        for (int j = 0; j < i; ++j) s -= sL[i * LDC + j] * sT[i * LDC + j];
        if (i < n) dbeta[be0 + (int64_t)i * ly.be_t] = s * sDb[i];
        sDa[i] = s * sDlam[i];
    }
    __syncthreads();
    // dL = -strict_lower(D W2) in place
    for (int idx = tid; idx < C * C; idx += NTH) {
        const int i = idx / C, j = idx - i * C;
        sT[i * LDC + j] = j < i ? -sAl[i] * sT[i * LDC + j] : 0.0f;
    }
    __syncthreads();
    // dQ += (M o W1) K;  dK += (M o W1)^T Q + dL K + dL^T K + 2 dlambda o K
    mm(aQ, sP, LDC, 1, sK, LDK, 1, C, w, lane);
    mm(aK, sP, 1, LDC, sQ, LDK, 1, C, w, lane);
    mm(aK, sT, LDC, 1, sK, LDK, 1, C, w, lane);
    mm(aK, sT, 1, LDC, sK, LDK, 1, C, w, lane);
    aQ.each(w, lane, [&](int i, int e, float& x) {
        if (i < n) dq[q0 + (int64_t)i * ly.q_t + e] = from_f32<E>(x);
    });
    aK.each(w, lane, [&](int i, int e, float& x) {
        if (i < n) dk[k0 + (int64_t)i * ly.k_t + e] = from_f32<E>(fmaf(2.0f * sDa[i], sK[i * LDK + e], x));
    });
}

// ------------------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------------------
struct BwdArgs {
    const void *q, *k, *v;
    const float* beta;
    const float* s0;
    const void* d_o;
    const float* d_final;
    void *dq, *dk, *dv;
    float* dbeta;
    float* d_initial;
    int BH, L, d_k, d_v, chunk, gate;
    void* tw;        // UT output (Ta), already written
    void* s_all;     // BH x NC x d_k x d_v: fp32, or bf16 when sbf
    void* ds_all;    // BH x NC x d_k x d_v: fp32, or bf16 when sbf
    void* tt;        // T^T of every chunk (BH x NC x chunk x chunk, storage type), or null
    // null: contiguous [B,H,L,d] tensors; else the strides of q, k, v, d_o (in o's place) and beta -- the
    // gradients dq, dk, dv, dbeta take those of their input -- and packed sequences (then the UT workspace,
    // s_all, ds_all and tt hold the chunks of the sequences in the layout's order)
    const TokLayout* layout = nullptr;
    // the per-chunk states in bf16: only where all three kernels after the UT launch run on bf16 matrix cores
    // (bf16, d_k >= 32, 64-token chunks, d_v a multiple of 32), whose per-chunk kernel rounds them to bf16 operands
    // anyway -- the same values, half the workspace and its traffic
    bool sbf = false;
};

// contiguous [B,H,L,d] tensors: every (batch, head) a sequence of L tokens
inline TokLayout bwd_layout(const BwdArgs& a) {
    return a.layout ? *a.layout : contiguous_layout(1, a.L, a.d_k, a.d_v);
}
// workgroups of a launch over every chunk of the workspace (packed sequences: an upper bound)
inline int64_t bwd_chunk_grid(const BwdArgs& a, int C) {
    const int64_t NC = (a.L + C - 1) / C;
    return a.layout && a.layout->cu_seqlens ? (int64_t)a.layout->H * (NC + a.layout->nseq) : (int64_t)a.BH * NC;
}

// The per-chunk gradient kernel on bf16 matrix cores (efla_bwd_mx.hpp) takes the shapes it supports by
// specialising this for bf16; launch() returns false where it does not apply.
template <typename E, int DK, int C>
struct BwdChunkFast {
    static bool launch(const BwdArgs&, hipStream_t, hipError_t*) { return false; }
};
// Likewise the state recompute and the state-gradient pass on bf16 matrix cores (efla_bwd_chain_mx.hpp).
template <typename E, int DK, int C>
struct BwdStatesFast {
    static bool launch(const BwdArgs&, hipStream_t, hipError_t*) { return false; }
};
template <typename E, int DK, int C>
struct BwdChainFast {
    static bool launch(const BwdArgs&, hipStream_t, hipError_t*) { return false; }
};

template <typename E, int DK, int C>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t s) {
    const E* q = static_cast<const E*>(a.q);
    const E* k = static_cast<const E*>(a.k);
    const E* v = static_cast<const E*>(a.v);
    const E* d_o = static_cast<const E*>(a.d_o);
    const E* tw = static_cast<const E*>(a.tw);
    const TokLayout ly = bwd_layout(a);
    // bf16 states are planned only where the matrix-core kernels run all three passes; check the pairing
    const bool fast_states = std::is_same<E, bf16>::value && DK >= 32 && C == 64;
    const bool fast_chunk = std::is_same<E, bf16>::value && DK >= 32 && C >= 32 && a.d_v % 32 == 0 && a.tt;
    if (a.sbf && !(fast_states && fast_chunk)) return hipErrorInvalidValue;
    if (a.L > 0) {
        hipError_t es = hipSuccess;
        if (BwdStatesFast<E, DK, C>::launch(a, s, &es)) {
            if (es != hipSuccess) return es;
        } else if (a.d_v >= 32) {
            const int nslab = a.d_v / 32;
            hipLaunchKernelGGL((bwd_states_kernel<E, DK, C, 32>), dim3((unsigned)(a.BH * nslab)), dim3(bwd::NT), 0, s, k,
                               v, tw, a.s0, static_cast<float*>(a.s_all), a.L, a.d_v, nslab, ly);
        } else {
            const int nslab = a.d_v / 16;
            hipLaunchKernelGGL((bwd_states_kernel<E, DK, C, 16>), dim3((unsigned)(a.BH * nslab)), dim3(bwd::NT), 0, s, k,
                               v, tw, a.s0, static_cast<float*>(a.s_all), a.L, a.d_v, nslab, ly);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipError_t ec = hipSuccess;
    if (BwdChainFast<E, DK, C>::launch(a, s, &ec)) {
        if (ec != hipSuccess) return ec;
    } else if (a.d_v >= 32) {
        const int nslab = a.d_v / 32;
        hipLaunchKernelGGL((bwd_chain_kernel<E, DK, C, 32>), dim3((unsigned)(a.BH * nslab)), dim3(kChainThreads), 0, s, q, k,
                           tw, d_o, a.d_final, static_cast<float*>(a.ds_all), static_cast<E*>(a.dv), a.d_initial, a.L, a.d_v, nslab,
                           ly);
    } else {
        const int nslab = a.d_v / 16;
        hipLaunchKernelGGL((bwd_chain_kernel<E, DK, C, 16>), dim3((unsigned)(a.BH * nslab)), dim3(kChainThreads), 0, s, q, k,
                           tw, d_o, a.d_final, static_cast<float*>(a.ds_all), static_cast<E*>(a.dv), a.d_initial, a.L, a.d_v, nslab,
                           ly);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.L == 0) return e;
    if (BwdChunkFast<E, DK, C>::launch(a, s, &e)) return e;
    constexpr int LDS = BwdChunkLds<E, DK, C>::BYTES;
    static_assert(LDS <= kMaxLdsBytes, "backward chunk kernel LDS too large");
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_chunk_kernel<E, DK, C>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_chunk_kernel<E, DK, C>), dim3((unsigned)bwd_chunk_grid(a, C)), dim3(kChunkThreads), LDS, s, q,
                       k, v, a.beta, d_o, static_cast<const float*>(a.s_all), static_cast<const float*>(a.ds_all),
                       static_cast<E*>(a.dq), static_cast<E*>(a.dk), a.dbeta,
                       a.L, a.d_v, a.gate, ly);
    return hipGetLastError();
}

template <typename E, int DK>
hipError_t launch_bwd_dk(const BwdArgs& a, hipStream_t s) {
    switch (a.chunk) {
        case 16: return launch_bwd_t<E, DK, 16>(a, s);
        case 32: return launch_bwd_t<E, DK, 32>(a, s);
        case 64: return launch_bwd_t<E, DK, 64>(a, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename E>
hipError_t launch_bwd_e(const BwdArgs& a, hipStream_t s) {
    switch (a.d_k) {
        case 16: return launch_bwd_dk<E, 16>(a, s);
        case 32: return launch_bwd_dk<E, 32>(a, s);
        case 64: return launch_bwd_dk<E, 64>(a, s);
        case 128: return launch_bwd_dk<E, 128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace efla

namespace efla {
hipError_t launch_bwd_f32(const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t s);
}  // namespace efla
