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
// parallel over all chunks.  All arithmetic is fp32 on the vector units through LDS tiles (a 16 x 16 thread
// grid of register micro-tiles); inputs of either storage type are widened on load.
#pragma once

#include "efla_common.hpp"
#include "efla_launch.hpp"

namespace efla {

namespace bwd {

constexpr int NT = 256;   // threads per workgroup: tx = tid & 15 (columns), ty = tid >> 4 (rows)

// acc[mi][nj] += sum_{k < K} A(ty + 16 mi, k) B(k, tx + 16 nj), A(i, k) = A[i * ars + k * acs],
// B(k, j) = B[k * brs + j * bcs] (LDS, fp32)
template <int MI, int NJ>
__device__ __forceinline__ void mm(float (&acc)[MI][NJ], const float* A, int ars, int acs, const float* B, int brs,
                                   int bcs, int K, int ty, int tx) {
    // unrolled so that the LDS reads of several steps are in flight together (one wave per SIMD here)
#pragma unroll 8
    for (int k = 0; k < K; ++k) {
        float a[MI], b[NJ];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) a[mi] = A[(ty + 16 * mi) * ars + k * acs];
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj) b[nj] = B[k * brs + (tx + 16 * nj) * bcs];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int nj = 0; nj < NJ; ++nj) acc[mi][nj] = fmaf(a[mi], b[nj], acc[mi][nj]);
    }
}

template <int MI, int NJ>
__device__ __forceinline__ void zero(float (&acc)[MI][NJ]) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj) acc[mi][nj] = 0.0f;
}

// ROWS x COLS of a row-major global matrix (row stride ld elements, 16-byte aligned rows) held in registers
// between a load (16 bytes per thread and request, all requests issued before any is used; rows >= n read as
// zeros) and a store into LDS (row stride sld) widened to fp32.  Loading the next tile before computing on
// the current one keeps its latency off the critical path.
template <typename E, int ROWS, int COLS>
struct Tile {
    typedef typename Vec16<E>::type V;
    static constexpr int VEC = Vec16<E>::N;
    static constexpr int VPR = COLS / VEC;
    static constexpr int TOT = ROWS * VPR;
    static constexpr int N = (TOT + NT - 1) / NT;
    static_assert(COLS % VEC == 0, "whole 16-byte vectors per row");
    V x[N];
    __device__ __forceinline__ void load(const E* g, int64_t ld, int n, int tid) {
#pragma unroll
        for (int it = 0; it < N; ++it) {
            const int idx = it * NT + tid, r = idx / VPR, c = (idx - r * VPR) * VEC;
            x[it] = (idx < TOT && r < n) ? *reinterpret_cast<const V*>(g + (int64_t)r * ld + c)
                                         : __builtin_bit_cast(V, u32x4{0u, 0u, 0u, 0u});
        }
    }
    __device__ __forceinline__ void store(float* s, int sld, int tid) const {
#pragma unroll
        for (int it = 0; it < N; ++it) {
            const int idx = it * NT + tid, r = idx / VPR, c = (idx - r * VPR) * VEC;
            if (TOT % NT == 0 || idx < TOT) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) s[r * sld + c + e] = to_f32<E>(x[it][e]);
            }
        }
    }
};

// The lower 16x16 blocks of one chunk's Ta from the UT workspace's operand order: block qi = rb (rb + 1) / 2 + kb
// (kb <= rb) holds at [lane = 16 g + r][j] the entry (16 rb + r, 16 kb + 4 g + j).  The blocks above the
// diagonal are never written here: zero_upper clears them once.
template <typename E, int C>
struct TaTile {
    static constexpr int NQ = (C / 16) * (C / 16 + 1) / 2;
    static constexpr int TOT = NQ * 64;   // 4-element groups
    static constexpr int N = (TOT + NT - 1) / NT;
    typedef E V4 __attribute__((ext_vector_type(4)));
    V4 x[N];
    __device__ __forceinline__ void load(const E* blk, int tid) {
#pragma unroll
        for (int it = 0; it < N; ++it) {
            const int idx = it * NT + tid;
            if (TOT % NT == 0 || idx < TOT) x[it] = *reinterpret_cast<const V4*>(blk + 4 * idx);
        }
    }
    __device__ __forceinline__ void store(float* s, int sld, int tid) const {
#pragma unroll
        for (int it = 0; it < N; ++it) {
            const int idx = it * NT + tid;
            if (TOT % NT == 0 || idx < TOT) {
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
        for (int idx = tid; idx < C * C; idx += NT) {
            const int row = idx / C, col = idx - row * C;
            if ((col >> 4) > (row >> 4)) s[row * sld + col] = 0.0f;
        }
    }
};

}  // namespace bwd

// ------------------------------------------------------------------------------------------------
// The state entering every chunk: s_all[bh][c][i][j] (fp32, d_k x d_v), from S_0 = s0 (or 0) and
// S <- S + K^T Ta (V - K S).  One workgroup per (head, slab of DVS state columns).
// ------------------------------------------------------------------------------------------------
template <typename E, int DK, int C, int DVS>
__global__ __launch_bounds__(bwd::NT) void bwd_states_kernel(const E* __restrict__ k, const E* __restrict__ v,
                                                             const E* __restrict__ tw, const float* __restrict__ s0,
                                                             float* __restrict__ s_all, int L, int DV, int nslab) {
    using namespace bwd;
    constexpr int LDK = DK + 1, LDV = DVS + 1, LDC = C + 1;
    constexpr int NQE = (C / 16) * (C / 16 + 1) / 2 * 256;
    __shared__ float sK[C * LDK], sV[C * LDV], sR[C * LDV], sT[C * LDC], sS[DK * LDV];
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int bh = blockIdx.x / nslab, slab = blockIdx.x - bh * nslab;
    const int col0 = slab * DVS;
    const int NC = (L + C - 1) / C;
    const int64_t tok0 = (int64_t)bh * L;
    float S[DK / 16][DVS / 16];
#pragma unroll
    for (int mi = 0; mi < DK / 16; ++mi)
#pragma unroll
        for (int nj = 0; nj < DVS / 16; ++nj)
            S[mi][nj] = s0 ? s0[((int64_t)bh * DK + ty + 16 * mi) * DV + col0 + tx + 16 * nj] : 0.0f;
    Tile<E, C, DK> tk;
    Tile<E, C, DVS> tv;
    TaTile<E, C> tt;
    auto load = [&](int c) {
        const int t0 = c * C, n = L - t0 < C ? L - t0 : C;
        tk.load(k + (tok0 + t0) * DK, DK, n, tid);
        tv.load(v + (tok0 + t0) * DV + col0, DV, n, tid);
        tt.load(tw + ((int64_t)bh * NC + c) * NQE, tid);
    };
    TaTile<E, C>::zero_upper(sT, LDC, tid);
    if (NC > 0) load(0);
    for (int c = 0; c < NC; ++c) {
        float* out = s_all + ((int64_t)bh * NC + c) * DK * DV;
#pragma unroll
        for (int mi = 0; mi < DK / 16; ++mi)
#pragma unroll
            for (int nj = 0; nj < DVS / 16; ++nj) {
                out[(ty + 16 * mi) * DV + col0 + tx + 16 * nj] = S[mi][nj];
                sS[(ty + 16 * mi) * LDV + tx + 16 * nj] = S[mi][nj];
            }
        tk.store(sK, LDK, tid);
        tv.store(sV, LDV, tid);
        tt.store(sT, LDC, tid);
        __syncthreads();
        if (c + 1 < NC) load(c + 1);
        {   // R = V - K S
            float a[C / 16][DVS / 16];
            zero(a);
            mm(a, sK, LDK, 1, sS, LDV, 1, DK, ty, tx);
#pragma unroll
            for (int mi = 0; mi < C / 16; ++mi)
#pragma unroll
                for (int nj = 0; nj < DVS / 16; ++nj) {
                    const int i = ty + 16 * mi, j = tx + 16 * nj;
                    sR[i * LDV + j] = sV[i * LDV + j] - a[mi][nj];
                }
        }
        __syncthreads();
        {   // Delta = Ta R  (into sV)
            float a[C / 16][DVS / 16];
            zero(a);
            mm(a, sT, LDC, 1, sR, LDV, 1, C, ty, tx);
#pragma unroll
            for (int mi = 0; mi < C / 16; ++mi)
#pragma unroll
                for (int nj = 0; nj < DVS / 16; ++nj) sV[(ty + 16 * mi) * LDV + tx + 16 * nj] = a[mi][nj];
        }
        __syncthreads();
        mm(S, sK, 1, LDK, sV, LDV, 1, C, ty, tx);   // S += K^T Delta
        __syncthreads();
    }
}

// ------------------------------------------------------------------------------------------------
// The state gradient, backwards over the chunks, for one (head, slab of DVS columns): ds_all[bh][c] =
// the gradient of the state leaving chunk c; dV of the slab; d_initial = the gradient of S_0.
// ------------------------------------------------------------------------------------------------
template <typename E, int DK, int C, int DVS>
__global__ __launch_bounds__(bwd::NT) void bwd_chain_kernel(const E* __restrict__ q, const E* __restrict__ k,
                                                            const E* __restrict__ tw, const E* __restrict__ d_o,
                                                            const float* __restrict__ d_final,
                                                            float* __restrict__ ds_all, E* __restrict__ dv,
                                                            float* __restrict__ d_initial, int L, int DV, int nslab) {
    using namespace bwd;
    constexpr int LDK = DK + 1, LDV = DVS + 1, LDC = C + 1;
    constexpr int NQE = (C / 16) * (C / 16 + 1) / 2 * 256;
    __shared__ float sQ[C * LDK], sK[C * LDK], sO[C * LDV], sD[C * LDV], sR[C * LDV], sT[C * LDC], sP[C * LDC],
        sS[DK * LDV];
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int bh = blockIdx.x / nslab, slab = blockIdx.x - bh * nslab;
    const int col0 = slab * DVS;
    const int NC = (L + C - 1) / C;
    const int64_t tok0 = (int64_t)bh * L;
    float dS[DK / 16][DVS / 16];
#pragma unroll
    for (int mi = 0; mi < DK / 16; ++mi)
#pragma unroll
        for (int nj = 0; nj < DVS / 16; ++nj)
            dS[mi][nj] = d_final ? d_final[((int64_t)bh * DK + ty + 16 * mi) * DV + col0 + tx + 16 * nj] : 0.0f;
    Tile<E, C, DK> tq, tk;
    Tile<E, C, DVS> to;
    TaTile<E, C> tt;
    auto load = [&](int c) {
        const int t0 = c * C, n = L - t0 < C ? L - t0 : C;
        tq.load(q + (tok0 + t0) * DK, DK, n, tid);
        tk.load(k + (tok0 + t0) * DK, DK, n, tid);
        to.load(d_o + (tok0 + t0) * DV + col0, DV, n, tid);
        tt.load(tw + ((int64_t)bh * NC + c) * NQE, tid);
    };
    TaTile<E, C>::zero_upper(sT, LDC, tid);
    if (NC > 0) load(NC - 1);
    for (int c = NC - 1; c >= 0; --c) {
        const int t0 = c * C, n = L - t0 < C ? L - t0 : C;
        float* out = ds_all + ((int64_t)bh * NC + c) * DK * DV;
#pragma unroll
        for (int mi = 0; mi < DK / 16; ++mi)
#pragma unroll
            for (int nj = 0; nj < DVS / 16; ++nj) {
                out[(ty + 16 * mi) * DV + col0 + tx + 16 * nj] = dS[mi][nj];
                sS[(ty + 16 * mi) * LDV + tx + 16 * nj] = dS[mi][nj];
            }
        tq.store(sQ, LDK, tid);
        tk.store(sK, LDK, tid);
        to.store(sO, LDV, tid);
        tt.store(sT, LDC, tid);
        __syncthreads();
        if (c > 0) load(c - 1);
        {   // P = lower_incl(Q K^T)
            float a[C / 16][C / 16];
            zero(a);
            mm(a, sQ, LDK, 1, sK, 1, LDK, DK, ty, tx);
#pragma unroll
            for (int mi = 0; mi < C / 16; ++mi)
#pragma unroll
                for (int nj = 0; nj < C / 16; ++nj) {
                    const int i = ty + 16 * mi, j = tx + 16 * nj;
                    sP[i * LDC + j] = j <= i ? a[mi][nj] : 0.0f;
                }
        }
        __syncthreads();
        {   // dDelta = P^T dO + K dS'
            float a[C / 16][DVS / 16];
            zero(a);
            mm(a, sP, 1, LDC, sO, LDV, 1, C, ty, tx);
            mm(a, sK, LDK, 1, sS, LDV, 1, DK, ty, tx);
#pragma unroll
            for (int mi = 0; mi < C / 16; ++mi)
#pragma unroll
                for (int nj = 0; nj < DVS / 16; ++nj) sD[(ty + 16 * mi) * LDV + tx + 16 * nj] = a[mi][nj];
        }
        __syncthreads();
        {   // dR = Ta^T dDelta = dV
            float a[C / 16][DVS / 16];
            zero(a);
            mm(a, sT, 1, LDC, sD, LDV, 1, C, ty, tx);
#pragma unroll
            for (int mi = 0; mi < C / 16; ++mi)
#pragma unroll
                for (int nj = 0; nj < DVS / 16; ++nj) {
                    const int i = ty + 16 * mi, j = tx + 16 * nj;
                    sR[i * LDV + j] = a[mi][nj];
                    if (i < n) dv[(tok0 + t0 + i) * DV + col0 + j] = from_f32<E>(a[mi][nj]);
                }
        }
        __syncthreads();
        {   // dS = dS' + Q^T dO - K^T dR
            float a[DK / 16][DVS / 16], b[DK / 16][DVS / 16];
            zero(a);
            zero(b);
            mm(a, sQ, 1, LDK, sO, LDV, 1, C, ty, tx);
            mm(b, sK, 1, LDK, sR, LDV, 1, C, ty, tx);
#pragma unroll
            for (int mi = 0; mi < DK / 16; ++mi)
#pragma unroll
                for (int nj = 0; nj < DVS / 16; ++nj) dS[mi][nj] += a[mi][nj] - b[mi][nj];
        }
        __syncthreads();
    }
    if (d_initial) {
#pragma unroll
        for (int mi = 0; mi < DK / 16; ++mi)
#pragma unroll
            for (int nj = 0; nj < DVS / 16; ++nj)
                d_initial[((int64_t)bh * DK + ty + 16 * mi) * DV + col0 + tx + 16 * nj] = dS[mi][nj];
    }
}

// ------------------------------------------------------------------------------------------------
// dQ, dK and dbeta of one chunk (one workgroup per (head, chunk)), from the chunk's entering state
// (s_all) and the gradient of its leaving state (ds_all); the d_v columns are taken 16 at a time.
// ------------------------------------------------------------------------------------------------
template <typename E, int DK, int C>
struct BwdChunkLds {
    static constexpr int LDK = DK + 1, LDC = C + 1, LDV = 17;
    static constexpr int BYTES = 4 * (2 * C * LDK + 3 * C * LDC + 2 * DK * LDV + 6 * C * LDV + 4 * C);
};

template <typename E, int DK, int C>
__global__ __launch_bounds__(bwd::NT) void bwd_chunk_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v, const float* __restrict__ beta,
    const E* __restrict__ d_o, const float* __restrict__ s_all, const float* __restrict__ ds_all, E* __restrict__ dq,
    E* __restrict__ dk, float* __restrict__ dbeta, int L, int DV, int gate) {
    using namespace bwd;
    typedef BwdChunkLds<E, DK, C> LY;
    constexpr int LDK = LY::LDK, LDC = LY::LDC, LDV = LY::LDV;
    constexpr int MC = C / 16, MK = DK / 16;
    extern __shared__ float smem[];
    float* sQ = smem;
    float* sK = sQ + C * LDK;
    float* sL = sK + C * LDK;    // K K^T (full)
    float* sP = sL + C * LDC;    // lower_incl(Q K^T); later M o (dO Delta^T)
    float* sT = sP + C * LDC;    // T; later dL
    float* sS = sT + C * LDC;    // S[:, slab]
    float* sG2 = sS + DK * LDV;  // dS'[:, slab]
    float* sV = sG2 + DK * LDV;  // V slab; then D R
    float* sO = sV + C * LDV;    // dO slab
    float* sDl = sO + C * LDV;   // Delta slab
    float* sDd = sDl + C * LDV;  // dDelta slab
    float* sGs = sDd + C * LDV;  // G slab
    float* sDr = sGs + C * LDV;  // dR slab
    float* sAl = sDr + C * LDV;  // alpha
    float* sDb = sAl + C;        // dalpha/dbeta
    float* sDlam = sDb + C;      // dalpha/dlambda
    float* sDa = sDlam + C;      // dalpha, then dlambda

    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int NC = (L + C - 1) / C;
    const int bh = blockIdx.x / NC, c = blockIdx.x - bh * NC;
    const int t0 = c * C, n = L - t0 < C ? L - t0 : C;
    const int64_t tok = (int64_t)bh * L + t0;
    const float* Sg = s_all + ((int64_t)bh * NC + c) * DK * DV;
    const float* dSg = ds_all + ((int64_t)bh * NC + c) * DK * DV;

    {
        Tile<E, C, DK> tq, tk;
        tq.load(q + tok * DK, DK, n, tid);
        tk.load(k + tok * DK, DK, n, tid);
        tq.store(sQ, LDK, tid);
        tk.store(sK, LDK, tid);
    }
    // the d_v slabs' tiles, loaded one slab ahead
    Tile<float, DK, 16> ts, tds;
    Tile<E, C, 16> tv, to;
    auto load_slab = [&](int col0) {
        ts.load(Sg + col0, DV, DK, tid);
        tds.load(dSg + col0, DV, DK, tid);
        tv.load(v + tok * DV + col0, DV, n, tid);
        to.load(d_o + tok * DV + col0, DV, n, tid);
    };
    load_slab(0);
    __syncthreads();
    if (tid < C) {   // gates of the chunk's tokens (rows past the end: zero keys, zero step)
        float lam = 0.0f;
        for (int e = 0; e < DK; ++e) lam = fmaf(sK[tid * LDK + e], sK[tid * LDK + e], lam);
        const float b = tid < n ? beta[tok + tid] : 0.0f;
        sAl[tid] = gate_alpha(b, lam, gate);
        float db, dl;
        gate_alpha_grad(b, lam, gate, &db, &dl);
        sDb[tid] = db;
        sDlam[tid] = dl;
    }
    {   // L = K K^T, P = lower_incl(Q K^T)
        float a[MC][MC], b[MC][MC];
        zero(a);
        zero(b);
        mm(a, sK, LDK, 1, sK, 1, LDK, DK, ty, tx);
        mm(b, sQ, LDK, 1, sK, 1, LDK, DK, ty, tx);
#pragma unroll
        for (int mi = 0; mi < MC; ++mi)
#pragma unroll
            for (int nj = 0; nj < MC; ++nj) {
                const int i = ty + 16 * mi, j = tx + 16 * nj;
                sL[i * LDC + j] = a[mi][nj];
                sP[i * LDC + j] = j <= i ? b[mi][nj] : 0.0f;
            }
    }
    __syncthreads();
    // T = (I + D strict_lower(L))^{-1} by forward substitution, one column per lane of wave 0 in registers:
    // T[i][j] = [i == j] - alpha_i sum_{j <= m < i} L[i][m] T[m][j]
    if (tid < 64) {
        const int j = tid;
        float t[C];
#pragma unroll
        for (int i = 0; i < C; ++i) {
            float s = 0.0f;
#pragma unroll
            for (int m = 0; m < i; ++m) s = fmaf(sL[i * LDC + m], t[m], s);
            t[i] = (i == j ? 1.0f : 0.0f) - sAl[i] * s;
            if (i < j) t[i] = 0.0f;
        }
        if (j < C) {
#pragma unroll
            for (int i = 0; i < C; ++i) sT[i * LDC + j] = t[i];
        }
    }
    __syncthreads();

    float aQ[MC][MK], aK[MC][MK], W1[MC][MC], W2[MC][MC];
    zero(aQ);
    zero(aK);
    zero(W1);
    zero(W2);
    float dap[MC];   // this thread's share of rowsum(G o R): rows ty + 16 mi, columns tx of every slab
#pragma unroll
    for (int mi = 0; mi < MC; ++mi) dap[mi] = 0.0f;

    for (int col0 = 0; col0 < DV; col0 += 16) {
        ts.store(sS, LDV, tid);
        tds.store(sG2, LDV, tid);
        tv.store(sV, LDV, tid);
        to.store(sO, LDV, tid);
        __syncthreads();
        if (col0 + 16 < DV) load_slab(col0 + 16);
        float r[MC];
        {   // R = V - K S; keep R, write D R over V
            float a[MC][1];
            zero(a);
            mm(a, sK, LDK, 1, sS, LDV, 1, DK, ty, tx);
#pragma unroll
            for (int mi = 0; mi < MC; ++mi) r[mi] = sV[(ty + 16 * mi) * LDV + tx] - a[mi][0];
        }
        __syncthreads();
#pragma unroll
        for (int mi = 0; mi < MC; ++mi) sV[(ty + 16 * mi) * LDV + tx] = sAl[ty + 16 * mi] * r[mi];
        __syncthreads();
        {   // Delta = T (D R); dDelta = P^T dO + K dS'
            float a[MC][1], b[MC][1];
            zero(a);
            zero(b);
            mm(a, sT, LDC, 1, sV, LDV, 1, C, ty, tx);
            mm(b, sP, 1, LDC, sO, LDV, 1, C, ty, tx);
            mm(b, sK, LDK, 1, sG2, LDV, 1, DK, ty, tx);
#pragma unroll
            for (int mi = 0; mi < MC; ++mi) {
                sDl[(ty + 16 * mi) * LDV + tx] = a[mi][0];
                sDd[(ty + 16 * mi) * LDV + tx] = b[mi][0];
            }
        }
        __syncthreads();
        {   // G = T^T dDelta; dR = D G
            float a[MC][1];
            zero(a);
            mm(a, sT, 1, LDC, sDd, LDV, 1, C, ty, tx);
#pragma unroll
            for (int mi = 0; mi < MC; ++mi) {
                const int i = ty + 16 * mi;
                sGs[i * LDV + tx] = a[mi][0];
                sDr[i * LDV + tx] = sAl[i] * a[mi][0];
                dap[mi] = fmaf(a[mi][0], r[mi], dap[mi]);
            }
        }
        __syncthreads();
        // dQ += dO S^T; dK += Delta dS'^T - dR S^T; W1 += dO Delta^T; W2 += G Delta^T
        mm(aQ, sO, LDV, 1, sS, 1, LDV, 16, ty, tx);
        mm(aK, sDl, LDV, 1, sG2, 1, LDV, 16, ty, tx);
        {
            float b[MC][MK];
            zero(b);
            mm(b, sDr, LDV, 1, sS, 1, LDV, 16, ty, tx);
#pragma unroll
            for (int mi = 0; mi < MC; ++mi)
#pragma unroll
                for (int nj = 0; nj < MK; ++nj) aK[mi][nj] -= b[mi][nj];
        }
        mm(W1, sO, LDV, 1, sDl, 1, LDV, 16, ty, tx);
        mm(W2, sGs, LDV, 1, sDl, 1, LDV, 16, ty, tx);
        __syncthreads();
    }

    // dalpha = rowsum(G o R) - rowsum(strict_lower(L) o W2): reduce over the 16 column threads of a row
    float dal[MC];
#pragma unroll
    for (int mi = 0; mi < MC; ++mi) {
        const int i = ty + 16 * mi;
        float s = dap[mi];
#pragma unroll
        for (int nj = 0; nj < MC; ++nj) {
            const int j = tx + 16 * nj;
            if (j < i) s -= sL[i * LDC + j] * W2[mi][nj];
        }
        s += __shfl_xor(s, 1, 16);
        s += __shfl_xor(s, 2, 16);
        s += __shfl_xor(s, 4, 16);
        s += __shfl_xor(s, 8, 16);
        dal[mi] = s;
    }
    // M o W1 into sP, dL = -strict_lower(D W2) into sT
#pragma unroll
    for (int mi = 0; mi < MC; ++mi)
#pragma unroll
        for (int nj = 0; nj < MC; ++nj) {
            const int i = ty + 16 * mi, j = tx + 16 * nj;
            sP[i * LDC + j] = j <= i ? W1[mi][nj] : 0.0f;
            sT[i * LDC + j] = j < i ? -sAl[i] * W2[mi][nj] : 0.0f;
        }
    if (tx == 0) {
#pragma unroll
        for (int mi = 0; mi < MC; ++mi) {
            const int i = ty + 16 * mi;
            const float db = dal[mi] * sDb[i];
            sDa[i] = dal[mi] * sDlam[i];   // dlambda
            if (i < n) dbeta[tok + i] = db;
        }
    }
    __syncthreads();
    // dQ += (M o W1) K;  dK += (M o W1)^T Q + dL K + dL^T K + 2 dlambda o K
    mm(aQ, sP, LDC, 1, sK, LDK, 1, C, ty, tx);
    mm(aK, sP, 1, LDC, sQ, LDK, 1, C, ty, tx);
    mm(aK, sT, LDC, 1, sK, LDK, 1, C, ty, tx);
    mm(aK, sT, 1, LDC, sK, LDK, 1, C, ty, tx);
#pragma unroll
    for (int mi = 0; mi < MC; ++mi) {
        const int i = ty + 16 * mi;
        if (i >= n) continue;
        const float dl2 = 2.0f * sDa[i];
#pragma unroll
        for (int nj = 0; nj < MK; ++nj) {
            const int e = tx + 16 * nj;
            dq[(tok + i) * DK + e] = from_f32<E>(aQ[mi][nj]);
            dk[(tok + i) * DK + e] = from_f32<E>(fmaf(dl2, sK[i * LDK + e], aK[mi][nj]));
        }
    }
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
    float* s_all;    // BH x NC x d_k x d_v
    float* ds_all;   // BH x NC x d_k x d_v
};

template <typename E, int DK, int C>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t s) {
    const int NC = (a.L + C - 1) / C;
    const E* q = static_cast<const E*>(a.q);
    const E* k = static_cast<const E*>(a.k);
    const E* v = static_cast<const E*>(a.v);
    const E* d_o = static_cast<const E*>(a.d_o);
    const E* tw = static_cast<const E*>(a.tw);
    if (a.L > 0) {
        if (a.d_v >= 32) {
            const int nslab = a.d_v / 32;
            hipLaunchKernelGGL((bwd_states_kernel<E, DK, C, 32>), dim3((unsigned)(a.BH * nslab)), dim3(bwd::NT), 0, s, k,
                               v, tw, a.s0, a.s_all, a.L, a.d_v, nslab);
        } else {
            const int nslab = a.d_v / 16;
            hipLaunchKernelGGL((bwd_states_kernel<E, DK, C, 16>), dim3((unsigned)(a.BH * nslab)), dim3(bwd::NT), 0, s, k,
                               v, tw, a.s0, a.s_all, a.L, a.d_v, nslab);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.d_v >= 32) {
        const int nslab = a.d_v / 32;
        hipLaunchKernelGGL((bwd_chain_kernel<E, DK, C, 32>), dim3((unsigned)(a.BH * nslab)), dim3(bwd::NT), 0, s, q, k,
                           tw, d_o, a.d_final, a.ds_all, static_cast<E*>(a.dv), a.d_initial, a.L, a.d_v, nslab);
    } else {
        const int nslab = a.d_v / 16;
        hipLaunchKernelGGL((bwd_chain_kernel<E, DK, C, 16>), dim3((unsigned)(a.BH * nslab)), dim3(bwd::NT), 0, s, q, k,
                           tw, d_o, a.d_final, a.ds_all, static_cast<E*>(a.dv), a.d_initial, a.L, a.d_v, nslab);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.L == 0) return e;
    constexpr int LDS = BwdChunkLds<E, DK, C>::BYTES;
    static_assert(LDS <= kMaxLdsBytes, "backward chunk kernel LDS too large");
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_chunk_kernel<E, DK, C>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_chunk_kernel<E, DK, C>), dim3((unsigned)((int64_t)a.BH * NC)), dim3(bwd::NT), LDS, s, q, k,
                       v, a.beta, d_o, a.s_all, a.ds_all, static_cast<E*>(a.dq), static_cast<E*>(a.dk), a.dbeta, a.L,
                       a.d_v, a.gate);
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
