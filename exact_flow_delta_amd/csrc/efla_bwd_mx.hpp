// efla_bwd_mx.hpp -- the per-chunk gradient kernel of the backward pass on bf16 matrix cores (bf16 inputs,
// d_k >= 32, chunks of 32 or 64 tokens, d_v a multiple of 32).
//
// Same chunk gradients as bwd_chunk_kernel (efla_bwd.hpp, where they are derived: the adjoint of the chunked form
// of "Error-Free Linear Attention is a Free Lunch" (howistudyai.com), Step 4), in the same phases, with every
// product a 16x16x32 bf16 matrix instruction accumulating in fp32 over bf16 tiles in LDS:
//   * Tiles are row-major bf16 with rows padded by 8 elements (16 bytes), so that the 16 rows of a fragment start
//     on different banks.
//   * An operand whose reduction index runs along its rows' contiguous elements is read 8 elements per lane with
//     one 16-byte read (lane (r, g): reduction indices 8 g .. 8 g + 7).  When either operand of a product has its
//     reduction index along columns instead, both take the other convention -- lane (r, g) carries reduction
//     indices 4 g .. 4 g + 3 and 16 + 4 g .. 16 + 4 g + 3 -- read with two 8-byte reads, or two transposing reads
//     (ds_read_tr16_b64) on the strided side.  The matrix instruction sums over whatever indices each slot holds,
//     as long as both operands agree.
//   * The d_v columns are taken 32 at a time (one reduction step of the products over d_v); the state and state
//     gradient slabs are read as bf16 from the workspace with 64-token chunks (the matrix-core state passes store
//     them rounded to bf16) and rounded to bf16 on the way into LDS from the fp32 workspace otherwise.
// T = (I + D strict_lower(L))^{-1} comes from the UT launch (its T^T export, bf16), and L = K K^T is formed only where
// dalpha needs it, on the tiles of W2 the wave holds, so no fp32 C x C matrix passes through LDS.
#pragma once

#include "efla_bwd.hpp"

namespace efla {

namespace bwdx {

typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

// 8 consecutive bf16 at a 16-byte aligned LDS address
__device__ __forceinline__ bf16x8 ld8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
// 4 consecutive bf16 at an 8-byte aligned LDS address
__device__ __forceinline__ bf16x4 ld4(const bf16* p) { return *reinterpret_cast<const bf16x4*>(p); }
// transposing read of a row-major bf16 block X (leading dimension baked into tr_off = Mma<bf16>::tr_offset):
// lane (r, g) receives X[4 g .. 4 g + 3][r]
__device__ __forceinline__ bf16x4 ldt(const bf16* X, int tr_off) {
    return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(X + tr_off)));
}

// acc += A B over a reduction of K (a multiple of 32) on the wave's tiles of an M x N product (tile assignment of
// bwd::Acc).  A(i, k) is A[i * lda + k] when AK (reduction index contiguous), else A[k * lda + i]; B(k, j) is
// B[j * ldb + k] when BK, else B[k * ldb + j].  Reduction steps in the outer loop, the wave's tiles inside, so that
// consecutive matrix instructions are independent.
template <int M, int N, int NWV, bool AK, bool BK, int K>
__device__ __forceinline__ void mmx(bwd::Acc<M, N, NWV>& acc, const bf16* A, int lda, const bf16* B, int ldb, int w,
                                    int lane) {
    typedef bwd::Acc<M, N, NWV> AC;
    constexpr int TPW = AC::TPW;
    static_assert(K % 32 == 0, "reduction in steps of 32");
    const int r = lane & 15, g = lane >> 4;
    const int tra = Mma<bf16>::tr_offset(lane, lda), trb = Mma<bf16>::tr_offset(lane, ldb);
    const bool last = AC::ALL || w + NWV * (TPW - 1) < AC::NTT;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 32) {
#pragma unroll
        for (int s = 0; s < TPW; ++s) {
            if (s == TPW - 1 && !last) continue;
            const int tt = w + NWV * s;
            const int ti = tt / AC::TN, tj = tt - ti * AC::TN;
            if constexpr (AK && BK) {
                const bf16x8 a = ld8(A + (16 * ti + r) * lda + k0 + 8 * g);
                const bf16x8 b = ld8(B + (16 * tj + r) * ldb + k0 + 8 * g);
                acc.t[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc.t[s], 0, 0, 0);
            } else {
                bf16x4 a0, a1, b0, b1;
                if constexpr (AK) {
                    const bf16* pa = A + (16 * ti + r) * lda + k0 + 4 * g;
                    a0 = ld4(pa);
                    a1 = ld4(pa + 16);
                } else {
                    a0 = ldt(A + k0 * lda + 16 * ti, tra);
                    a1 = ldt(A + (k0 + 16) * lda + 16 * ti, tra);
                }
                if constexpr (BK) {
                    const bf16* pb = B + (16 * tj + r) * ldb + k0 + 4 * g;
                    b0 = ld4(pb);
                    b1 = ld4(pb + 16);
                } else {
                    b0 = ldt(B + k0 * ldb + 16 * tj, trb);
                    b1 = ldt(B + (k0 + 16) * ldb + 16 * tj, trb);
                }
                Mma<bf16>::mma2(acc.t[s], a0, a1, b0, b1);
            }
        }
    }
}

// The wave's tiles of C^T for an M x N product C formed with its operands exchanged (an Acc<N, M>): lane (r, g) of
// tile (ti, tj) holds C[16 tj + r][16 ti + 4 g .. + 3], four consecutive columns of one row of C, so that the
// row-major LDS tiles take them with one 8-byte access.  f(row, col0, x) for each of the wave's tiles.
template <int MT, int NT, int NWV, class F>
__device__ __forceinline__ void rows4(bwd::Acc<MT, NT, NWV>& at, int w, int lane, F f) {
    typedef bwd::Acc<MT, NT, NWV> AC;
#pragma unroll
    for (int s = 0; s < AC::TPW; ++s) {
        const int tt = w + NWV * s;
        if (AC::ALL || tt < AC::NTT) {
            const int ti = tt / AC::TN, tj = tt - ti * AC::TN;
            f(16 * tj + (lane & 15), 16 * ti + 4 * (lane >> 4), at.t[s]);
        }
    }
}
__device__ __forceinline__ void st4(bf16* p, const f32x4& x) { *reinterpret_cast<bf16x4*>(p) = Mma<bf16>::cvt(x); }
__device__ __forceinline__ f32x4 ld4f(const bf16* p) {
    const bf16x4 h = ld4(p);
    return f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
}

// ROWS x COLS of a row-major global matrix (row stride ld elements, 16-byte aligned rows) in registers between a
// load (16 bytes per thread and request; rows >= n read as zeros) and a store into a bf16 LDS tile (row stride sld,
// a multiple of 8).
template <typename E, int ROWS, int COLS, int NTH>
struct TileB {
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
    __device__ __forceinline__ void store(bf16* s, int sld, int tid) const {
#pragma unroll
        for (int it = 0; it < N; ++it) {
            const int idx = it * NTH + tid, r = idx / VPR, c = (idx - r * VPR) * VEC;
            if (TOT % NTH == 0 || idx < TOT) {
                if constexpr (VEC == 8) {
                    *reinterpret_cast<bf16x8*>(s + r * sld + c) = x[it];
                } else {
                    bf16x4 h;
#pragma unroll
                    for (int e = 0; e < 4; ++e) h[e] = (bf16)x[it][e];
                    *reinterpret_cast<bf16x4*>(s + r * sld + c) = h;
                }
            }
        }
    }
};

// LDS of the kernel (byte offsets): bf16 tiles Q, K (C x DK), P and T^T (C x C), the d_v slab tiles S, dS' (DK x NV)
// and V (then D R), dO, Delta, dDelta, G, -dR (C x NV); four fp32 C-vectors; the fp32 row sums behind dalpha, one C-vector per
// 16-column tile column of G o R (NV / 16) and of strict_lower(L) o W2 (C / 16), each element written by one lane.
template <int DK, int C, int NV_>
struct BwdXLds {
    static constexpr int NV = NV_;   // d_v columns per slab (32 or 64)
    static constexpr int LDK = DK + 8, LDC = C + 8, LDV = NV + 16;   // row padding (elements) measured best
    static constexpr int Q = 0;
    static constexpr int K = Q + C * LDK * 2;
    static constexpr int P = K + C * LDK * 2;
    static constexpr int T = P + C * LDC * 2;
    static constexpr int S = T + C * LDC * 2;
    static constexpr int G2 = S + DK * LDV * 2;
    static constexpr int V = G2 + DK * LDV * 2;
    static constexpr int O = V + C * LDV * 2;
    static constexpr int DL = O + C * LDV * 2;
    static constexpr int DD = DL + C * LDV * 2;
    static constexpr int GS = DD + C * LDV * 2;
    static constexpr int DRN = GS + C * LDV * 2;
    static constexpr int AL = DRN + C * LDV * 2;
    static constexpr int RS = AL + 4 * C * 4;
    static constexpr int BYTES = RS + (NV / 16 + C / 16) * C * 4;
};

}  // namespace bwdx

constexpr int kChunkXThreads = 512;   // eight waves

template <int DK, int C, int NVS>
__global__ __launch_bounds__(kChunkXThreads) void bwd_chunk_mx_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v, const float* __restrict__ beta,
    const bf16* __restrict__ d_o, const void* __restrict__ s_all, const void* __restrict__ ds_all,
    const bf16* __restrict__ tt, bf16* __restrict__ dq, bf16* __restrict__ dk, float* __restrict__ dbeta, int L, int DV,
    int gate, TokLayout ly) {
    using namespace bwd;
    using namespace bwdx;
    constexpr int NWV = kChunkXThreads / 64;
    constexpr int NTH = kChunkXThreads;
    typedef BwdXLds<DK, C, NVS> LY;
    constexpr int NV = LY::NV, LDK = LY::LDK, LDC = LY::LDC, LDV = LY::LDV;
    static_assert(DK % 32 == 0 && C % 32 == 0, "d_k and chunk multiples of 32");
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_x[];
    bf16* sQ = reinterpret_cast<bf16*>(smem_x + LY::Q);
    bf16* sK = reinterpret_cast<bf16*>(smem_x + LY::K);
    bf16* sP = reinterpret_cast<bf16*>(smem_x + LY::P);    // lower_incl(Q K^T); later M o W1
    bf16* sT = reinterpret_cast<bf16*>(smem_x + LY::T);    // T^T; later dL
    bf16* sS = reinterpret_cast<bf16*>(smem_x + LY::S);    // S[:, slab]
    bf16* sG2 = reinterpret_cast<bf16*>(smem_x + LY::G2);  // dS'[:, slab]
    bf16* sV = reinterpret_cast<bf16*>(smem_x + LY::V);    // V slab; then D R
    bf16* sO = reinterpret_cast<bf16*>(smem_x + LY::O);    // dO slab
    bf16* sDl = reinterpret_cast<bf16*>(smem_x + LY::DL);  // Delta slab
    bf16* sDd = reinterpret_cast<bf16*>(smem_x + LY::DD);  // dDelta slab
    bf16* sGs = reinterpret_cast<bf16*>(smem_x + LY::GS);  // G slab
    bf16* sDr = reinterpret_cast<bf16*>(smem_x + LY::DRN); // -dR slab
    float* sAl = reinterpret_cast<float*>(smem_x + LY::AL);
    float* sDb = sAl + C;
    float* sDlam = sDb + C;
    float* sDa = sDlam + C;
    float* sGR = reinterpret_cast<float*>(smem_x + LY::RS);   // [NV / 16][C]: rowsum(G o R) by tile column
    float* sLW = sGR + (NV / 16) * C;                         // [C / 16][C]: rowsum(strict_lower(L) o W2) likewise

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int bh, c;
    SeqView sv;
    if (!chunk_at(ly, blockIdx.x, L, C, bh, c, sv)) return;
    (void)bh;
    const int t0 = c * C, n = sv.len - t0 < C ? sv.len - t0 : C;
    const int64_t q0 = sv.q0 + (int64_t)t0 * ly.q_t, k0 = sv.k0 + (int64_t)t0 * ly.k_t;   // the chunk's first rows
    const int64_t v0 = sv.v0 + (int64_t)t0 * ly.v_t, o0 = sv.o0 + (int64_t)t0 * ly.o_t;
    const int64_t be0 = sv.be0 + (int64_t)t0 * ly.be_t;
    const int64_t u = blockIdx.x;   // workgroup u works on chunk u of the workspace
    // the chunk's entering state and leaving state gradient: bf16 with 64-token chunks (the state passes on
    // matrix cores store them rounded as this kernel would), else fp32
    typedef typename std::conditional<C == 64, bf16, float>::type SE;
    const SE* Sg = static_cast<const SE*>(s_all) + u * DK * DV;
    const SE* dSg = static_cast<const SE*>(ds_all) + u * DK * DV;

    {
        TileB<bf16, C, DK, NTH> tq, tk;
        TileB<bf16, C, C, NTH> ttl;
        tq.load(q + q0, ly.q_t, n, tid);
        tk.load(k + k0, ly.k_t, n, tid);
        ttl.load(tt + u * C * C, C, C, tid);
        tq.store(sQ, LDK, tid);
        tk.store(sK, LDK, tid);
        ttl.store(sT, LDC, tid);
    }
    // the d_v slabs' tiles, loaded one slab ahead
    TileB<SE, DK, NV, NTH> ts, tds;
    TileB<bf16, C, NV, NTH> tv, to;
    auto load_slab = [&](int col0) {
        ts.load(Sg + col0, DV, DK, tid);
        tds.load(dSg + col0, DV, DK, tid);
        tv.load(v + v0 + col0, ly.v_t, n, tid);
        to.load(d_o + o0 + col0, ly.o_t, n, tid);
    };
    load_slab(0);
    if (tid < (NV / 16) * C) sGR[tid] = 0.0f;
    __syncthreads();
    if (tid < C) {   // gates of the chunk's tokens (rows past the end: zero keys, zero step)
        float lam = 0.0f;   // exact bf16 squares summed in fp32, 16 bytes of the key row per read
#pragma unroll
        for (int e = 0; e < DK; e += 8) lam += sum_sq(ld8(sK + tid * LDK + e));
        const float b = tid < n ? beta[be0 + (int64_t)tid * ly.be_t] : 0.0f;
        sAl[tid] = gate_alpha(b, lam, gate);
        float db, dl;
        gate_alpha_grad(b, lam, gate, &db, &dl);
        sDb[tid] = db;
        sDlam[tid] = dl;
    }
    // Every product below is formed with its operands exchanged (C^T = B^T A^T), so that each lane's accumulator
    // elements are four consecutive columns of one row of C (rows4).
    {   // P = lower_incl(Q K^T)
        Acc<C, C, NWV> b;
        b.zero();
        mmx<C, C, NWV, true, true, DK>(b, sK, LDK, sQ, LDK, w, lane);
        rows4(b, w, lane, [&](int i, int j0, f32x4& x) {
            f32x4 y;
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = j0 + e <= i ? x[e] : 0.0f;
            st4(sP + i * LDC + j0, y);
        });
    }
    __syncthreads();

    Acc<DK, C, NWV> aQ, aK;   // dQ^T, dK^T
    Acc<C, C, NWV> W1, W2;
    aQ.zero();
    aK.zero();
    W1.zero();
    W2.zero();
    for (int col0 = 0; col0 < DV; col0 += NV) {
        ts.store(sS, LDV, tid);
        tds.store(sG2, LDV, tid);
        tv.store(sV, LDV, tid);
        to.store(sO, LDV, tid);
        __syncthreads();
        if (col0 + NV < DV) load_slab(col0 + NV);
        // phase A: R = V - K S (kept for dalpha; D R over V) and dDelta = K dS' + P^T dO -- the two share the key
        // fragments and need nothing from each other
        Acc<NV, C, NWV> R, dD;   // R^T, dDelta^T
        R.zero();
        dD.zero();
        mmx<NV, C, NWV, false, true, DK>(R, sS, LDV, sK, LDK, w, lane);
        mmx<NV, C, NWV, false, true, DK>(dD, sG2, LDV, sK, LDK, w, lane);
        mmx<NV, C, NWV, false, false, C>(dD, sO, LDV, sP, LDC, w, lane);
        // each element of sV is read and then overwritten by the one lane that holds it in R: no barrier between
        rows4(R, w, lane, [&](int i, int j0, f32x4& x) {
            x = ld4f(sV + i * LDV + j0) - x;
            st4(sV + i * LDV + j0, sAl[i] * x);
        });
        rows4(dD, w, lane, [&](int i, int j0, f32x4& x) { st4(sDd + i * LDV + j0, x); });
        __syncthreads();
        {   // phase B: Delta = T (D R); G = T^T dDelta; -dR = -D G; dalpha += rowsum(G o R)
            Acc<NV, C, NWV> a, gg;   // Delta^T, G^T
            a.zero();
            gg.zero();
            mmx<NV, C, NWV, false, false, C>(a, sV, LDV, sT, LDC, w, lane);
            mmx<NV, C, NWV, false, true, C>(gg, sDd, LDV, sT, LDC, w, lane);
            rows4(a, w, lane, [&](int i, int j0, f32x4& x) { st4(sDl + i * LDV + j0, x); });
            rows4(gg, w, lane, [&](int i, int j0, f32x4& x) {
                st4(sGs + i * LDV + j0, x);
                st4(sDr + i * LDV + j0, -sAl[i] * x);
            });
            // rows of this lane's elements: the same (tile, row) for gg and R, summed over the tile's 16 columns (the
            // lane's four, then across the four lane rows) into the tile column's row sums (a tile belongs to the
            // same wave in every slab: one writer per element, and a fixed order of the sums, so the gradients do not
            // depend on the waves' timing)
            typedef Acc<NV, C, NWV> AN;
#pragma unroll
            for (int s = 0; s < AN::TPW; ++s) {
                const int tt = w + NWV * s;
                if (AN::ALL || tt < AN::NTT) {
                    const int ti = tt / AN::TN, tj = tt - ti * AN::TN;
                    float p = (gg.t[s][0] * R.t[s][0] + gg.t[s][1] * R.t[s][1]) +
                              (gg.t[s][2] * R.t[s][2] + gg.t[s][3] * R.t[s][3]);
                    p = cross_row_sum(p);
                    if ((lane >> 4) == 0) sGR[ti * C + 16 * tj + (lane & 15)] += p;
                }
            }
        }
        __syncthreads();
        // dQ += dO S^T; dK += Delta dS'^T - dR S^T; W1 += dO Delta^T; W2 += G Delta^T (reduction over the slab)
        mmx<DK, C, NWV, true, true, NV>(aQ, sS, LDV, sO, LDV, w, lane);
        mmx<DK, C, NWV, true, true, NV>(aK, sG2, LDV, sDl, LDV, w, lane);
        mmx<DK, C, NWV, true, true, NV>(aK, sS, LDV, sDr, LDV, w, lane);
        mmx<C, C, NWV, true, true, NV>(W1, sDl, LDV, sO, LDV, w, lane);
        mmx<C, C, NWV, true, true, NV>(W2, sDl, LDV, sGs, LDV, w, lane);
        __syncthreads();
    }

    // M o W1 into sP; dL = -strict_lower(D W2) into sT (T is no longer needed); the row sums of strict_lower(L) o W2
    // by tile column, with L = K K^T formed on the wave's tiles of W2
    rows4(W1, w, lane, [&](int i, int j0, f32x4& x) {
        f32x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = j0 + e <= i ? x[e] : 0.0f;
        st4(sP + i * LDC + j0, y);
    });
    rows4(W2, w, lane, [&](int i, int j0, f32x4& x) {
        f32x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = j0 + e < i ? -sAl[i] * x[e] : 0.0f;
        st4(sT + i * LDC + j0, y);
    });
    {
        typedef Acc<C, C, NWV> AC;
        AC Lt;   // L = K K^T is symmetric: its tiles line up with those of W2^T element by element
        Lt.zero();
        mmx<C, C, NWV, true, true, DK>(Lt, sK, LDK, sK, LDK, w, lane);
#pragma unroll
        for (int s = 0; s < AC::TPW; ++s) {
            const int tt2 = w + NWV * s;
            if (AC::ALL || tt2 < AC::NTT) {
                const int ti = tt2 / AC::TN, tj = tt2 - ti * AC::TN;
                const int row = 16 * tj + (lane & 15), col0 = 16 * ti + 4 * (lane >> 4);
                float q[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) q[e] = col0 + e < row ? Lt.t[s][e] * W2.t[s][e] : 0.0f;
                float p = (q[0] + q[1]) + (q[2] + q[3]);
                p = cross_row_sum(p);
                if ((lane >> 4) == 0) sLW[ti * C + row] = p;
            }
        }
    }
    __syncthreads();
    // dalpha = rowsum(G o R) - rowsum(strict_lower(L) o W2), tile columns summed in order; dbeta; dlambda
    if (tid < C) {
        const int i = tid;
        float gr = 0.0f, lw = 0.0f;
#pragma unroll
        for (int j = 0; j < NV / 16; ++j) gr += sGR[j * C + i];
#pragma unroll
        for (int j = 0; j < C / 16; ++j) lw += sLW[j * C + i];
        const float s = gr - lw;
        if (i < n) dbeta[be0 + (int64_t)i * ly.be_t] = s * sDb[i];
        sDa[i] = s * sDlam[i];
    }
    __syncthreads();
    // dQ += (M o W1) K;  dK += (M o W1)^T Q + dL K + dL^T K + 2 dlambda o K
    mmx<DK, C, NWV, false, true, C>(aQ, sK, LDK, sP, LDC, w, lane);
    mmx<DK, C, NWV, false, false, C>(aK, sQ, LDK, sP, LDC, w, lane);
    mmx<DK, C, NWV, false, true, C>(aK, sK, LDK, sT, LDC, w, lane);
    mmx<DK, C, NWV, false, false, C>(aK, sK, LDK, sT, LDC, w, lane);
    // dQ and dK staged as bf16 tiles in the slab tiles' space (no product reads it any more), then written as
    // 16-byte pieces of the chunk's rows
    static_assert(2 * C * LDK * 2 <= LY::AL - LY::S, "dQ and dK tiles fit where the slab tiles were");
    bf16* sDQ = reinterpret_cast<bf16*>(smem_x + LY::S);
    bf16* sDK = sDQ + C * LDK;
    rows4(aQ, w, lane, [&](int i, int e0, f32x4& x) { st4(sDQ + i * LDK + e0, x); });
    rows4(aK, w, lane, [&](int i, int e0, f32x4& x) {
        const f32x4 kr = ld4f(sK + i * LDK + e0);
        f32x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = fmaf(2.0f * sDa[i], kr[e], x[e]);
        st4(sDK + i * LDK + e0, y);
    });
    __syncthreads();
    for (int idx = tid; idx < C * (DK / 8); idx += NTH) {
        const int r = idx / (DK / 8), c8 = (idx - r * (DK / 8)) * 8;
        if (r < n) {
            *reinterpret_cast<bf16x8*>(dq + q0 + (int64_t)r * ly.q_t + c8) = ld8(sDQ + r * LDK + c8);
            *reinterpret_cast<bf16x8*>(dk + k0 + (int64_t)r * ly.k_t + c8) = ld8(sDK + r * LDK + c8);
        }
    }
}

template <int DK, int C, int NV>
hipError_t launch_bwd_chunk_mx_nv(const BwdArgs& a, hipStream_t s) {
    constexpr int LDS = bwdx::BwdXLds<DK, C, NV>::BYTES;
    static_assert(LDS <= kMaxLdsBytes, "matrix-core chunk kernel LDS too large");
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_chunk_mx_kernel<DK, C, NV>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_chunk_mx_kernel<DK, C, NV>), dim3((unsigned)bwd_chunk_grid(a, C)), dim3(kChunkXThreads), LDS,
                       s, static_cast<const bf16*>(a.q), static_cast<const bf16*>(a.k), static_cast<const bf16*>(a.v),
                       a.beta, static_cast<const bf16*>(a.d_o), a.s_all, a.ds_all, static_cast<const bf16*>(a.tt),
                       static_cast<bf16*>(a.dq), static_cast<bf16*>(a.dk), a.dbeta, a.L, a.d_v, a.gate, bwd_layout(a));
    return hipGetLastError();
}

// Launches the matrix-core chunk kernel when it applies (bf16, d_k >= 32, chunk 32 or 64, d_v a multiple of 32, and
// the UT launch wrote T^T); returns false otherwise, leaving the launch to bwd_chunk_kernel.  The d_v columns are
// taken 64 at a time where d_v allows (the products over a slab then reuse each operand fragment for two tiles of
// a wave, and a chunk has half as many slab phases), else 32.
template <int DK, int C>
bool launch_bwd_chunk_mx(const BwdArgs& a, hipStream_t s, hipError_t* err) {
    if constexpr (DK < 32 || C < 32) {
        (void)a;
        (void)s;
        (void)err;
        return false;
    } else {
        if (a.d_v % 32 != 0 || a.tt == nullptr) return false;
        if ((C == 64) != a.sbf) {   // the kernel reads bf16 states exactly with 64-token chunks
            *err = hipErrorInvalidValue;
            return true;
        }
        *err = a.d_v % 64 == 0 ? launch_bwd_chunk_mx_nv<DK, C, 64>(a, s) : launch_bwd_chunk_mx_nv<DK, C, 32>(a, s);
        return true;
    }
}

template <int DK, int C>
struct BwdChunkFast<bf16, DK, C> {
    static bool launch(const BwdArgs& a, hipStream_t s, hipError_t* e) { return launch_bwd_chunk_mx<DK, C>(a, s, e); }
};

}  // namespace efla
