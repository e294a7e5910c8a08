// efla_chunk_fwd.hpp -- fused chunkwise-parallel EFLA forward for gfx950 (one kernel, one pass over HBM).
//
// The recurrence S_t = (I - alpha_t k_t k_t^T) S_{t-1} + alpha_t k_t v_t^T, o_t = S_t^T q_t keeps the
// rank-1 delta-rule structure, so it can be regrouped over chunks of C tokens ("Exact Flow Linear
// Attention" (gist.science), Metodologia item 3; "Error-Free Linear Attention is a Free Lunch"
// (howistudyai.com), Step 4).  With S the state entering a chunk and K, Q, V, alpha its rows:
//   A     = strict_lower(diag(alpha) K K^T)             (C x C)
//   T     = (I + A)^{-1}                                (unit lower triangular)
//   R     = V - K S                                     (C x d_v)
//   Delta = T diag(alpha) R                             (row t: the rank-1 write u_t of token t)
//   O     = Q S + lower_incl(Q K^T) Delta               (readout after each token's update)
//   S    <- S + K^T Delta
// (Unrolling u_t = alpha_t (v_t - S_{t-1}^T k_t) inside the chunk gives (I + A) Delta = diag(alpha) R.)
//
// Work split.  One workgroup per (batch*head, slab of DVS state columns); the columns of S evolve
// independently, so slabs never talk to each other.  Each wave owns 16 columns of the slab and keeps
// its d_k x 16 piece of S in fp32 accumulator registers for the whole sequence.  Per chunk:
//   1. the chunk's Q, K, V slab (prefetched into registers during the previous chunk) go to LDS, with
//      lambda = ||k||^2 reduced across the lanes holding a key row; the next chunk's global loads are
//      issued right after;
//   2. per wave: alpha for 16 tokens, a Gram block row alpha_i k_i.k_j (upper tiles, stored transposed =
//      lower) and a block row of Q K^T on the matrix cores; the wave then solves its 16x16 diagonal block
//      of T by right-looking forward substitution in fp32 (lane r carries column r; step m reads column m
//      of the block as one broadcast LDS row);
//   3. the off-diagonal blocks of T, one block column per wave, walked down the column with the blocks
//      found so far kept in registers: T_IJ = -T_II sum_m A_Im T_mJ on the matrix cores; T diag(alpha)
//      is written as a matrix-core operand;
//   4. per wave: K S and (Q S)^T, R = V - K S, Delta = T diag(alpha) R, O^T = (Q S)^T + Delta^T P^T
//      (stored, four consecutive outputs per lane), S += K^T Delta -- all on the matrix cores with the
//      state as an in-register operand.
// Operands that must be read "down a column" (K^T, V) are fetched with the transposing LDS read, so K and
// V live in LDS once, row-major.  T and T diag(alpha) are stored transposed (every writer then emits
// contiguous runs) and read back with plain or transposing quad reads as the product needs.
// bf16 inputs use the 16x16x32 bf16 instruction with fp32 accumulation (S, R, Delta and T diag(alpha)
// are rounded to bf16 only as instruction operands; the carried state stays fp32); fp32 inputs use the
// 16x16x4 fp32 instruction throughout.
#pragma once

#include "efla_common.hpp"
#include "efla_launch.hpp"
#include "efla_ut.hpp"

namespace efla {

// LDS carve-up of one workgroup.  Row strides of the storage-type matrices are padded by 20 elements
// for bf16 (40 bytes: quad reads of 16 consecutive rows hit distinct banks and the transposing reads
// of 4 rows at most pair up) and by 4 elements for fp32.
template <int ESIZE, int DK, int C, int DVS>
struct ChunkLayout {
    static constexpr int PAD = ESIZE == 2 ? 20 : 4;
    static constexpr int LD_DK = DK + PAD;   // sQ, sK   [C][LD_DK]   storage type, row-major
    static constexpr int LD_V = DVS + PAD;   // sV       [C][LD_V]    storage type
    static constexpr int LD_CE = C + PAD;    // sA, sTt, sTat, sP [C][LD_CE] storage type
    static constexpr int OFF_Q = 0;
    static constexpr int OFF_K = OFF_Q + C * LD_DK * ESIZE;
    static constexpr int OFF_V = OFF_K + C * LD_DK * ESIZE;
    static constexpr int OFF_A = OFF_V + C * LD_V * ESIZE;    // alpha_i k_i.k_j, off-diagonal blocks
    static constexpr int OFF_AT = OFF_A + C * LD_CE * ESIZE;
    static constexpr int OFF_TT = OFF_AT + C * kLdAt * 4;       // T^T (diagonal blocks used)
    static constexpr int OFF_TAT = OFF_TT + C * LD_CE * ESIZE;  // (T diag(alpha))^T
    static constexpr int OFF_P = OFF_TAT + C * LD_CE * ESIZE;
    static constexpr int OFF_LB = OFF_P + C * LD_CE * ESIZE;   // lambda[C], beta[C] (fp32)
    static constexpr int OFF_ALPHA = OFF_LB + 2 * C * 4;
    static constexpr int BYTES = OFF_ALPHA + C * 4;
};

// host-side mirror of ChunkLayout::BYTES
template <int ESIZE>
constexpr int chunk_layout_bytes(int dk, int c, int dvs) {
    const int pad = ESIZE == 2 ? 20 : 4;
    return c * (dk + pad) * ESIZE * 2 + c * (dvs + pad) * ESIZE + c * (c + pad) * ESIZE * 4 + c * 20 * 4 + c * 4 * 3;
}

// global -> register staging of one chunk; prefetched when it fits in a few registers per thread
template <typename E, int DK, int C, int DVS, int NT>
struct ChunkStage {
    typedef typename Vec16<E>::type V16;
    static constexpr int VEC = Vec16<E>::N;
    static constexpr int VPR = DK / VEC;            // 16-byte vectors per key row (2..32, divides 64)
    static constexpr int NQK = (C * VPR + NT - 1) / NT;
    static constexpr int VPRV = DVS / VEC;
    static constexpr int NV = (C * VPRV + NT - 1) / NT;
    V16 q[NQK], k[NQK], v[NV];
    float beta[NQK];

    __device__ __forceinline__ void load(const E* __restrict__ gq, const E* __restrict__ gk, const E* __restrict__ gv,
                                         const float* __restrict__ gbeta, int64_t tok, int n, int DV, int slab_col,
                                         int tid) {
        // chunk base pointers are uniform; lanes add 32-bit offsets
        const E* q0 = gq + tok * DK;
        const E* k0 = gk + tok * DK;
        const E* v0 = gv + tok * DV + slab_col;
        const float* b0 = gbeta + tok;
#pragma unroll
        for (int it = 0; it < NQK; ++it) {
            const int idx = it * NT + tid;
            const int t = idx / VPR;
            const int cv = idx % VPR;
            q[it] = V16{};
            k[it] = V16{};
            beta[it] = 0.0f;
            if (idx < C * VPR && t < n) {
                q[it] = *reinterpret_cast<const V16*>(q0 + (t * DK + cv * VEC));
                k[it] = *reinterpret_cast<const V16*>(k0 + (t * DK + cv * VEC));
                if (cv == 0) beta[it] = b0[t];
            }
        }
#pragma unroll
        for (int it = 0; it < NV; ++it) {
            const int idx = it * NT + tid;
            const int t = idx / VPRV;
            const int cv = idx % VPRV;
            v[it] = V16{};
            if (idx < C * VPRV && t < n) v[it] = *reinterpret_cast<const V16*>(v0 + (t * DV + cv * VEC));
        }
    }
};

template <typename E, int DK, int C, int DVS>
__global__ __launch_bounds__(DVS / 16 * 64) void chunk_fwd_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v, const float* __restrict__ beta,
    E* __restrict__ o, const float* s0, float* sf, int BH, int L, int DV, int nslab, int gate) {
    typedef ChunkLayout<sizeof(E), DK, C, DVS> LY;
    typedef Mma<E> M;
    typedef typename M::quad quad;
    constexpr int NW = DVS / 16;
    constexpr int NT = NW * 64;
    constexpr int NB = C / 16;
    constexpr int NKD = DK / 16;
    constexpr int LD_DK = LY::LD_DK, LD_V = LY::LD_V, LD_CE = LY::LD_CE;
    typedef ChunkStage<E, DK, C, DVS, NT> Stage;
    // prefetching keeps one chunk in registers: only when that is a few registers per thread
    constexpr bool kPrefetch = (2 * Stage::NQK + Stage::NV) <= 12;
    static_assert(LY::BYTES <= kMaxLdsBytes, "chunk kernel LDS too large");

    __shared__ __attribute__((aligned(16))) unsigned char smem[LY::BYTES];
    E* sQ = reinterpret_cast<E*>(smem + LY::OFF_Q);
    E* sK = reinterpret_cast<E*>(smem + LY::OFF_K);
    E* sV = reinterpret_cast<E*>(smem + LY::OFF_V);
    E* sA = reinterpret_cast<E*>(smem + LY::OFF_A);
    float* sLam = reinterpret_cast<float*>(smem + LY::OFF_LB);
    float* sBeta = sLam + C;
    float* sAt = reinterpret_cast<float*>(smem + LY::OFF_AT);
    E* sTt = reinterpret_cast<E*>(smem + LY::OFF_TT);
    E* sTat = reinterpret_cast<E*>(smem + LY::OFF_TAT);
    E* sP = reinterpret_cast<E*>(smem + LY::OFF_P);
    float* sAlpha = reinterpret_cast<float*>(smem + LY::OFF_ALPHA);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int r = lane & 15;
    const int g = lane >> 4;
    const int tr_dk = M::tr_offset(lane, LD_DK);
    const int tr_v = M::tr_offset(lane, LD_V);
    const int tr_ce = M::tr_offset(lane, LD_CE);

    // Workgroup -> (batch*head, slab).  Consecutive workgroups go to different XCDs (round robin over 8),
    // so the slabs of one head are placed 8 apart to share an XCD and its L2 (they read the same Q, K).
    const int bid = blockIdx.x;
    const int slab = (bid >> 3) % nslab;
    const int bh = ((bid >> 3) / nslab) * 8 + (bid & 7);
    if (bh >= BH) return;
    const int slab_col = slab * DVS;
    const int colw = slab_col + 16 * w;     // first state column owned by this wave
    const int64_t tok0 = (int64_t)bh * L;

    // this wave's piece of the state: S[16 rt + 4g + i][colw + r]
    f32x4 S[NKD];
#pragma unroll
    for (int rt = 0; rt < NKD; ++rt) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[rt][i] = s0 ? s0[((int64_t)bh * DK + 16 * rt + 4 * g + i) * DV + colw + r] : 0.0f;
    }

    Stage st;
    if constexpr (kPrefetch) {
        if (L > 0) st.load(q, k, v, beta, tok0, L < C ? L : C, DV, slab_col, tid);
    }

    for (int t0 = 0; t0 < L; t0 += C) {
        const int n = (L - t0 < C) ? (L - t0) : C;

        // ---- 1. chunk -> LDS; lambda and alpha per token; next chunk's loads in flight -------------
        {
            if constexpr (!kPrefetch) st.load(q, k, v, beta, tok0 + t0, n, DV, slab_col, tid);
#pragma unroll
            for (int it = 0; it < Stage::NQK; ++it) {
                const int idx = it * NT + tid;
                const int t = idx / Stage::VPR;
                const int cv = idx % Stage::VPR;
                const float ss = group_sum<Stage::VPR>(sum_sq(st.k[it]));
                if (idx < C * Stage::VPR) {
                    lds_store_vec16(sQ + t * LD_DK + cv * Stage::VEC, st.q[it]);
                    lds_store_vec16(sK + t * LD_DK + cv * Stage::VEC, st.k[it]);
                    if (cv == 0) {
                        sLam[t] = ss;
                        sBeta[t] = st.beta[it];
                    }
                }
            }
#pragma unroll
            for (int it = 0; it < Stage::NV; ++it) {
                const int idx = it * NT + tid;
                if (idx < C * Stage::VPRV) {
                    const int t = idx / Stage::VPRV;
                    const int cv = idx % Stage::VPRV;
                    lds_store_vec16(sV + t * LD_V + cv * Stage::VEC, st.v[it]);
                }
            }
            if constexpr (kPrefetch) {
                const int t1 = t0 + C;
                if (t1 < L) st.load(q, k, v, beta, tok0 + t1, (L - t1 < C) ? (L - t1) : C, DV, slab_col, tid);
            }
        }
        __syncthreads();

        // ---- 2. per wave: Gram block row hi (-> A; its diagonal block is solved right here for T_hh) and
        //         Q K^T block row NB-1-hi (-> P).  Both rows share the A-side K blocks; each row keeps its
        //         B-side block (K_hi, Q_hp) in registers across its tiles.
        ut_rows<E, DK, C, NW, LD_DK, LD_CE, true>(sQ, sK, sLam, sBeta, sA, sAt, sTt, sTat, sP, sAlpha, w, r, g, gate);
        __syncthreads();

        // ---- 3. off-diagonal blocks of T, one block column J per wave, walked down the column with the
        //         blocks already found kept in registers: T_IJ = -T_II sum_{m=J}^{I-1} A_Im T_mJ
        ut_offdiag<E, C, NW, LD_CE>(sA, sTt, sTat, sAlpha, w, r, g, tr_ce);
        __syncthreads();

        // ---- 4. the state-dependent part, per wave on its 16 columns ---------------------------------
        {
            quad Sq[NKD];
#pragma unroll
            for (int rt = 0; rt < NKD; ++rt) Sq[rt] = M::cvt(S[rt]);
            // Ot = (Q S)^T accumulates O transposed: lane (r, g), element e = O[16 rb + r][colw + 4g + e], so each
            // lane later stores four consecutive outputs of one token.  (Q S)^T = S^T Q^T takes the state quads
            // as the A operand and the same row quads of Q as the B operand.
            f32x4 Ot[NB];
            quad Rq[NB];
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) {
                f32x4 xk = {0.f, 0.f, 0.f, 0.f};
                Ot[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
                const E* pq = sQ + (16 * rb + r) * LD_DK + 4 * g;
                const E* pk = sK + (16 * rb + r) * LD_DK + 4 * g;
#pragma unroll
                for (int kd = 0; kd + 1 < NKD; kd += 2) {
                    M::mma2(Ot[rb], Sq[kd], Sq[kd + 1], M::lds_quad(pq + 16 * kd), M::lds_quad(pq + 16 * kd + 16));
                    M::mma2(xk, M::lds_quad(pk + 16 * kd), M::lds_quad(pk + 16 * kd + 16), Sq[kd], Sq[kd + 1]);
                }
                if constexpr (NKD & 1) {
                    M::mma1(Ot[rb], Sq[NKD - 1], M::lds_quad(pq + 16 * (NKD - 1)));
                    M::mma1(xk, M::lds_quad(pk + 16 * (NKD - 1)), Sq[NKD - 1]);
                }
                // R = V - K S: lane (r, g), element e: row 16 rb + 4g + e, column 16 w + r of the slab
                const quad vq = M::lds_quad_t(sV + 16 * rb * LD_V + 16 * w, LD_V, tr_v);
                f32x4 rr;
#pragma unroll
                for (int e = 0; e < 4; ++e) rr[e] = to_f32<E>(vq[e]) - xk[e];
                Rq[rb] = M::cvt(rr);
            }
            // Delta = T diag(alpha) R, block-lower-triangular product
            quad Dq[NB];
            static_for<NB>([&](auto rbc) {
                constexpr int rb = decltype(rbc)::value;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                // A quads of T diag(alpha) = column quads of its stored transpose
                const E* pt = sTat + 16 * rb;
                static_for<(rb + 1) / 2>([&](auto hc) {
                    constexpr int kb = 2 * decltype(hc)::value;
                    M::mma2(acc, M::lds_quad_t(pt + 16 * kb * LD_CE, LD_CE, tr_ce),
                            M::lds_quad_t(pt + 16 * (kb + 1) * LD_CE, LD_CE, tr_ce), Rq[kb], Rq[kb + 1]);
                });
                if constexpr ((rb + 1) & 1) M::mma1(acc, M::lds_quad_t(pt + 16 * rb * LD_CE, LD_CE, tr_ce), Rq[rb]);
                Dq[rb] = M::cvt(acc);
            });
            // O^T = (Q S)^T + Delta^T lower_incl(Q K^T)^T: Delta quads as the A operand, row quads of P as B;
            // each lane stores four consecutive outputs of token 16 rb + r with one vector store
            static_for<NB>([&](auto rbc) {
                constexpr int rb = decltype(rbc)::value;
                const E* pp = sP + (16 * rb + r) * LD_CE + 4 * g;
                static_for<(rb + 1) / 2>([&](auto hc) {
                    constexpr int kb = 2 * decltype(hc)::value;
                    M::mma2(Ot[rb], Dq[kb], Dq[kb + 1], M::lds_quad(pp + 16 * kb), M::lds_quad(pp + 16 * kb + 16));
                });
                if constexpr ((rb + 1) & 1) M::mma1(Ot[rb], Dq[rb], M::lds_quad(pp + 16 * rb));
                const int t = 16 * rb + r;
                if (t < n) *reinterpret_cast<quad*>(o + (tok0 + t0 + t) * DV + colw + 4 * g) = M::cvt(Ot[rb]);
            });
            // S += K^T Delta (K^T blocks fetched down the columns of K)
#pragma unroll
            for (int rt = 0; rt < NKD; ++rt) {
                const E* pk = sK + 16 * rt;
#pragma unroll
                for (int kb = 0; kb + 1 < NB; kb += 2)
                    M::mma2(S[rt], M::lds_quad_t(pk + 16 * kb * LD_DK, LD_DK, tr_dk),
                            M::lds_quad_t(pk + 16 * (kb + 1) * LD_DK, LD_DK, tr_dk), Dq[kb], Dq[kb + 1]);
                if constexpr (NB & 1) M::mma1(S[rt], M::lds_quad_t(pk + 16 * (NB - 1) * LD_DK, LD_DK, tr_dk), Dq[NB - 1]);
            }
        }
        __syncthreads();
    }

    if (sf) {
#pragma unroll
        for (int rt = 0; rt < NKD; ++rt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) sf[((int64_t)bh * DK + 16 * rt + 4 * g + i) * DV + colw + r] = S[rt][i];
        }
    }
}

template <typename E, int DK, int C, int DVS>
hipError_t launch_chunk_t(const void* q, const void* k, const void* v, const float* beta, void* o, const float* s0,
                          float* sf, int BH, int L, int DV, int gate, hipStream_t stream) {
    if constexpr (ChunkLayout<sizeof(E), DK, C, DVS>::BYTES > kMaxLdsBytes) {
        return hipErrorInvalidConfiguration;
    } else {
        const int nslab = DV / DVS;
        const int64_t grid = (int64_t)((BH + 7) / 8) * 8 * nslab;
        hipLaunchKernelGGL((chunk_fwd_kernel<E, DK, C, DVS>), dim3((unsigned)grid), dim3(DVS / 16 * 64), 0, stream,
                           static_cast<const E*>(q), static_cast<const E*>(k), static_cast<const E*>(v), beta,
                           static_cast<E*>(o), s0, sf, BH, L, DV, nslab, gate);
        return hipGetLastError();
    }
}

template <typename E, int DK, int C>
hipError_t launch_chunk_dvs(const ChunkArgs& a, hipStream_t s) {
    switch (a.dvs) {
        case 16: return launch_chunk_t<E, DK, C, 16>(a.q, a.k, a.v, a.beta, a.o, a.s0, a.sf, a.BH, a.L, a.d_v, a.gate, s);
        case 32: return launch_chunk_t<E, DK, C, 32>(a.q, a.k, a.v, a.beta, a.o, a.s0, a.sf, a.BH, a.L, a.d_v, a.gate, s);
        case 64: return launch_chunk_t<E, DK, C, 64>(a.q, a.k, a.v, a.beta, a.o, a.s0, a.sf, a.BH, a.L, a.d_v, a.gate, s);
    }
    return hipErrorInvalidValue;
}

template <typename E, int DK>
hipError_t launch_chunk_c(const ChunkArgs& a, hipStream_t s) {
    switch (a.chunk) {
        case 16: return launch_chunk_dvs<E, DK, 16>(a, s);
        case 32: return launch_chunk_dvs<E, DK, 32>(a, s);
        case 64: return launch_chunk_dvs<E, DK, 64>(a, s);
    }
    return hipErrorInvalidValue;
}

template <typename E>
hipError_t launch_chunk_e(const ChunkArgs& a, hipStream_t s) {
    switch (a.d_k) {
        case 16: return launch_chunk_c<E, 16>(a, s);
        case 32: return launch_chunk_c<E, 32>(a, s);
        case 64: return launch_chunk_c<E, 64>(a, s);
        case 128: return launch_chunk_c<E, 128>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace efla
