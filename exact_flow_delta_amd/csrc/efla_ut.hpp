// efla_ut.hpp -- the intra-chunk (state-independent) part of the chunkwise EFLA forward, as device
// phases shared by the fused chunk kernel and the stand-alone UT kernel.
//
// For one chunk of C tokens with keys K (rows k_t) and gates alpha_t:
//   A = strict_lower(diag(alpha) K K^T),   T = (I + A)^{-1}  (unit lower triangular),
// and the product the state pass needs is T diag(alpha).  ("Exact Flow Linear Attention"
// (gist.science), Metodologia item 3: the update keeps the delta-rule rank-1 form, so the WY/UT
// chunk scheme applies; "Error-Free Linear Attention is a Free Lunch" (howistudyai.com), Step 4:
// the within-chunk transforms do not depend on the state.)
//
// LDS operands (storage type E unless noted), row strides LD_DK / LD_CE as the caller lays them out:
//   sK [C][LD_DK]  keys, row-major;  sQ [C][LD_DK] queries (only with WITH_P)
//   sLam, sBeta [C] fp32: ||k_t||^2 and beta_t;  sAlpha [C] fp32: alpha_t (written)
//   sA  [C][LD_CE]: off-diagonal 16x16 blocks of A (written)
//   sAt [C][20] fp32: diagonal blocks of A, transposed (written, scratch)
//   sTt [C][LD_CE]: T^T, diagonal blocks and (after ut_offdiag) nothing else needed;  sTat: (T diag(alpha))^T
//   sP  [C][LD_CE]: lower_incl(Q K^T) (only with WITH_P)
#pragma once

#include <type_traits>

#include "efla_common.hpp"

namespace efla {

constexpr int kLdAt = 16 + 4;   // row stride of sAt (fp32)

// Per wave: for every block row hi with hi % NW == w, alpha of its 16 tokens, the Gram block row
// alpha_i k_i.k_j (off-diagonal blocks -> sA, the diagonal block -> sAt transposed) and, with WITH_P,
// block row NB-1-hi of lower_incl(Q K^T) (-> sP); then the wave solves its diagonal block
// T_hh = (I + A_hh)^{-1} by right-looking forward substitution in fp32: lane r carries column r and
// step m reads column m of the block as one broadcast row of sAt.  T_hh^T and (T_hh diag(alpha))^T
// go to sTt / sTat.  Both block rows share the A-side K blocks; each keeps its B-side block in registers.
template <typename E, int DK, int C, int NW, int LD_DK, int LD_CE, bool WITH_P>
__device__ __forceinline__ void ut_rows(const E* sQ, const E* sK, const float* sLam, const float* sBeta, E* sA,
                                        float* sAt, E* sTt, E* sTat, E* sP, float* sAlpha, int w, int r, int g,
                                        int gate) {
    typedef Mma<E> M;
    typedef typename M::quad quad;
    constexpr int NB = C / 16;
    constexpr int NKD = DK / 16;
    static_for<NB>([&](auto hc) {
        constexpr int hi = decltype(hc)::value;
        constexpr int hp = NB - 1 - hi;
        if (hi % NW == w) {
            // alpha of this block row's tokens (lane r: token 16 hi + r)
            const float ar = gate_alpha(sBeta[16 * hi + r], sLam[16 * hi + r], gate);
            if (g == 0) sAlpha[16 * hi + r] = ar;
            quad bk[NKD], bq[NKD];
#pragma unroll
            for (int kd = 0; kd < NKD; ++kd) {
                bk[kd] = M::lds_quad(sK + (16 * hi + r) * LD_DK + 4 * g + 16 * kd);
                if constexpr (WITH_P) bq[kd] = M::lds_quad(sQ + (16 * hp + r) * LD_DK + 4 * g + 16 * kd);
            }
            static_for<NB>([&](auto lc) {
                constexpr int lo = decltype(lc)::value;
                if constexpr (lo <= hi || (WITH_P && lo <= hp)) {
                    quad ak[NKD];
#pragma unroll
                    for (int kd = 0; kd < NKD; ++kd) ak[kd] = M::lds_quad(sK + (16 * lo + r) * LD_DK + 4 * g + 16 * kd);
                    const int col = 16 * lo + 4 * g;
                    if constexpr (lo <= hi) {
                        // acc lane (r, g), element i: (K K^T)[16 hi + r][16 lo + 4g + i]
                        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int kd = 0; kd + 1 < NKD; kd += 2) M::mma2(acc, ak[kd], ak[kd + 1], bk[kd], bk[kd + 1]);
                        if constexpr (NKD & 1) M::mma1(acc, ak[NKD - 1], bk[NKD - 1]);
                        const int row = 16 * hi + r;
                        f32x4 out;
#pragma unroll
                        for (int i = 0; i < 4; ++i) out[i] = (col + i < row) ? ar * acc[i] : 0.0f;
                        if constexpr (lo < hi) {
                            M::lds_store_quad(sA + row * LD_CE + col, M::cvt(out));
                        } else {
                            // diagonal block, transposed: At[16 hi + m][i] = A[16 hi + i][16 hi + m]
#pragma unroll
                            for (int i = 0; i < 4; ++i) sAt[(col + i) * kLdAt + r] = out[i];
                        }
                    }
                    if constexpr (WITH_P && lo <= hp) {
                        // acc lane (r, g), element i: (Q K^T)[16 hp + r][16 lo + 4g + i]
                        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int kd = 0; kd + 1 < NKD; kd += 2) M::mma2(acc, ak[kd], ak[kd + 1], bq[kd], bq[kd + 1]);
                        if constexpr (NKD & 1) M::mma1(acc, ak[NKD - 1], bq[NKD - 1]);
                        const int row = 16 * hp + r;
                        f32x4 out;
#pragma unroll
                        for (int i = 0; i < 4; ++i) out[i] = (col + i <= row) ? acc[i] : 0.0f;
                        M::lds_store_quad(sP + row * LD_CE + col, M::cvt(out));
                    }
                }
            });
            // sAt rows were written by this wave just above; LDS operations of one wave complete in order.
            __asm__ volatile("" ::: "memory");
            {
                const float* at = sAt + 16 * hi * kLdAt;
                float sv[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) sv[i] = (i == r) ? 1.0f : 0.0f;
                // rows of At are read three steps ahead of their use
                f32x4 ring[4][4];
#pragma unroll
                for (int m = 0; m < 3; ++m) {
#pragma unroll
                    for (int i4 = 0; i4 < 4; ++i4) ring[m][i4] = *reinterpret_cast<const f32x4*>(at + m * kLdAt + 4 * i4);
                }
#pragma unroll
                for (int m = 0; m < 15; ++m) {
                    if (m + 3 < 15) {
#pragma unroll
                        for (int i4 = (m + 3) / 4; i4 < 4; ++i4)
                            ring[(m + 3) & 3][i4] = *reinterpret_cast<const f32x4*>(at + (m + 3) * kLdAt + 4 * i4);
                    }
#pragma unroll
                    for (int i = m + 1; i < 16; ++i) sv[i] -= ring[m & 3][i / 4][i % 4] * sv[m];
                }
                // lane (r, g) writes T[16 hi + 4g + e][16 hi + r], e = 0..3: four consecutive entries of row
                // 16 hi + r of T^T, and the same scaled by alpha_{16 hi + r}
                f32x4 mine;
#pragma unroll
                for (int e = 0; e < 4; ++e) mine[e] = g == 0 ? sv[e] : g == 1 ? sv[4 + e] : g == 2 ? sv[8 + e] : sv[12 + e];
                const int b0 = 16 * hi;
                M::lds_store_quad(sTt + (b0 + r) * LD_CE + b0 + 4 * g, M::cvt(mine));
                M::lds_store_quad(sTat + (b0 + r) * LD_CE + b0 + 4 * g, M::cvt(mine * ar));
            }
        }
    });
}

// Off-diagonal blocks of T, one block column J per wave (J % NW == w), walked down the column with the
// blocks already found kept in registers: T_IJ = -T_II sum_{m=J}^{I-1} A_Im T_mJ on the matrix cores.
// (T diag(alpha))^T is completed in sTat.  Needs sA, sTt (diagonal blocks), sAlpha of every wave.
template <typename E, int C, int NW, int LD_CE>
__device__ __forceinline__ void ut_offdiag(const E* sA, const E* sTt, E* sTat, const float* sAlpha, int w, int r,
                                           int g, int tr_ce) {
    typedef Mma<E> M;
    typedef typename M::quad quad;
    constexpr int NB = C / 16;
    static_for<NB - 1>([&](auto jc) {
        constexpr int J = decltype(jc)::value;
        if (J % NW == w) {
            quad Tq[NB];
            Tq[J] = M::lds_quad(sTt + (16 * J + r) * LD_CE + 16 * J + 4 * g);   // T_JJ as B: row quad of T^T
            const float aj = sAlpha[16 * J + r];
            static_for<NB>([&](auto ic) {
                constexpr int I = decltype(ic)::value;
                if constexpr (I > J) {
                    const E* pa = sA + (16 * I + r) * LD_CE + 4 * g;
                    f32x4 y = {0.f, 0.f, 0.f, 0.f};
                    static_for<(I - J) / 2>([&](auto pc) {
                        constexpr int m = J + 2 * decltype(pc)::value;
                        M::mma2(y, M::lds_quad(pa + 16 * m), M::lds_quad(pa + 16 * m + 16), Tq[m], Tq[m + 1]);
                    });
                    if constexpr ((I - J) & 1) M::mma1(y, M::lds_quad(pa + 16 * (I - 1)), Tq[I - 1]);
                    f32x4 z = {0.f, 0.f, 0.f, 0.f};
                    // T_II as A: column quad of T^T
                    M::mma1(z, M::lds_quad_t(sTt + 16 * I * LD_CE + 16 * I, LD_CE, tr_ce), M::cvt_neg(y));
                    // z lane (r, g), element e: T[16 I + 4g + e][16 J + r] = T^T[16 J + r][16 I + 4g + e]
                    Tq[I] = M::cvt(z);
                    M::lds_store_quad(sTat + (16 * J + r) * LD_CE + 16 * I + 4 * g, M::cvt(z * aj));
                }
            });
        }
    });
}

}  // namespace efla
