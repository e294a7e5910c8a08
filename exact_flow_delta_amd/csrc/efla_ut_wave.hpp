// efla_ut_wave.hpp -- the UT transform for bf16 keys with d_k in {32, 64, 128}: one wave per (batch*head,
// chunk), no workgroup barriers.
//
// For a chunk of C tokens with keys K (rows k_t) and gates alpha_t ("Exact Flow Linear Attention"
// (gist.science), Metodologia items 2-3; "Error-Free Linear Attention is a Free Lunch" (howistudyai.com),
// Step 4):
//   A = strict_lower(diag(alpha) K K^T),  T = (I + A)^{-1},  output Ta = T diag(alpha)
// in the operand order the state pass reads (block qi = rb (rb + 1) / 2 + kb, lane 16 g + r, element e =
// Ta[16 rb + r][16 kb + 4 g + e]).
//
// The keys go straight from global memory into the registers that feed the matrix cores: lane (r, g)
// holds row 16 rb + r, d_k 32 kp + 8 g .. +7 of the key tile, which is at once the A and the B operand of
// the Gram blocks K_lo K_hi^T, so the Gram needs no LDS at all.  ||k_t||^2 is summed from the same
// registers.  The off-diagonal blocks of A stay in registers as the A operands of the block substitution.
// Only the small pieces that change hands between lanes pass through a private 7 KiB slice of LDS:
// the diagonal blocks of A (fp32, transposed) for the 16x16 solves, which run for all C/16 blocks at once
// (lane (r, g): column r of block g, right-looking substitution in fp32), the solved diagonal blocks of
// T (bf16, transposed, read back as either operand), and Ta^T for the export (in the space of the
// A blocks, which are dead by then).
//
// DG (diagonal 32-blocks only, C = 64): a state pass that steps a 64-token chunk as two 32-token halves
// reads only the two diagonal 32 x 32 blocks of Ta -- each is the Ta of its half on its own, because the
// diagonal blocks of the inverse of a block lower triangular matrix are the inverses of its diagonal blocks.
// With DG the Gram blocks, the block substitution and the export skip the off-diagonal 32 x 32 block (quads
// (2,0), (2,1), (3,0), (3,1)), which is left unwritten; the six quads written are bit-identical to the full
// transform's.
//
// The grid is persistent: each wave walks chunks u, u + W, u + 2W, ... (W waves in the grid) and loads
// the next chunk's keys into the operand registers once the current chunk's Gram blocks and diagonal
// solves are done, so that the load runs under the off-diagonal blocks and the export.  Several waves per SIMD hide the rest.
#pragma once

#include "efla_common.hpp"
#include "efla_launch.hpp"
#include "efla_ut.hpp"

namespace efla {

template <int DK, int C>
struct UtWaveShape {
    static constexpr int NB = C / 16;
    static constexpr int NQ = NB * (NB + 1) / 2;
    static constexpr int LDAT = 20;                   // row stride (floats) of a transposed diagonal A block
    static constexpr int ATB = 16 * LDAT + 4;         // block stride (floats): blocks start on different banks
    static constexpr int OFF_AT = 0;                  // fp32 [NB][ATB]
    static constexpr int OFF_TAT = 0;                 // bf16 [NQ][16][16]: Ta_qi^T, over the dead A blocks
    static constexpr int OFF_TT = (NB * ATB * 4 > NQ * 512 ? NB * ATB * 4 : NQ * 512);   // bf16 [NB][16][16]: T_bb^T
    static constexpr int BYTES = (OFF_TT + NB * 512 + 15) / 16 * 16;   // per wave
    static constexpr int WPB = 4;                     // waves per workgroup (the launch bounds assume 4)
};

// block (hi, lo) of a chunk's Ta is formed: all of them, or with DG those inside a diagonal 32 x 32 block
template <bool DG>
__host__ __device__ constexpr bool ut_block_used(int hi, int lo) { return !DG || (hi >> 1) == (lo >> 1); }

// tt (optional, not with DG): T^T of every chunk as a row-major C x C bf16 matrix (tt[u][j][i] = T[i][j], zeros below
// the diagonal), for the backward pass.
template <int DK, int C, bool VL, bool DG>
__global__ __launch_bounds__(256, 3) void ut_wave_kernel(
    const bf16* __restrict__ k, const float* __restrict__ beta, bf16* __restrict__ tw, int L, int NC, int BH,
    int gate, TokLayout ly, bf16* __restrict__ tt_out) {
    typedef UtWaveShape<DK, C> SH;
    typedef Mma<bf16> M;
    typedef M::quad quad;
    typedef bf16x8 bx8;
    constexpr int NB = SH::NB;
    constexpr int NKP = DK / 32;
    static_assert(DK == 32 || DK == 64 || DK == 128, "d_k of 32, 64 or 128");
    static_assert(C == 16 || C == 32 || C == 64, "chunk of 16, 32 or 64");
    static_assert(SH::WPB * 64 == 256, "launch bounds");
    static_assert(!DG || C == 64, "diagonal 32-blocks only for 64-token chunks");

    __shared__ __attribute__((aligned(16))) unsigned char smem[SH::WPB * SH::BYTES];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15;
    const int g = lane >> 4;
    const int stride = gridDim.x * SH::WPB;
    const int total = ut_chunks<VL>(ly, BH, NC);
    int u = blockIdx.x * SH::WPB + w;
    if (u >= total) return;   // whole wave
    float* sAt = reinterpret_cast<float*>(smem + w * SH::BYTES + SH::OFF_AT);
    bf16* sTt = reinterpret_cast<bf16*>(smem + w * SH::BYTES + SH::OFF_TT);
    bf16* sTat = reinterpret_cast<bf16*>(smem + w * SH::BYTES + SH::OFF_TAT);

    const int tr = M::tr_offset(lane, 16);

    // ---- keys of chunk uu into operand registers, and the step of token `lane` ------------------------
    // (uu >= total: an empty range, zeros, no memory access -- the registers are written either way, so the
    // previous chunk's keys are not kept alive across a conditional load)
    bx8 kf[NB][NKP];
    float beta_mine;
    auto load = [&](int uu) __attribute__((always_inline)) {
        const bool any = uu < total;
        if (!any) uu = 0;
        int bh, c;
        chunk_of<VL>(ly, uu, NC, bh, c);
        const SeqView sv = seq_view_t<VL>(ly, bh, L, C);
        const int t0 = c * C;
        const int n = !any ? 0 : (sv.len - t0 < C) ? (sv.len - t0) : C;   // valid rows; the rest read as zeros
        const int kt = (int)ly.k_t, bt = (int)ly.be_t;
        // one range per row block (wave-uniform), so that the only per-lane offset is that of row r
        const int lane_off = (r * kt + 8 * g) * 2;
#pragma unroll
        for (int rb = 0; rb < NB; ++rb) {
            const int nr = n - 16 * rb;   // valid rows of this block
            const __amdgpu_buffer_rsrc_t rk =
                buffer_rsrc(k + sv.k0 + (int64_t)(t0 + 16 * rb) * kt, nr > 0 ? ((nr - 1) * kt + DK) * 2 : 0);
#pragma unroll
            for (int kp = 0; kp < NKP; ++kp)
                kf[rb][kp] = __builtin_bit_cast(bx8, buffer_load<u32x4>(rk, lane_off + 64 * kp));
        }
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(beta + sv.be0 + (int64_t)t0 * bt, n > 0 ? ((n - 1) * bt + 1) * 4 : 0);
        beta_mine = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, lane * bt * 4, 0, 0));
    };
    load(u);
    for (; u < total; u += stride) {

        // ---- lambda of rows 16 rb + r (fp32 sum of exact bf16 squares; the four lanes of a row combined) ----
        float lam[NB];
#pragma unroll
        for (int rb = 0; rb < NB; ++rb) {
            float s = 0.0f;
#pragma unroll
            for (int kp = 0; kp < NKP; ++kp) s += sum_sq(kf[rb][kp]);
            lam[rb] = cross_row_sum(s);
        }
        // gate of token 16 g + r on lane (r, g) (lanes past the chunk compute an unused value), then the gate
        // of row 16 rb + r on every lane of row r
        float lam_mine = lam[0];
#pragma unroll
        for (int rb = 1; rb < NB; ++rb) lam_mine = g == rb ? lam[rb] : lam_mine;
        const float alpha_mine = gate_alpha(beta_mine, lam_mine, gate);
        float ar[4];
        rows_bcast4(alpha_mine, ar);

        // ---- Gram blocks: acc lane (r, g), element i = (K K^T)[16 hi + r][16 lo + 4 g + i] --------------------
        quad Aq[SH::NQ];   // off-diagonal blocks of A (row order, qi = hi (hi + 1) / 2 + lo), bf16 A operands
        static_for<NB>([&](auto hc) {
            constexpr int hi = decltype(hc)::value;
            static_for<hi + 1>([&](auto lc) {
                constexpr int lo = decltype(lc)::value;
                if constexpr (!ut_block_used<DG>(hi, lo)) return;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kp = 0; kp < NKP; ++kp) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[lo][kp], kf[hi][kp], acc, 0, 0, 0);
                if constexpr (lo < hi) {
                    Aq[hi * (hi + 1) / 2 + lo] = M::cvt(acc * ar[hi]);
                } else {
                    // strict lower part, transposed: At[m][i] = A[16 hi + i][16 hi + m]
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        sAt[hi * SH::ATB + (4 * g + i) * SH::LDAT + r] = (4 * g + i < r) ? ar[hi] * acc[i] : 0.0f;
                }
            });
        });
        // sAt was written by this wave; its LDS operations complete in order
        __asm__ volatile("" ::: "memory");

        // ---- diagonal solves, all blocks at once: lane (r, g) carries column r of T_gg --------------------------
        const int blk = g < NB ? g : 0;   // lanes of groups past the last block repeat block 0 and store nothing
        const float* at = sAt + blk * SH::ATB;
        float sv[16];
        {
            // lane r reads row r of its block of At (column r of A); the substitution takes column m from lane m
            // of the row by row broadcast
            float acol[16];
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const f32x4 a = *reinterpret_cast<const f32x4*>(at + r * SH::LDAT + 4 * i4);
#pragma unroll
                for (int e = 0; e < 4; ++e) acol[4 * i4 + e] = a[e];
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) sv[i] = (i == r) ? 1.0f : 0.0f;
            tri_solve_row_bcast<0, 15>(acol, sv);
        }
        // the keys are consumed: fetch the next chunk's (after the solves, which hold the most registers)
        load(u + stride);
        if (g < NB) {
            // row r of T_gg^T and of Ta_gg^T (column r scaled by the gate of token 16 g + r)
            bx8 t0v, t1v, a0v, a1v;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                t0v[i] = (bf16)sv[i];
                t1v[i] = (bf16)sv[8 + i];
                a0v[i] = (bf16)(sv[i] * alpha_mine);
                a1v[i] = (bf16)(sv[8 + i] * alpha_mine);
            }
            bf16* tt = sTt + g * 256 + r * 16;
            *reinterpret_cast<bx8*>(tt) = t0v;
            *reinterpret_cast<bx8*>(tt + 8) = t1v;
            if (tt_out) {   // row r of T_gg^T is row 16 g + r of T^T, columns 16 g .. 16 g + 15
                bf16* o = tt_out + (int64_t)u * (C * C) + (16 * g + r) * C + 16 * g;
                *reinterpret_cast<bx8*>(o) = t0v;
                *reinterpret_cast<bx8*>(o + 8) = t1v;
            }
            // diagonal block qi = g (g + 3) / 2
            bf16* ta = sTat + (g * (g + 3) / 2) * 256 + r * 16;
            *reinterpret_cast<bx8*>(ta) = a0v;
            *reinterpret_cast<bx8*>(ta + 8) = a1v;
        }
        __asm__ volatile("" ::: "memory");

        // ---- off-diagonal blocks, down each block column J: T_IJ = -T_II sum_{m=J}^{I-1} A_Im T_mJ ------------
        // B operands (column quads, lane (r, g): T_mJ[4 g + e][r]) of the blocks found so far stay in registers
        static_for<NB - 1>([&](auto jc) {
            constexpr int J = decltype(jc)::value;
            quad Tq[NB];
            Tq[J] = M::lds_quad(sTt + J * 256 + r * 16 + 4 * g);   // T_JJ[4g + e][r] = T_JJ^T[r][4g + e]
            static_for<NB>([&](auto ic) {
                constexpr int I = decltype(ic)::value;
                if constexpr (I > J && ut_block_used<DG>(I, J)) {
                    f32x4 y = {0.f, 0.f, 0.f, 0.f};
                    static_for<(I - J) / 2>([&](auto pc) {
                        constexpr int m = J + 2 * decltype(pc)::value;
                        M::mma2(y, Aq[I * (I + 1) / 2 + m], Aq[I * (I + 1) / 2 + m + 1], Tq[m], Tq[m + 1]);
                    });
                    if constexpr ((I - J) & 1) M::mma1(y, Aq[I * (I + 1) / 2 + I - 1], Tq[I - 1]);
                    // T_II as the A operand: lane (r, g) <- T_II[r][4g + e] = T_II^T[4g + e][r]
                    f32x4 z = {0.f, 0.f, 0.f, 0.f};
                    M::mma1(z, M::lds_quad_t(sTt + I * 256, 16, tr), M::cvt_neg(y));
                    // z lane (r, g), element e = T_IJ[4g + e][r]: row r of Ta_IJ^T after the column gate of token 16 J + r
                    Tq[I] = M::cvt(z);
                    M::lds_store_quad(sTat + (I * (I + 1) / 2 + J) * 256 + r * 16 + 4 * g, M::cvt(z * ar[J]));
                    if (tt_out) {   // T_IJ[4g + e][r] = T^T[16 J + r][16 I + 4 g + e]; zeros at T^T block (I, J)
                        bf16* o = tt_out + (int64_t)u * (C * C);
                        *reinterpret_cast<quad*>(o + (16 * J + r) * C + 16 * I + 4 * g) = Tq[I];
                        *reinterpret_cast<quad*>(o + (16 * I + r) * C + 16 * J + 4 * g) = M::zero();
                    }
                }
            });
        });
        __asm__ volatile("" ::: "memory");

        // ---- export: lane (r, g) of block qi takes Ta[16 rb + r][16 kb + 4 g + e] = Ta^T[4 g + e][r] -----------
        bf16* dst = tw + (int64_t)u * (SH::NQ * 256) + lane * 4;
        static_for<NB>([&](auto rc) {
            constexpr int rb = decltype(rc)::value;
            static_for<rb + 1>([&](auto kc) {
                constexpr int kb = decltype(kc)::value;
                constexpr int qi = rb * (rb + 1) / 2 + kb;
                if constexpr (ut_block_used<DG>(rb, kb))
                    *reinterpret_cast<quad*>(dst + qi * 256) = M::lds_quad_t(sTat + qi * 256, 16, tr);
            });
        });
        __asm__ volatile("" ::: "memory");   // the next chunk's A blocks overwrite Ta^T
    }
}

}  // namespace efla
