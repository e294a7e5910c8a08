// efla_bwd_chain_mx.hpp -- the state-gradient pass of the backward on bf16 matrix cores (bf16 inputs, d_k >= 32,
// 64-token chunks): dS carried backwards over the chunks, dV, the gradient of the state leaving every chunk and
// the initial state's.
//
// The adjoint of the chunked form ("Error-Free Linear Attention is a Free Lunch" (howistudyai.com), Step 4; the
// gradients are derived in efla_bwd.hpp).  A 64-token chunk is taken as two 32-token halves, last half first: each
// half is a chunk of its own whose T diag(alpha) is a diagonal 32 x 32 block of the chunk's (as in the forward
// state pass), so per half, with dS the gradient of the state leaving it, P = lower_incl(Q K^T) and Ta its diagonal
// block:
//   dDelta = P^T dO + K dS,   dR = Ta^T dDelta (= dV),   dS <- dS + Q^T dO - K^T dR.
// The organisation is the forward state pass's (efla_chain_bf16.hpp): one workgroup per (head, slab of DVS
// gradient columns), DVS / 16 compute waves each holding 16 columns of dS in fp32 registers, one producer wave that
// issues the next chunks' Q, K, dO slab and Ta blocks as buffer loads straight into three LDS buffers (two chunks
// ahead, in reverse order), the same swizzled tiles and the same operand reads:
//   * K dS takes the key fragments and the gradient's bf16 copy as in K S;
//   * P^T comes from Q K^T with the operands exchanged, which leaves its accumulator in the A-operand layout of P^T;
//   * dO enters as the column quads of the transposing read (as V does in the forward), for P^T dO and Q^T dO;
//   * Ta^T is read with the transposing read straight from the operand layout in which the UT transform stores
//     Ta (each 8-byte run there is four consecutive columns of one row);
//   * Q^T and K^T are the transposing reads of the update S += K^T Delta.
#pragma once

#include "efla_bwd.hpp"
#include "efla_chain_bf16.hpp"

namespace efla {

template <int DK, int DVS>
__global__ __launch_bounds__(DVS / 16 * 64 + 64) void bwd_chain_mx_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ tw, const bf16* __restrict__ d_o,
    const float* __restrict__ d_final, void* __restrict__ ds_all, bf16* __restrict__ dv, float* __restrict__ d_initial,
    int BH, int L, int DV, int nslab, TokLayout ly, int sbf) {
    constexpr int C = 64;
    typedef ChainBf16Shape<DK, C, DVS, 0> SH;
    typedef Mma<bf16> M;
    typedef M::quad quad;
    typedef bf16x8 bx8;
    constexpr int NW = DVS / 16;
    constexpr int NKD = DK / 16;
    constexpr int NKP = DK / 32;
    constexpr int NQ = TaShape<C>::NQ;
    constexpr int QE = TaShape<C>::QE;
    constexpr int NCV = DVS / 8;
    static_assert(DK == 32 || DK == 64 || DK == 128, "d_k of 32, 64 or 128");
    static_assert(SH::NBUF == 3, "three chunk buffers");
    static_assert(SH::NLT == 5, "Ta of a 64-token chunk is five 1 KiB loads");
    __shared__ __attribute__((aligned(1024))) unsigned char buf0_[SH::BUF];
    __shared__ __attribute__((aligned(1024))) unsigned char buf1_[SH::BUF];
    __shared__ __attribute__((aligned(1024))) unsigned char buf2_[SH::BUF];
    lds_u8* const buf0 = (lds_u8*)buf0_;
    lds_u8* const buf1 = (lds_u8*)buf1_;
    lds_u8* const buf2 = (lds_u8*)buf2_;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15;
    const int g = lane >> 4;
    const int bid = blockIdx.x;
    const int slab = (bid >> 3) % nslab;
    const int bh = ((bid >> 3) / nslab) * 8 + (bid & 7);
    if (bh >= BH) return;
    const int slab_col = slab * DVS;
    const bool producer = w == NW;
    const int colw = slab_col + 16 * (producer ? 0 : w);
    const SeqView sv = seq_view(ly, bh, L, C);   // this sequence's tokens and first chunk
    const int len = sv.len;
    const int NC = (len + C - 1) / C;
    const int64_t qs = ly.q_t, ks = ly.k_t, vs = ly.v_t, os = ly.o_t;   // token strides (elements)
    const bf16* twh = tw + (int64_t)sv.chunk0 * (NQ * QE);

    // ---- loads (producer wave): chunk c's Q, K, dO slab and Ta blocks into one buffer, as the forward state pass
    //      lays them out (wave load j of a tile covers its bytes [1024 j, 1024 j + 1024); lane L writes 16 bytes at
    //      1024 j + 16 L, physical chunk p of row t holding logical chunk p ^ sw(t)); rows past the end of the
    //      sequence are outside the buffer range and land as zeros
    constexpr int NLOAD = 2 * SH::NLQ + SH::NLV + SH::NLT - 1;   // Ta quads 6 and 7 are not read
    auto issue_chunk = [&](int c, lds_u8* buf) __attribute__((always_inline)) {
        const int t = c * C;
        const int n = (len - t < C) ? (len - t) : C;
        const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(q + sv.q0 + t * qs, (int)((n - 1) * qs + DK) * 2);
        const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(k + sv.k0 + t * ks, (int)((n - 1) * ks + DK) * 2);
        const __amdgpu_buffer_rsrc_t ro = buffer_rsrc(d_o + sv.o0 + t * os + slab_col, (int)((n - 1) * os + DVS) * 2);
        const __amdgpu_buffer_rsrc_t rt = buffer_rsrc(twh + (int64_t)c * (NQ * QE), SH::TBYTES);
        static_for<2 * SH::NLQ + SH::NLV + SH::NLT>([&](auto kc) {
            constexpr int kk = decltype(kc)::value;
            constexpr int tile = kk < SH::NLQ ? 0 : kk < 2 * SH::NLQ ? 1 : kk < 2 * SH::NLQ + SH::NLV ? 2 : 3;
            constexpr int j = tile == 0 ? kk : tile == 1 ? kk - SH::NLQ : tile == 2 ? kk - 2 * SH::NLQ
                                                                                  : kk - 2 * SH::NLQ - SH::NLV;
            constexpr int RB = tile < 2 ? SH::RBQ : SH::RBV;
            constexpr int off = tile == 0 ? SH::OFF_Q : tile == 1 ? SH::OFF_K : tile == 2 ? SH::OFF_V : SH::OFF_T;
            lds_void* dst = (lds_void*)(buf + off + 1024 * j);
            const int p = 1024 * j + 16 * lane;
            if constexpr (tile == 3 && j == 3) {
                return;   // bytes [3072, 4096) of Ta: quads 6 and 7, outside the diagonal 32 x 32 blocks
            } else if constexpr (tile == 3) {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rt, dst, 16, p, 0, 0, 0);
            } else {
                const int tr = p / RB;
                const int lc = ((p % RB) / 16) ^ (tile == 2 ? sw_v<DVS>(tr) : sw_qk_tr<DK>(tr));
                const int ld = (int)(tile == 2 ? os : tile == 1 ? ks : qs);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(tile == 0 ? rq : tile == 1 ? rk : ro, dst, 16,
                                                         (tr * ld + 8 * lc) * 2, 0, 0, 0);
            }
        });
    };
    auto wait_vm = [&](auto n_c) __attribute__((always_inline)) {
        constexpr int N = decltype(n_c)::value;
        static_assert(N >= 0 && N < 64, "vector-memory count field");
        __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
    };
    typedef std::integral_constant<int, 0> I0;
    typedef std::integral_constant<int, NLOAD> ILOAD;

    if (producer) {
        // step s works on chunk NC - 1 - s in buffer s mod 3; its tiles go out in step s - 2 (the first two before
        // the first barrier), and those of step s + 1 have landed by the end of step s
        if (NC > 0) {
            issue_chunk(NC - 1, buf0);
            if (NC > 1) {
                issue_chunk(NC - 2, buf1);
                wait_vm(ILOAD{});
            } else {
                wait_vm(I0{});
            }
            __builtin_amdgcn_s_barrier();
        }
        auto pstep = [&](int s, lds_u8* nxt) __attribute__((always_inline)) {
            if (s + 2 < NC) {
                issue_chunk(NC - 3 - s, nxt);
                wait_vm(ILOAD{});
            } else {
                wait_vm(I0{});
            }
            __builtin_amdgcn_s_barrier();
        };
        for (int s = 0; s < NC; s += 3) {
            pstep(s, buf2);
            if (s + 1 < NC) pstep(s + 1, buf0);
            if (s + 2 < NC) pstep(s + 2, buf1);
        }
        return;
    }

    // ---- the state gradient: dS[32 kp + 8 g + 4 h + i][colw + r] in tile rt = 2 kp + h, element i ------------------
    auto srow = [&](int rt, int i) __attribute__((always_inline)) { return 32 * (rt >> 1) + 8 * g + 4 * (rt & 1) + i; };
    f32x4 dS[NKD];
#pragma unroll
    for (int rt = 0; rt < NKD; ++rt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) dS[rt][i] = d_final ? d_final[((int64_t)bh * DK + srow(rt, i)) * DV + colw + r] : 0.0f;
    }

    // per-lane LDS offsets, as in the forward state pass
    const int swr = sw_qk_tr<DK>(r);
    const int te = 4 * g + ((lane >> 2) & 3);
    const int tc = lane & 3;
    const int swt = sw_qk_tr<DK>(te);
    const int o_off = te * SH::RBV + 16 * (((2 * w + (tc >> 1)) % NCV) ^ sw_v<DVS>(te)) + 8 * (tc & 1);
    // Ta^T from the stored operand layout: lane 4 e + c of group g reads stored lane 16 c + 4 g + e of the block
    const int ta_off = 8 * (16 * (lane & 3) + 4 * g + ((lane >> 2) & 3));
    // byte offsets of this lane's state-gradient and dV elements (row 8 g or 4 g, column colw + r)
    const int ds_lane = (8 * g * DV + colw + r) * (sbf ? 2 : 4);
    const int dv_lane = (int)(4 * g * vs + colw + r) * 2;

    auto step = [&](int c, const lds_u8* cQ, const lds_u8* cK, const lds_u8* cO, const lds_u8* cT)
                    __attribute__((always_inline)) {
        typedef quad __attribute__((address_space(3))) lds_quad;
        (void)sizeof(lds_quad);
        const int t0 = c * C;
        const int n = (len - t0 < C) ? (len - t0) : C;
        // the gradient of the state leaving chunk c, for the per-chunk gradients: element i of tile rt is row
        // 32 kp + 8 g + 4 h + i, i.e. the lane's offset plus a wave-uniform one (buffer stores with a scalar offset,
        // so that no per-element address stays live across the chunk loop; every row is inside the chunk's state)
        if (sbf) {   // rounded to bf16 as the per-chunk kernel rounds its operands
            const __amdgpu_buffer_rsrc_t rs =
                buffer_rsrc(static_cast<bf16*>(ds_all) + ((int64_t)sv.chunk0 + c) * DK * DV, DK * DV * 2);
#pragma unroll
            for (int rt = 0; rt < NKD; ++rt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bf16 x = (bf16)dS[rt][i];
                    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, x), rs, ds_lane,
                                                          (32 * (rt >> 1) + 4 * (rt & 1) + i) * DV * 2, 0);
                }
            }
        } else {
            const __amdgpu_buffer_rsrc_t rs =
                buffer_rsrc(static_cast<float*>(ds_all) + ((int64_t)sv.chunk0 + c) * DK * DV, DK * DV * 4);
#pragma unroll
            for (int rt = 0; rt < NKD; ++rt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float x = dS[rt][i];   // one element to a scalar first: a bit cast of a vector element
                                                 // directly yields element 0 with this toolchain
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, x), rs, ds_lane,
                                                          (32 * (rt >> 1) + 4 * (rt & 1) + i) * DV * 4, 0);
                }
            }
        }
        auto frag = [&](const lds_u8* tile, int rb, int kp) __attribute__((always_inline)) {
            return bx8(*reinterpret_cast<const lds_bf16x8*>(tile + (16 * rb + r) * SH::RBQ + 16 * ((4 * kp + g) ^ swr)));
        };
        auto pair = [&](quad a, quad b) __attribute__((always_inline)) -> bx8 { return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7); };
        // transposed Q or K block: tile rt of d_k rows, tokens 16 kb .. 16 kb + 15
        auto tr_qk = [&](const lds_u8* tile, int rt, int kb) __attribute__((always_inline)) {
            const int off = te * SH::RBQ + 16 * ((4 * (rt >> 1) + tc) ^ swt) + 8 * (rt & 1);
            return __builtin_bit_cast(quad, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                (lds_s16x4*)(const_cast<lds_u8*>(tile) + 16 * kb * SH::RBQ + off)));
        };
        // Ta^T block (rb, kb) = the transpose of the stored block (kb, rb), kb >= rb
        auto ta_t = [&](int rb, int kb) __attribute__((always_inline)) {
            const int qi = kb * (kb + 1) / 2 + rb;
            return __builtin_bit_cast(quad, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                (lds_s16x4*)(const_cast<lds_u8*>(cT) + 512 * qi + ta_off)));
        };
        // the halves, last first
        static_for<2>([&](auto hc) {
            constexpr int b0 = 2 * (1 - decltype(hc)::value);   // first row block of the half
            bx8 Gq[NKP];   // dS as the B operand: lane (r, g) holds dS[32 kp + 8 g .. +7][colw + r]
#pragma unroll
            for (int kp = 0; kp < NKP; ++kp) Gq[kp] = pair(M::cvt(dS[2 * kp]), M::cvt(dS[2 * kp + 1]));
            // row block 0, then row block 1 (its key fragments kept for the off-diagonal block of P^T); dD[j] = K dS
            f32x4 dD[2];
            quad oq[2];
            quad pt00, pt01, pt11;
            bx8 kq0[NKP];
            {
                bx8 qq0[NKP];
#pragma unroll
                for (int kp = 0; kp < NKP; ++kp) {
                    qq0[kp] = frag(cQ, b0, kp);
                    kq0[kp] = frag(cK, b0, kp);
                }
                f32x4 a00 = {0.f, 0.f, 0.f, 0.f};
                dD[0] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kp = 0; kp < NKP; ++kp) {
                    dD[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kq0[kp], Gq[kp], dD[0], 0, 0, 0);
                    a00 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qq0[kp], kq0[kp], a00, 0, 0, 0);
                }
                // P^T blocks (jk, jq), jk <= jq: Q_jq K_jk^T with the operands exchanged; lane (r, g), element e =
                // P[16 (b0 + jq) + 4 g + e][16 (b0 + jk) + r], the A operand of P^T; the diagonal blocks keep
                // key <= query
#pragma unroll
                for (int e = 0; e < 4; ++e) a00[e] = (r <= 4 * g + e) ? a00[e] : 0.0f;
                pt00 = M::cvt(a00);
            }
            {
                bx8 qq1[NKP], kq1[NKP];
#pragma unroll
                for (int kp = 0; kp < NKP; ++kp) {
                    qq1[kp] = frag(cQ, b0 + 1, kp);
                    kq1[kp] = frag(cK, b0 + 1, kp);
                }
                f32x4 a01 = {0.f, 0.f, 0.f, 0.f}, a11 = {0.f, 0.f, 0.f, 0.f};
                dD[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kp = 0; kp < NKP; ++kp) {
                    dD[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kq1[kp], Gq[kp], dD[1], 0, 0, 0);
                    a01 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qq1[kp], kq0[kp], a01, 0, 0, 0);
                    a11 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qq1[kp], kq1[kp], a11, 0, 0, 0);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) a11[e] = (r <= 4 * g + e) ? a11[e] : 0.0f;
                pt01 = M::cvt(a01);
                pt11 = M::cvt(a11);
            }
            // dO rows 16 rb + 4 g + e, column 16 w + r of the slab
#pragma unroll
            for (int j = 0; j < 2; ++j)
                oq[j] = __builtin_bit_cast(quad, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                     (lds_s16x4*)(const_cast<lds_u8*>(cO) + 16 * (b0 + j) * SH::RBV + o_off)));
            // dDelta = K dS + P^T dO
            M::mma2(dD[0], pt00, pt01, oq[0], oq[1]);
            M::mma1(dD[1], pt11, oq[1]);
            const quad dq0 = M::cvt(dD[0]), dq1 = M::cvt(dD[1]);
            // dR = Ta^T dDelta: lane (r, g), element e = dR[16 (b0 + j) + 4 g + e][colw + r]
            f32x4 dR0 = {0.f, 0.f, 0.f, 0.f}, dR1 = {0.f, 0.f, 0.f, 0.f};
            M::mma2(dR0, ta_t(b0, b0), ta_t(b0, b0 + 1), dq0, dq1);
            M::mma1(dR1, ta_t(b0 + 1, b0 + 1), dq1);
            // dV = dR: rows 16 (b0 + j) + 4 g + e of the chunk; those past its end fall outside the buffer range (the
            // row is in the per-lane offset, which the range check covers) and are dropped
            {
                const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(dv + sv.v0 + t0 * vs, (int)((n - 1) * vs + DV) * 2);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bf16 x0 = (bf16)dR0[e], x1 = (bf16)dR1[e];
                    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, x0), rv,
                                                          dv_lane + (16 * b0 + e) * (int)vs * 2, 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, x1), rv,
                                                          dv_lane + (16 * b0 + 16 + e) * (int)vs * 2, 0, 0);
                }
            }
            // dS += Q^T dO - K^T dR over the half; the tiles' chains interleaved
            const quad nr0 = M::cvt_neg(dR0), nr1 = M::cvt_neg(dR1);
#pragma unroll
            for (int rt = 0; rt < NKD; ++rt) {
                M::mma2(dS[rt], tr_qk(cQ, rt, b0), tr_qk(cQ, rt, b0 + 1), oq[0], oq[1]);
                M::mma2(dS[rt], tr_qk(cK, rt, b0), tr_qk(cK, rt, b0 + 1), nr0, nr1);
            }
        });
        wait_vm(I0{});   // this wave's LDS reads and its stores are done
        __builtin_amdgcn_s_barrier();
    };
    auto stepb = [&](int s, const lds_u8* b) __attribute__((always_inline)) {
        step(NC - 1 - s, b + SH::OFF_Q, b + SH::OFF_K, b + SH::OFF_V, b + SH::OFF_T);
    };
    if (NC > 0) __builtin_amdgcn_s_barrier();   // the producer's prologue
    for (int s = 0; s < NC; s += 3) {
        stepb(s, buf0);
        if (s + 1 < NC) stepb(s + 1, buf1);
        if (s + 2 < NC) stepb(s + 2, buf2);
    }
    if (d_initial) {
#pragma unroll
        for (int rt = 0; rt < NKD; ++rt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) d_initial[((int64_t)bh * DK + srow(rt, i)) * DV + colw + r] = dS[rt][i];
        }
    }
}

// The state entering every chunk, s_all[bh][c] (d_k x d_v; bf16 when sbf, else fp32), for the per-chunk gradients: the forward state
// pass again without outputs (per 32-token half: R = V - K S, Delta = Ta R, S <- S + K^T Delta), organised as
// bwd_chain_mx_kernel but in chunk order, with only K, the V slab and Ta loaded.
template <int DK, int DVS>
__global__ __launch_bounds__(DVS / 16 * 64 + 64) void bwd_states_mx_kernel(
    const bf16* __restrict__ k, const bf16* __restrict__ v, const bf16* __restrict__ tw, const float* __restrict__ s0,
    void* __restrict__ s_all, int BH, int L, int DV, int nslab, TokLayout ly, int sbf) {
    constexpr int C = 64;
    typedef ChainBf16Shape<DK, C, DVS, 0> SH;
    typedef Mma<bf16> M;
    typedef M::quad quad;
    typedef bf16x8 bx8;
    constexpr int NW = DVS / 16;
    constexpr int NKD = DK / 16;
    constexpr int NKP = DK / 32;
    constexpr int NQ = TaShape<C>::NQ;
    constexpr int QE = TaShape<C>::QE;
    constexpr int NCV = DVS / 8;
    static_assert(DK == 32 || DK == 64 || DK == 128, "d_k of 32, 64 or 128");
    static_assert(SH::NLT == 5, "Ta of a 64-token chunk is five 1 KiB loads");
    // one buffer: K tile, V slab, Ta (no Q tile)
    constexpr int OK_ = 0, OV_ = SH::NLQ * 1024, OT_ = (SH::NLQ + SH::NLV) * 1024;
    constexpr int BUFB = (SH::NLQ + SH::NLV + SH::NLT) * 1024;
    __shared__ __attribute__((aligned(1024))) unsigned char buf0_[BUFB];
    __shared__ __attribute__((aligned(1024))) unsigned char buf1_[BUFB];
    __shared__ __attribute__((aligned(1024))) unsigned char buf2_[BUFB];
    lds_u8* const buf0 = (lds_u8*)buf0_;
    lds_u8* const buf1 = (lds_u8*)buf1_;
    lds_u8* const buf2 = (lds_u8*)buf2_;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15;
    const int g = lane >> 4;
    const int bid = blockIdx.x;
    const int slab = (bid >> 3) % nslab;
    const int bh = ((bid >> 3) / nslab) * 8 + (bid & 7);
    if (bh >= BH) return;
    const int slab_col = slab * DVS;
    const bool producer = w == NW;
    const int colw = slab_col + 16 * (producer ? 0 : w);
    const SeqView sv = seq_view(ly, bh, L, C);   // this sequence's tokens and first chunk
    const int len = sv.len;
    const int NC = (len + C - 1) / C;
    const int64_t ks = ly.k_t, vs = ly.v_t;   // token strides (elements)
    const bf16* twh = tw + (int64_t)sv.chunk0 * (NQ * QE);

    constexpr int NLOAD = SH::NLQ + SH::NLV + SH::NLT - 1;   // Ta quads 6 and 7 are not read
    auto issue_chunk = [&](int c, lds_u8* buf) __attribute__((always_inline)) {
        const int t = c * C;
        const int n = (len - t < C) ? (len - t) : C;
        const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(k + sv.k0 + t * ks, (int)((n - 1) * ks + DK) * 2);
        const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(v + sv.v0 + t * vs + slab_col, (int)((n - 1) * vs + DVS) * 2);
        const __amdgpu_buffer_rsrc_t rt = buffer_rsrc(twh + (int64_t)c * (NQ * QE), SH::TBYTES);
        static_for<SH::NLQ + SH::NLV + SH::NLT>([&](auto kc) {
            constexpr int kk = decltype(kc)::value;
            constexpr int tile = kk < SH::NLQ ? 1 : kk < SH::NLQ + SH::NLV ? 2 : 3;
            constexpr int j = tile == 1 ? kk : tile == 2 ? kk - SH::NLQ : kk - SH::NLQ - SH::NLV;
            constexpr int RB = tile == 1 ? SH::RBQ : SH::RBV;
            constexpr int off = tile == 1 ? OK_ : tile == 2 ? OV_ : OT_;
            lds_void* dst = (lds_void*)(buf + off + 1024 * j);
            const int p = 1024 * j + 16 * lane;
            if constexpr (tile == 3 && j == 3) {
                return;
            } else if constexpr (tile == 3) {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rt, dst, 16, p, 0, 0, 0);
            } else {
                const int tr = p / RB;
                const int lc = ((p % RB) / 16) ^ (tile == 2 ? sw_v<DVS>(tr) : sw_qk_tr<DK>(tr));
                const int ld = (int)(tile == 2 ? vs : ks);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(tile == 1 ? rk : rv, dst, 16, (tr * ld + 8 * lc) * 2, 0, 0, 0);
            }
        });
    };
    auto wait_vm = [&](auto n_c) __attribute__((always_inline)) {
        constexpr int N = decltype(n_c)::value;
        static_assert(N >= 0 && N < 64, "vector-memory count field");
        __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
    };
    typedef std::integral_constant<int, 0> I0;
    typedef std::integral_constant<int, NLOAD> ILOAD;

    if (producer) {
        if (NC > 0) {
            issue_chunk(0, buf0);
            if (NC > 1) {
                issue_chunk(1, buf1);
                wait_vm(ILOAD{});
            } else {
                wait_vm(I0{});
            }
            __builtin_amdgcn_s_barrier();
        }
        auto pstep = [&](int c, lds_u8* nxt) __attribute__((always_inline)) {
            if (c + 2 < NC) {
                issue_chunk(c + 2, nxt);
                wait_vm(ILOAD{});
            } else {
                wait_vm(I0{});
            }
            __builtin_amdgcn_s_barrier();
        };
        for (int c = 0; c < NC; c += 3) {
            pstep(c, buf2);
            if (c + 1 < NC) pstep(c + 1, buf0);
            if (c + 2 < NC) pstep(c + 2, buf1);
        }
        return;
    }

    auto srow = [&](int rt, int i) __attribute__((always_inline)) { return 32 * (rt >> 1) + 8 * g + 4 * (rt & 1) + i; };
    f32x4 S[NKD];
#pragma unroll
    for (int rt = 0; rt < NKD; ++rt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) S[rt][i] = s0 ? s0[((int64_t)bh * DK + srow(rt, i)) * DV + colw + r] : 0.0f;
    }
    const int swr = sw_qk_tr<DK>(r);
    const int te = 4 * g + ((lane >> 2) & 3);
    const int tc = lane & 3;
    const int swt = sw_qk_tr<DK>(te);
    const int v_off = te * SH::RBV + 16 * (((2 * w + (tc >> 1)) % NCV) ^ sw_v<DVS>(te)) + 8 * (tc & 1);
    const int s_lane = (8 * g * DV + colw + r) * (sbf ? 2 : 4);

    auto step = [&](int c, const lds_u8* cK, const lds_u8* cV, const lds_u8* cT) __attribute__((always_inline)) {
        typedef quad __attribute__((address_space(3))) lds_quad;
        if (sbf) {   // the state entering chunk c, rounded to bf16 as the per-chunk kernel rounds its operands
            const __amdgpu_buffer_rsrc_t rs =
                buffer_rsrc(static_cast<bf16*>(s_all) + ((int64_t)sv.chunk0 + c) * DK * DV, DK * DV * 2);
#pragma unroll
            for (int rt = 0; rt < NKD; ++rt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bf16 x = (bf16)S[rt][i];
                    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, x), rs, s_lane,
                                                          (32 * (rt >> 1) + 4 * (rt & 1) + i) * DV * 2, 0);
                }
            }
        } else {   // the state entering chunk c
            const __amdgpu_buffer_rsrc_t rs =
                buffer_rsrc(static_cast<float*>(s_all) + ((int64_t)sv.chunk0 + c) * DK * DV, DK * DV * 4);
#pragma unroll
            for (int rt = 0; rt < NKD; ++rt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float x = S[rt][i];   // to a scalar before the bit cast (see bwd_chain_mx_kernel)
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, x), rs, s_lane,
                                                          (32 * (rt >> 1) + 4 * (rt & 1) + i) * DV * 4, 0);
                }
            }
        }
        auto frag = [&](int rb, int kp) __attribute__((always_inline)) {
            return bx8(*reinterpret_cast<const lds_bf16x8*>(cK + (16 * rb + r) * SH::RBQ + 16 * ((4 * kp + g) ^ swr)));
        };
        auto pair = [&](quad a, quad b) __attribute__((always_inline)) -> bx8 { return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7); };
        auto kt = [&](int rt, int kb) __attribute__((always_inline)) {
            const int off = te * SH::RBQ + 16 * ((4 * (rt >> 1) + tc) ^ swt) + 8 * (rt & 1);
            return __builtin_bit_cast(quad, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                (lds_s16x4*)(const_cast<lds_u8*>(cK) + 16 * kb * SH::RBQ + off)));
        };
        auto ta = [&](int rb, int kb) __attribute__((always_inline)) {
            return *reinterpret_cast<const lds_quad*>(cT + 512 * (rb * (rb + 1) / 2 + kb) + 8 * lane);
        };
        static_for<2>([&](auto hc) {
            constexpr int b0 = 2 * decltype(hc)::value;
            bx8 Sq[NKP];
#pragma unroll
            for (int kp = 0; kp < NKP; ++kp) Sq[kp] = pair(M::cvt(S[2 * kp]), M::cvt(S[2 * kp + 1]));
            quad Rq[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                f32x4 xk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kp = 0; kp < NKP; ++kp) xk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(frag(b0 + j, kp), Sq[kp], xk, 0, 0, 0);
                const quad vq = __builtin_bit_cast(quad, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                             (lds_s16x4*)(const_cast<lds_u8*>(cV) + 16 * (b0 + j) * SH::RBV + v_off)));
                f32x4 rr;
#pragma unroll
                for (int e = 0; e < 4; ++e) rr[e] = (float)vq[e] - xk[e];
                Rq[j] = M::cvt(rr);
            }
            // Delta = Ta R over the half (its diagonal 32 x 32 block of Ta)
            f32x4 d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
            M::mma1(d0, ta(b0, b0), Rq[0]);
            M::mma2(d1, ta(b0 + 1, b0), ta(b0 + 1, b0 + 1), Rq[0], Rq[1]);
            const quad D0 = M::cvt(d0), D1 = M::cvt(d1);
            // S += K^T Delta
#pragma unroll
            for (int rt = 0; rt < NKD; ++rt) M::mma2(S[rt], kt(rt, b0), kt(rt, b0 + 1), D0, D1);
        });
        wait_vm(I0{});
        __builtin_amdgcn_s_barrier();
    };
    auto stepb = [&](int c, const lds_u8* b) __attribute__((always_inline)) { step(c, b + OK_, b + OV_, b + OT_); };
    if (NC > 0) __builtin_amdgcn_s_barrier();
    for (int c = 0; c < NC; c += 3) {
        stepb(c, buf0);
        if (c + 1 < NC) stepb(c + 1, buf1);
        if (c + 2 < NC) stepb(c + 2, buf2);
    }
}

// Launches the matrix-core state-gradient pass when it applies (bf16, d_k >= 32, 64-token chunks); returns false
// otherwise, leaving the launch to bwd_chain_kernel.
template <int DK, int C>
bool launch_bwd_chain_mx(const BwdArgs& a, hipStream_t s, hipError_t* err) {
    if constexpr (DK < 32 || C != 64) {
        (void)a;
        (void)s;
        (void)err;
        return false;
    } else {
        // slab width as the forward state pass: the widest that still gives enough workgroups
        int dvs = a.d_v < 64 ? a.d_v : 64;
        while (dvs > 16 && (int64_t)a.BH * (a.d_v / dvs) < 256) dvs /= 2;
        const int nslab = a.d_v / dvs;
        const int64_t grid = (int64_t)((a.BH + 7) / 8) * 8 * nslab;
        const bf16* q = static_cast<const bf16*>(a.q);
        const bf16* k = static_cast<const bf16*>(a.k);
        const bf16* tw = static_cast<const bf16*>(a.tw);
        const bf16* d_o = static_cast<const bf16*>(a.d_o);
        bf16* dv = static_cast<bf16*>(a.dv);
        const TokLayout ly = bwd_layout(a);
        switch (dvs) {
            case 16:
                hipLaunchKernelGGL((bwd_chain_mx_kernel<DK, 16>), dim3((unsigned)grid), dim3(16 / 16 * 64 + 64), 0, s, q,
                                   k, tw, d_o, a.d_final, a.ds_all, dv, a.d_initial, a.BH, a.L, a.d_v, nslab, ly,
                                   (int)a.sbf);
                break;
            case 32:
                hipLaunchKernelGGL((bwd_chain_mx_kernel<DK, 32>), dim3((unsigned)grid), dim3(32 / 16 * 64 + 64), 0, s, q,
                                   k, tw, d_o, a.d_final, a.ds_all, dv, a.d_initial, a.BH, a.L, a.d_v, nslab, ly,
                                   (int)a.sbf);
                break;
            default:
                hipLaunchKernelGGL((bwd_chain_mx_kernel<DK, 64>), dim3((unsigned)grid), dim3(64 / 16 * 64 + 64), 0, s, q,
                                   k, tw, d_o, a.d_final, a.ds_all, dv, a.d_initial, a.BH, a.L, a.d_v, nslab, ly,
                                   (int)a.sbf);
                break;
        }
        *err = hipGetLastError();
        return true;
    }
}

// Launches the matrix-core state recompute when it applies (bf16, d_k >= 32, 64-token chunks).
template <int DK, int C>
bool launch_bwd_states_mx(const BwdArgs& a, hipStream_t s, hipError_t* err) {
    if constexpr (DK < 32 || C != 64) {
        (void)a;
        (void)s;
        (void)err;
        return false;
    } else {
        int dvs = a.d_v < 64 ? a.d_v : 64;
        while (dvs > 16 && (int64_t)a.BH * (a.d_v / dvs) < 256) dvs /= 2;
        const int nslab = a.d_v / dvs;
        const int64_t grid = (int64_t)((a.BH + 7) / 8) * 8 * nslab;
        const bf16* k = static_cast<const bf16*>(a.k);
        const bf16* v = static_cast<const bf16*>(a.v);
        const bf16* tw = static_cast<const bf16*>(a.tw);
        const TokLayout ly = bwd_layout(a);
        switch (dvs) {
            case 16:
                hipLaunchKernelGGL((bwd_states_mx_kernel<DK, 16>), dim3((unsigned)grid), dim3(16 / 16 * 64 + 64), 0, s,
                                   k, v, tw, a.s0, a.s_all, a.BH, a.L, a.d_v, nslab, ly,
                                   (int)a.sbf);
                break;
            case 32:
                hipLaunchKernelGGL((bwd_states_mx_kernel<DK, 32>), dim3((unsigned)grid), dim3(32 / 16 * 64 + 64), 0, s,
                                   k, v, tw, a.s0, a.s_all, a.BH, a.L, a.d_v, nslab, ly,
                                   (int)a.sbf);
                break;
            default:
                hipLaunchKernelGGL((bwd_states_mx_kernel<DK, 64>), dim3((unsigned)grid), dim3(64 / 16 * 64 + 64), 0, s,
                                   k, v, tw, a.s0, a.s_all, a.BH, a.L, a.d_v, nslab, ly,
                                   (int)a.sbf);
                break;
        }
        *err = hipGetLastError();
        return true;
    }
}

template <int DK, int C>
struct BwdStatesFast<bf16, DK, C> {
    static bool launch(const BwdArgs& a, hipStream_t s, hipError_t* e) { return launch_bwd_states_mx<DK, C>(a, s, e); }
};

template <int DK, int C>
struct BwdChainFast<bf16, DK, C> {
    static bool launch(const BwdArgs& a, hipStream_t s, hipError_t* e) { return launch_bwd_chain_mx<DK, C>(a, s, e); }
};

}  // namespace efla
