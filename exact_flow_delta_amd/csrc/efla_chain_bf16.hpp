// efla_chain_bf16.hpp -- the inter-chunk state pass for bf16 inputs with d_k in {32, 64, 128}.
//
// Same arithmetic as the generic state-pass kernel (per chunk, with S the state entering it and
// Ta = T diag(alpha) read from the UT transform's output:
//   R = V - K S,  Delta = Ta R,  O = Q S + lower_incl(Q K^T) Delta,  S <- S + K^T Delta;
// "Error-Free Linear Attention is a Free Lunch" (howistudyai.com), Step 4; "Exact Flow Linear
// Attention" (gist.science), Metodologia item 3), organised around three gfx950 features:
//
//  * Direct global -> LDS loads.  The next chunk's Q, K, V slab and Ta blocks are fetched with buffer
//    loads that write LDS themselves (16 bytes per lane, one contiguous KiB per wave instruction), so
//    staging takes no registers and no LDS store instructions, and the only vector-memory traffic of a
//    chunk is that prefetch and the output stores.  Lanes whose rows lie past the end of the sequence
//    are outside the buffer range and write zeros.
//  * 16-byte LDS fragment reads.  Every 32-wide slice of d_k is split among the four lane groups as
//    eight consecutive elements each, which makes each Q or K matrix-core fragment one ds_read_b128.
//    The reduction index must run in the same order in the state operand, so the state tile rows are
//    permuted to match: accumulator tile rt = 2 kp + h, lane (r, g), element i holds
//    S[32 kp + 8 g + 4 h + i][column r].  The K^T operand of the state update is read with the
//    transposing LDS read, addressed with the same permutation.
//  * XOR-swizzled, unpadded tiles.  Row t of a tile keeps its 16-byte chunk c at position c ^ sw(t),
//    with sw chosen per row width by measurement (sw_qk below) so that fragment reads and the transposing reads
//    of the state update lose as few cycles as possible to bank conflicts.
//
// One workgroup per (batch*head, slab of DVS state columns): DVS/16 compute waves (16 state columns each; on the
// 128-column slab without outputs, four of 32 columns) and one producer wave that only issues the tile loads and waits for them, so the compute waves never
// stall on the address unit.  All waves meet at one barrier per chunk.  Tiles are fetched two chunks
// ahead into three LDS buffers when they fit (else one chunk ahead into two); the chunk loops are unrolled
// so that the buffers rotate as distinct arrays, which also lets the compiler see that loads into one
// never alias reads of another.  A chunk's outputs are stored a row block at a time while the following
// chunk is computed.
//
// UTW (in-workgroup UT transform, 64-token chunks): more waves form each chunk's Ta in the workgroup itself,
// ahead of the compute waves, from the key tile and the betas already staged in LDS; the keys cross HBM once and
// no workspace is written or read.  Only the diagonal 32 x 32 blocks of Ta are formed (the half-chunk steps read
// no other).
//   UTW = 2: four UT waves, in pairs on alternate chunks, each half-chunk transform cut into two parts run in
//            steps c - 2 and c - 1 for chunk c; the waves running part 1 also issue the loads; LDS rings of
//            their own (keys and betas four chunks deep, queries and V slab two deep), and Ta read by the compute
//            waves from the UT waves' private LDS, where part 2 leaves it.
#pragma once

#include "efla_chunk_split.hpp"

namespace efla {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef bf16x8 __attribute__((address_space(3))) lds_bf16x8;
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) bf16 lds_b16;
typedef f32x4 __attribute__((address_space(3))) lds_f32x4;
typedef bf16x4 __attribute__((address_space(3))) lds_b16x4;

// LDS of one in-workgroup UT wave: two transposed fp32 diagonal blocks of A, then T_bb^T (bf16); Ta^T (three
// bf16 quads) reuses the space of the A blocks
constexpr int kUtHalfAtb = 16 * 20 + 4;                       // floats per transposed diagonal block of A
constexpr int kUtHalfOffTt = 2 * kUtHalfAtb * 4;
constexpr int kUtHalfBytes = kUtHalfOffTt + 2 * 512;

// UTW: 0 none (the UT launch's Ta is read), 2 four in-workgroup UT waves over separate rings (below)
template <int DK, int C, int DVS, int UTW = 0>
struct ChainBf16Shape {
    static constexpr int RBQ = DK * 2;                       // bytes per Q / K row
    static constexpr int RBV = DVS * 2;                      // bytes per V-slab row
    static constexpr int QBYTES = C * RBQ;
    static constexpr int VBYTES = C * RBV;
    static constexpr int NLQ = (QBYTES + 1023) / 1024;       // wave loads (1 KiB each) per Q or K tile
    static constexpr int NLV = (VBYTES + 1023) / 1024;
    static constexpr int TBYTES = TaShape<C>::NQ * TaShape<C>::QE * 2;   // T diag(alpha) blocks of one chunk
    static constexpr int NLT = (TBYTES + 1023) / 1024;
    static constexpr int OFF_Q = 0;
    static constexpr int OFF_K = NLQ * 1024;
    static constexpr int OFF_V = 2 * NLQ * 1024;
    static constexpr int OFF_T = (2 * NLQ + NLV) * 1024;
    static constexpr int BUF = (2 * NLQ + NLV + NLT) * 1024;   // one buffer (each tile rounded up to 1 KiB)
    static constexpr int NBUF = 3 * BUF <= kMaxLdsBytes ? 3 : 2;   // prefetch distance NBUF - 1 chunks
    // UTW == 2: rings of their own -- keys and betas four deep, queries and values two deep -- and four UT
    // waves' private LDS (which also holds the Ta blocks the compute waves read)
    static constexpr int KBS = NLQ * 1024 + 1024;            // K tile, then the betas
    static constexpr int QVS = (NLQ + NLV) * 1024;           // Q tile, then the V slab
    static constexpr int RING2 = 4 * KBS + 2 * QVS + 4 * kUtHalfBytes;
    static constexpr int BYTES = UTW == 2 ? RING2 : NBUF * BUF;
};

// shape of one tile for the load routine: row bytes, wave loads, whether it is a V tile
template <int RB_, int NL_, int ISV_>
struct TileTag {
    static constexpr int RB = RB_;
    static constexpr int NL = NL_;
    static constexpr int ISV = ISV_;
};

// chunk swizzles (16-byte chunks within a row).  256-byte rows (d_k = 128): row t's chunk c sits at c ^ sw(t), sw a
// linear map of the row's low four bits (bits 1, 2, 4, 8 -> masks 3, 10, 5, 4), chosen by timing all 20,160
// invertible maps on gfx950: conflict-free 16-byte fragment reads (16 rows, four chunks each) and the fewest
// conflict cycles of the transposing reads of four rows by four chunks.
template <int DK>
__device__ __forceinline__ int sw_qk(int t) {
    if constexpr (DK == 128) return ((t & 1) ? 3 : 0) ^ ((t & 2) ? 10 : 0) ^ ((t & 4) ? 5 : 0) ^ ((t & 8) ? 4 : 0);
    else if constexpr (DK == 64) return 4 * ((t >> 1) & 1) + ((t >> 2) & 3);
    else return (t >> 2) & 3;
}
// The earlier 256-byte-row swizzle (4 (t & 3) + (t >> 2 & 3)): fewer cycles where transposing reads dominate (the
// backward's state passes measured faster with it)
template <int DK>
__device__ __forceinline__ int sw_qk_tr(int t) {
    if constexpr (DK == 128) return 4 * (t & 3) + ((t >> 2) & 3);
    else return sw_qk<DK>(t);
}
template <int DVS>
__device__ __forceinline__ int sw_v(int t) {
    if constexpr (DVS == 128) return 2 * (t & 7);   // 256-byte rows: 8 rows' chunk pairs on distinct banks
    else if constexpr (DVS == 64) return 2 * ((t >> 1) & 1);
    else return 0;
}

// The UT transform of one 32-token half of a 64-token chunk, from the chunk's key tile (the state pass's
// swizzled layout) and betas in LDS.  The diagonal 32 x 32 blocks of the chunk's Ta = T diag(alpha),
// T = (I + strict_lower(diag(alpha) K K^T))^{-1}, are the halves' own Ta (the diagonal blocks of the inverse of a
// block lower triangular matrix are the inverses of its diagonal blocks), and they are all the half-chunk steps
// of the state pass read; half h is blocks 2h and 2h + 1.  Rows past the end of the sequence hold zero keys and
// betas: their alpha is 0, their rows of T those of I.  One wave runs it in two parts in consecutive chunk steps
// (two pairs of UT waves take alternate chunks, so each has two steps per chunk).
// Part 1 (registers only, no LDS writes): the keys, the Gram blocks (whose diagonals give lambda), the gates,
// A_10 and the two diagonal blocks of A.  Part 2: the diagonal blocks of A into the wave's private LDS, both
// 16 x 16 substitutions by row broadcast, T_bb^T and Ta^T, then T_10.  Ta^T stays in the private LDS for the
// compute waves of the next step, which read it transposed; part 1 of the wave's next chunk, run in that step,
// writes no LDS, and its part 2 comes a step later.  The split point was measured: every substitution step moved
// into part 1, or the gates moved into part 2, made the step slower.
struct UtCarry {
    bf16x4 A10;          // A_10 as a bf16 A operand
    float ar0, ar1;      // gates of rows 16 j + r
    float alpha_mine;    // gate of token 32 h + 16 (g & 1) + r
    f32x4 at0, at1;      // lane (r, g): A_jj[r][4 g + i] of the two diagonal blocks, zero on and above the diagonal
};

template <int DK>
__device__ __forceinline__ void ut_half_part1(const lds_u8* cK, const lds_u8* cB, int gate, int lane, int h,
                                              UtCarry& u) {
    constexpr int NKP = DK / 32;
    constexpr int RBQ = DK * 2;
    typedef Mma<bf16> M;
    typedef bf16x8 bx8;
    const int r = lane & 15;
    const int g = lane >> 4;
    const int gb = g & 1;
    const int swr = sw_qk<DK>(r);
    bx8 kf[2][NKP];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int kp = 0; kp < NKP; ++kp)
            kf[j][kp] = bx8(*reinterpret_cast<const lds_bf16x8*>(cK + (32 * h + 16 * j + r) * RBQ + 16 * ((4 * kp + g) ^ swr)));
    }
    const float beta_mine = reinterpret_cast<const lds_f32*>(cB)[32 * h + (lane & 31)];
    // the three Gram blocks of the half-chunk, (0, 0), (1, 1) and (1, 0): lane (r, g) holds entries (4 g + i, r)
    f32x4 gr[3] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kp = 0; kp < NKP; ++kp) {
        gr[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][kp], kf[0][kp], gr[0], 0, 0, 0);
        gr[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][kp], kf[1][kp], gr[1], 0, 0, 0);
        gr[2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][kp], kf[1][kp], gr[2], 0, 0, 0);
    }
    // lambda of row 16 j + r is the diagonal entry (r, r) of block (j, j), held by lane (r, r / 4) as element r % 4:
    // row r / 4 of the wave, taken to its whole column by two row swaps
    auto diag = [&](const f32x4& blk) __attribute__((always_inline)) {
        float e, o, lo, hi;
        row_swap16(blk[r & 3], e, o);
        row_swap32((r >> 2) & 1 ? o : e, lo, hi);
        return (r >> 3) & 1 ? hi : lo;
    };
    const float lam0 = diag(gr[0]);
    const float lam1 = diag(gr[1]);
    u.alpha_mine = gate_alpha(beta_mine, gb ? lam1 : lam0, gate);
    row_swap16(u.alpha_mine, u.ar0, u.ar1);   // rows 0 and 2 hold block 0's tokens, rows 1 and 3 block 1's
    u.A10 = M::cvt(gr[2] * u.ar1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        u.at0[i] = (4 * g + i < r) ? u.ar0 * gr[0][i] : 0.0f;
        u.at1[i] = (4 * g + i < r) ? u.ar1 * gr[1][i] : 0.0f;
    }
}

// part 2; `scr` is the wave's private kUtHalfBytes, which ends holding Ta^T: quads (0, 0), (1, 0), (1, 1) of the
// half-chunk at bytes 0, 512 and 1024, each a row-major 16 x 16 bf16 block (row c = column c of Ta)
__device__ __forceinline__ void ut_half_part2(lds_u8* scr, int lane, const UtCarry& u) {
    constexpr int LDAT = 20;
    typedef Mma<bf16> M;
    typedef M::quad quad;
    typedef bf16x8 bx8;
    const int r = lane & 15;
    const int g = lane >> 4;
    const int gb = g & 1;
    lds_f32* const sAt = (lds_f32*)scr;
    lds_b16* const sTt = (lds_b16*)(scr + kUtHalfOffTt);
    lds_b16* const sTat = (lds_b16*)scr;
    const int tr = M::tr_offset(lane, 16);
    // transposed diagonal blocks of A (At[m][i] = A[i][m]); lane r then reads row r of its block, column r of A
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        sAt[(4 * g + i) * LDAT + r] = u.at0[i];
        sAt[kUtHalfAtb + (4 * g + i) * LDAT + r] = u.at1[i];
    }
    __asm__ volatile("" ::: "memory");   // this wave's LDS operations complete in order
    float sv[16];   // column r of the lane group's diagonal block of T
    {
        float acol[16];
        const lds_f32* at = sAt + gb * kUtHalfAtb + r * LDAT;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const f32x4 a = *reinterpret_cast<const lds_f32x4*>(at + 4 * i4);
#pragma unroll
            for (int e = 0; e < 4; ++e) acol[4 * i4 + e] = a[e];
        }
        __asm__ volatile("" ::: "memory");   // the block of A is read before Ta^T overwrites it
#pragma unroll
        for (int i = 0; i < 16; ++i) sv[i] = (i == r) ? 1.0f : 0.0f;
        tri_solve_row_bcast<0, 15>(acol, sv);   // rows 2 and 3 repeat rows 0 and 1
    }
    if (g < 2) {
        // row r of T_gg^T and of Ta_gg^T (column r scaled by the gate of token 32 h + 16 g + r)
        bx8 t0v, t1v, a0v, a1v;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            t0v[i] = (bf16)sv[i];
            t1v[i] = (bf16)sv[8 + i];
            a0v[i] = (bf16)(sv[i] * u.alpha_mine);
            a1v[i] = (bf16)(sv[8 + i] * u.alpha_mine);
        }
        lds_b16* tt = sTt + g * 256 + r * 16;
        *reinterpret_cast<lds_bf16x8*>(tt) = t0v;
        *reinterpret_cast<lds_bf16x8*>(tt + 8) = t1v;
        lds_b16* tq = sTat + (2 * g) * 256 + r * 16;   // local quads: 0 = (0, 0), 1 = (1, 0), 2 = (1, 1)
        *reinterpret_cast<lds_bf16x8*>(tq) = a0v;
        *reinterpret_cast<lds_bf16x8*>(tq + 8) = a1v;
    }
    __asm__ volatile("" ::: "memory");
    // T_10 = -T_11 (A_10 T_00)
    {
        const quad T00 = *reinterpret_cast<const lds_b16x4*>(sTt + r * 16 + 4 * g);   // T_00[4g + e][r]
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
        M::mma1(y, u.A10, T00);
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const quad T11 = __builtin_bit_cast(quad, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sTt + 256 + tr)));
        M::mma1(z, T11, M::cvt_neg(y));   // T_11 as the A operand
        // z lane (r, g), element e = T_10[4g + e][r]: row r of Ta_10^T after the column gate of token 32 h + r
        *reinterpret_cast<lds_b16x4*>(sTat + 256 + r * 16 + 4 * g) = M::cvt(z * u.ar0);
    }
    __asm__ volatile("" ::: "memory");
}

// OUT = false: no outputs (the first pass of the segment-parallel forward needs only the final states), so no
// Q tile, no Q S, no Q K^T and no O -- 38 matrix instructions per chunk and wave instead of 100.
// UTW = 2: the in-workgroup UT transform (tw unused; beta and gate read); 64-token chunks with outputs, one
// segment; four UT waves, which also issue the loads, over separate rings (keys and betas four chunks deep, so that
// a UT wave has two steps per chunk).
// State columns per compute wave: 32 on the 128-column slab without outputs (the first pass of the segment-parallel
// forward at d_k = 128: four compute waves, each key fragment read feeding the products of two column tiles, which
// halves the LDS reads that bound that pass), else 16.
template <int DVS, bool OUT, int UTW>
constexpr int chain_cols_per_wave() { return (!OUT && UTW == 0 && DVS == 128) ? 32 : 16; }
template <int DVS, bool OUT, int UTW>
constexpr int chain_threads() { return DVS / chain_cols_per_wave<DVS, OUT, UTW>() * 64 + (UTW == 2 ? 256 : 64); }

template <int DK, int C, int DVS, bool OUT, int UTW = 0>
__global__ __launch_bounds__((chain_threads<DVS, OUT, UTW>())) void chain_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v, const bf16* __restrict__ tw,
    bf16* __restrict__ o, const float* s0, float* sf, int BH, int L, int DV, int nslab, ChainSeg sg,
    TokLayout ly, const float* __restrict__ beta, int gate) {
    typedef ChainBf16Shape<DK, C, DVS, UTW> SH;
    typedef Mma<bf16> M;
    typedef M::quad quad;
    constexpr int CPW = chain_cols_per_wave<DVS, OUT, UTW>();
    constexpr int NW = DVS / CPW;   // compute waves
    static_assert(CPW == 16 || (DK == 128 && C == 64), "32-column waves: d_k = 128, 64-token chunks");
    constexpr int NB = C / 16;
    constexpr int NKD = DK / 16;   // state tiles (16 d_k rows each)
    constexpr int NKP = DK / 32;   // 32-wide d_k slices
    constexpr int NQ = TaShape<C>::NQ;
    constexpr int QE = TaShape<C>::QE;
    constexpr int NCV = DVS / 8;   // 16-byte chunks per V row
    constexpr int NSUB = C > 32 ? C / 32 : 1;   // sub-chunks of at most 32 tokens per chunk
    constexpr int NBS = NB / NSUB;              // row blocks per sub-chunk
    static_assert(DK == 32 || DK == 64 || DK == 128, "d_k of 32, 64 or 128");
    static_assert(SH::BYTES <= kMaxLdsBytes, "state pass LDS too large");
    static_assert(UTW == 0 || (C == 64 && OUT), "in-workgroup UT: 64-token chunks with outputs");
    static_assert(UTW == 0 || UTW == 2, "no in-workgroup UT, or four UT waves");

    constexpr int PD = SH::NBUF - 1;   // chunks fetched ahead
    __shared__ __attribute__((aligned(1024))) unsigned char buf0_[UTW == 2 ? 16 : SH::BUF];
    __shared__ __attribute__((aligned(1024))) unsigned char buf1_[UTW == 2 ? 16 : SH::BUF];
    __shared__ __attribute__((aligned(1024))) unsigned char buf2_[UTW != 2 && PD == 2 ? SH::BUF : 16];
    __shared__ __attribute__((aligned(1024))) unsigned char ring_[UTW == 2 ? SH::RING2 - 4 * kUtHalfBytes : 16];
    __shared__ __attribute__((aligned(16))) unsigned char uts_[UTW == 2 ? 4 * kUtHalfBytes : 16];
    // LDS is addressed only through LDS-space pointers (no generic pointer ever points into it)
    lds_u8* const buf0 = (lds_u8*)buf0_;
    lds_u8* const buf1 = (lds_u8*)buf1_;
    lds_u8* const buf2 = (lds_u8*)buf2_;
    lds_u8* const ring = (lds_u8*)ring_;
    // UTW == 2: chunk x's keys and betas, queries and V slab, and the private LDS of the UT pair that forms its Ta
    auto kbslot = [&](int x) __attribute__((always_inline)) { return ring + (x & 3) * SH::KBS; };
    auto qvslot = [&](int x) __attribute__((always_inline)) { return ring + 4 * SH::KBS + (x & 1) * SH::QVS; };
    auto tpair = [&](int x) __attribute__((always_inline)) { return (const lds_u8*)uts_ + 2 * (x & 1) * kUtHalfBytes; };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15;
    const int g = lane >> 4;

    const int bid = blockIdx.x;
    const int slab = (bid >> 3) % nslab;
    const int bh = ((bid >> 3) / nslab) * 8 + (bid & 7);
    if (bh >= BH) return;
    const int slab_col = slab * DVS;               // column of the state (value columns first, then transition)
    const bool trans = slab >= sg.nslab_v;         // transition slab: zero values, identity start, no outputs
    const bool producer = w == NW;                 // the extra wave: it only fetches
    const int colw = slab_col + CPW * (producer ? 0 : w);
    const SeqView sv = seq_view(ly, bh, L, C);      // this head's tokens: offsets, row strides, length
    const int len = sv.len;
    const int NC = (len + C - 1) / C;
    const int64_t qs = ly.q_t, ks = ly.k_t, vs = ly.v_t, os = ly.o_t;
    const int seg = blockIdx.y, nseg = gridDim.y;
    const int c0 = seg * sg.seg_chunks;            // this workgroup's chunks [c0, c1)
    const int c1 = NC < c0 + sg.seg_chunks ? NC : c0 + sg.seg_chunks;
    const bf16* twh = tw + (int64_t)sv.chunk0 * (NQ * QE);

    // ---- per-lane LDS byte offsets, fixed for the whole sequence ---------------------------------
    // fragment reads: row 16 rb + r, logical chunk 4 kp + g  ->  + 16 * ((4 kp + g) ^ sw(row))
    // (sw of rows 16 rb + r depends on r only, since 16 rb leaves the low four bits alone)
    const int swr = sw_qk<DK>(r);
    // transposing K^T reads: lane (g, e, c) = (lane >> 4, (lane >> 2) & 3, lane & 3): row 16 kb + 4 g + e,
    // logical chunk 4 kp + c, byte 8 h within it; sw of that row depends on (g, e) only
    const int te = 4 * g + ((lane >> 2) & 3);
    const int tc = lane & 3;
    const int swt = sw_qk<DK>(te);
    // transposing V reads: row 16 rb + 4 g + e, columns 16 w + 4 c .. +3: logical chunk 2 w + (c >> 1), byte 8 (c & 1)
    const int v_off = te * SH::RBV + 16 * (((2 * w + (tc >> 1)) % NCV) ^ sw_v<DVS>(te)) + 8 * (tc & 1);
    const int ta_tr = 2 * M::tr_offset(lane, 16);   // transposing reads of a row-major 16 x 16 bf16 block (bytes)

    // ---- loads (producer wave only): wave load j of a tile covers its bytes [1024 j, 1024 j + 1024); lane L
    //      writes 16 bytes at 1024 j + 16 L, i.e. physical chunk p of row t, holding logical chunk p ^ sw(t)
    constexpr int NLOAD = 2 * SH::NLQ + SH::NLV + SH::NLT;   // loads of a chunk's tiles
    // the ones issued: no Q tile without outputs, and no load of Ta quads 6 and 7 with half-chunk steps
    constexpr int NISSUE = NLOAD - (OUT ? 0 : SH::NLQ) - (NSUB == 2 ? 1 : 0);
    // with UTW: the keys and betas of a chunk (issued first), then its queries and values (NQV loads); no Ta load
    constexpr int NQV = SH::NLQ + SH::NLV;
    static_assert(NSUB != 2 || SH::NLT == 5, "Ta of a 64-token chunk is five 1 KiB loads");
    // part 0: every tile of the chunk (Q, K, V, Ta); part 1 (UTW): K and the betas; part 2 (UTW): Q and V
    auto issue_to = [&](int c, lds_u8* dQ, lds_u8* dK, lds_u8* dV, lds_u8* dT, lds_u8* dB, auto part_c)
                        __attribute__((always_inline)) {
        constexpr int PART = decltype(part_c)::value;
        const int t = c * C;
        const int n = (len - t < C) ? (len - t) : C;   // <= 0 past the end: an empty range, zeros
        const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(q + sv.q0 + t * qs, n > 0 ? ((n - 1) * qs + DK) * 2 : 0);
        const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(k + sv.k0 + t * ks, n > 0 ? ((n - 1) * ks + DK) * 2 : 0);
        const __amdgpu_buffer_rsrc_t rv =
            buffer_rsrc(v + sv.v0 + t * vs + slab_col, n > 0 && !trans ? ((n - 1) * vs + DVS) * 2 : 0);
        const __amdgpu_buffer_rsrc_t rt = buffer_rsrc(twh + (int64_t)c * (NQ * QE), SH::TBYTES);
        static_for<NLOAD>([&](auto kc) {
            constexpr int kk = decltype(kc)::value;
            constexpr int tile = kk < SH::NLQ ? 0 : kk < 2 * SH::NLQ ? 1 : kk < 2 * SH::NLQ + SH::NLV ? 2 : 3;
            constexpr int j = tile == 0 ? kk : tile == 1 ? kk - SH::NLQ : tile == 2 ? kk - 2 * SH::NLQ
                                                                                  : kk - 2 * SH::NLQ - SH::NLV;
            constexpr int RB = tile < 2 ? SH::RBQ : SH::RBV;
            lds_void* dst = (lds_void*)((tile == 0 ? dQ : tile == 1 ? dK : tile == 2 ? dV : dT) + 1024 * j);
            const int p = 1024 * j + 16 * lane;
            if constexpr (tile == 0 && !OUT) {
                return;
            } else if constexpr ((PART == 1 && tile != 1) || (PART == 2 && tile != 0 && tile != 2)) {
                return;
            } else if constexpr (tile == 3 && NSUB == 2 && j == 3) {
                // bytes [3072, 4096) of Ta are quads 6 and 7, blocks (3, 0) and (3, 1) of the off-diagonal
                // 32 x 32 block, which the half-chunk steps never read
                return;
            } else if constexpr (tile == 3) {
                // Ta blocks: contiguous in the workspace, copied as they are
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rt, dst, 16, p, 0, 0, 0);
            } else {
                // rows >= C (slack of a last partial load) and rows >= n are out of range and land as zeros
                const int tr = p / RB;
                const int lc = ((p % RB) / 16) ^ (tile == 2 ? sw_v<DVS>(tr) : sw_qk<DK>(tr));
                const int ld = (int)(tile == 2 ? vs : tile == 1 ? ks : qs);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(tile == 0 ? rq : tile == 1 ? rk : rv, dst, 16,
                                                         (tr * ld + 8 * lc) * 2, 0, 0, 0);
            }
        });
        if constexpr (PART == 1) {
            // beta of token t + lane -> 4 bytes at dB + 4 lane (zero past the end)
            const int64_t bt = ly.be_t;
            const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(beta + sv.be0 + t * bt, n > 0 ? (int)(((n - 1) * bt + 1) * 4) : 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)dB, 4, (int)(lane * bt * 4), 0, 0, 0);
        }
    };
    auto issue_chunk = [&](int c, lds_u8* buf) __attribute__((always_inline)) {
        issue_to(c, buf + SH::OFF_Q, buf + SH::OFF_K, buf + SH::OFF_V, buf + SH::OFF_T, buf, std::integral_constant<int, 0>{});
    };
    // wait until at most N vector-memory operations of this wave are in flight and all its LDS operations
    // are done (N is an immediate of the wait instruction; operations retire in issue order)
    auto wait_vm = [&](auto n_c) __attribute__((always_inline)) {
        constexpr int N = decltype(n_c)::value;
        static_assert(N >= 0 && N < 64, "vector-memory count field");
        __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
    };
    typedef std::integral_constant<int, 0> I0;
    typedef std::integral_constant<int, NISSUE> ILOAD;
    typedef std::integral_constant<int, NB> INB;

    if constexpr (UTW == 2) {
        if (w >= NW) {
            // UT wave u: pair u >> 1 takes the chunks of that parity, u & 1 is its half.  In step c (c0 - 2 <= c < c1)
            // pair c & 1 runs part 1 of chunk c + 2 and the other pair part 2 of chunk c + 1 (which writes its Ta).
            // The UT waves also issue the loads: wave 0 before the first barrier the keys and betas of chunks
            // c0 .. c0 + 2 and the queries and values of c0; in step c >= c0 the pair running part 1, its first wave
            // the keys and betas of c + 3 and its second the queries and values of c + 1, each landed by the end of
            // the step (issued by the part-2 pair instead, they measured slower).
            typedef std::integral_constant<int, 1> I1;
            typedef std::integral_constant<int, 2> I2;
            const int u = w - NW;
            const int pair = u >> 1, half = u & 1;
            const bool prod = u == 0;
            lds_u8* const scr = (lds_u8*)uts_ + u * kUtHalfBytes;
            auto issue_kb = [&](int x) __attribute__((always_inline)) {
                lds_u8* d = kbslot(x);
                issue_to(x, d, d, d, d, d + SH::NLQ * 1024, I1{});
            };
            auto issue_qv = [&](int x) __attribute__((always_inline)) {
                lds_u8* d = qvslot(x);
                issue_to(x, d, d, d + SH::NLQ * 1024, d, d, I2{});
            };
            UtCarry uc;
            if (c1 > c0) {
                if (prod) {
                    issue_kb(c0);
                    if (c0 + 1 < c1) issue_kb(c0 + 1);
                    if (c0 + 2 < c1) issue_kb(c0 + 2);
                    issue_qv(c0);
                    wait_vm(I0{});
                }
                __builtin_amdgcn_s_barrier();
                for (int c = c0 - 2; c < c1; ++c) {
                    if (u == 2 * (c & 1) && c >= c0 && c + 3 < c1) issue_kb(c + 3);
                    if (u == 2 * (c & 1) + 1 && c >= c0 && c + 1 < c1) issue_qv(c + 1);
                    if ((c & 1) == pair) {
                        if (c + 2 < c1) {
                            lds_u8* kb = kbslot(c + 2);
                            ut_half_part1<DK>(kb, kb + SH::NLQ * 1024, gate, lane, half, uc);
                        }
                    } else if (c + 1 >= c0 && c + 1 < c1) {
                        ut_half_part2(scr, lane, uc);
                    }
                    wait_vm(I0{});   // this step's loads have landed and this wave's LDS writes are done
                    __builtin_amdgcn_s_barrier();
                }
            }
            return;
        }
    } else if (producer) {
        // Chunk c's tiles go out at the step of chunk c - PD (the prologue fetches the first PD).  At the end
        // of the step of chunk c those of chunk c + 1 must have landed; with PD = 2 the ones issued during
        // the step (chunk c + 2) may still be in flight.  One barrier per step, as the compute waves.
        if (c1 > c0) {
            issue_chunk(c0, buf0);
            if (PD == 2 && c0 + 1 < c1) {
                issue_chunk(c0 + 1, buf1);
                wait_vm(ILOAD{});
            } else {
                wait_vm(I0{});
            }
            __builtin_amdgcn_s_barrier();
        }
        auto pstep = [&](int c, lds_u8* nxt) __attribute__((always_inline)) {
            if (c + PD < c1) {
                issue_chunk(c + PD, nxt);
                if constexpr (PD == 2) wait_vm(ILOAD{}); else wait_vm(I0{});
            } else {
                wait_vm(I0{});
            }
            __builtin_amdgcn_s_barrier();
        };
        if constexpr (PD == 2) {
            for (int c = c0; c < c1; c += 3) {
                pstep(c, buf2);
                if (c + 1 < c1) pstep(c + 1, buf0);
                if (c + 2 < c1) pstep(c + 2, buf1);
            }
        } else {
            for (int c = c0; c < c1; c += 2) {
                pstep(c, buf1);
                if (c + 1 < c1) pstep(c + 1, buf0);
            }
        }
        return;
    }

    // ---- the state: S[32 kp + 8 g + 4 h + i][colw + r] in tile rt = 2 kp + h, element i ------------------
    auto srow = [&](int rt, int i) __attribute__((always_inline)) { return 32 * (rt >> 1) + 8 * g + 4 * (rt & 1) + i; };

    if constexpr (CPW == 32) {
        // Two 16-column state tiles per wave (columns colw .. +15 and colw + 16 .. +31), no outputs: per 32-token
        // sub-chunk R = V - K S, Delta = Ta R, S += K^T Delta for both tiles, every key fragment, transposed key block
        // and Ta block read once for the two.
        typedef bf16x8 bx8;
        typedef quad __attribute__((address_space(3))) lds_quad;
        f32x4 S2[2][NKD];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const int col = colw + 16 * ct;
#pragma unroll
            for (int rt = 0; rt < NKD; ++rt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = srow(rt, i);
                    S2[ct][rt][i] = trans ? (row == col - DV + r ? 1.0f : 0.0f)
                                          : s0 ? s0[(((int64_t)bh * nseg + seg) * DK + row) * DV + col + r] : 0.0f;
                }
            }
        }
        // transposing V reads of tile ct: row 16 rb + 4 g + e, columns 32 w + 16 ct + 4 c .. +3 of the slab
        int v_off2[2];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
            v_off2[ct] = te * SH::RBV + 16 * (((2 * (2 * w + ct) + (tc >> 1)) % NCV) ^ sw_v<DVS>(te)) + 8 * (tc & 1);
        auto pair = [&](quad a, quad b) __attribute__((always_inline)) -> bx8 { return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7); };
        auto step32 = [&](const lds_u8* cK, const lds_u8* cV, const lds_u8* cT) __attribute__((always_inline)) {
            auto frag = [&](int rb, int kp) __attribute__((always_inline)) {   // row 16 rb + r, d_k 32 kp + 8 g .. +7
                return bx8(*reinterpret_cast<const lds_bf16x8*>(cK + (16 * rb + r) * SH::RBQ + 16 * ((4 * kp + g) ^ swr)));
            };
            auto kt = [&](int rt, int kb) __attribute__((always_inline)) {
                const int off = te * SH::RBQ + 16 * ((4 * (rt >> 1) + tc) ^ swt) + 8 * (rt & 1);
                return __builtin_bit_cast(quad, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                    (lds_s16x4*)(const_cast<lds_u8*>(cK) + 16 * kb * SH::RBQ + off)));
            };
            auto ta = [&](int rb, int kb) __attribute__((always_inline)) {
                return *reinterpret_cast<const lds_quad*>(cT + 512 * (rb * (rb + 1) / 2 + kb) + 8 * lane);
            };
            auto vblk = [&](int rb, int ct) __attribute__((always_inline)) {
                return __builtin_bit_cast(quad, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                    (lds_s16x4*)(const_cast<lds_u8*>(cV) + 16 * rb * SH::RBV + v_off2[ct])));
            };
            static_for<NSUB>([&](auto hc) {
                constexpr int b0 = decltype(hc)::value * NBS;
                bx8 Sq[2][NKP];
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                    for (int kp = 0; kp < NKP; ++kp) Sq[ct][kp] = pair(M::cvt(S2[ct][2 * kp]), M::cvt(S2[ct][2 * kp + 1]));
                quad Rq[2][NBS];
                static_for<NBS>([&](auto jc) {
                    constexpr int rb = b0 + decltype(jc)::value;
                    bx8 kq[NKP];
#pragma unroll
                    for (int kp = 0; kp < NKP; ++kp) kq[kp] = frag(rb, kp);
                    f32x4 xk[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
                    for (int kp = 0; kp < NKP; ++kp)
#pragma unroll
                        for (int ct = 0; ct < 2; ++ct)
                            xk[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kq[kp], Sq[ct][kp], xk[ct], 0, 0, 0);   // K S
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) {
                        const quad vq = vblk(rb, ct);
                        f32x4 rr;
#pragma unroll
                        for (int e = 0; e < 4; ++e) rr[e] = (float)vq[e] - xk[ct][e];
                        Rq[ct][decltype(jc)::value] = M::cvt(rr);
                    }
                });
                quad Dq[2][NBS];
                static_for<NBS>([&](auto jc) {
                    constexpr int j = decltype(jc)::value;
                    constexpr int rb = b0 + j;
                    f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
                    static_for<(j + 1) / 2>([&](auto pc) {
                        constexpr int i = 2 * decltype(pc)::value;
                        const quad a0 = ta(rb, b0 + i), a1 = ta(rb, b0 + i + 1);
#pragma unroll
                        for (int ct = 0; ct < 2; ++ct) M::mma2(acc[ct], a0, a1, Rq[ct][i], Rq[ct][i + 1]);
                    });
                    if constexpr ((j + 1) & 1) {
                        const quad a = ta(rb, rb);
#pragma unroll
                        for (int ct = 0; ct < 2; ++ct) M::mma1(acc[ct], a, Rq[ct][j]);
                    }
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) Dq[ct][j] = M::cvt(acc[ct]);
                });
                static_assert(NBS == 2, "two row blocks per sub-chunk");
                quad k0[NKD], k1[NKD];
#pragma unroll
                for (int rt = 0; rt < NKD; ++rt) {
                    k0[rt] = kt(rt, b0);
                    k1[rt] = kt(rt, b0 + 1);
                }
#pragma unroll
                for (int rt = 0; rt < NKD; ++rt)
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) M::mma2(S2[ct][rt], k0[rt], k1[rt], Dq[ct][0], Dq[ct][1]);
            });
            wait_vm(I0{});   // LDS reads done
            __builtin_amdgcn_s_barrier();
        };
        auto stepb32 = [&](const lds_u8* b) __attribute__((always_inline)) {
            step32(b + SH::OFF_K, b + SH::OFF_V, b + SH::OFF_T);
        };
        static_assert(PD == 2, "three buffers");
        if (c1 > c0) __builtin_amdgcn_s_barrier();   // the producer's prologue
        for (int c = c0; c < c1; c += 3) {
            stepb32(buf0);
            if (c + 1 < c1) stepb32(buf1);
            if (c + 2 < c1) stepb32(buf2);
        }
        if (sf && (sg.sf_all || seg == nseg - 1)) {
            const int64_t base = sg.sf_all ? (int64_t)bh * nseg + seg : bh;
            const int ld = sg.sf_all ? sg.ld_sf : DV;
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int rt = 0; rt < NKD; ++rt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) sf[(base * DK + srow(rt, i)) * ld + colw + 16 * ct + r] = S2[ct][rt][i];
        }
        return;
    }
    f32x4 S[NKD];
#pragma unroll
    for (int rt = 0; rt < NKD; ++rt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = srow(rt, i);
            S[rt][i] = trans ? (row == colw - DV + r ? 1.0f : 0.0f)
                             : s0 ? s0[(((int64_t)bh * nseg + seg) * DK + row) * DV + colw + r] : 0.0f;
        }
    }
    const bool write_o = o != nullptr && !trans;

    f32x4 Ot[NB];
#pragma unroll
    for (int rb = 0; rb < NB; ++rb) Ot[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
    int pend_t0 = 0, pend_n = 0;   // the computed chunk whose outputs are still to be stored (none: n = 0)
    // row block rb of those outputs, through a buffer range ending at the chunk's last valid row (an
    // empty range before the first chunk)
    auto store_pending = [&](int rb) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t ors =
            buffer_rsrc(o + sv.o0 + pend_t0 * os + colw, pend_n > 0 ? ((pend_n - 1) * os + 16) * 2 : 0);
        buffer_store<quad>(ors, ((16 * rb + r) * (int)os + 4 * g) * 2, M::cvt(Ot[rb]));
    };

    // one chunk of the compute waves: the previous chunk's outputs are stored a row block at a time while
    // this one is computed
    auto step = [&](int c, const lds_u8* cQ, const lds_u8* cK, const lds_u8* cV, const lds_u8* cT)
                    __attribute__((always_inline)) {
        typedef bf16x8 bx8;
        auto frag = [&](const lds_u8* tile, int rb, int kp) __attribute__((always_inline)) {   // row 16 rb + r, d_k 32 kp + 8 g .. +7
            return bx8(*reinterpret_cast<const lds_bf16x8*>(tile + (16 * rb + r) * SH::RBQ + 16 * ((4 * kp + g) ^ swr)));
        };
        auto pair = [&](quad a, quad b) __attribute__((always_inline)) -> bx8 { return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7); };

        // S += K^T Delta: tile rt = 2 kp + h takes, as A operand, the transposed K block whose lane (g, e, c)
        // points at row 16 kb + 4 g + e, logical chunk 4 kp + c, byte 8 h
        auto kt = [&](int rt, int kb) __attribute__((always_inline)) {
            const int off = te * SH::RBQ + 16 * ((4 * (rt >> 1) + tc) ^ swt) + 8 * (rt & 1);
            return __builtin_bit_cast(quad, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                (lds_s16x4*)(const_cast<lds_u8*>(cK) + 16 * kb * SH::RBQ + off)));
        };
        typedef quad __attribute__((address_space(3))) lds_quad;
        // The chunk is stepped through in sub-chunks of NBS row blocks (32 tokens): the sub-chunks' T diag(alpha)
        // are the diagonal 32 x 32 blocks of the chunk's (the diagonal blocks of the inverse of a block lower
        // triangular matrix are the inverses of its diagonal blocks), so the same UT output serves, and the
        // intra-chunk products shrink: Q K^T, Delta and O take 32 instead of 52 matrix instructions per 64 tokens.
        static_for<NSUB>([&](auto hc) {
            constexpr int b0 = decltype(hc)::value * NBS;   // first row block of the sub-chunk
            bx8 Sq[NKP];   // state operand: lane (r, g) holds S[32 kp + 8 g .. +7][colw + r]
#pragma unroll
            for (int kp = 0; kp < NKP; ++kp) Sq[kp] = pair(M::cvt(S[2 * kp]), M::cvt(S[2 * kp + 1]));
            quad Rq[NBS];
            bx8 kq[NBS][NKP];
            quad Pq[NBS * (NBS + 1) / 2];   // block (j, lo) of the sub-chunk at j (j + 1) / 2 + lo
            // Delta = Ta R over the sub-chunk; Ta block (rb, kb) of the chunk is quad qi = rb (rb + 1) / 2 + kb,
            // lane (r, g)'s at byte 512 qi + 8 lane
            auto ta = [&](int rb, int kb) __attribute__((always_inline)) {
                if constexpr (UTW == 2) {
                    // from the private LDS of the half's UT wave: its Ta^T quads (0, 0), (1, 0), (1, 1), read
                    // transposed
                    const int hh = rb / NBS, lr = rb - hh * NBS, lk = kb - hh * NBS;
                    return __builtin_bit_cast(quad, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4*)(const_cast<lds_u8*>(cT) + hh * kUtHalfBytes + 512 * (lr * (lr + 1) / 2 + lk) + ta_tr)));
                } else {
                    return *reinterpret_cast<const lds_quad*>(cT + 512 * (rb * (rb + 1) / 2 + kb) + 8 * lane);
                }
            };
            // R = V - K S: lane (r, g), element e of row block rb: row 16 rb + 4g + e, column 16 w + r of the slab
            auto vblk = [&](int rb) __attribute__((always_inline)) {
                return __builtin_bit_cast(quad, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                    (lds_s16x4*)(const_cast<lds_u8*>(cV) + 16 * rb * SH::RBV + v_off)));
            };
            static_for<NBS>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                constexpr int rb = b0 + j;
                if constexpr (OUT) store_pending(rb);
                bx8 qq[NKP];
#pragma unroll
                for (int kp = 0; kp < NKP; ++kp) {
                    if constexpr (OUT) qq[kp] = frag(cQ, rb, kp);
                    kq[j][kp] = frag(cK, rb, kp);
                }
                f32x4 xk = {0.f, 0.f, 0.f, 0.f};
                Ot[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kp = 0; kp < NKP; ++kp) {
                    if constexpr (OUT) Ot[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Sq[kp], qq[kp], Ot[rb], 0, 0, 0);   // (Q S)^T
                    xk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kq[j][kp], Sq[kp], xk, 0, 0, 0);       // K S
                }
                const quad vq = vblk(rb);
                f32x4 rr;
#pragma unroll
                for (int e = 0; e < 4; ++e) rr[e] = (float)vq[e] - xk[e];
                Rq[j] = M::cvt(rr);
                if constexpr (!OUT) return;
                // block row rb of lower_incl(Q K^T) within the sub-chunk: acc lane (r, g), element e =
                // (Q K^T)[16 rb + r][16 (b0 + lo) + 4g + e]; the blocks' chains are interleaved (reduction step
                // outer) so that consecutive matrix instructions are independent
                f32x4 pacc[j + 1];
#pragma unroll
                for (int lo = 0; lo <= j; ++lo) pacc[lo] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kp = 0; kp < NKP; ++kp) {
#pragma unroll
                    for (int lo = 0; lo <= j; ++lo)
                        pacc[lo] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kq[lo][kp], qq[kp], pacc[lo], 0, 0, 0);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) pacc[j][e] = (4 * g + e <= r) ? pacc[j][e] : 0.0f;
#pragma unroll
                for (int lo = 0; lo <= j; ++lo) Pq[j * (j + 1) / 2 + lo] = M::cvt(pacc[lo]);
            });
            // the transposed key blocks of the state update depend on nothing computed in the sub-chunk: with the
            // UT waves in the workgroup, read them all here, ahead of the Delta products, and keep the scheduler
            // from sinking them to their uses (measured faster there, slower in the state pass on its own)
            constexpr bool kKtEarly = UTW == 2;
            quad kte[NBS][NKD];
            if constexpr (kKtEarly) {
#pragma unroll
                for (int rt = 0; rt < NKD; ++rt)
#pragma unroll
                    for (int i = 0; i < NBS; ++i) kte[i][rt] = kt(rt, b0 + i);
                __builtin_amdgcn_sched_barrier(0);
            }
            auto ktb = [&](int rt, int kb) __attribute__((always_inline)) {
                if constexpr (kKtEarly) return kte[kb - b0][rt];
                else return kt(rt, kb);
            };
            quad Dq[NBS];
            static_for<NBS>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                constexpr int rb = b0 + j;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                static_for<(j + 1) / 2>([&](auto pc) {
                    constexpr int i = 2 * decltype(pc)::value;
                    M::mma2(acc, ta(rb, b0 + i), ta(rb, b0 + i + 1), Rq[i], Rq[i + 1]);
                });
                if constexpr ((j + 1) & 1) M::mma1(acc, ta(rb, rb), Rq[j]);
                Dq[j] = M::cvt(acc);
            });
            // O^T += Delta^T lower_incl(Q K^T)^T within the sub-chunk (stored with the next chunk)
            if constexpr (OUT) {
                static_for<NBS>([&](auto jc) {
                    constexpr int j = decltype(jc)::value;
                    constexpr int p0 = j * (j + 1) / 2;
                    static_for<(j + 1) / 2>([&](auto pc) {
                        constexpr int i = 2 * decltype(pc)::value;
                        M::mma2(Ot[b0 + j], Dq[i], Dq[i + 1], Pq[p0 + i], Pq[p0 + i + 1]);
                    });
                    if constexpr ((j + 1) & 1) M::mma1(Ot[b0 + j], Dq[j], Pq[p0 + j]);
                });
            }
            // S += K^T Delta over the sub-chunk; the tiles' chains are interleaved
#pragma unroll
            for (int i = 0; i + 1 < NBS; i += 2) {
                quad k0[NKD], k1[NKD];
#pragma unroll
                for (int rt = 0; rt < NKD; ++rt) {
                    k0[rt] = ktb(rt, b0 + i);
                    k1[rt] = ktb(rt, b0 + i + 1);
                }
#pragma unroll
                for (int rt = 0; rt < NKD; ++rt) M::mma2(S[rt], k0[rt], k1[rt], Dq[i], Dq[i + 1]);
            }
            if constexpr (NBS & 1) {
#pragma unroll
                for (int rt = 0; rt < NKD; ++rt) M::mma1(S[rt], ktb(rt, b0 + NBS - 1), Dq[NBS - 1]);
            }
        });
        pend_t0 = c * C;
        pend_n = !write_o ? 0 : (len - pend_t0 < C) ? (len - pend_t0) : C;
        wait_vm(INB{});   // LDS reads done; only this chunk's stores may still be in flight
        __builtin_amdgcn_s_barrier();
    };

    auto stepb = [&](int c, const lds_u8* b) __attribute__((always_inline)) {
        step(c, b + SH::OFF_Q, b + SH::OFF_K, b + SH::OFF_V, b + SH::OFF_T);
    };
    if constexpr (UTW == 2) {
        if (c1 > c0) {
            // the loads' prologue, then the two steps in which the UT waves start chunks c0 and c0 + 1
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_s_barrier();
        }
        // one segment (c0 = 0): unrolled over the key ring's four slots, so that every slot is a constant offset
        auto stepr = [&](int c, int i) __attribute__((always_inline)) {
            const lds_u8* qv = qvslot(i);
            step(c, qv, kbslot(i), qv + SH::NLQ * 1024, tpair(i));
        };
        for (int c = 0; c < c1; c += 4) {
            stepr(c, 0);
            if (c + 1 < c1) stepr(c + 1, 1);
            if (c + 2 < c1) stepr(c + 2, 2);
            if (c + 3 < c1) stepr(c + 3, 3);
        }
    } else {
        if (c1 > c0) {
            __builtin_amdgcn_s_barrier();   // the producer's prologue
        }
        if constexpr (PD == 2) {
            for (int c = c0; c < c1; c += 3) {
                stepb(c, buf0);
                if (c + 1 < c1) stepb(c + 1, buf1);
                if (c + 2 < c1) stepb(c + 2, buf2);
            }
        } else {
            for (int c = c0; c < c1; c += 2) {
                stepb(c, buf0);
                if (c + 1 < c1) stepb(c + 1, buf1);
            }
        }
    }
    if constexpr (OUT) {
#pragma unroll
        for (int rb = 0; rb < NB; ++rb) store_pending(rb);
    }

    if (sf && (sg.sf_all || seg == nseg - 1)) {
        const int64_t base = sg.sf_all ? (int64_t)bh * nseg + seg : bh;
        const int ld = sg.sf_all ? sg.ld_sf : DV;
#pragma unroll
        for (int rt = 0; rt < NKD; ++rt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) sf[(base * DK + srow(rt, i)) * ld + colw + r] = S[rt][i];
        }
    }
}

template <int DK, int C, int DVS>
hipError_t launch_chain_bf16(const SplitArgs& a, hipStream_t stream) {
    if constexpr (DVS == 128) {
        // the 128-column slab (eight compute waves) is built for the pass without outputs only
        if (a.o != nullptr) return hipErrorInvalidValue;
    }
    const ChainSeg sg = chain_seg(a, DK, C, DVS);
    const TokLayout ly = a.layout ? *a.layout : contiguous_layout(1, a.L, DK, a.d_v);
    const int nslab = (a.d_v + (a.aug ? DK : 0)) / DVS;
    const int64_t grid = (int64_t)((a.BH + 7) / 8) * 8 * nslab;
    const dim3 g3((unsigned)grid, (unsigned)(a.nseg > 0 ? a.nseg : 1));
    if (a.o == nullptr)
        hipLaunchKernelGGL((chain_bf16_kernel<DK, C, DVS, false>), g3, dim3(chain_threads<DVS, false, 0>()), 0, stream,
                           static_cast<const bf16*>(a.q), static_cast<const bf16*>(a.k), static_cast<const bf16*>(a.v),
                           static_cast<const bf16*>(a.tw), static_cast<bf16*>(a.o), a.s0, a.sf, a.BH, a.L, a.d_v, nslab,
                           sg, ly, nullptr, 0);
    else if constexpr (DVS != 128)
        hipLaunchKernelGGL((chain_bf16_kernel<DK, C, DVS, true>), g3, dim3(chain_threads<DVS, true, 0>()), 0, stream,
                           static_cast<const bf16*>(a.q), static_cast<const bf16*>(a.k), static_cast<const bf16*>(a.v),
                           static_cast<const bf16*>(a.tw), static_cast<bf16*>(a.o), a.s0, a.sf, a.BH, a.L, a.d_v, nslab,
                           sg, ly, nullptr, 0);
    return hipGetLastError();
}

// LDS bytes of the one-launch forward (mirror of ChainBf16Shape<.., 2>)
constexpr int chain_ut_bf16_bytes(int dk, int dvs) {
    const int nlq = (64 * dk * 2 + 1023) / 1024, nlv = (64 * dvs * 2 + 1023) / 1024;
    return 4 * (nlq + 1) * 1024 + 2 * (nlq + nlv) * 1024 + 4 * kUtHalfBytes;
}

// The whole chunked forward in one launch (bf16, d_k >= 32, 64-token chunks; contiguous [B,H,L,d], or the strided
// views and packed sequences of a.layout): the state pass with its own UT waves in every workgroup.
template <int DK, int DVS>
hipError_t launch_chain_ut_bf16_t(const ChunkArgs& a, hipStream_t stream) {
    typedef ChainBf16Shape<DK, 64, DVS, 2> SH;
    static_assert(SH::BYTES == chain_ut_bf16_bytes(DK, DVS), "host mirror of the LDS size");
    SplitArgs sa{};
    sa.BH = a.BH;
    sa.L = a.L;
    sa.d_k = DK;
    sa.d_v = a.d_v;
    sa.chunk = 64;
    sa.dvs = DVS;
    const ChainSeg sg = chain_seg(sa, DK, 64, DVS);
    const TokLayout ly = a.layout ? *a.layout : contiguous_layout(1, a.L, DK, a.d_v);
    const int nslab = a.d_v / DVS;
    const int64_t grid = (int64_t)((a.BH + 7) / 8) * 8 * nslab;
    const int threads = DVS / 16 * 64 + 256;
    hipLaunchKernelGGL((chain_bf16_kernel<DK, 64, DVS, true, 2>), dim3((unsigned)grid), dim3(threads),
                       0, stream, static_cast<const bf16*>(a.q), static_cast<const bf16*>(a.k),
                       static_cast<const bf16*>(a.v), nullptr, static_cast<bf16*>(a.o), a.s0, a.sf, a.BH, a.L, a.d_v,
                       nslab, sg, ly, a.beta, a.gate);
    return hipGetLastError();
}

template <int DK>
hipError_t launch_chain_ut_bf16_dvs(const ChunkArgs& a, hipStream_t stream) {
    switch (a.dvs) {
        case 16: return launch_chain_ut_bf16_t<DK, 16>(a, stream);
        case 32: return launch_chain_ut_bf16_t<DK, 32>(a, stream);
        case 64: return launch_chain_ut_bf16_t<DK, 64>(a, stream);
    }
    return hipErrorInvalidValue;
}

inline hipError_t launch_chain_ut_bf16(const ChunkArgs& a, hipStream_t stream) {
    switch (a.d_k) {
        case 32: return launch_chain_ut_bf16_dvs<32>(a, stream);
        case 64: return launch_chain_ut_bf16_dvs<64>(a, stream);
        case 128: return launch_chain_ut_bf16_dvs<128>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace efla
