// efla_chunk_split.hpp -- the chunkwise EFLA forward as two kernels: the intra-chunk UT transform over
// every (head, chunk) at once, then the inter-chunk state pass.
//
// Per chunk of C tokens (rows k_t, q_t, v_t, gates alpha_t) with S the state entering it:
//   A = strict_lower(diag(alpha) K K^T),  T = (I + A)^{-1},  Ta = T diag(alpha)           [UT kernel]
//   R = V - K S,  Delta = Ta R,  O = Q S + lower_incl(Q K^T) Delta,  S <- S + K^T Delta   [chain kernel]
// ("Exact Flow Linear Attention" (gist.science), Metodologia item 3: the rank-1 delta-rule form is kept,
// so the WY/UT chunk scheme applies; "Error-Free Linear Attention is a Free Lunch" (howistudyai.com),
// Step 4: within-chunk transforms in parallel, chunks joined by passing the state.)
//
// The UT transform does not depend on the state, so it runs as its own launch with one workgroup per
// (batch*head, chunk) -- thousands of small independent workgroups, several per compute unit, which hide
// each other's latency -- and the sequential state pass no longer carries it.  Ta travels through a
// workspace in the exact register layout in which the state pass consumes it as a matrix-core operand:
//   tw[bh][c][qi][lane][j],  qi = rb (rb + 1) / 2 + kb for kb <= rb < C/16,  lane = 16 g + r,
//   element j = Ta[16 rb + r][16 kb + 4 g + j]          (storage type of q/k/v; 256 elements per block)
// so each wave of the state pass loads its operands with plain coalesced vector loads, no LDS staging.
//
// State pass: one workgroup per (batch*head, slab of DVS state columns); each wave owns 16 columns and
// keeps its d_k x 16 piece of S in fp32 registers for the whole sequence.  Q, K and the V slab of the
// next chunk are staged into a second LDS buffer while the current chunk is being processed (one
// barrier per chunk).  Each wave forms the block-lower Q K^T of the chunk from the Q and K fragments it
// reads for Q S and K S anyway, so that product costs no LDS traffic and no exchange between waves.
#pragma once

#include <type_traits>

#include "efla_common.hpp"
#include "efla_launch.hpp"
#include "efla_ut.hpp"
#include "efla_ut_wave.hpp"

namespace efla {

// rows [0, n) of a C x W tile of a row-major matrix (leading dimension ld) in 16-byte vectors spread
// over NT threads; rows n .. C-1 (and the idle slots of a last partial pass) read as zeros through the
// range check of a buffer resource covering exactly the valid rows
template <typename E, int C, int W, int NT>
struct TileRegs {
    typedef typename Vec16<E>::type V16;
    static constexpr int VEC = Vec16<E>::N;
    static constexpr int VPR = W / VEC;
    static constexpr int N = (C * VPR + NT - 1) / NT;
    V16 x[N];

    // Rows >= n read as zeros: the range ends at row n - 1, and with a row stride ld >= W every later row
    // starts past it.
    __device__ __forceinline__ void load(const E* __restrict__ base, int ld, int n, int tid) {
        if constexpr (NT % VPR == 0) {
            // pass `it` covers rows it * RPI + tid / VPR: one (wave-uniform) range per pass, so that a
            // single per-lane offset serves every pass whatever the row stride
            constexpr int RPI = NT / VPR;
            const int lane_off = ((tid / VPR) * ld + (tid % VPR) * VEC) * (int)sizeof(E);
#pragma unroll
            for (int it = 0; it < N; ++it) {
                const int nr = n - it * RPI;
                const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(base + (int64_t)it * RPI * ld,
                                                              nr > 0 ? ((nr - 1) * ld + W) * (int)sizeof(E) : 0);
                x[it] = buffer_load<V16>(rs, lane_off);
            }
        } else {
            const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(base, n > 0 ? ((n - 1) * ld + W) * (int)sizeof(E) : 0);
#pragma unroll
            for (int it = 0; it < N; ++it) {
                const int idx = it * NT + tid;   // idx >= C * VPR lands on a row >= C >= n: out of range
                x[it] = buffer_load<V16>(rs, ((idx / VPR) * ld + (idx % VPR) * VEC) * (int)sizeof(E));
            }
        }
    }
    __device__ __forceinline__ void store(E* s, int lds_ld, int tid) const {
#pragma unroll
        for (int it = 0; it < N; ++it) {
            const int idx = it * NT + tid;
            // only a last partial pass has idle slots (tid < NT is not visible to the compiler)
            if ((C * VPR) % NT == 0 || it + 1 < N || idx < C * VPR)
                lds_store_vec16(s + (idx / VPR) * lds_ld + (idx % VPR) * VEC, x[it]);
        }
    }
};

template <int C>
struct TaShape {
    static constexpr int NB = C / 16;
    static constexpr int NQ = NB * (NB + 1) / 2;   // 16x16 blocks of the lower triangle
    static constexpr int QE = 256;                  // elements per block in the workspace
};

// ------------------------------------------------------------------------------------------------
// UT kernel.  C/16 waves per workgroup; a grid of a few workgroups per compute unit walks the
// (batch*head, chunk) pairs u = blockIdx.x, blockIdx.x + gridDim.x, ..., prefetching the next pair's
// keys and steps into registers while the current one is transformed.
// ------------------------------------------------------------------------------------------------
template <int ESIZE, int DK, int C>
struct UtLayout {
    static constexpr int PAD = ESIZE == 2 ? 20 : 4;
    static constexpr int LD_DK = DK + PAD;
    static constexpr int LD_CE = C + PAD;
    static constexpr int OFF_K = 0;
    static constexpr int OFF_A = OFF_K + C * LD_DK * ESIZE;
    static constexpr int OFF_AT = OFF_A + C * LD_CE * ESIZE;
    static constexpr int OFF_TT = OFF_AT + C * kLdAt * 4;
    static constexpr int OFF_TAT = OFF_TT + C * LD_CE * ESIZE;
    static constexpr int OFF_LB = OFF_TAT + C * LD_CE * ESIZE;   // lambda[C], beta[C]
    static constexpr int OFF_ALPHA = OFF_LB + 2 * C * 4;
    static constexpr int BYTES = OFF_ALPHA + C * 4;
};

// host-side mirror of UtLayout::BYTES
template <int ESIZE>
constexpr int ut_layout_bytes(int dk, int c) {
    const int pad = ESIZE == 2 ? 20 : 4;
    return c * (dk + pad) * ESIZE + 3 * c * (c + pad) * ESIZE + c * kLdAt * 4 + 3 * c * 4;
}

// Gram blocks and diagonal solves of one chunk, balanced over NW = C/16 waves: wave w forms the diagonal
// block (w, w) of A and solves T_ww = (I + A_ww)^{-1} from it; the off-diagonal blocks (hi, lo), lo < hi,
// numbered in row order, go round-robin to the waves.  Every wave evaluates the gate of all C tokens once
// (lane 16 g + r: token 16 g + r) and takes the ones it needs from the owning lanes; wave 0 publishes them
// for the off-diagonal phase.  The solve is right-looking forward substitution in fp32 (lane r carries
// column r; step m reads column m of the block as one broadcast row of At), with every row of At read
// before the first step so that the substitution runs at arithmetic speed.
template <typename E, int DK, int C, int LD_DK, int LD_CE>
__device__ __forceinline__ void ut_rows_balanced(const E* sK, const float* sLam, const float* sBeta, float* sAlpha,
                                                 E* sA, float* sAt, E* sTt, E* sTat, int w, int r, int g, int gate) {
    typedef Mma<E> M;
    typedef typename M::quad quad;
    constexpr int NB = C / 16;
    constexpr int NW = NB;
    constexpr int NKD = DK / 16;
    const int lane = 16 * g + r;
    const float a_mine = lane < C ? gate_alpha(sBeta[lane < C ? lane : 0], sLam[lane < C ? lane : 0], gate) : 0.0f;
    if (w == 0 && lane < C) sAlpha[lane] = a_mine;
    auto alpha_of_row = [&](int blk) { return __shfl(a_mine, 16 * blk + r, 64); };   // alpha of token 16 blk + r
    auto gram = [&](int hi, int lo, f32x4& acc) {   // acc lane (r, g), element i: (K K^T)[16 hi + r][16 lo + 4g + i]
        const E* pa = sK + (16 * lo + r) * LD_DK + 4 * g;
        const E* pb = sK + (16 * hi + r) * LD_DK + 4 * g;
        quad qa[NKD], qb[NKD];
#pragma unroll
        for (int kd = 0; kd < NKD; ++kd) {
            qa[kd] = M::lds_quad(pa + 16 * kd);
            qb[kd] = M::lds_quad(pb + 16 * kd);
        }
        acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kd = 0; kd + 1 < NKD; kd += 2) M::mma2(acc, qa[kd], qa[kd + 1], qb[kd], qb[kd + 1]);
        if constexpr (NKD & 1) M::mma1(acc, qa[NKD - 1], qb[NKD - 1]);
    };
    // off-diagonal blocks of A: alpha_i k_i . k_j with i the row token
    static_for<NB>([&](auto hc) {
        constexpr int hi = decltype(hc)::value;
        static_for<hi>([&](auto lc) {
            constexpr int lo = decltype(lc)::value;
            constexpr int idx = hi * (hi - 1) / 2 + lo;
            if (idx % NW == w) {
                f32x4 acc;
                gram(hi, lo, acc);
                const float ar = alpha_of_row(hi);
                M::lds_store_quad(sA + (16 * hi + r) * LD_CE + 16 * lo + 4 * g, M::cvt(acc * ar));
            }
        });
    });
    // diagonal block w: strict lower part, stored transposed in fp32: At[16 w + m][i] = A[16 w + i][16 w + m]
    const int b0 = 16 * w;
    const float ar = alpha_of_row(w);
    {
        f32x4 acc;
        gram(w, w, acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) sAt[(b0 + 4 * g + i) * kLdAt + r] = (4 * g + i < r) ? ar * acc[i] : 0.0f;
    }
    // sAt rows were written by this wave just above; LDS operations of one wave complete in order
    __asm__ volatile("" ::: "memory");
    const float* at = sAt + b0 * kLdAt;
    f32x4 rows[15][4];
#pragma unroll
    for (int m = 0; m < 15; ++m) {
#pragma unroll
        for (int i4 = (m + 1) / 4; i4 < 4; ++i4) rows[m][i4] = *reinterpret_cast<const f32x4*>(at + m * kLdAt + 4 * i4);
    }
    float sv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) sv[i] = (i == r) ? 1.0f : 0.0f;
#pragma unroll
    for (int m = 0; m < 15; ++m) {
#pragma unroll
        for (int i = m + 1; i < 16; ++i) sv[i] -= rows[m][i / 4][i % 4] * sv[m];
    }
    // lane (r, g) writes T[b0 + 4g + e][b0 + r], e = 0..3 (row b0 + r of T^T) and the same scaled by alpha_{b0 + r}
    f32x4 mine;
#pragma unroll
    for (int e = 0; e < 4; ++e) mine[e] = g == 0 ? sv[e] : g == 1 ? sv[4 + e] : g == 2 ? sv[8 + e] : sv[12 + e];
    M::lds_store_quad(sTt + (b0 + r) * LD_CE + b0 + 4 * g, M::cvt(mine));
    M::lds_store_quad(sTat + (b0 + r) * LD_CE + b0 + 4 * g, M::cvt(mine * ar));
}

template <typename E, int DK, int C, bool VL>
__global__ __launch_bounds__(C / 16 * 64) void ut_kernel(const E* __restrict__ k, const float* __restrict__ beta,
                                                         E* __restrict__ tw, int L, int NC, int BH, int gate,
                                                         TokLayout ly) {
    typedef UtLayout<sizeof(E), DK, C> LY;
    typedef Mma<E> M;
    typedef typename M::quad quad;
    constexpr int NW = C / 16;
    constexpr int NT = NW * 64;
    constexpr int NB = C / 16;
    constexpr int LD_DK = LY::LD_DK, LD_CE = LY::LD_CE;
    typedef TileRegs<E, C, DK, NT> KT;

    __shared__ __attribute__((aligned(16))) unsigned char smem[LY::BYTES];
    E* sK = reinterpret_cast<E*>(smem + LY::OFF_K);
    E* sA = reinterpret_cast<E*>(smem + LY::OFF_A);
    float* sAt = reinterpret_cast<float*>(smem + LY::OFF_AT);
    E* sTt = reinterpret_cast<E*>(smem + LY::OFF_TT);
    E* sTat = reinterpret_cast<E*>(smem + LY::OFF_TAT);
    float* sLam = reinterpret_cast<float*>(smem + LY::OFF_LB);
    float* sBeta = sLam + C;
    float* sAlpha = reinterpret_cast<float*>(smem + LY::OFF_ALPHA);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15;
    const int g = lane >> 4;
    const int tr_ce = M::tr_offset(lane, LD_CE);

    // keys (16-byte vectors over the threads) and, for the thread holding the first vector of a key row,
    // that token's step; rows past the end of the sequence read as zero keys with zero step
    KT kt;
    float bt[KT::N];
    const int total = ut_chunks<VL>(ly, BH, NC);
    auto load = [&](int u) {
        int bh, c;
        chunk_of<VL>(ly, u, NC, bh, c);
        const SeqView sv = seq_view_t<VL>(ly, bh, L, C);
        const int t0 = c * C;
        const int n = (sv.len - t0 < C) ? (sv.len - t0) : C;
        const int ks = (int)ly.k_t, bs = (int)ly.be_t;
        kt.load(k + sv.k0 + (int64_t)t0 * ks, ks, n, tid);
        const __amdgpu_buffer_rsrc_t brs = buffer_rsrc(beta + sv.be0 + (int64_t)t0 * bs, n > 0 ? ((n - 1) * bs + 1) * 4 : 0);
#pragma unroll
        for (int it = 0; it < KT::N; ++it)
            bt[it] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(brs, ((it * NT + tid) / KT::VPR) * bs * 4, 0, 0));
    };
    int u = blockIdx.x;
    if (u < total) load(u);
    for (; u < total; u += gridDim.x) {
        // keys -> LDS; lambda = ||k||^2 reduced across the lanes holding one key row, and beta, per token
#pragma unroll
        for (int it = 0; it < KT::N; ++it) {
            const int idx = it * NT + tid;
            const float lam = group_sum<KT::VPR>(sum_sq(kt.x[it]));
            if ((C * KT::VPR) % NT == 0 || it + 1 < KT::N || idx < C * KT::VPR) {
                const int t = idx / KT::VPR;
                const int cv = idx % KT::VPR;
                lds_store_vec16(sK + t * LD_DK + cv * KT::VEC, kt.x[it]);
                if (cv == 0) {
                    sLam[t] = lam;
                    sBeta[t] = bt[it];
                }
            }
        }
        if (u + (int)gridDim.x < total) load(u + gridDim.x);
        __syncthreads();   // also: every wave is done with the previous pair's LDS
        ut_rows_balanced<E, DK, C, LD_DK, LD_CE>(sK, sLam, sBeta, sAlpha, sA, sAt, sTt, sTat, w, r, g, gate);
        __syncthreads();
        ut_offdiag<E, C, NW, LD_CE>(sA, sTt, sTat, sAlpha, w, r, g, tr_ce);
        __syncthreads();
        // export: the A-operand quads of Ta are the column quads of its stored transpose
        E* dst = tw + (int64_t)u * (TaShape<C>::NQ * TaShape<C>::QE) + lane * 4;
        static_for<NB>([&](auto rbc) {
            constexpr int rb = decltype(rbc)::value;
            static_for<rb + 1>([&](auto kbc) {
                constexpr int kb = decltype(kbc)::value;
                constexpr int qi = rb * (rb + 1) / 2 + kb;
                if (qi % NW == w) {
                    const quad x = M::lds_quad_t(sTat + 16 * kb * LD_CE + 16 * rb, LD_CE, tr_ce);
                    *reinterpret_cast<quad*>(dst + qi * TaShape<C>::QE) = x;
                }
            });
        });
    }
}

// ------------------------------------------------------------------------------------------------
// State-pass (chain) kernel
// ------------------------------------------------------------------------------------------------
template <int ESIZE, int DK, int C, int DVS>
struct ChainLayout {
    static constexpr int PAD = ESIZE == 2 ? 20 : 4;
    static constexpr int LD_DK = DK + PAD;   // sQ, sK [C][LD_DK]
    static constexpr int LD_V = DVS + PAD;   // sV     [C][LD_V]
    static constexpr int OFF_Q = 0;
    static constexpr int OFF_K = OFF_Q + C * LD_DK * ESIZE;
    static constexpr int OFF_V = OFF_K + C * LD_DK * ESIZE;
    static constexpr int BUF = OFF_V + C * LD_V * ESIZE;   // one buffer; two when they fit
    static constexpr int NBUF = 2 * BUF <= kMaxLdsBytes ? 2 : 1;
    static constexpr int BYTES = NBUF * BUF;
};

// LDS of the bf16 state pass for d_k >= 32 (three buffers of Q, K, V-slab and Ta tiles when they fit, else
// two; each tile rounded up to 1 KiB)
constexpr int chain_bf16_bytes(int dk, int c, int dvs) {
    const int buf = (2 * ((c * dk * 2 + 1023) / 1024) + (c * dvs * 2 + 1023) / 1024 +
                     ((c / 16) * (c / 16 + 1) / 2 * 512 + 1023) / 1024) * 1024;
    return (3 * buf <= kMaxLdsBytes ? 3 : 2) * buf + (3 * buf <= kMaxLdsBytes ? 0 : 1024);
}

// The bf16 state pass for d_k >= 32 (direct global -> LDS staging, swizzled tiles); defined in
// efla_chain_bf16.hpp, which the bf16 translation unit includes.
template <int DK, int C, int DVS>
hipError_t launch_chain_bf16(const SplitArgs& a, hipStream_t stream);

// host-side mirror of the state pass's LDS bytes
template <int ESIZE>
constexpr int chain_layout_bytes(int dk, int c, int dvs) {
    if (ESIZE == 2 && dk >= 32) return chain_bf16_bytes(dk, c, dvs);
    const int pad = ESIZE == 2 ? 20 : 4;
    const int buf = c * (2 * (dk + pad) + (dvs + pad)) * ESIZE;
    return 2 * buf <= kMaxLdsBytes ? 2 * buf : buf;
}

template <typename E, int DK, int C, int DVS>
__global__ __launch_bounds__(DVS / 16 * 64) void chain_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v, const E* __restrict__ tw,
    E* __restrict__ o, const float* s0, float* sf, int BH, int L, int DV, int nslab, ChainSeg sg, TokLayout ly) {
    typedef ChainLayout<sizeof(E), DK, C, DVS> LY;
    typedef Mma<E> M;
    typedef typename M::quad quad;
    constexpr int NW = DVS / 16;
    constexpr int NT = NW * 64;
    constexpr int NB = C / 16;
    constexpr int NKD = DK / 16;
    constexpr int NQ = TaShape<C>::NQ;
    constexpr int QE = TaShape<C>::QE;
    constexpr int LD_DK = LY::LD_DK, LD_V = LY::LD_V;
    constexpr bool DB = LY::NBUF == 2;
    static_assert(LY::BYTES <= kMaxLdsBytes, "chain kernel LDS too large");

    __shared__ __attribute__((aligned(16))) unsigned char smem[LY::BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15;
    const int g = lane >> 4;
    const int tr_dk = M::tr_offset(lane, LD_DK);
    const int tr_v = M::tr_offset(lane, LD_V);

    // Workgroup -> (batch*head, slab): the slabs of one head are 8 workgroups apart, i.e. on one XCD
    // (consecutive workgroups go to different XCDs), so they share that XCD's L2 for Q, K and Ta.
    const int bid = blockIdx.x;
    const int slab = (bid >> 3) % nslab;
    const int bh = ((bid >> 3) / nslab) * 8 + (bid & 7);
    if (bh >= BH) return;
    const int slab_col = slab * DVS;              // column of the state (value columns first, then transition)
    const bool trans = slab >= sg.nslab_v;        // transition slab: zero values, identity start, no outputs
    const int colw = slab_col + 16 * w;
    const SeqView sv = seq_view(ly, bh, L, C);     // this head's tokens: offsets, row strides, length
    const int len = sv.len;
    const int NC = (len + C - 1) / C;
    const int64_t qs = ly.q_t, ks = ly.k_t, vs = ly.v_t, os = ly.o_t;
    const int seg = blockIdx.y, nseg = gridDim.y;
    const int c0 = seg * sg.seg_chunks;           // this workgroup's chunks [c0, c1)
    const int c1 = NC < c0 + sg.seg_chunks ? NC : c0 + sg.seg_chunks;
    const bool write_o = o != nullptr && !trans;
    const E* twh = tw + (int64_t)sv.chunk0 * (NQ * QE) + lane * 4;

    auto sQ = [&](int b) { return reinterpret_cast<E*>(smem + b * LY::BUF + LY::OFF_Q); };
    auto sK = [&](int b) { return reinterpret_cast<E*>(smem + b * LY::BUF + LY::OFF_K); };
    auto sV = [&](int b) { return reinterpret_cast<E*>(smem + b * LY::BUF + LY::OFF_V); };

    TileRegs<E, C, DK, NT> rq, rk;
    TileRegs<E, C, DVS, NT> rv;
    auto load_stage = [&](int c) {
        const int t = c * C;
        const int n = (len - t < C) ? (len - t) : C;
        rq.load(q + sv.q0 + t * qs, (int)qs, n, tid);
        rk.load(k + sv.k0 + t * ks, (int)ks, n, tid);
        rv.load(v + sv.v0 + t * vs + slab_col, (int)vs, trans ? 0 : n, tid);
    };
    auto store_stage = [&](int b) {
        rq.store(sQ(b), LD_DK, tid);
        rk.store(sK(b), LD_DK, tid);
        rv.store(sV(b), LD_V, tid);
    };
    auto load_ta = [&](quad* dst, int c) {
        const E* p = twh + (int64_t)c * (NQ * QE);
#pragma unroll
        for (int i = 0; i < NQ; ++i) dst[i] = *reinterpret_cast<const quad*>(p + i * QE);
    };
    // this wave's piece of the state: S[16 rt + 4g + i][colw + r]
    f32x4 S[NKD];
#pragma unroll
    for (int rt = 0; rt < NKD; ++rt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * rt + 4 * g + i;
            S[rt][i] = trans ? (row == colw - DV + r ? 1.0f : 0.0f)
                             : s0 ? s0[(((int64_t)bh * nseg + seg) * DK + row) * DV + colw + r] : 0.0f;
        }
    }

    quad ta[NQ];
    if (c1 > c0) {
        load_ta(ta, c0);
        load_stage(c0);
        if constexpr (DB) {
            store_stage(0);
            load_stage(c0 + 1);
            __syncthreads();
        }
    }

    for (int c = c0; c < c1; ++c) {
        const int t0 = c * C;
        const int n = (len - t0 < C) ? (len - t0) : C;
        const int b = DB ? ((c - c0) & 1) : 0;
        if constexpr (DB) {
            // Straight-line on purpose (no branch for the last chunks): past the end of the sequence the
            // buffer ranges are empty, so chunk c+1's stage and chunk c+2's loads are zeros that nobody reads.
            store_stage(b ^ 1);
            load_stage(c + 2);
        } else {
            if (c > c0) __syncthreads();   // the previous chunk is done with the buffer
            store_stage(0);
            if (c + 1 < c1) load_stage(c + 1);
            __syncthreads();
        }
        const E* cQ = sQ(b);
        const E* cK = sK(b);
        const E* cV = sV(b);

        // Per row block rb of the chunk, from the same Q and K fragments: (Q S)^T, K S, R = V - K S, and block
        // row rb of lower_incl(Q K^T).  Every wave forms all of Q K^T itself: the fragments are in its
        // registers already, and the blocks come out as exactly the operand quads the O product takes.
        quad Sq[NKD];
#pragma unroll
        for (int rt = 0; rt < NKD; ++rt) Sq[rt] = M::cvt(S[rt]);
        // Ot accumulates O transposed: lane (r, g), element e = O[16 rb + r][colw + 4g + e]
        f32x4 Ot[NB];
        quad Rq[NB];
        quad kq[NB][NKD];          // K row quads: lane (r, g) holds K[16 rb + r][16 kd + 4g .. +3]
        quad Pq[NB * (NB + 1) / 2];   // P row quads: lane (r, g) holds P[16 hp + r][16 lo + 4g .. +3]
        static_for<NB>([&](auto rbc) {
            constexpr int rb = decltype(rbc)::value;
            quad qq[NKD];
            const E* pq = cQ + (16 * rb + r) * LD_DK + 4 * g;
            const E* pk = cK + (16 * rb + r) * LD_DK + 4 * g;
#pragma unroll
            for (int kd = 0; kd < NKD; ++kd) {
                qq[kd] = M::lds_quad(pq + 16 * kd);
                kq[rb][kd] = M::lds_quad(pk + 16 * kd);
            }
            f32x4 xk = {0.f, 0.f, 0.f, 0.f};
            Ot[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kd = 0; kd + 1 < NKD; kd += 2) {
                M::mma2(Ot[rb], Sq[kd], Sq[kd + 1], qq[kd], qq[kd + 1]);
                M::mma2(xk, kq[rb][kd], kq[rb][kd + 1], Sq[kd], Sq[kd + 1]);
            }
            if constexpr (NKD & 1) {
                M::mma1(Ot[rb], Sq[NKD - 1], qq[NKD - 1]);
                M::mma1(xk, kq[rb][NKD - 1], Sq[NKD - 1]);
            }
            // R: lane (r, g), element e: row 16 rb + 4g + e, column 16 w + r of the slab
            const quad vq = M::lds_quad_t(cV + 16 * rb * LD_V + 16 * w, LD_V, tr_v);
            f32x4 rr;
#pragma unroll
            for (int e = 0; e < 4; ++e) rr[e] = to_f32<E>(vq[e]) - xk[e];
            Rq[rb] = M::cvt(rr);
            // P block (rb, lo): acc lane (r, g), element e = (Q K^T)[16 rb + r][16 lo + 4g + e]
            static_for<rb + 1>([&](auto lc) {
                constexpr int lo = decltype(lc)::value;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kd = 0; kd + 1 < NKD; kd += 2) M::mma2(acc, kq[lo][kd], kq[lo][kd + 1], qq[kd], qq[kd + 1]);
                if constexpr (NKD & 1) M::mma1(acc, kq[lo][NKD - 1], qq[NKD - 1]);
                if constexpr (lo == rb) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[e] = (4 * g + e <= r) ? acc[e] : 0.0f;
                }
                Pq[rb * (rb + 1) / 2 + lo] = M::cvt(acc);
            });
        });
        // Delta = T diag(alpha) R, block-lower-triangular product
        quad Dq[NB];
        static_for<NB>([&](auto rbc) {
            constexpr int rb = decltype(rbc)::value;
            constexpr int q0 = rb * (rb + 1) / 2;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            static_for<(rb + 1) / 2>([&](auto hc) {
                constexpr int kb = 2 * decltype(hc)::value;
                M::mma2(acc, ta[q0 + kb], ta[q0 + kb + 1], Rq[kb], Rq[kb + 1]);
            });
            if constexpr ((rb + 1) & 1) M::mma1(acc, ta[q0 + rb], Rq[rb]);
            Dq[rb] = M::cvt(acc);
        });
        // the next chunk's T diag(alpha) operands go into the registers just consumed: a whole iteration
        // covers their latency (the last chunk reloads its own, unused)
        load_ta(ta, c + 1 < c1 ? c + 1 : c);
        // O^T = (Q S)^T + Delta^T lower_incl(Q K^T)^T; four consecutive outputs of one token per lane, stored
        // through a buffer resource that ends at the chunk's last valid row
        const __amdgpu_buffer_rsrc_t ors =
            buffer_rsrc(o + sv.o0 + t0 * os + colw, write_o ? ((n - 1) * (int)os + 16) * (int)sizeof(E) : 0);
        static_for<NB>([&](auto rbc) {
            constexpr int rb = decltype(rbc)::value;
            constexpr int p0 = rb * (rb + 1) / 2;
            static_for<(rb + 1) / 2>([&](auto hc) {
                constexpr int kb = 2 * decltype(hc)::value;
                M::mma2(Ot[rb], Dq[kb], Dq[kb + 1], Pq[p0 + kb], Pq[p0 + kb + 1]);
            });
            if constexpr ((rb + 1) & 1) M::mma1(Ot[rb], Dq[rb], Pq[p0 + rb]);
            buffer_store<quad>(ors, ((16 * rb + r) * (int)os + 4 * g) * (int)sizeof(E), M::cvt(Ot[rb]));
        });
        // S += K^T Delta (K^T blocks fetched down the columns of K)
#pragma unroll
        for (int rt = 0; rt < NKD; ++rt) {
            const E* pk = cK + 16 * rt;
#pragma unroll
            for (int kb = 0; kb + 1 < NB; kb += 2)
                M::mma2(S[rt], M::lds_quad_t(pk + 16 * kb * LD_DK, LD_DK, tr_dk),
                        M::lds_quad_t(pk + 16 * (kb + 1) * LD_DK, LD_DK, tr_dk), Dq[kb], Dq[kb + 1]);
            if constexpr (NB & 1) M::mma1(S[rt], M::lds_quad_t(pk + 16 * (NB - 1) * LD_DK, LD_DK, tr_dk), Dq[NB - 1]);
        }
        if constexpr (DB) __syncthreads();   // buffer b is free and chunk c+1's stage is in LDS
    }

    if (sf && (sg.sf_all || seg == nseg - 1)) {
        const int64_t base = sg.sf_all ? (int64_t)bh * nseg + seg : bh;
        const int ld = sg.sf_all ? sg.ld_sf : DV;
#pragma unroll
        for (int rt = 0; rt < NKD; ++rt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) sf[(base * DK + 16 * rt + 4 * g + i) * ld + colw + r] = S[rt][i];
        }
    }
}

// ------------------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------------------
// diag32: only the diagonal 32 x 32 blocks of every 64-token chunk's Ta are needed (the bf16 state pass
// reads no other); the wave kernel then skips the rest (other kernels form the whole transform regardless)
// tt (bf16 with d_k >= 32 only, not with diag32): also T^T of every chunk, row-major C x C (the backward pass)
template <typename E, int DK, int C, bool VL>
hipError_t launch_ut_vl(const void* k, const float* beta, void* tw, int BH, int L, int gate, const TokLayout& ly,
                        bool diag32, hipStream_t stream, void* tt = nullptr) {
    static_assert(UtLayout<sizeof(E), DK, C>::BYTES <= kMaxLdsBytes, "UT kernel LDS too large");
    const int NC = (L + C - 1) / C;
    // chunks of the workspace (with packed sequences an upper bound; the kernel reads the exact count)
    const int64_t total = VL ? (int64_t)ly.H * (NC + ly.nseq) : (int64_t)BH * NC;
    if (total == 0) return hipSuccess;
    if constexpr (std::is_same<E, bf16>::value && DK >= 32) {
        // one wave per (batch*head, chunk) at a time; as many waves as the device holds at once
        constexpr int WPB = UtWaveShape<DK, C>::WPB;
        constexpr bool CAN_DG = C == 64;
        const bool dg = CAN_DG && diag32;
        const void* kfn = dg ? reinterpret_cast<const void*>(&ut_wave_kernel<DK, C, VL, CAN_DG>)
                             : reinterpret_cast<const void*>(&ut_wave_kernel<DK, C, VL, false>);
        int dev = 0, cus = 0, per_cu = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kfn, WPB * 64, 0);
        if (e != hipSuccess) return e;
        const int64_t resident = (int64_t)(cus < 1 ? 1 : cus) * (per_cu < 1 ? 1 : per_cu);
        const int64_t need = (total + WPB - 1) / WPB;
        const dim3 grid((unsigned)(need < resident ? need : resident));
        if (dg)
            hipLaunchKernelGGL((ut_wave_kernel<DK, C, VL, CAN_DG>), grid, dim3(WPB * 64), 0, stream,
                               static_cast<const bf16*>(k), beta, static_cast<bf16*>(tw), L, NC, BH, gate, ly, nullptr);
        else
            hipLaunchKernelGGL((ut_wave_kernel<DK, C, VL, false>), grid, dim3(WPB * 64), 0, stream,
                               static_cast<const bf16*>(k), beta, static_cast<bf16*>(tw), L, NC, BH, gate, ly,
                               static_cast<bf16*>(tt));
        return hipGetLastError();
    }
    // as many workgroups as the device holds at once, each walking several pairs
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(&ut_kernel<E, DK, C, VL>),
                                                          C / 16 * 64, 0);
    if (e != hipSuccess) return e;
    const int64_t resident = (int64_t)(cus < 1 ? 1 : cus) * (per_cu < 1 ? 1 : per_cu);
    const int64_t grid = total < resident ? total : resident;
    hipLaunchKernelGGL((ut_kernel<E, DK, C, VL>), dim3((unsigned)grid), dim3(C / 16 * 64), 0, stream,
                       static_cast<const E*>(k), beta, static_cast<E*>(tw), L, NC, BH, gate, ly);
    return hipGetLastError();
}

template <typename E, int DK, int C>
hipError_t launch_ut_t(const void* k, const float* beta, void* tw, int BH, int L, int gate, const TokLayout* lyp,
                       hipStream_t stream, bool diag32 = false, void* tt = nullptr) {
    const TokLayout ly = lyp ? *lyp : contiguous_layout(1, L, DK, DK);   // contiguous: every (batch, head) is a "batch"
    return ly.cu_seqlens ? launch_ut_vl<E, DK, C, true>(k, beta, tw, BH, L, gate, ly, diag32, stream, tt)
                         : launch_ut_vl<E, DK, C, false>(k, beta, tw, BH, L, gate, ly, diag32, stream, tt);
}

template <typename E, int DK, int C, int DVS>
hipError_t launch_chain_t(const SplitArgs& a, hipStream_t stream) {
    if constexpr (std::is_same<E, bf16>::value && DK >= 32) {
        return launch_chain_bf16<DK, C, DVS>(a, stream);
    } else if constexpr (ChainLayout<sizeof(E), DK, C, DVS>::BYTES > kMaxLdsBytes) {
        return hipErrorInvalidConfiguration;
    } else {
        const ChainSeg sg = chain_seg(a, DK, C, DVS);
        const TokLayout ly = a.layout ? *a.layout : contiguous_layout(1, a.L, DK, a.d_v);
        const int nslab = (a.d_v + (a.aug ? DK : 0)) / DVS;
        const int64_t grid = (int64_t)((a.BH + 7) / 8) * 8 * nslab;
        hipLaunchKernelGGL((chain_kernel<E, DK, C, DVS>), dim3((unsigned)grid, (unsigned)(a.nseg > 0 ? a.nseg : 1)),
                           dim3(DVS / 16 * 64), 0, stream, static_cast<const E*>(a.q), static_cast<const E*>(a.k),
                           static_cast<const E*>(a.v), static_cast<const E*>(a.tw), static_cast<E*>(a.o), a.s0, a.sf,
                           a.BH, a.L, a.d_v, nslab, sg, ly);
        return hipGetLastError();
    }
}

template <typename E, int DK, int C>
hipError_t launch_split_c(const SplitArgs& a, bool with_ut, hipStream_t s) {
    if (with_ut && a.L > 0) {
        // the bf16 state pass (d_k >= 32) steps 64-token chunks in 32-token halves and reads only the
        // diagonal 32 x 32 blocks of Ta
        constexpr bool diag32 = std::is_same<E, bf16>::value && DK >= 32 && C == 64;
        const hipError_t e = launch_ut_t<E, DK, C>(a.k, a.beta, a.tw, a.BH, a.L, a.gate, a.layout, s, diag32);
        if (e != hipSuccess) return e;
    }
    switch (a.dvs) {
        case 16: return launch_chain_t<E, DK, C, 16>(a, s);
        case 32: return launch_chain_t<E, DK, C, 32>(a, s);
        case 64: return launch_chain_t<E, DK, C, 64>(a, s);
        case 128:
            // the first pass of the segment-parallel forward at d_k 128 (bf16, 64-token chunks, no outputs)
            if constexpr (std::is_same<E, bf16>::value && DK == 128 && C == 64) return launch_chain_t<E, DK, C, 128>(a, s);
            break;
    }
    return hipErrorInvalidValue;
}

template <typename E, int DK>
hipError_t launch_split_dk(const SplitArgs& a, bool with_ut, hipStream_t s) {
    switch (a.chunk) {
        case 16: return launch_split_c<E, DK, 16>(a, with_ut, s);
        case 32: return launch_split_c<E, DK, 32>(a, with_ut, s);
        case 64: return launch_split_c<E, DK, 64>(a, with_ut, s);
    }
    return hipErrorInvalidValue;
}

// with_ut: run the UT launch into a.tw first; otherwise a.tw already holds it
template <typename E>
hipError_t launch_split_e(const SplitArgs& a, bool with_ut, hipStream_t s) {
    switch (a.d_k) {
        case 16: return launch_split_dk<E, 16>(a, with_ut, s);
        case 32: return launch_split_dk<E, 32>(a, with_ut, s);
        case 64: return launch_split_dk<E, 64>(a, with_ut, s);
        case 128: return launch_split_dk<E, 128>(a, with_ut, s);
    }
    return hipErrorInvalidValue;
}

template <typename E, int DK>
hipError_t launch_ut_dk(const void* k, const float* beta, void* tw, int BH, int L, int chunk, int gate, hipStream_t s,
                        void* tt, const TokLayout* ly) {
    switch (chunk) {
        case 16: return launch_ut_t<E, DK, 16>(k, beta, tw, BH, L, gate, ly, s, false, tt);
        case 32: return launch_ut_t<E, DK, 32>(k, beta, tw, BH, L, gate, ly, s, false, tt);
        case 64: return launch_ut_t<E, DK, 64>(k, beta, tw, BH, L, gate, ly, s, false, tt);
    }
    return hipErrorInvalidValue;
}

template <typename E>
hipError_t launch_ut_e(const void* k, const float* beta, void* tw, int BH, int L, int d_k, int chunk, int gate,
                       hipStream_t s, void* tt = nullptr, const TokLayout* ly = nullptr) {
    switch (d_k) {
        case 16: return launch_ut_dk<E, 16>(k, beta, tw, BH, L, chunk, gate, s, tt, ly);
        case 32: return launch_ut_dk<E, 32>(k, beta, tw, BH, L, chunk, gate, s, tt, ly);
        case 64: return launch_ut_dk<E, 64>(k, beta, tw, BH, L, chunk, gate, s, tt, ly);
        case 128: return launch_ut_dk<E, 128>(k, beta, tw, BH, L, chunk, gate, s, tt, ly);
    }
    return hipErrorInvalidValue;
}

}  // namespace efla
