// efla_common.hpp -- shared device helpers of the EFLA HIP kernels (gfx950 / CDNA4).
//
// Matrix-core conventions used by every kernel here (16x16 output tiles, 64-wide wavefront):
//   lane = 16*g + r with r = lane & 15, g = lane >> 4.
//   An A operand fragment of a 16x16 block (rows m, reduction index k) is a "quad": lane (r, g)
//   holds A[r][4g .. 4g+3].  A B operand fragment (rows k, columns n) is a quad too: lane (r, g)
//   holds B[4g .. 4g+3][r].  The 16x16 fp32 accumulator D has lane (r, g) holding D[4g+i][r],
//   i = 0..3 -- i.e. an accumulator tile is already a B-operand quad of the same matrix.
// The matrix instructions reduce over whatever k each (lane group, slot) carries, as long as the
// A and B fragments agree, so two quads (two 16-wide k blocks) feed one 16x16x32 bf16 instruction,
// a single quad goes through 16x16x32 with a zero second half, and one fp32 quad feeds four 16x16x4
// fp32 instructions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace efla {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef s16x4 __attribute__((address_space(3))) lds_s16x4;

constexpr int kMaxLdsBytes = 160 * 1024;   // LDS of one gfx950 compute unit

// ------------------------------------------------------------------------------------------------
// Buffer resources (CDNA raw buffers: stride 0, byte-granular range check).  A load whose offset
// falls outside [0, bytes) returns zeros and such a store is dropped by the address unit, so a
// ragged tail needs neither a branch nor an exec mask, and the compiler can count outstanding
// memory operations exactly.  Third descriptor word as for every gfx9-family part.
// ------------------------------------------------------------------------------------------------
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
template <typename V>
__device__ __forceinline__ V buffer_load(__amdgpu_buffer_rsrc_t rs, int byte_off) {
    static_assert(sizeof(V) == 16 || sizeof(V) == 8, "8- or 16-byte vectors");
    if constexpr (sizeof(V) == 16) {
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off, 0, 0));
    } else {
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b64(rs, byte_off, 0, 0));
    }
}
template <typename V>
__device__ __forceinline__ void buffer_store(__amdgpu_buffer_rsrc_t rs, int byte_off, V x) {
    static_assert(sizeof(V) == 16 || sizeof(V) == 8, "8- or 16-byte vectors");
    if constexpr (sizeof(V) == 16) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), rs, byte_off, 0, 0);
    } else {
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, x), rs, byte_off, 0, 0);
    }
}

// ------------------------------------------------------------------------------------------------
// The exact gate.  alpha = (1 - e^{-beta lambda}) / lambda, evaluated as -expm1(-x)/lambda with
// x = beta*lambda so that small x does not cancel; x == 0 (lambda == 0 or beta == 0) gives the
// limit beta.  Large x: expm1 -> -1 and alpha -> 1/lambda.
// ("Exact Flow Linear Attention", Metodologia item 3; "Error-Free Linear Attention is a Free
// Lunch", Step 1.)
// ------------------------------------------------------------------------------------------------
__device__ __forceinline__ float exact_alpha(float beta, float lambda) {
    const float x = beta * lambda;
    if (x == 0.0f) return beta;
    return -expm1f(-x) / lambda;
}

// The coefficient of the update for one of the integrators of the same dynamics dS/dt = -k k^T S + k v^T
// over a step beta ("Error-Free Linear Attention guida completa" (mauroscia.it), the section on RK-infinity:
// Euler and Runge-Kutta steps of rising order approach the exact flow; "Error-Free Linear Attention is a
// Free Lunch" (howistudyai.com), building blocks "Delta Rule" and "Runge-Kutta Methods").
//   gate == 0: the exact flow, exact_alpha above.
//   gate == p in 1 .. kMaxGate: a p-th order Runge-Kutta step, whose update keeps the same rank-1 form
//     (the p-th degree Taylor polynomial of e^{-beta k k^T}, with (k k^T)^n = lambda^{n-1} k k^T) with
//     alpha_p = beta sum_{n=0}^{p-1} (-beta lambda)^n / (n+1)!   -- p = 1 is the delta rule's alpha = beta.
// Horner's scheme in fp32.
constexpr int kMaxGate = 16;
__device__ __forceinline__ float gate_alpha(float beta, float lambda, int gate) {
    if (gate == 0) return exact_alpha(beta, lambda);
    const float mx = -beta * lambda;
    float s = 1.0f;
    for (int n = gate - 1; n >= 1; --n) s = 1.0f + s * mx / (float)(n + 1);
    return beta * s;
}

// Derivatives of the gate for the backward pass: *da_db = d alpha / d beta, *da_dl = d alpha / d lambda.
// Writing alpha = beta phi(y), y = beta lambda:  d/dbeta = phi(y) + y phi'(y),  d/dlambda = beta^2 phi'(y).
//   gate 0: phi(y) = (1 - e^{-y}) / y, so d/dbeta = e^{-y} and phi'(y) = (y e^{-y} - (1 - e^{-y})) / y^2,
//           taken from its series sum_{n>=0} (-1)^{n+1} (n+1)/(n+2)! y^n below y = 1/2 (the closed form
//           cancels there), phi'(0) = -1/2.
//   gate p: phi(y) = sum_{n=0}^{p-1} (-y)^n / (n+1)!, differentiated term by term.
__device__ __forceinline__ void gate_alpha_grad(float beta, float lambda, int gate, float* da_db, float* da_dl) {
    const float y = beta * lambda;
    float dphi;
    if (gate == 0) {
        *da_db = expf(-y);
        if (y < 0.5f) {
            // Horner over n = 10 .. 0 of c_n y^n, c_n = (-1)^{n+1} (n+1) / (n+2)!
            float f = 1.0f;   // 1/(n+2)!, built for n = 10 first
            for (int m = 3; m <= 12; ++m) f /= (float)m;   // 1/12! * 2
            f *= 0.5f;
            float acc = 0.0f;
            for (int n = 10; n >= 0; --n) {
                const float c = ((n & 1) ? 1.0f : -1.0f) * (float)(n + 1) * f;
                acc = acc * y + c;
                f *= (float)(n + 2);   // 1/(n+1)!
            }
            dphi = acc;
        } else {
            dphi = (y * expf(-y) + expm1f(-y)) / (y * y);
        }
    } else {
        float phi = 0.0f, d = 0.0f, yn = 1.0f, fact = 1.0f;   // y^n, (n+1)!
        for (int n = 0; n < gate; ++n) {
            fact *= (float)(n + 1);
            const float sgn = (n & 1) ? -1.0f : 1.0f;
            phi += sgn * yn / fact;
            if (n + 1 < gate) d += -sgn * (float)(n + 1) * yn / (fact * (float)(n + 2));   // term n+1
            yn *= y;
        }
        dphi = d;
        *da_db = phi + y * dphi;
    }
    *da_dl = beta * beta * dphi;
}

// ------------------------------------------------------------------------------------------------
// element conversion
// ------------------------------------------------------------------------------------------------
template <typename E> __device__ __forceinline__ float to_f32(E x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<bf16>(bf16 x) { return (float)x; }

template <typename E> __device__ __forceinline__ E from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE

// 16-byte vector of storage elements (8 bf16 or 4 fp32)
template <typename E> struct Vec16;
template <> struct Vec16<float> { typedef f32x4 type; static constexpr int N = 4; };
template <> struct Vec16<bf16> { typedef bf16x8 type; static constexpr int N = 8; };

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// sum of squares of a 16-byte vector, accumulated in fp32 (bf16 products are exact in fp32)
__device__ __forceinline__ float sum_sq(f32x4 x) { return x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3]; }
__device__ __forceinline__ float sum_sq(bf16x8 x) {
    float s = 0.0f;
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1), __builtin_shufflevector(x, x, 0, 1), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3), __builtin_shufflevector(x, x, 2, 3), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5), __builtin_shufflevector(x, x, 4, 5), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7), __builtin_shufflevector(x, x, 6, 7), s, false);
    return s;
}

// store a 16-byte vector to an LDS address that is only 8-byte aligned (two 8-byte halves)
__device__ __forceinline__ void lds_store_vec16(float* p, f32x4 x) { *reinterpret_cast<f32x4*>(p) = x; }
__device__ __forceinline__ void lds_store_vec16(bf16* p, bf16x8 x) {
    *reinterpret_cast<bf16x4*>(p) = __builtin_shufflevector(x, x, 0, 1, 2, 3);
    *reinterpret_cast<bf16x4*>(p + 4) = __builtin_shufflevector(x, x, 4, 5, 6, 7);
}

// ------------------------------------------------------------------------------------------------
// matrix-core policy per operand type
// ------------------------------------------------------------------------------------------------
template <typename E> struct Mma;

template <> struct Mma<bf16> {
    typedef bf16x4 quad;
    static __device__ __forceinline__ quad cvt(f32x4 v) {
        quad q;
        q[0] = (bf16)v[0]; q[1] = (bf16)v[1]; q[2] = (bf16)v[2]; q[3] = (bf16)v[3];
        return q;
    }
    static __device__ __forceinline__ quad cvt_neg(f32x4 v) { return cvt(-v); }
    static __device__ __forceinline__ quad zero() { return cvt(f32x4{0.f, 0.f, 0.f, 0.f}); }
    // acc += [A0 A1](16 x 32) * [B0; B1](32 x 16)
    static __device__ __forceinline__ void mma2(f32x4& acc, quad a0, quad a1, quad b0, quad b1) {
        bf16x8 a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
        bf16x8 b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
    // acc += A(16 x 16) * B(16 x 16), issued as 16x16x32 with a zero upper k half.  Every accumulator
    // chain stays on the one instruction shape: a 16x16x16 bf16 instruction reading, as its C operand,
    // the result of a 16x16x32 bf16 instruction a few cycles earlier gave wrong sums with this
    // toolchain (the generated code left too few wait states between the two shapes).
    static __device__ __forceinline__ void mma1(f32x4& acc, quad a, quad b) { mma2(acc, a, zero(), b, zero()); }
    static __device__ __forceinline__ quad lds_quad(const bf16* p) {  // 8-byte aligned
        return *reinterpret_cast<const quad*>(p);
    }
    static __device__ __forceinline__ void lds_store_quad(bf16* p, quad q) { *reinterpret_cast<quad*>(p) = q; }
    // Column quad of a row-major 16x16 LDS block X (leading dimension ld): lane (r, g) receives
    // X[4g .. 4g+3][r].  One transposing LDS read: within each 16-lane group, lane i gets element i%4
    // of the 8-byte runs addressed by lanes 4e + i/4 (e = 0..3), so lane 16g + 4e + c points at
    // X[4g + e][4c .. 4c+3].  The per-lane offset (4g + e) * ld + 4c comes from tr_offset().
    static __device__ __forceinline__ int tr_offset(int lane, int ld) {
        const int j = lane & 15;
        return (4 * (lane >> 4) + (j >> 2)) * ld + 4 * (j & 3);
    }
    static __device__ __forceinline__ quad lds_quad_t(const bf16* X, int ld, int tr_off) {
        (void)ld;
        const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(X + tr_off));
        return __builtin_bit_cast(quad, v);
    }
};

template <> struct Mma<float> {
    typedef f32x4 quad;
    static __device__ __forceinline__ quad cvt(f32x4 v) { return v; }
    static __device__ __forceinline__ quad cvt_neg(f32x4 v) { return -v; }
    static __device__ __forceinline__ quad zero() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
    static __device__ __forceinline__ void mma1(f32x4& acc, quad a, quad b) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
    }
    static __device__ __forceinline__ void mma2(f32x4& acc, quad a0, quad a1, quad b0, quad b1) {
        mma1(acc, a0, b0);
        mma1(acc, a1, b1);
    }
    static __device__ __forceinline__ quad lds_quad(const float* p) {  // 16-byte aligned
        return *reinterpret_cast<const quad*>(p);
    }
    static __device__ __forceinline__ void lds_store_quad(float* p, quad q) { *reinterpret_cast<quad*>(p) = q; }
    // Column quad of a row-major 16x16 LDS block X: lane (r, g) receives X[4g .. 4g+3][r] (four reads).
    static __device__ __forceinline__ int tr_offset(int lane, int ld) { return 4 * (lane >> 4) * ld + (lane & 15); }
    static __device__ __forceinline__ quad lds_quad_t(const float* X, int ld, int tr_off) {
        const float* p = X + tr_off;
        return quad{p[0], p[ld], p[2 * ld], p[3 * ld]};
    }
};

// x from another lane of the same 16-lane row, through a DPP lane move (no LDS traffic)
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// gfx950 row swaps between the 16-lane rows of a wave (v_permlane16_swap / v_permlane32_swap, vector ALU, no
// LDS), both operands x.  row_swap16: `even` holds, in rows 0..3, rows 0, 0, 2, 2 of x and `odd` rows 1, 1, 3, 3.
// row_swap32: `lo` holds rows 0, 1, 0, 1 and `hi` rows 2, 3, 2, 3.  Every lane of the wave must be active.
// The two results leave the builtin's vector by value (__uint_as_float): a bit cast of a subscripted element of a
// vector lvalue reads element 0 in this compiler.
__device__ __forceinline__ void row_swap16(float x, float& even, float& odd) {
    const unsigned u = __float_as_uint(x);
    const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    even = __uint_as_float(p[0]);
    odd = __uint_as_float(p[1]);
}
__device__ __forceinline__ void row_swap32(float x, float& lo, float& hi) {
    const unsigned u = __float_as_uint(x);
    const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    lo = __uint_as_float(p[0]);
    hi = __uint_as_float(p[1]);
}
// Sum of the four lanes r, 16 + r, 32 + r, 48 + r, on each of them: (x0 + x1) + (x2 + x3), as a butterfly
// over lane distances 16 and 32 pairs them.
__device__ __forceinline__ float cross_row_sum(float x) {
    float a, b;
    row_swap16(x, a, b);
    row_swap32(a + b, a, b);
    return a + b;
}
// out[i] = x of lane 16 i + r, on every lane of column r.
__device__ __forceinline__ void rows_bcast4(float x, float out[4]) {
    float e, o;
    row_swap16(x, e, o);
    row_swap32(e, out[0], out[2]);
    row_swap32(o, out[1], out[3]);
}

// f(integral_constant<int, i>) for i = 0 .. N - 1, unrolled at compile time
template <int I, int N, class F>
__device__ __forceinline__ void static_for_impl(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for_impl<I + 1, N>(f);
    }
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl<0, N>(f);
}

// x -= (a of lane M of this lane's 16-lane row) * y: v_fmac_f32 with the row_newbcast:M data-parallel modifier
// and a negated broadcast operand (the compiler folds row broadcasts into adds but not into multiply-adds).  A DPP
// instruction may not read a VGPR that a vector instruction wrote in the two instructions before it; NOP leads with
// those two wait states.  Vector ALU only.
template <int M, bool NOP>
__device__ __forceinline__ void fmac_row_bcast_neg(float& x, float a, float y) {
    static_assert(M >= 0 && M < 16, "lane of a 16-lane row");
    if constexpr (NOP)
        asm volatile("s_nop 1\n\tv_fmac_f32_dpp %0, -%1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
                     : "+v"(x) : "v"(a), "v"(y), "i"(M));
    else
        asm volatile("v_fmac_f32_dpp %0, -%1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
                     : "+v"(x) : "v"(a), "v"(y), "i"(M));
}

// Steps m = M0 .. M1 - 1 of the right-looking forward substitution for one column of (I + A)^-1, A strictly lower
// 16 x 16: step m subtracts A[i][m] x[m] from x[i] for every i > m.  Each 16-lane row of the wave solves its own
// block; lane m of the row holds column m of that block (acol[i] = A[i][m], zero for i <= m) and lane r column r of
// the inverse in x (x = e_r before step 0).  Step m takes A[i][m] from lane m by row broadcast, so no lane reads the
// block from memory.  The first multiply-add of a step leads with the wait states (it reads x[m], written by the
// step before), and so does every one of the first step, whose x registers the compiler may have just set.
template <int M0, int M1>
__device__ __forceinline__ void tri_solve_row_bcast(const float* acol, float* x) {
    static_assert(M0 >= 0 && M0 <= M1 && M1 <= 15, "substitution steps of a 16 x 16 block");
    static_for<M1 - M0>([&](auto mc) {
        constexpr int m = M0 + decltype(mc)::value;
        static_for<15 - m>([&](auto jc) {
            constexpr int i = m + 1 + decltype(jc)::value;
            fmac_row_bcast_neg<m, i == m + 1 || m == M0>(x[i], acol[i], x[m]);
        });
    });
}

// Sum over aligned groups of WIDTH consecutive lanes (WIDTH a power of two <= 64); every lane of a
// group receives the group's sum.  Within a 16-lane row the partners come from DPP moves: swap
// neighbours (quad_perm 1,0,3,2), swap pairs (quad_perm 2,3,0,1), mirror each half row, mirror the
// row; wider groups add the row swaps.
template <int WIDTH>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (WIDTH >= 2) x += dpp_mov<0xB1>(x);
    if constexpr (WIDTH >= 4) x += dpp_mov<0x4E>(x);
    if constexpr (WIDTH >= 8) x += dpp_mov<0x141>(x);
    if constexpr (WIDTH >= 16) x += dpp_mov<0x140>(x);
    if constexpr (WIDTH >= 32) {
        float e, o;
        row_swap16(x, e, o);
        x = e + o;
    }
    if constexpr (WIDTH >= 64) {
        float lo, hi;
        row_swap32(x, lo, hi);
        x = lo + hi;
    }
    return x;
}

}  // namespace efla
